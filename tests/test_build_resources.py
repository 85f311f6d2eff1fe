"""Register placement of the built kernels (the spill marks of Fig. 12).

The build records the compiler's per-kernel resource usage next to the
library.  The walk kernels of every Markov configuration and of the int8
recurrent head up to batch bucket 8 must not spill: a spill would move W
tiles or working values that the residency plan keeps in registers into
scratch memory.  That includes the whole-shard bf16 kernels of one and two
batch rows (11 register tiles of 8 KiB per wave); at four rows they spill a
few registers.  (Known exceptions: the recurrent head with bf16 W
at B >= 4 streams 8 KiB tiles through a 256-register wave, and the int8
recurrent head at B = 16 with T = 1; the log-normaliser variants may spill a
few registers.)
"""
import json
import os

import pytest

RES = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "serial_draft_head_persistent_amd", "libwts.resources.json")


def _load():
    if not os.path.exists(RES):
        pytest.skip("library not built (python -m serial_draft_head_persistent_amd.build)")
    with open(RES) as fh:
        return json.load(fh)


def _args(label):
    return [a.strip() for a in label.partition("<")[2].rstrip(">").split(",")]


def test_every_kernel_variant_is_recorded():
    r = _load()
    walks = [k for k in r if k.startswith("walk_kernel<")]
    steps = [k for k in r if k.startswith("step_kernel<")]
    # wtype x bucket x head x T x lse, plus the whole-shard bf16 Markov kernels
    # (buckets 1, 2, 4 x T x lse); and wtype x bucket x T x lse
    assert len(walks) == 2 * 5 * 2 * 2 * 2 + 3 * 4 and len(steps) == 2 * 5 * 2 * 2
    for k in walks + steps:
        assert {"vgpr", "agpr", "scratch", "vgpr_spill"} <= set(r[k]), k


def test_walk_kernels_do_not_spill():
    r = _load()
    bad = []
    for k, v in r.items():
        if not k.startswith(("walk_kernel<", "step_kernel<")):
            continue
        a = _args(k)
        if k.startswith("walk_kernel<"):
            wt, bb, head, temp, lse, whole = int(a[0]), int(a[1]), int(a[2]), int(a[3]), a[4] == "true", \
                a[5] == "true"
            if lse or (head == 1 and (wt == 1 or bb == 16)):
                continue
            if whole and bb == 4:   # 11 register tiles of 8 KiB and four batch rows: a few spills
                assert v["vgpr_spill"] <= 16, (k, v)
                continue
        if v["vgpr_spill"] != 0 or v["scratch"] != 0:
            bad.append((k, v["vgpr_spill"], v["scratch"]))
    assert not bad, bad


def test_headline_kernel_keeps_two_waves_per_simd():
    # int8 walks run 8 waves per workgroup (two per SIMD), so each may use at most 256 VGPRs
    r = _load()
    for bb in (1, 2, 4, 8, 16):
        v = r[f"walk_kernel<0, {bb}, 0, 0, false, false>"]
        assert v["vgpr"] + v["agpr"] <= 256 and v["occupancy"] >= 2, (bb, v)
