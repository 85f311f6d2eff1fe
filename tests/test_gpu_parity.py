"""GPU parity: the HIP walk (through the C ABI) against the CPU oracle.

int8 W: tokens and bf16 logits bit-identical.  Every execution mode and
residency split must give the same bits.
"""
import numpy as np
import pytest

import datagen
from gpu_helpers import make_head, run, oracle_walk, assert_exact
from conftest import cached_inputs

pytestmark = pytest.mark.gpu


def _print_case(**kw):
    print("CASE", " ".join(f"{k}={v}" for k, v in kw.items()), flush=True)


@pytest.mark.parametrize("exec_", ["resident", "stream", "stepwise"])
def test_config0_exact(exec_):
    d = cached_inputs(0)
    _print_case(cfg=0, exec=exec_)
    h, t = make_head(d)
    got = run(h, t, exec=exec_)
    assert_exact(got, oracle_walk(d), f"config0 {exec_}")
    h.close()


@pytest.mark.parametrize("V", [12, 17, 4099])
@pytest.mark.parametrize("B", [1, 3])
@pytest.mark.parametrize("T", [0, 1])
def test_ragged_vocab_exact(V, B, T):
    d = datagen.make_inputs(V, 256, B, 5, seed=V + B)
    _print_case(V=V, B=B, T=T)
    h, t = make_head(d)
    ref = oracle_walk(d, temperature=T, seed=7)
    for ex in ("resident", "stream", "stepwise"):
        assert_exact(run(h, t, exec=ex, temperature=T, seed=7), ref, f"V={V} B={B} T={T} {ex}")
    h.close()


@pytest.mark.parametrize("B", [1, 2, 3, 4, 5, 8, 11, 16])
@pytest.mark.parametrize("T", [0, 1])
def test_batch_buckets_exact(B, T):
    d = datagen.make_inputs(20000, 256, B, 6, seed=100 + B)
    _print_case(V=20000, B=B, T=T)
    h, t = make_head(d)
    ref = oracle_walk(d, temperature=T, seed=3, step_offset=2)
    assert_exact(run(h, t, temperature=T, seed=3, step_offset=2), ref, f"B={B} T={T}")
    h.close()


def test_config1_full_size_exact():
    d = cached_inputs(1)
    _print_case(cfg=1)
    h, t = make_head(d)
    p = h.plan(1)
    assert p["stream_tiles"] == 0 and p["resident_bytes"] >= p["w_bytes"], p
    assert_exact(run(h, t), oracle_walk(d), "config1")
    h.close()


@pytest.mark.parametrize("reg,lds", [(0, 0), (1, 0), (2, 1), (3, 2), (0, 4), (5, 0)])
def test_partial_residency_bitwise(reg, lds):
    d = datagen.make_inputs(30011, 256, 2, 4, seed=5)
    _print_case(reg=reg, lds=lds)
    h, t = make_head(d, resident_tiles=reg, lds_tiles=lds)
    ref = oracle_walk(d)
    assert_exact(run(h, t), ref, f"reg={reg} lds={lds}")
    h.close()


def test_recurrent_small_exact():
    d = datagen.make_inputs(5000, 256, 2, 5, head="recurrent", seed=9)
    _print_case(head="recurrent", V=5000)
    h, t = make_head(d)
    for T in (0, 1):
        assert_exact(run(h, t, temperature=T, seed=4), oracle_walk(d, temperature=T, seed=4), f"rec T={T}")
    h.close()


def test_x0_out_of_range_is_latched():
    import torch
    d = datagen.make_inputs(1000, 256, 1, 3, seed=2)
    h, t = make_head(d)
    bad = torch.tensor([1000], dtype=torch.int32, device="cuda")
    h.walk(t["base"], bad)
    assert h.error() == "WTS_ERR_TOKEN_RANGE"
    assert h.error() == "WTS_OK"
    assert_exact(run(h, t), oracle_walk(d), "after error")
    h.close()


def test_watchdog_latches_timeout_and_grid_drains():
    # A 1 us limit on every wait cannot hold one step's exchange (the last
    # workgroup arrives ~0.5 us after the first, and a key needs ~0.8 us to
    # cross both levels), so the walk latches WTS_ERR_TIMEOUT; every
    # workgroup leaves its wait by itself and the launch completes.
    import torch
    d = cached_inputs(0)
    _print_case(test="watchdog", watchdog_us=1)
    h, t = make_head(d, watchdog_us=1)
    h.walk(t["base"], t["x0"])
    torch.cuda.synchronize()
    assert h.error() == "WTS_ERR_TIMEOUT"
    assert h.error() == "WTS_OK"
    # the step-wise path has no waits inside a launch: it still runs on this context
    assert_exact(run(h, t, exec="stepwise"), oracle_walk(d), "step-wise after time-out")
    h.close()
    # and a context with the default limit computes the walk
    h2, t2 = make_head(d, t)
    assert_exact(run(h2, t2), oracle_walk(d), "after time-out")
    h2.close()


def test_log_ratio_shortcut_is_exact_everywhere():
    # The noise kernels form the portable log's f / (2 + f) from a reciprocal
    # estimate and one fused-multiply-add correction.  Over every argument that
    # log can produce (all 2^23 reduced mantissas) it must equal the IEEE
    # quotient bit for bit, or the T=1 walks could part from the oracle.
    from serial_draft_head_persistent_amd import check_log_ratio
    _print_case(test="log_ratio_exhaustive")
    assert check_log_ratio(0) == 0
