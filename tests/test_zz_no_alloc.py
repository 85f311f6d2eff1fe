"""wts_walk_noalloc: the walk with its scratch in the library's fixed per-GPU
array, against wts_walk on the same inputs, through the C ABI.  Two calls in
a row, the second smaller; tokens, logits, lse and state must be identical
(int8 W: the same kernels, so the same bits)."""
import numpy as np
import pytest

import datagen
from conftest import cached_inputs
from gpu_helpers import make_head, oracle_walk, assert_exact

pytestmark = pytest.mark.gpu


def _case(**kw):
    print("CASE", " ".join(f"{k}={v}" for k, v in kw.items()), flush=True)


def _walk(h, base, x0, noalloc, **kw):
    import torch
    o = h.walk(base, x0, logits=True, noalloc=noalloc, **kw)
    torch.cuda.synchronize()
    assert h.error() == "WTS_OK"
    return {k: (v.view(torch.int16) if v.dtype == torch.bfloat16 else v).cpu().numpy() for k, v in o.items()}


def _same(a, b, what):
    for k in a:
        assert np.array_equal(a[k].view(np.uint8), b[k].view(np.uint8)), f"{what}: {k} differs"


def test_noalloc_matches_walk_full_size_two_calls():
    d = cached_inputs(2)                       # V=151,936, int8, B=16
    h, t = make_head(d)
    calls = [dict(B=4, gamma=16, temperature=1, seed=7, lse=True),
             dict(B=1, gamma=7, temperature=0, seed=0, lse=False)]
    for c in calls:
        _case(test="noalloc_full", **c)
        B, g = c["B"], c["gamma"]
        base, x0 = t["base"][:B, :g].contiguous(), t["x0"][:B].contiguous()
        kw = dict(temperature=c["temperature"], seed=c["seed"], lse=c["lse"])
        ref = _walk(h, base, x0, False, **kw)
        got = _walk(h, base, x0, True, **kw)
        _same(got, ref, f"B={B} gamma={g}")
        ds = dict(d)
        ds["base"], ds["x0"] = d["base"][:B, :g], d["x0"][:B]
        assert_exact({"tokens": got["tokens"], "logits": got["logits"].view(np.uint16)},
                     oracle_walk(ds, temperature=c["temperature"], seed=c["seed"]), f"noalloc B={B}")
    h.close()


@pytest.mark.parametrize("exec_", ["resident", "stream", "stepwise"])
def test_noalloc_matches_walk_each_mode(exec_):
    d = datagen.make_inputs(20011, 256, 5, 6, seed=71)
    _case(test="noalloc_modes", exec=exec_)
    h, t = make_head(d)
    for B, g in ((5, 6), (2, 3)):
        base, x0 = t["base"][:B, :g].contiguous(), t["x0"][:B].contiguous()
        ref = _walk(h, base, x0, False, exec=exec_, temperature=1, seed=3, lse=True)
        got = _walk(h, base, x0, True, exec=exec_, temperature=1, seed=3, lse=True)
        _same(got, ref, f"{exec_} B={B} gamma={g}")
    h.close()


def test_noalloc_recurrent_two_calls():
    d = datagen.make_inputs(9001, 256, 3, 5, head="recurrent", seed=72)
    _case(test="noalloc_recurrent")
    h, t = make_head(d)
    for B, g in ((3, 5), (1, 2)):
        base, x0, h0 = t["base"][:B, :g].contiguous(), t["x0"][:B].contiguous(), t["h0"][:B].contiguous()
        ref = _walk(h, base, x0, False, h0=h0, state=True)
        got = _walk(h, base, x0, True, h0=h0, state=True)
        _same(got, ref, f"recurrent B={B}")
    h.close()


def test_noalloc_and_walk_interleaved_across_contexts():
    # two contexts on one GPU share the array; calls in turn (never
    # overlapping) alternate its walk parity independently of each context's
    d = datagen.make_inputs(7001, 256, 2, 5, seed=73)
    _case(test="noalloc_interleaved")
    h1, t = make_head(d)
    h2, _ = make_head(d, t)
    ref = _walk(h1, t["base"], t["x0"], False)
    for h in (h1, h2, h2, h1, h2):
        _same(_walk(h, t["base"], t["x0"], True), ref, "interleaved")
        _same(_walk(h, t["base"], t["x0"], False), ref, "interleaved plain")
    h1.close()
    h2.close()


def test_noalloc_rejects_partials_beyond_the_array():
    import torch
    from serial_draft_head_persistent_amd import WtsError, _abi
    d = cached_inputs(2)                       # V=151,936: 1,187 step-wise workgroups
    _case(test="noalloc_limit")
    h, t = make_head(d)
    groups = -(-h.plan(16)["tiles"] // 8)
    assert 16 * 16 * groups * 8 > _abi.NOALLOC_LSE_BYTES
    out = {"tokens": torch.full((16, 16), -5, dtype=torch.int32, device="cuda"),
           "lse": torch.full((16, 16), -5.0, dtype=torch.float32, device="cuda")}
    with pytest.raises(WtsError, match="UNSUPPORTED"):
        h.walk(t["base"], t["x0"], exec="stepwise", lse=True, out=out, noalloc=True)
    torch.cuda.synchronize()
    assert int(out["tokens"].min()) == -5 and float(out["lse"].max()) == -5.0   # nothing enqueued
    # the same walk without lse, and the persistent walk with it, fit
    ref = _walk(h, t["base"], t["x0"], False, lse=True)
    _same(_walk(h, t["base"], t["x0"], True, lse=True), ref, "persistent lse at the limit")
    h.close()
