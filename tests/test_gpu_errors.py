"""Host-detected errors of wts_walk on a live context: each bad argument
returns a status before any launch, leaves the caller's outputs untouched,
and does not disturb the context (a correct walk follows)."""
import ctypes

import numpy as np
import pytest

from gpu_helpers import make_head, run, oracle_walk, assert_exact
from conftest import cached_inputs

pytestmark = pytest.mark.gpu

SENTINEL = -7


def _params(_abi, t, tokens, B, gamma, over):
    import torch
    p = _abi.WalkParams(B=B, gamma=gamma, step_offset=0, temperature=0, seed=0,
                        base=t["base"].data_ptr(), x0=t["x0"].data_ptr(), h0=None,
                        tokens_out=tokens.data_ptr(), logits_out=None, state_out=None, exec=0, flags=0,
                        stream=ctypes.c_void_p(torch.cuda.current_stream().cuda_stream),
                        trace_out=None, lse_out=None)
    for k, v in over.items():
        setattr(p, k, v)
    return p


@pytest.mark.parametrize("case,kw,status", [
    ("B=0 (empty batch)", {"B": 0}, 1),
    ("B above max_batch", {"B": 5}, 1),
    ("gamma=0 (empty walk)", {"gamma": 0}, 1),
    ("gamma above max_steps", {"gamma": 9}, 1),
    ("temperature 2", {"temperature": 2}, 1),
    ("negative step_offset", {"step_offset": -1}, 1),
    ("unknown flag", {"flags": 4}, 1),
    ("unknown exec", {"exec": 3}, 1),
    ("null tokens_out", {"tokens_out": None}, 1),
    ("null base", {"base": None}, 1),
    ("null x0", {"x0": None}, 1),
    ("odd base address", {"base": "odd"}, 1),
    ("odd winners_out address", {"winners_out": "odd"}, 1),
])
def test_walk_rejects_bad_arguments_and_leaves_outputs(case, kw, status):
    import torch
    from serial_draft_head_persistent_amd import _abi
    print("CASE", case, flush=True)
    d = cached_inputs(0)
    h, t = make_head(d, max_batch=4, max_steps=8)
    B, gamma = d["base"].shape[0], d["base"].shape[1]
    tokens = torch.full((4, 8), SENTINEL, dtype=torch.int32, device="cuda")
    if kw.get("base") == "odd":
        kw = {"base": t["base"].data_ptr() + 1}
    if kw.get("winners_out") == "odd":
        kw = {"winners_out": tokens.data_ptr() + 4}
    p = _params(_abi, t, tokens, B, gamma, kw)
    assert _abi.lib().wts_walk(h._h, ctypes.byref(p)) == status
    torch.cuda.synchronize()
    assert h.error() == "WTS_OK"
    assert (tokens.cpu().numpy() == SENTINEL).all()
    # the context still walks correctly
    assert_exact(run(h, t), oracle_walk(d), f"after {case}")
    h.close()


def test_plan_rejects_bad_arguments():
    import torch  # noqa: F401
    from serial_draft_head_persistent_amd import _abi
    d = cached_inputs(0)
    h, _ = make_head(d, max_batch=4, max_steps=8)
    plan = _abi.Plan()
    lib = _abi.lib()
    for B, ex, T in [(0, 0, 0), (5, 0, 0), (1, 3, 0), (1, 0, 2)]:
        assert lib.wts_get_plan(h._h, B, ex, T, ctypes.byref(plan)) == 1, (B, ex, T)
    assert lib.wts_get_plan(h._h, 4, 0, 1, ctypes.byref(plan)) == 0
    assert plan.grid >= 1 and plan.tiles * 16 >= d["W"].shape[0]
    h.close()

