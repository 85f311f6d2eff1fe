"""The cross-workgroup exchange's hardware assumption and its fallback, and
the limits of smaller grids, through the C ABI.

The first level of the selection exchange (Fig. 8) runs through one XCD's L2
only if workgroup g is dispatched to the same XCD as g mod 16; wts_create
checks this by reading every workgroup's XCC_ID and otherwise falls back to
device scope, which a create flag can also force.  Both must give the
oracle's bits."""
import numpy as np
import pytest

import datagen
from conftest import cached_inputs
from gpu_helpers import make_head, run, oracle_walk, assert_exact

pytestmark = pytest.mark.gpu


def _case(**kw):
    print("CASE", " ".join(f"{k}={v}" for k, v in kw.items()), flush=True)


def test_dispatch_check_keeps_groups_inside_an_xcd():
    # on MI355X (eight XCDs, workgroups dealt round-robin) the check passes
    d = cached_inputs(0)
    _case(test="xcd_check")
    h, t = make_head(d)
    assert h.plan(1)["exchange"] == 0
    assert_exact(run(h, t), oracle_walk(d), "xcd-local exchange")
    h.close()


def test_device_scope_exchange_full_size_exact():
    d = cached_inputs(1)
    _case(test="device_scope_exchange", cfg=1)
    h, t = make_head(d, exchange="device")
    assert h.plan(1)["exchange"] == 1
    assert_exact(run(h, t), oracle_walk(d), "device-scope exchange, headline workload")
    h.close()


@pytest.mark.parametrize("B,T", [(1, 1), (3, 1), (16, 0)])
@pytest.mark.parametrize("exec_", ["resident", "stream"])
def test_device_scope_exchange_exact(B, T, exec_):
    d = datagen.make_inputs(20011, 256, B, 6, seed=90 + B)
    _case(test="device_scope_exchange", B=B, T=T, exec=exec_)
    h, t = make_head(d, exchange="device")
    assert_exact(run(h, t, exec=exec_, temperature=T, seed=2), oracle_walk(d, temperature=T, seed=2),
                 f"device scope B={B} T={T} {exec_}")
    h.close()


def test_device_scope_exchange_recurrent():
    d = datagen.make_inputs(5003, 256, 2, 5, head="recurrent", seed=95)
    _case(test="device_scope_exchange", head="recurrent")
    h, t = make_head(d, exchange="device")
    assert_exact(run(h, t), oracle_walk(d), "device scope recurrent")
    h.close()


@pytest.mark.parametrize("grid,B", [(1, 1), (8, 4), (37, 4)])
def test_smaller_grids_exact(grid, B):
    # fewer workgroups, each with a larger shard (more LDS and streamed tiles);
    # one workgroup holds all 20,016 rows, whose T=1 noise fits LDS for one row
    d = datagen.make_inputs(20011, 256, B, 5, seed=96)
    _case(test="small_grid", grid=grid, B=B)
    h, t = make_head(d, grid=grid)
    assert h.plan(B)["grid"] == grid
    for T in (0, 1):
        assert_exact(run(h, t, temperature=T, seed=5), oracle_walk(d, temperature=T, seed=5), f"grid={grid} T={T}")
    h.close()


def test_noise_that_does_not_fit_in_lds_is_rejected():
    # 8 workgroups of 20,011 rows: a T=1 walk of 16 rows would need 16 x 2,512 x 4
    # bytes of noise in LDS, more than the 160 KiB; T=0 and fewer rows fit
    import torch
    from serial_draft_head_persistent_amd import WtsError
    d = datagen.make_inputs(20011, 256, 16, 3, seed=97)
    _case(test="noise_lds_limit")
    h, t = make_head(d, grid=8)
    with pytest.raises(WtsError, match="UNSUPPORTED"):
        h.plan(16, temperature=1)
    out = {"tokens": torch.full((16, 3), -7, dtype=torch.int32, device="cuda")}
    with pytest.raises(WtsError, match="UNSUPPORTED"):
        h.walk(t["base"], t["x0"], temperature=1, out=out)
    torch.cuda.synchronize()
    assert int(out["tokens"].max()) == -7          # nothing enqueued
    assert_exact(run(h, t), oracle_walk(d), "grid 8, T=0, B=16")
    h.close()


def test_row_field_limit_at_create():
    # two workgroups over 151,936 rows would each own 75,968 rows (> 65,535)
    from serial_draft_head_persistent_amd import WtsError
    d = cached_inputs(0, V=151936)
    _case(test="row_field_limit")
    with pytest.raises(WtsError, match="UNSUPPORTED"):
        make_head(d, grid=2)
    h, _ = make_head(d, grid=3)                    # 50,656 rows each: fits
    h.close()
