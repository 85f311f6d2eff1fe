"""The cross-workgroup selection (Fig. 8) under forced arrival delays, with
every workgroup's observed winner recorded, through the C ABI.

WTS_WALK_STRESS makes each workgroup wait a pseudo-random time before each
step's exchange, so keys reach the first- and second-level lines in orders an
unperturbed walk rarely produces; winners_out records the key each workgroup
took.  Every workgroup must take the same key at every step, that key must
name the token the walk wrote, and the walk must still give the oracle's
bits.  The crafted ties of the selection tests (equal maxima inside one
group, across groups and across XCDs) are run the same way.
"""
import numpy as np
import pytest

import datagen
from conftest import cached_inputs
from gpu_helpers import make_head, run, oracle_walk, assert_exact

pytestmark = pytest.mark.gpu


def _case(**kw):
    print("CASE", " ".join(f"{k}={v}" for k, v in kw.items()), flush=True)


def _check_winners(got, what):
    w = got["winners"]                          # [gamma, B, grid] uint64
    gamma, B, G = w.shape
    assert np.all(w != 0), f"{what}: a workgroup recorded no winner"
    agree = np.all(w == w[:, :, :1], axis=2)
    assert agree.all(), f"{what}: workgroups disagree at (step, row) {np.argwhere(~agree)[:5].tolist()}"
    tok = 0x3FFFF - (w[:, :, 0] & np.uint64(0x3FFFF)).astype(np.int64)
    assert np.array_equal(tok.T, got["tokens"]), f"{what}: recorded winner is not the written token"


@pytest.mark.parametrize("B,T", [(1, 0), (16, 0), (4, 1)])
@pytest.mark.parametrize("exchange", ["auto", "device"])
def test_stress_int8_exact(B, T, exchange):
    d = cached_inputs(1, B=B, gamma=8, seed=41 + B)
    _case(test="stress", B=B, T=T, exchange=exchange)
    h, t = make_head(d, exchange=exchange)
    ref = oracle_walk(d, temperature=T, seed=9)
    for rep in range(2):                        # back to back: both walk parities
        got = run(h, t, temperature=T, seed=9, stress=True, winners=True)
        assert_exact(got, ref, f"stress B={B} T={T} {exchange} rep={rep}")
        _check_winners(got, f"B={B} T={T} {exchange} rep={rep}")
    h.close()


@pytest.mark.parametrize("exec_", ["resident", "stream"])
def test_stress_streamed_and_staged(exec_):
    # B=1 stages the winner's embedding row during the exchange (candidate path)
    d = datagen.make_inputs(20011, 256, 1, 8, seed=43)
    _case(test="stress", exec=exec_)
    h, t = make_head(d)
    got = run(h, t, exec=exec_, stress=True, winners=True)
    assert_exact(got, oracle_walk(d), f"stress {exec_}")
    _check_winners(got, exec_)
    h.close()


def test_stress_recurrent():
    d = datagen.make_inputs(5003, 256, 2, 6, head="recurrent", seed=44)
    _case(test="stress", head="recurrent")
    h, t = make_head(d)
    got = run(h, t, stress=True, winners=True)
    assert_exact(got, oracle_walk(d), "stress recurrent")
    _check_winners(got, "recurrent")
    h.close()


def test_stress_crafted_ties():
    # equal maxima inside one group, across groups of one XCD and across XCDs
    from test_gpu_selection import crafted_inputs
    d, expected = crafted_inputs()
    _case(test="stress", scenario="crafted_ties")
    h, t = make_head(d)
    for T in (0, 1):
        got = run(h, t, temperature=T, seed=13, stress=True, winners=True)
        if T == 0:
            assert np.array_equal(got["tokens"], expected)
        assert_exact(got, oracle_walk(d, temperature=T, seed=13), f"stress crafted T={T}")
        _check_winners(got, f"crafted T={T}")
    h.close()


def test_winner_record_without_stress_and_stepwise_rejected():
    import torch
    from serial_draft_head_persistent_amd import WtsError
    d = datagen.make_inputs(20011, 256, 3, 5, seed=45)
    _case(test="winners", stress=False)
    h, t = make_head(d)
    got = run(h, t, winners=True)
    assert_exact(got, oracle_walk(d), "winners, no stress")
    _check_winners(got, "no stress")
    out = {"tokens": torch.full((3, 5), -7, dtype=torch.int32, device="cuda")}
    for kw in ({"stress": True}, {"winners": True}):
        with pytest.raises(WtsError, match="UNSUPPORTED"):
            h.walk(t["base"], t["x0"], exec="stepwise", out=out if "stress" in kw else None, **kw)
    torch.cuda.synchronize()
    assert int(out["tokens"].max()) == -7        # nothing enqueued
    h.close()
