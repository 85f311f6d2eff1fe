"""Cross-workgroup selection (Fig. 8) on crafted maxima, through the C ABI.

With E = 0 every latent is zero, so each logit is exactly 0 * s_w[v] + base
(+0 or -0 plus the base logit): the walk reduces to a per-step argmax of the
base logits, and the winner of each step can be written down by hand.  The
maxima are placed in chosen workgroups of the persistent grid: exact bf16
ties inside one first-level group (one XCD), across groups on one XCD, across
XCDs, a +0 / -0 top (rows with a negative row scale give -0 logits), many
ties, the last row, ties inside one workgroup, and negative maxima.  The
lowest index must win everywhere; the oracle must agree bit for bit, in the
resident, fused-streaming and step-wise executions, at T=0 and T=1.
"""
import numpy as np
import pytest

import datagen
from oracle.fp import bf16_rne
from gpu_helpers import make_head, run, oracle_walk, assert_exact

pytestmark = pytest.mark.gpu

V = 151936
GAMMA = 10


def _case(**kw):
    print("CASE", " ".join(f"{k}={v}" for k, v in kw.items()), flush=True)


def _rows(g, tiles, G):
    """Vocabulary rows [lo, hi) of persistent workgroup g."""
    tb, te = g * tiles // G, (g + 1) * tiles // G
    return 16 * tb, min(16 * te, V)


def _scenarios(tiles, G, shift):
    """Ten crafted steps, as ({row: value}, winner, rows whose logit is -0).

    Workgroup numbers are moved by `shift` (a multiple of 16, so groups and
    XCDs keep their relations); ties go to the lowest row (min)."""
    R = lambda g: _rows((g + shift) % G, tiles, G)
    first = lambda g: R(g)[0]
    last = lambda g: R(g)[1] - 1
    mid = lambda g: (R(g)[0] + R(g)[1]) // 2
    out = []
    # 0: ties inside one first-level group (workgroups 17, 33, 241: group 1, one XCD)
    vals = {last(33): 9.0, first(241): 9.0, mid(17): 9.0}
    out.append((vals, min(vals), ()))
    # 1: ties in two groups of one XCD (workgroups 3 and 11)
    vals = {first(11): 7.5, last(3): 7.5}
    out.append((vals, min(vals), ()))
    # 2: ties on three XCDs (workgroups 5, 6, 200)
    vals = {first(200): 6.25, last(6): 6.25, mid(5): 6.25}
    out.append((vals, min(vals), ()))
    # 3: +0 / -0 at the top, all else negative: the lower row holds -0
    lo, hi = sorted((mid(40), mid(41)))
    out.append(({lo: -0.0, hi: 0.0}, lo, (lo,)))
    # 4: the lower row holds +0, the higher -0 (workgroups 60 and 188)
    lo, hi = sorted((first(60), last(188)))
    out.append(({lo: 0.0, hi: -0.0}, lo, (hi,)))
    # 5: two hundred ties spread over the vocabulary
    idx = np.random.default_rng(5).choice(V, 200, replace=False)
    out.append(({int(i): 11.0 for i in idx}, int(idx.min()), ()))
    # 6: a unique maximum on the last row, one bf16 ulp above a value on row 0
    out.append(({V - 1: 8.0, 0: 7.96875}, V - 1, ()))
    # 7: ties inside one workgroup: rows of its first two tiles (two waves)
    #    and two rows of one tile (two lanes)
    b100 = first(100)
    out.append(({b100 + 16 + 3: 5.0, b100 + 3: 5.0, b100 + 7: 5.0}, b100 + 3, ()))
    # 8: negative maxima tied across the last two workgroups
    vals = {first(255): -1.5, last(254): -1.5}
    out.append((vals, min(vals), ()))
    # 9: the first and the last row tied
    out.append(({0: 4.0, V - 1: 4.0}, 0, ()))
    return out


def crafted_inputs():
    """Inputs of the crafted scenarios (16 batch rows) and the hand winners."""
    d = datagen.make_inputs(V, 256, 16, GAMMA, seed=81)
    d["E"][:] = 0.0
    h, t = make_head(d)
    G, tiles = h.plan(1)["grid"], h.plan(1)["tiles"]
    h.close()
    rng = np.random.default_rng(82)
    expected = np.zeros((16, GAMMA), np.int64)
    # background: bf16 values in [-8, -4), below every crafted value
    d["base"][:] = bf16_rne(rng.uniform(-8.0, -4.0, size=d["base"].shape).astype(np.float32))
    neg_rows = set()
    for b in range(16):
        for t_ in range(GAMMA):
            # rows of one batch row walk the scenarios in another order; the
            # workgroups move by 16 b (same group and XCD relations)
            scen = _scenarios(tiles, G, 16 * b)
            vals, win, negs = scen[(t_ + b) % len(scen)]
            for i, v in vals.items():
                d["base"][b, t_, i] = bf16_rne(np.float32(v))
            neg_rows.update(negs)
            expected[b, t_] = win
    s_w = d["s_w"].copy()
    for i in neg_rows:
        s_w[i] = -s_w[i]
    d["s_w"] = s_w
    return d, expected


@pytest.fixture(scope="module")
def crafted():
    return crafted_inputs()


def test_crafted_oracle_matches_hand_winners(crafted):
    d, expected = crafted
    ref = oracle_walk(d)
    assert np.array_equal(ref["tokens"], expected)
    # the logits are the base logits, with -0 where the scale is negative and the base is -0
    assert np.array_equal(ref["logits"] & 0x7FFF, d["base"] & 0x7FFF)
    neg = np.flatnonzero(d["s_w"] < 0)
    assert neg.size and np.any(ref["logits"][:, :, neg] == 0x8000)


@pytest.mark.parametrize("B", [1, 16])
@pytest.mark.parametrize("exec_", ["resident", "stream", "stepwise"])
def test_crafted_ties_greedy(crafted, B, exec_):
    d, expected = crafted
    _case(test="crafted_ties", B=B, exec=exec_, T=0)
    ds = dict(d)
    ds["base"], ds["x0"] = d["base"][:B], d["x0"][:B]
    h, t = make_head(ds)
    got = run(h, t, exec=exec_)
    assert np.array_equal(got["tokens"], expected[:B]), np.argwhere(got["tokens"] != expected[:B])[:5]
    assert_exact(got, oracle_walk(ds), f"crafted B={B} {exec_}")
    h.close()


@pytest.mark.parametrize("B", [1, 16])
@pytest.mark.parametrize("exec_", ["resident", "stepwise"])
def test_crafted_ties_gumbel(crafted, B, exec_):
    d, _ = crafted
    _case(test="crafted_ties", B=B, exec=exec_, T=1)
    ds = dict(d)
    ds["base"], ds["x0"] = d["base"][:B], d["x0"][:B]
    h, t = make_head(ds)
    assert_exact(run(h, t, exec=exec_, temperature=1, seed=13), oracle_walk(ds, temperature=1, seed=13),
                 f"crafted T=1 B={B} {exec_}")
    h.close()
