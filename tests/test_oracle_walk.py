"""Pins of the oracle walk: brute force on the Fig. 2 toy shape, closed forms,
tie-break, key order, resume invariance, recurrent update, bf16 projection."""
from fractions import Fraction

import numpy as np
import pytest

import datagen
import oracle
from oracle.fp import bf16_to_f32, bf16_rne, tanh_p
from fp32emu import rnd32, rnd_bf16, rint_even, f32_to_frac


def _F(x):
    return f32_to_frac(np.float32(x))


def _brute_quant(u):
    uf = [_F(x) for x in u]
    amax = max(abs(x) for x in uf)
    if amax == 0:
        return [0] * len(u), [0] * len(u), Fraction(0), Fraction(0)
    s_hi = rnd32(amax / 127)
    inv = rnd32(Fraction(127) / amax)
    inv256 = rnd32(inv * 256)
    hi = [max(-127, min(127, rint_even(rnd32(x * inv)))) for x in uf]
    lo = []
    for x, h in zip(uf, hi):
        res = rnd32(x - rnd32(s_hi * h))
        lo.append(max(-127, min(127, rint_even(rnd32(res * inv256)))))
    return hi, lo, s_hi, s_hi / 256


def _brute_walk(d, temperature=0, seed=0, step_offset=0, fixed=False):
    """Every operation of the int8 Markov / recurrent walk with exact rationals.

    fixed: the fixed-latent probe (Fig. 13b) -- the state of step 0 is kept."""
    W, s_w, E, base, x0 = d["W"], d["s_w"], d["E"], d["base"], d["x0"]
    B, gamma, V = base.shape
    r = W.shape[1]
    toks = np.zeros((B, gamma), np.int64)
    logits = np.zeros((B, gamma, V), np.uint16)
    for b in range(B):
        x = int(x0[b])
        h = None if d["head"] == "markov" else [np.float32(v) for v in d["h0"][b]]
        for t in range(gamma):
            if d["head"] == "markov":
                lat = E[x]
            elif fixed and t > 0:
                lat = np.array(h, np.float32)
            else:
                A = bf16_to_f32(d["A"])
                hn = []
                for j in range(r):
                    acc = Fraction(0)         # one chain in ascending k, product and sum rounded apart
                    for k in range(r):
                        acc = rnd32(acc + rnd32(_F(A[j, k]) * _F(h[k])))
                    pre = rnd32(rnd32(acc + _F(E[x, j])) + _F(d["c"][j]))
                    hn.append(tanh_p(np.float32(float(pre))))
                h = hn
                lat = np.array(h, np.float32)
            hi, lo, s_hi, s_lo = _brute_quant(lat)
            scores = []
            for v in range(V):
                ah = sum(int(W[v, k]) * hi[k] for k in range(r))
                al = sum(int(W[v, k]) * lo[k] for k in range(r))
                z = rnd32(rnd32(ah * s_hi) + rnd32(al * s_lo))
                z = rnd32(z * _F(s_w[v]))
                z = rnd32(z + _F(bf16_to_f32(base[b, t, v])))
                lg = rnd_bf16(z)
                logits[b, t, v] = bf16_rne(np.float32(float(lg)))
                if temperature == 1:
                    g = oracle.gumbel_noise(seed, b, step_offset + t, np.array([v]))[0]
                    lg = rnd32(lg + _F(g))
                scores.append((-lg, v))
            toks[b, t] = min(scores)[1]
            if not fixed:
                x = int(toks[b, t])
    return toks, logits


@pytest.mark.parametrize("temperature", [0, 1])
@pytest.mark.parametrize("head", ["markov", "recurrent"])
def test_toy_walk_brute_force(temperature, head):
    # Fig. 2 toy shape: V=12, r=4, three steps (two batch rows)
    d = datagen.make_inputs(12, 4, 2, 3, head=head, seed=11)
    toks, lg = _brute_walk(d, temperature, seed=3)
    o = oracle.walk(d["W"], d["E"], d["base"], d["x0"], s_w=d["s_w"], head=head,
                    A=d["A"], c=d["c"], h0=d["h0"], temperature=temperature, seed=3)
    assert np.array_equal(o["tokens"], toks)
    assert np.array_equal(o["logits"], lg)


def test_toy_walk_brute_force_ties():
    # bf16 base values drawn from a tiny set and E = 0 -> many exact ties at the top
    d = datagen.make_inputs(12, 4, 1, 3, seed=12)
    d["E"][:] = 0
    d["E"][:, 0] = np.float32(1e-3)
    d["base"][:] = bf16_rne(np.float32(1.0))
    d["base"][0, 1, 5] = d["base"][0, 1, 9] = bf16_rne(np.float32(2.0))
    toks, lg = _brute_walk(d)
    o = oracle.walk(d["W"], d["E"], d["base"], d["x0"], s_w=d["s_w"])
    assert np.array_equal(o["tokens"], toks) and np.array_equal(o["logits"], lg)


def test_project_int8_exact_bruteforce():
    rng = np.random.default_rng(9)
    W = rng.integers(-127, 128, size=(37, 256)).astype(np.int8)
    hi = rng.integers(-127, 128, size=(2, 256)).astype(np.int8)
    lo = rng.integers(-127, 128, size=(2, 256)).astype(np.int8)
    ah, al = oracle.project_int8(W.astype(np.float64), hi, lo)
    for b in range(2):
        for v in range(37):
            assert ah[b, v] == sum(int(W[v, k]) * int(hi[b, k]) for k in range(256))
            assert al[b, v] == sum(int(W[v, k]) * int(lo[b, k]) for k in range(256))
    # the worst case stays below 2^24, so the conversion to binary32 is exact
    full = oracle.project_int8(np.full((1, 256), 127.0), np.full(256, 127, np.int8), np.full(256, -127, np.int8))
    assert full[0][0] == 256 * 127 * 127 < 2 ** 24 and full[1][0] == -256 * 127 * 127


def test_epilogue_matches_rational_emulation():
    rng = np.random.default_rng(10)
    n = 4000
    ah = rng.integers(-4_129_024, 4_129_025, n)
    al = rng.integers(-4_129_024, 4_129_025, n)
    s_hi = np.float32(rng.uniform(1e-4, 1e-2))
    s_lo = np.float32(s_hi / 256)
    s_w = rng.uniform(1e-3, 0.1, n).astype(np.float32)
    base = bf16_rne(rng.normal(0, 1.4, n).astype(np.float32))
    lg, z = oracle.epilogue_int8(ah, al, s_hi, s_lo, s_w, base)
    for i in range(n):
        q = rnd32(rnd32(int(ah[i]) * _F(s_hi)) + rnd32(int(al[i]) * _F(s_lo)))
        q = rnd32(q * _F(s_w[i]))
        q = rnd32(q + _F(bf16_to_f32(base[i])))
        assert Fraction(float(z[i])) == q
        assert Fraction(float(bf16_to_f32(lg[i]))) == rnd_bf16(q)


def test_select_and_key_order_with_ties():
    rng = np.random.default_rng(11)
    vals = np.array([0.0, -0.0, 1.5, -2.0, 1.5, 3.25, -0.0], np.float32)
    for trial in range(200):
        s = rng.choice(vals, size=rng.integers(1, 40)).astype(np.float32)
        idx = np.arange(s.size)
        lex = np.lexsort((idx, -s.astype(np.float64)))[0]
        assert oracle.select_token(s) == lex == int(np.argmax(s))
        keys = oracle.order_key(s, idx)
        assert int(np.argmax(keys)) == lex
    # -0 and +0 are equal: the lower index wins whichever sign it carries
    assert oracle.select_token(np.array([-0.0, 0.0], np.float32)) == 0
    assert oracle.select_token(np.array([0.0, -0.0], np.float32)) == 0
    k = oracle.order_key(np.array([-0.0, 0.0], np.float32), np.array([5, 5]))
    assert k[0] == k[1]
    # key order: negative < -0 == +0 < positive; and below any finite key sits 0
    k = oracle.order_key(np.array([-1e30, -1.0, 0.0, 1e-30, 2.0], np.float32), np.zeros(5, np.int64))
    assert np.all(np.diff(k.astype(object)) > 0) and np.all(k > 0)


def test_closed_form_zero_embedding_is_per_step_argmax():
    d = datagen.make_inputs(300, 16, 3, 5, seed=13)
    d["E"][:] = 0
    o = oracle.walk(d["W"], d["E"], d["base"], d["x0"], s_w=d["s_w"])
    want = np.argmax(bf16_to_f32(d["base"]), axis=-1)
    assert np.array_equal(o["tokens"], want)
    assert np.array_equal(o["logits"], d["base"])


def test_closed_form_cyclic_successor():
    V, r = 12, 4
    th = 2 * np.pi * np.arange(V) / V
    d = datagen.make_inputs(V, r, 4, 6, seed=14)
    d["W"] = np.zeros((V, r), np.int8)
    d["W"][:, 0] = np.rint(127 * np.cos(th))
    d["W"][:, 1] = np.rint(127 * np.sin(th))
    d["s_w"] = np.full(V, 1 / 127, np.float32)
    d["E"] = np.zeros((V, r), np.float32)
    d["E"][:, 0] = np.cos(np.roll(th, -1))
    d["E"][:, 1] = np.sin(np.roll(th, -1))
    d["base"][:] = 0
    d["x0"] = np.array([0, 5, 11, 7], np.int32)
    o = oracle.walk(d["W"], d["E"], d["base"], d["x0"], s_w=d["s_w"])
    want = (d["x0"][:, None] + np.arange(1, 7)[None, :]) % V
    assert np.array_equal(o["tokens"], want)


def test_closed_form_recurrent():
    d = datagen.make_inputs(50, 8, 2, 4, head="recurrent", seed=15)
    d["A"][:] = 0
    d["c"][:] = 0
    o = oracle.walk(d["W"], d["E"], d["base"], d["x0"], s_w=d["s_w"], head="recurrent",
                    A=d["A"], c=d["c"], h0=d["h0"])
    last_in = o["tokens"][:, -2]
    assert np.array_equal(o["state"], tanh_p(d["E"][last_in]))
    d["E"][:] = 0
    o = oracle.walk(d["W"], d["E"], d["base"], d["x0"], s_w=d["s_w"], head="recurrent",
                    A=d["A"], c=d["c"], h0=d["h0"])
    assert np.array_equal(o["state"], np.broadcast_to(tanh_p(d["c"]), (2, 8)))


@pytest.mark.parametrize("head", ["markov", "recurrent"])
def test_resume_invariance(head):
    d = datagen.make_inputs(500, 32, 2, 16, head=head, seed=16)
    kw = dict(s_w=d["s_w"], head=head, A=d["A"], c=d["c"], temperature=1, seed=99)
    full = oracle.walk(d["W"], d["E"], d["base"], d["x0"], h0=d["h0"], **kw)
    a = oracle.walk(d["W"], d["E"], d["base"][:, :7], d["x0"], h0=d["h0"], **kw)
    b = oracle.walk(d["W"], d["E"], d["base"][:, 7:], a["tokens"][:, -1], h0=a["state"],
                    step_offset=7, **kw)
    assert np.array_equal(np.concatenate([a["tokens"], b["tokens"]], 1), full["tokens"])
    assert np.array_equal(np.concatenate([a["logits"], b["logits"]], 1), full["logits"])


def test_batch_rows_independent():
    # Rows of a batch share only W and E (and A, c): at T=0 row b of a batched
    # walk is the walk of row b alone.  At T=1 the noise is keyed by the batch
    # index, so batch row 0 equals a lone walk, and row b equals a lone walk
    # that draws row b's noise -- checked through the Gumbel-max rule itself:
    # each chosen token is the argmax of fp32(logit + g(seed, b, t, v)).
    d = datagen.make_inputs(400, 32, 3, 5, seed=17)
    greedy = oracle.walk(d["W"], d["E"], d["base"], d["x0"], s_w=d["s_w"])
    hot = oracle.walk(d["W"], d["E"], d["base"], d["x0"], s_w=d["s_w"], temperature=1, seed=5)
    for b in range(3):
        one = oracle.walk(d["W"], d["E"], d["base"][b:b + 1], d["x0"][b:b + 1], s_w=d["s_w"])
        assert np.array_equal(greedy["tokens"][b:b + 1], one["tokens"])
        assert np.array_equal(greedy["logits"][b:b + 1], one["logits"])
        lone = oracle.walk(d["W"], d["E"], d["base"][b:b + 1], d["x0"][b:b + 1], s_w=d["s_w"],
                           temperature=1, seed=5)
        if b == 0:
            assert np.array_equal(hot["tokens"][:1], lone["tokens"])
        for t in range(5):
            g = oracle.gumbel_noise(5, b, t, np.arange(400))
            sc = (bf16_to_f32(hot["logits"][b, t]) + g).astype(np.float32)
            assert hot["tokens"][b, t] == int(np.argmax(sc))
    # the T=1 walks of rows 1 and 2 take other noise than a lone row would
    assert not all(np.array_equal(hot["tokens"][b], oracle.walk(
        d["W"], d["E"], d["base"][b:b + 1], d["x0"][b:b + 1], s_w=d["s_w"], temperature=1,
        seed=5)["tokens"][0]) for b in (1, 2))


def test_project_bf16_exact_sum():
    rng = np.random.default_rng(18)
    W = bf16_rne(rng.standard_t(4, (20, 64)).astype(np.float32))
    u = bf16_rne(rng.normal(0, 0.1, 64).astype(np.float32))
    p = oracle.project_bf16(bf16_to_f32(W).astype(np.float64), u)
    Wf, uf = bf16_to_f32(W), bf16_to_f32(u)
    for v in range(20):
        s = sum(_F(Wf[v, k]) * _F(uf[k]) for k in range(64))
        assert Fraction(float(p[v])) == rnd32(s)


def test_bf16_walk_bruteforce_small():
    d = datagen.make_inputs(16, 8, 1, 3, wtype="bf16", seed=19)
    o = oracle.walk(d["W"], d["E"], d["base"], d["x0"], wtype="bf16", keep_z=True)
    Wf = bf16_to_f32(d["W"])
    x = int(d["x0"][0])
    for t in range(3):
        u = bf16_to_f32(bf16_rne(d["E"][x]))
        sc = []
        for v in range(16):
            z = rnd32(rnd32(sum(_F(Wf[v, k]) * _F(u[k]) for k in range(8))) + _F(bf16_to_f32(d["base"][0, t, v])))
            assert Fraction(float(o["z"][0, t, v])) == z
            sc.append((-rnd_bf16(z), v))
        x = min(sc)[1]
        assert o["tokens"][0, t] == x


@pytest.mark.parametrize("temperature", [0, 1])
@pytest.mark.parametrize("head", ["markov", "recurrent"])
def test_fixed_latent_brute_force(temperature, head):
    # the probe of Fig. 13b on the toy shape: every op with exact rationals
    d = datagen.make_inputs(12, 4, 2, 4, head=head, seed=21)
    toks, lg = _brute_walk(d, temperature, seed=4, fixed=True)
    o = oracle.walk(d["W"], d["E"], d["base"], d["x0"], s_w=d["s_w"], head=head, A=d["A"],
                    c=d["c"], h0=d["h0"], temperature=temperature, seed=4, fixed_latent=True)
    assert np.array_equal(o["tokens"], toks)
    assert np.array_equal(o["logits"], lg)


def test_fixed_latent_cyclic_successor():
    # the cyclic-successor head walks x0+1, x0+2, ...; with the latent fixed at
    # E[x0] every step picks x0+1
    V, r = 12, 4
    th = 2 * np.pi * np.arange(V) / V
    d = datagen.make_inputs(V, r, 3, 5, seed=22)
    d["W"] = np.zeros((V, r), np.int8)
    d["W"][:, 0] = np.rint(127 * np.cos(th))
    d["W"][:, 1] = np.rint(127 * np.sin(th))
    d["s_w"] = np.full(V, 1 / 127, np.float32)
    d["E"] = np.zeros((V, r), np.float32)
    d["E"][:, 0] = np.cos(np.roll(th, -1))
    d["E"][:, 1] = np.sin(np.roll(th, -1))
    d["base"][:] = 0
    d["x0"] = np.array([3, 11, 6], np.int32)
    o = oracle.walk(d["W"], d["E"], d["base"], d["x0"], s_w=d["s_w"], fixed_latent=True)
    assert np.array_equal(o["tokens"], np.repeat(((d["x0"] + 1) % V)[:, None], 5, axis=1))


@pytest.mark.parametrize("head", ["markov", "recurrent"])
def test_fixed_latent_steps_are_one_step_walks(head):
    # step t of the probe is the first step of a walk from x0 that reads base row t
    d = datagen.make_inputs(300, 32, 2, 5, head=head, seed=23)
    kw = dict(s_w=d["s_w"], head=head, A=d["A"], c=d["c"], h0=d["h0"])
    o = oracle.walk(d["W"], d["E"], d["base"], d["x0"], fixed_latent=True, **kw)
    for t in range(5):
        one = oracle.walk(d["W"], d["E"], d["base"][:, t:t + 1], d["x0"], **kw)
        assert np.array_equal(o["tokens"][:, t], one["tokens"][:, 0])
        assert np.array_equal(o["logits"][:, t], one["logits"][:, 0])


def test_log_normaliser_closed_forms():
    from oracle.walk import log_normaliser
    import math
    # equal logits: ln(V e^c) = c + ln V
    for c, V in [(1.5, 1000), (-7.25, 1), (12.0, 151936)]:
        lg = np.full(V, bf16_rne(np.float32(c)), np.uint16)
        assert abs(log_normaliser(lg) - (c + math.log(V))) < 1e-12 * max(1.0, abs(c))
    # two values: k copies of a, n - k of b
    a, b, k, n = 3.0, -2.5, 7, 5000
    lg = np.full(n, bf16_rne(np.float32(b)), np.uint16)
    lg[:k] = bf16_rne(np.float32(a))
    want = a + math.log(k + (n - k) * math.exp(b - a))
    assert abs(log_normaliser(lg) - want) < 1e-12
    # exact shift invariance for bf16-exact shifts
    rng = np.random.default_rng(24)
    q = rng.integers(-64, 64, 3000).astype(np.float32) / 8
    assert abs(log_normaliser(bf16_rne(q + 4)) - log_normaliser(bf16_rne(q)) - 4) < 1e-12


def test_log_normaliser_matches_library():
    from oracle.walk import log_normaliser
    from scipy.special import logsumexp, softmax
    rng = np.random.default_rng(25)
    lg = bf16_rne(rng.normal(0, 2, 20000).astype(np.float32))
    l64 = bf16_to_f32(lg).astype(np.float64)
    lse = log_normaliser(lg)
    assert abs(lse - logsumexp(l64)) < 1e-11
    # q = exp(l - lse) is the softmax of the logits and sums to one
    assert np.allclose(np.exp(l64 - lse), softmax(l64), rtol=1e-12, atol=0)
    assert abs(np.exp(l64 - lse).sum() - 1.0) < 1e-12


def test_walk_lse_is_normaliser_of_its_logits():
    d = datagen.make_inputs(700, 32, 2, 4, seed=26)
    o = oracle.walk(d["W"], d["E"], d["base"], d["x0"], s_w=d["s_w"], temperature=1, seed=2,
                    keep_lse=True)
    from oracle.walk import log_normaliser
    for b in range(2):
        for t in range(4):
            assert o["lse"][b, t] == log_normaliser(o["logits"][b, t])


# ---- the recurrent sum order (pins by hand-derived IEEE results) ----
# The pages give h = tanh(A h + E[x] + c) with no summation order (Fig. 13);
# the oracle takes one ascending chain with a rounding after every product
# and every addition, then (acc + E[x]) + c.  Each case below has a result
# worked out by hand from the binary32 rounding rule, and a summation in
# any other grouping, with fused multiply-adds, or in higher precision gives
# a different number.

def _preact(A_rows, h, e=0.0, c=0.0):
    A = np.asarray(A_rows, np.float32)
    n = A.shape[1]
    return oracle.recurrent_preact(A, np.asarray(h, np.float32), np.full(A.shape[0], e, np.float32),
                                   np.full(A.shape[0], c, np.float32))


def test_recurrent_sum_is_ascending_chain():
    # 1 followed by 255 terms of 2^-24 (half an ulp of 1): each addition to 1
    # is an exact tie and rounds to the even neighbour, 1, so the ascending
    # chain ends at exactly 1.  Summed in any order that adds small terms
    # together first (reversed, pairwise, interleaved partial sums) or exactly
    # and rounded once, the result is 1 + 2^-16 (127.5 ulps of 1, a tie that
    # rounds to the even 128).
    h = np.full(256, 2.0 ** -24, np.float32)
    h[0] = 1.0
    A = np.ones((1, 256), np.float32)
    assert _preact(A, h)[0] == np.float32(1.0)
    # reversed rows: the tiny terms first, then 1 at the end
    assert _preact(A[:, ::-1], h[::-1])[0] == np.float32(1.0 + 2.0 ** -16)
    # the terms before k = 0 matter the same way: 2^-24 terms then 1 (ascending chain
    # sums them exactly to 255 * 2^-24 first)
    h2 = np.full(256, 2.0 ** -24, np.float32)
    h2[255] = 1.0
    assert _preact(A, h2)[0] == np.float32(1.0 + 2.0 ** -16)


def test_recurrent_products_rounded_before_the_sum():
    # A[0] = -1, h[0] = 1 + 2^-7 + 2^-23 (exact in binary32), then
    # A[1] = 1 + 2^-7 (exact in bf16), h[1] = 1 + 2^-23: the exact product is
    # 1 + 2^-7 + 2^-23 + 2^-30, which rounds to 1 + 2^-7 + 2^-23 (the 2^-30
    # bit is below half an ulp), so the chain ends at exactly +0.  A fused
    # multiply-add would keep the 2^-30.
    h = np.zeros(256, np.float32)
    A = np.zeros((1, 256), np.float32)
    A[0, 0], h[0] = -1.0, np.float32(1.0 + 2.0 ** -7 + 2.0 ** -23)
    A[0, 1], h[1] = np.float32(1.0 + 2.0 ** -7), np.float32(1.0 + 2.0 ** -23)
    assert float(A[0, 1]) == float(bf16_to_f32(bf16_rne(A[0, 1])))
    got = _preact(A, h)[0]
    assert got == np.float32(0.0) and not np.signbit(got)


def test_recurrent_pre_adds_embedding_then_bias():
    # acc = 1 (A = e_0, h_0 = 1), E[x] = c = 2^-24: (1 + 2^-24) ties to 1,
    # then + 2^-24 ties to 1 again; adding E[x] + c first would give
    # 1 + 2^-23.
    h = np.zeros(256, np.float32)
    h[0] = 1.0
    A = np.zeros((1, 256), np.float32)
    A[0, 0] = 1.0
    assert _preact(A, h, e=2.0 ** -24, c=2.0 ** -24)[0] == np.float32(1.0)
    # and with E[x] = -1, c = 2^-24: (1 - 1) + 2^-24 = 2^-24 exactly
    assert _preact(A, h, e=-1.0, c=2.0 ** -24)[0] == np.float32(2.0 ** -24)


def test_recurrent_chain_starts_from_positive_zero():
    # all products -0 (A = -1, h = +0): +0 + (-0) = +0 in round-to-nearest
    A = -np.ones((3, 256), np.float32)
    got = _preact(A, np.zeros(256, np.float32))
    assert np.all(got == 0) and not np.any(np.signbit(got))
