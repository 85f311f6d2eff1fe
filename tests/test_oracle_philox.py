"""Pins of the counter-based noise: published known answer, uniformity, Gumbel-max law."""
import numpy as np
from scipy import stats

import oracle
from oracle.philox import philox4x32_10, uniform24, gumbel_noise


def test_philox_known_answer_zero():
    # Known-answer vector published with Philox4x32-10 (Salmon et al., SC'11):
    # counter (0,0,0,0), key (0,0)
    out = philox4x32_10(np.zeros(4, np.uint32), np.zeros(2, np.uint32))
    assert [int(v) for v in out] == [0x6627E8D5, 0xE169C58D, 0xBC57AC4C, 0x9B00DBD8]


def test_philox_known_answer_vectors():
    # all published known-answer vectors (tests/golden/philox4x32_10_kat.txt)
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", "philox4x32_10_kat.txt")
    rows = [l.split() for l in open(path) if l.strip() and not l.startswith("#")]
    assert len(rows) == 3
    for r in rows:
        w = [int(x, 16) for x in r]
        out = philox4x32_10(np.array(w[:4], np.uint32), np.array(w[4:6], np.uint32))
        assert [int(v) for v in out] == w[6:], r


def test_philox_deterministic_and_key_sensitive():
    ctr = np.array([[7, 3, 1, 0], [8, 3, 1, 0]], np.uint32)
    a = philox4x32_10(ctr, np.array([1, 2], np.uint32))
    b = philox4x32_10(ctr, np.array([1, 2], np.uint32))
    c = philox4x32_10(ctr, np.array([1, 3], np.uint32))
    assert np.array_equal(a, b) and not np.array_equal(a, c)
    assert not np.array_equal(a[0], a[1])


def test_philox_words_uniform():
    ctr = np.zeros((250_000, 4), np.uint32)
    ctr[:, 0] = np.arange(250_000)
    w = philox4x32_10(ctr, np.array([123, 456], np.uint32)).ravel()
    ks = stats.kstest(w.astype(np.float64) / 2.0 ** 32, "uniform")
    assert ks.pvalue > 1e-4
    bits = np.unpackbits(w.view(np.uint8)).mean()
    assert abs(bits - 0.5) < 1e-3


def test_uniform24_exact_open_interval():
    w = np.array([0, 511, 512, 0xFFFFFFFF], np.uint32)
    u = uniform24(w).astype(np.float64)
    assert u[0] == 2.0 ** -24 and u[1] == 2.0 ** -24 and u[2] == 3 * 2.0 ** -24
    assert u[3] == 1.0 - 2.0 ** -24


def test_gumbel_noise_layout():
    # consecutive v share one Philox call: v and v^1 use the same counter, other words
    v = np.arange(16)
    g = gumbel_noise(5, 2, 3, v)
    out = philox4x32_10(np.array([[i, 3, 2, 0] for i in range(4)], np.uint32), np.array([5, 0], np.uint32))
    y = -oracle.log_p(uniform24(out.ravel()))
    assert np.array_equal(g, -oracle.log_p(y))
    # 64-bit seed: high word is the second key word
    g2 = gumbel_noise(5 + (9 << 32), 2, 3, v)
    out2 = philox4x32_10(np.array([[i, 3, 2, 0] for i in range(4)], np.uint32), np.array([5, 9], np.uint32))
    assert np.array_equal(g2, -oracle.log_p(-oracle.log_p(uniform24(out2.ravel()))))


def test_gumbel_max_samples_softmax():
    # argmax(l + g) over independent keys is distributed as softmax(l)
    logits = np.array([0.0, 1.0, -0.5, 2.0, 0.3], np.float32)
    n = 200_000
    v = np.arange(5)
    g = gumbel_noise(77, 0, np.arange(n)[:, None], v[None, :])
    counts = np.bincount(np.argmax(logits[None, :] + g, axis=1), minlength=5).astype(np.float64)
    p = np.exp(logits.astype(np.float64))
    p /= p.sum()
    chi = stats.chisquare(counts, n * p)
    assert chi.pvalue > 1e-3, (counts, n * p)
