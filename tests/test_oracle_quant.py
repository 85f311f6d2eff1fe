"""Pins of the hi/lo latent quantiser: exact reconstruction bound, special cases."""
from fractions import Fraction

import numpy as np

from oracle.quant import quant_hilo


def _check_bound(u):
    hi, lo, s_hi, s_lo = quant_hilo(u)
    assert hi.dtype == np.int8 and lo.dtype == np.int8
    assert np.all(np.abs(hi.astype(int)) <= 127) and np.all(np.abs(lo.astype(int)) <= 127)
    sl = Fraction(float(s_lo))
    assert Fraction(float(s_hi)) == 256 * sl          # the two scales differ by exactly 2^8
    for k in range(u.shape[0]):
        uk = Fraction(float(u[k]))
        rec = sl * (256 * int(hi[k]) + int(lo[k]))
        assert abs(uk - rec) <= sl + abs(uk) * Fraction(1, 2 ** 23), (k, float(uk), float(rec))


def test_reconstruction_bound_random():
    rng = np.random.default_rng(5)
    for trial in range(20):
        scale = 10.0 ** rng.uniform(-4, 3)
        u = (rng.standard_normal(256) * scale).astype(np.float32)
        _check_bound(u)


def test_reconstruction_heavy_tail_and_small_r():
    rng = np.random.default_rng(6)
    _check_bound(rng.standard_t(2, 256).astype(np.float32))
    _check_bound(np.array([0.5, -0.25, 1e-6, 0.0], dtype=np.float32))


def test_hi_is_rounded_u_over_s_hi():
    # hi equals round(u * 127 / amax) whenever that product is not near a tie
    rng = np.random.default_rng(7)
    u = rng.standard_normal(256).astype(np.float32)
    hi, lo, s_hi, s_lo = quant_hilo(u)
    amax = np.max(np.abs(u.astype(np.float64)))
    t = u.astype(np.float64) * 127.0 / amax
    far = np.abs(np.abs(t - np.floor(t)) - 0.5) > 1e-4
    assert np.array_equal(hi[far], np.rint(t[far]).astype(np.int8))
    assert abs(int(hi[np.argmax(np.abs(u))])) == 127


def test_zero_vector():
    hi, lo, s_hi, s_lo = quant_hilo(np.zeros(256, np.float32))
    assert not hi.any() and not lo.any() and s_hi == 0 and s_lo == 0


def test_odd_symmetry_and_batch():
    rng = np.random.default_rng(8)
    u = rng.standard_normal((3, 256)).astype(np.float32)
    a = quant_hilo(u)
    b = quant_hilo(-u)
    assert np.array_equal(a[0], -b[0]) and np.array_equal(a[1], -b[1])
    assert np.array_equal(a[2], b[2])
    for i in range(3):
        one = quant_hilo(u[i])
        assert np.array_equal(one[0], a[0][i]) and np.array_equal(one[1], a[1][i]) and one[2] == a[2][i]
