"""Pins of the oracle's float helpers: bf16 rounding vs torch, log/exp/tanh vs fp64 libm."""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle.fp import bf16_rne, bf16_to_f32, log_p, exp_p, tanh_p

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _ulp32(x):
    x = np.abs(np.asarray(x, np.float64))
    e = np.floor(np.log2(np.maximum(x, 2.0 ** -126)))
    return 2.0 ** (e - 23)


def test_bf16_rne_matches_torch_random():
    rng = np.random.default_rng(1)
    bits = rng.integers(0, 2 ** 32, size=2_000_000, dtype=np.uint64).astype(np.uint32)
    x = bits.view(np.float32)
    x = x[np.isfinite(x)]
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(bf16_rne(x), ref)


def test_bf16_rne_edge_cases():
    # exact halfway points (ties to even), just above/below, zero signs, largest finite
    base = np.array([0x3F800000, 0x3F808000, 0x3F818000, 0x3F808001, 0x3F807FFF,
                     0x00000000, 0x80000000, 0x7F7FFFFF, 0xFF7FFFFF, 0x00008000,
                     0x00018000, 0x7F7F8000, 0x80008000], dtype=np.uint32)
    x = base.view(np.float32)
    ref = torch.from_numpy(x.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(bf16_rne(x), ref)
    assert bf16_rne(np.float32(1.0)) == 0x3F80
    assert bf16_rne(np.array([0x3F808000], np.uint32).view(np.float32))[0] == 0x3F80  # tie -> even
    assert bf16_rne(np.array([0x3F818000], np.uint32).view(np.float32))[0] == 0x3F82  # tie -> even


def test_bf16_roundtrip_exact():
    u = np.arange(0, 65536, dtype=np.uint32).astype(np.uint16)
    f = bf16_to_f32(u)
    ok = np.isfinite(f)
    assert np.array_equal(bf16_rne(f[ok]), u[ok])


def test_log_p_ulp_bound_dense():
    rng = np.random.default_rng(2)
    x = np.concatenate([
        np.exp(rng.uniform(np.log(2.0 ** -24), np.log(20.0), 400_000)),
        1.0 + rng.uniform(-1e-3, 1e-3, 100_000),
        rng.uniform(0.5, 2.0, 200_000),
        np.float32(2.0) ** np.arange(-60, 60, dtype=np.float64),
    ]).astype(np.float32)
    got = log_p(x).astype(np.float64)
    ref = np.log(x.astype(np.float64))
    err = np.abs(got - ref) / _ulp32(ref)
    nz = ref != 0
    assert np.max(err[nz]) <= 4.0
    assert log_p(np.float32(1.0)) == 0.0


def test_exp_p_ulp_bound_dense():
    rng = np.random.default_rng(3)
    y = np.concatenate([rng.uniform(-20.0, 0.0, 500_000), -np.arange(0, 20, 0.25)]).astype(np.float32)
    got = exp_p(y).astype(np.float64)
    ref = np.exp(y.astype(np.float64))
    assert np.max(np.abs(got - ref) / _ulp32(ref)) <= 4.0
    assert exp_p(np.float32(0.0)) == 1.0


def test_tanh_p_ulp_bound_and_symmetry():
    rng = np.random.default_rng(4)
    x = np.concatenate([rng.uniform(-12, 12, 500_000), rng.uniform(-0.3, 0.3, 200_000),
                        np.array([0.25, -0.25, 9.99, 10.0, -10.0, 1e-30], dtype=np.float64)]).astype(np.float32)
    got = tanh_p(x).astype(np.float64)
    ref = np.tanh(x.astype(np.float64))
    nz = ref != 0
    assert np.max(np.abs(got - ref)[nz] / _ulp32(ref[nz])) <= 4.0
    assert np.array_equal(tanh_p(-x), -tanh_p(x))
    assert tanh_p(np.float32(0.0)) == 0.0


def test_log_p_gumbel_domain_monotone():
    # the Gumbel construction needs -log_p(U) > 0 for every U in (0, 1)
    w = np.arange(0, 2 ** 23, 97, dtype=np.uint32) << np.uint32(9)
    u = oracle.uniform24(w)
    y = -log_p(u)
    assert np.all(y > 0) and np.all(np.isfinite(-log_p(y)))
    assert np.all(np.diff(y) <= 0)  # U increasing -> -log U non-increasing
