"""Float helpers of the oracle: bf16 rounding and portable log/exp/tanh.

Test infrastructure only (see ``oracle/__init__``).

Weights That Stay, Fig. 7: the projection result is rounded to bf16 a single
time.  bf16 here is the upper 16 bits of an IEEE binary32 value, rounded to
nearest even.

log_p / exp_p / tanh_p are *specifications* of the elementary functions used
by T=1 Gumbel noise (Fig. 10, bottom row) and by the recurrent head's tanh
(Fig. 13).  The pages do not fix them; both this oracle and the HIP kernels
implement the same sequence of binary32 operations, written separately from
this description:

  log_p(x), x > 0 normal:
    x = m * 2^e with m in [0.5, 1) (from the exponent bits);
    if m < 0.70710677: m = 2m, e = e - 1;      (m now in [0.7071, 1.4142))
    f = m - 1 (exact);  s = f / (2 + f);  z = s*s
    p = (((z/9 + 1/7) z + 1/5) z + 1/3) z     (coefficients rounded to fp32)
    lm = 2 (s + s p)                          (series of 2 atanh(s))
    return e*LN2_HI + (e*LN2_LO + lm)        (Cody-Waite split of ln 2)
  exp_p(y), -20 <= y <= 0:
    n = rint(y * (1/ln2));  f = (y - n LN2_HI) - n LN2_LO
    p = degree-8 Taylor polynomial of e^f in Horner form;  return p * 2^n
  tanh_p(x), a = |x|:
    a >= 10: 1;  a < 0.25: odd Taylor series through x^11 (Horner in x^2);
    else q = exp_p(-2a), r = (1 - q) / (1 + q);  result carries the sign of x.

Pinned in tests/test_oracle_fp.py against fp64 libm (ulp bounds) and, for
bf16, against torch's CPU float->bfloat16 conversion.
"""
import numpy as np

F32 = np.float32


def _f32(x):
    return np.asarray(x, dtype=np.float32)


def bf16_rne(x):
    """float32 -> bf16 bits (uint16), round to nearest, ties to even.

    Finite inputs only (the walk never produces NaN); overflow gives +-inf.
    """
    b = _f32(x).view(np.uint32).astype(np.uint64)
    r = (b + np.uint64(0x7FFF) + ((b >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return r.astype(np.uint16)


def bf16_to_f32(u):
    """bf16 bits (uint16) -> float32, exact."""
    return (np.asarray(u, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


# fp32 constants (each the binary32 value nearest to the stated rational)
LN2_HI = np.array([0x3F317200], dtype=np.uint32).view(np.float32)[0]   # 0.693145751953125
LN2_LO = F32(np.log(2.0) - float(LN2_HI))
INV_LN2 = F32(1.0 / np.log(2.0))
SQRT_HALF = F32(0.70710677)
_LOG_C = [F32(1.0 / 9.0), F32(1.0 / 7.0), F32(1.0 / 5.0), F32(1.0 / 3.0)]
_EXP_C = [F32(1.0 / 40320.0), F32(1.0 / 5040.0), F32(1.0 / 720.0), F32(1.0 / 120.0),
          F32(1.0 / 24.0), F32(1.0 / 6.0), F32(0.5), F32(1.0), F32(1.0)]
_TANH_C = [F32(-1382.0 / 155925.0), F32(62.0 / 2835.0), F32(-17.0 / 315.0),
           F32(2.0 / 15.0), F32(-1.0 / 3.0)]


def log_p(x):
    """Portable natural log of positive normal binary32 values (see module doc)."""
    x = _f32(x)
    bits = x.view(np.uint32)
    e = ((bits >> np.uint32(23)) & np.uint32(0xFF)).astype(np.int32) - 126
    m = ((bits & np.uint32(0x007FFFFF)) | np.uint32(0x3F000000)).view(np.float32)
    small = m < SQRT_HALF
    m = np.where(small, m * F32(2.0), m).astype(np.float32)
    e = np.where(small, e - 1, e)
    f = m - F32(1.0)
    s = f / (F32(2.0) + f)
    z = s * s
    p = _LOG_C[0] * z
    p = (p + _LOG_C[1]) * z
    p = (p + _LOG_C[2]) * z
    p = (p + _LOG_C[3]) * z
    lm = F32(2.0) * (s + s * p)
    ef = e.astype(np.float32)
    return (ef * LN2_HI + (ef * LN2_LO + lm)).astype(np.float32)


def exp_p(y):
    """Portable e^y for binary32 y in [-20, 0] (see module doc)."""
    y = _f32(y)
    n = np.rint(y * INV_LN2).astype(np.float32)
    f = (y - n * LN2_HI) - n * LN2_LO
    p = _EXP_C[0]
    for c in _EXP_C[1:]:
        p = p * f + c
    scale = ((n.astype(np.int32) + 127).astype(np.uint32) << np.uint32(23)).view(np.float32)
    return (p * scale).astype(np.float32)


def tanh_p(x):
    """Portable tanh of binary32 values (see module doc)."""
    x = _f32(x)
    a = np.abs(x)
    # mid range: (1 - q) / (1 + q), q = e^{-2a}
    am = np.minimum(a, F32(10.0))
    q = exp_p(F32(-2.0) * am)
    mid = (F32(1.0) - q) / (F32(1.0) + q)
    # small range: odd Taylor series, Horner in x^2
    x2 = x * x
    t = _TANH_C[0]
    for c in _TANH_C[1:]:
        t = t * x2 + c
    small = x + x * (x2 * t)
    r = np.where(a >= F32(10.0), F32(1.0), mid)
    r = np.where(x < 0, -r, r).astype(np.float32)
    return np.where(a < F32(0.25), small, r).astype(np.float32)
