"""Two-int8-vector (hi/lo) representation of the latent -- oracle side.

Test infrastructure only (see ``oracle/__init__``).

Weights That Stay, Fig. 7: the latent u is represented by two int8 vectors
that are multiplied by W together; their scaled results are summed.  The
pages do not give the scales.  Reading used here (symmetric, power-of-two
ratio between the two scales, so that s_lo * (256 hi + lo) reconstructs u):

    amax  = max_k |u_k|                     (if 0: hi = lo = 0, scales 0)
    s_hi  = fp32(amax / 127)
    inv   = fp32(127 / amax)
    hi_k  = clamp(rint(fp32(u_k * inv)), -127, 127)
    res_k = fp32(u_k - fp32(s_hi * hi_k))
    lo_k  = clamp(rint(fp32(res_k * fp32(inv * 256))), -127, 127)
    s_lo  = s_hi * 2^-8                     (exact)

rint rounds half to even.  Pinned in tests/test_oracle_quant.py by the exact
reconstruction bound |u_k - s_lo (256 hi_k + lo_k)| <= s_lo + 2^-23 |u_k|
(evaluated with Fractions), by the zero vector, and by symmetry.
"""
import numpy as np

F32 = np.float32


def quant_hilo(u):
    """u: float32[..., r] -> (hi int8[..., r], lo int8[..., r], s_hi f32[...], s_lo f32[...])."""
    u = np.asarray(u, dtype=np.float32)
    amax = np.max(np.abs(u), axis=-1)
    zero = amax == F32(0.0)
    safe = np.where(zero, F32(1.0), amax).astype(np.float32)
    s_hi = (safe / F32(127.0)).astype(np.float32)
    inv = (F32(127.0) / safe).astype(np.float32)
    hi = np.clip(np.rint(u * inv[..., None]), -127, 127).astype(np.float32)
    res = u - s_hi[..., None] * hi
    lo = np.clip(np.rint(res * (inv * F32(256.0))[..., None]), -127, 127).astype(np.float32)
    s_hi = np.where(zero, F32(0.0), s_hi).astype(np.float32)
    hi = np.where(zero[..., None], F32(0.0), hi)
    lo = np.where(zero[..., None], F32(0.0), lo)
    s_lo = (s_hi * F32(1.0 / 256.0)).astype(np.float32)
    return hi.astype(np.int8), lo.astype(np.int8), s_hi, s_lo
