"""Counter-based noise for T=1 Gumbel-max selection -- oracle side.

Test infrastructure only (see ``oracle/__init__``).

The pages measure T=1 walks (Weights That Stay, Fig. 10, bottom row) without
giving the sampler.  Reading used here: Gumbel-max with Philox4x32-10 noise
(Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as easy as 1, 2, 3",
SC'11), written from the paper's round function:

    round:  (c0, c1, c2, c3), key (k0, k1)
            hi0:lo0 = M0 * c0,  hi1:lo1 = M1 * c2       (32x32 -> 64 bit)
            -> (hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0)
    key schedule between rounds: k0 += W0, k1 += W1 (mod 2^32); 10 rounds.
    M0 = 0xD2511F53, M1 = 0xCD9E8D57, W0 = 0x9E3779B9, W1 = 0xBB67AE85.

Noise for batch row b, walk step s (step_offset + t) and vocabulary index v:
counter = (v >> 2, s, b, 0), key = (seed & 0xFFFFFFFF, seed >> 32); word
w = output[v & 3];  U = (2 (w >> 9) + 1) * 2^-24  (exact in binary32, in
(0, 1));  g = -log_p(-log_p(U)).

Pinned by the published all-zero known-answer vector of Philox4x32-10 and,
for the Gumbel-max sampler, by a chi-square test of token frequencies
against softmax(logits) (tests/test_oracle_philox.py).
"""
import numpy as np

from .fp import log_p

M0 = np.uint64(0xD2511F53)
M1 = np.uint64(0xCD9E8D57)
W0 = np.uint32(0x9E3779B9)
W1 = np.uint32(0xBB67AE85)
_MASK = np.uint64(0xFFFFFFFF)


def philox4x32_10(ctr, key):
    """ctr: uint32[..., 4], key: uint32[..., 2] (broadcastable) -> uint32[..., 4]."""
    ctr = np.asarray(ctr, dtype=np.uint32)
    key = np.asarray(key, dtype=np.uint32)
    c0, c1, c2, c3 = (ctr[..., i].astype(np.uint64) for i in range(4))
    k0 = key[..., 0].astype(np.uint64)
    k1 = key[..., 1].astype(np.uint64)
    for rnd in range(10):
        if rnd > 0:
            k0 = (k0 + np.uint64(W0)) & _MASK
            k1 = (k1 + np.uint64(W1)) & _MASK
        p0 = M0 * c0
        p1 = M1 * c2
        hi0, lo0 = p0 >> np.uint64(32), p0 & _MASK
        hi1, lo1 = p1 >> np.uint64(32), p1 & _MASK
        c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0
    return np.stack([c0, c1, c2, c3], axis=-1).astype(np.uint32)


def uniform24(w):
    """uint32 word -> binary32 U = (2 (w >> 9) + 1) * 2^-24, exactly."""
    w = np.asarray(w, dtype=np.uint32)
    n = (w >> np.uint32(9)).astype(np.uint32) * np.uint32(2) + np.uint32(1)
    return (n.astype(np.float32) * np.float32(2.0 ** -24)).astype(np.float32)


def gumbel_noise(seed, b, step, v):
    """Gumbel noise g(seed, b, step, v) (binary32); b, step, v broadcast together."""
    v, step, b = np.broadcast_arrays(np.asarray(v, dtype=np.int64),
                                     np.asarray(step, dtype=np.int64),
                                     np.asarray(b, dtype=np.int64))
    seed = int(seed)
    ctr = np.zeros(v.shape + (4,), dtype=np.uint32)
    ctr[..., 0] = (v >> 2).astype(np.uint32)
    ctr[..., 1] = (step & 0xFFFFFFFF).astype(np.uint32)
    ctr[..., 2] = b.astype(np.uint32)
    key = np.array([seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF], dtype=np.uint32)
    out = philox4x32_10(ctr, key)
    w = np.take_along_axis(out, (v & 3)[..., None], axis=-1)[..., 0]
    u = uniform24(w)
    y = -log_p(u)
    return (-log_p(y)).astype(np.float32)
