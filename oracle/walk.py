"""The serial draft walk, step by step -- oracle side.

Test infrastructure only (see ``oracle/__init__``).

Weights That Stay (arXiv 2611.00506): each step of the serial head projects a
small state through the same vocabulary-sized matrix W, adds base logits,
selects one token over the whole vocabulary and advances the state (abstract;
Fig. 2).  Markov head: the latent of step t is the embedding row of the token
chosen before it.  Recurrent head (Fig. 13): h_t = tanh(A h_{t-1} + E[x_{t-1}]
+ c) and the latent is h_t.  int8 W with per-row scales uses the two-int8
latent of Fig. 7; bf16 W (Fig. 14) uses the latent rounded once to bf16.

Readings of what the pages leave open (each one is listed with its reason in
the design notes):
  * step t (0-based) reads base[b, t, :] and emits token x_{t+1}; x_0 is an
    input; the walk emits gamma tokens.
  * int8 epilogue, binary32, in this order (one rounding per operation):
        z = fp32(acc_hi) * s_hi + fp32(acc_lo) * s_lo;  z = z * s_w[v]
        z = z + fp32(base[b, t, v]);  logit = bf16_rne(z)
    (acc_* are exact int32 dot products; |acc| <= 256*127^2 < 2^24, so the
    conversion to binary32 is exact.)
  * bf16 projection: exact sum of the bf16 x bf16 products (fp64), rounded
    once to binary32, then + base, then bf16_rne.  The GPU accumulates in
    fp32 in its own order, so the bf16 path is compared within a tolerance.
  * selection is on the returned bf16 logit widened to binary32 (T=0), or on
    fp32(logit + g) with the Gumbel noise g of ``oracle.philox`` (T=1);
    the largest score wins, ties go to the lowest index, -0 equals +0.
  * recurrent pre-activation: the pages give h = tanh(A h + E[x] + c) and no
    summation order, so the plainest one is taken: acc_j = sum_k A[j,k] h[k]
    as one chain in ascending k starting from +0, each term multiplied and
    then added with one binary32 rounding per operation (no fused
    multiply-add); pre = (acc_j + E[x][j]) + c[j]; h_j = tanh_p(pre).
  * fixed-latent probe (Fig. 13b): every step projects and selects with the
    latent of step 0 (Markov: E[x_0]; recurrent: h_1); the chosen tokens are
    emitted but do not feed back.
  * per-step normaliser of the draft distribution: at T=1 the Gumbel-max
    choice samples q(v) = exp(l_v) / sum_u exp(l_u) over the returned bf16
    logits l (widened exactly); its log normaliser lse = ln sum_u exp(l_u) is
    an optional output, taken here in float64.
"""
import math

import numpy as np

from .fp import bf16_rne, bf16_to_f32, tanh_p
from .quant import quant_hilo
from .philox import gumbel_noise

F32 = np.float32


def order_key(score, v):
    """64-bit selection key: larger key <=> larger score, then lower index.

    ord32 maps binary32 bits to an unsigned order (-0 first canonicalised to
    +0); the low word is 0xFFFFFFFF - v.  Used by tests to check that a key
    maximum and (value, -index) lexicographic order agree.
    """
    s = np.asarray(score, dtype=np.float32) + F32(0.0)       # -0 -> +0
    bits = s.view(np.uint32).astype(np.uint64)
    neg = (bits >> np.uint64(31)) == 1
    o = np.where(neg, bits ^ np.uint64(0xFFFFFFFF), bits ^ np.uint64(0x80000000))
    return (o << np.uint64(32)) | (np.uint64(0xFFFFFFFF) - np.asarray(v, dtype=np.uint64))


def select_token(scores):
    """Index of the maximum of a binary32 vector; lowest index among equals."""
    scores = np.asarray(scores, dtype=np.float32)
    m = np.max(scores)
    return int(np.flatnonzero(scores == m)[0])


def project_int8(Wq_f64, hi, lo):
    """Exact int32 dot products W_q[v,:] . hi and W_q[v,:] . lo for all v.

    Wq_f64: W_q as float64 [V, r]; hi, lo: int8 [r] or [B, r].
    Every partial sum is an integer below 2^53 in magnitude, so the fp64
    product is exact whatever order BLAS adds in.  Returns int64 arrays.
    """
    h = np.asarray(hi, dtype=np.float64)
    lw = np.asarray(lo, dtype=np.float64)
    acc_hi = (Wq_f64 @ h.T).T
    acc_lo = (Wq_f64 @ lw.T).T
    return acc_hi.astype(np.int64), acc_lo.astype(np.int64)


def epilogue_int8(acc_hi, acc_lo, s_hi, s_lo, s_w, base_bits):
    """Fig. 7 epilogue: scaled sums, row scale, + base, one bf16 rounding.

    Returns (logit bits uint16, z float32) with z the value before rounding.
    """
    z = acc_hi.astype(np.float32) * F32(s_hi) + acc_lo.astype(np.float32) * F32(s_lo)
    z = z * np.asarray(s_w, dtype=np.float32)
    z = z + bf16_to_f32(base_bits)
    return bf16_rne(z), z.astype(np.float32)


def project_bf16(Wb_f64, u_bits):
    """sum_k W[v,k] * u[k] over bf16 operands, rounded once to binary32.

    Wb_f64: bf16 W widened to float64 [V, r]; u_bits: bf16 latent bits [r].
    bf16 x bf16 products are exact in fp64; the fp64 sum is the reference
    (its own rounding is far below the bf16 tolerance).
    """
    u = bf16_to_f32(u_bits).astype(np.float64)
    return (Wb_f64 @ u).astype(np.float32)


def recurrent_preact(A_f32, h, e_row, c):
    """Pre-activation of the recurrent state, ((sum_k A[:,k] h[k]) + e_row) + c.

    Weights That Stay, Fig. 13 (recurrent heads): the state update is
    h = tanh(A h + E[x] + c); no summation order is given, so the sum is one
    binary32 chain in ascending k from +0: acc = RN(acc + RN(A[j,k] h[k])),
    a separate rounding for every product and every addition.  A_f32 holds
    the bf16 matrix widened exactly to binary32 ([r, r], row j = output j).
    """
    acc = np.zeros(A_f32.shape[0], dtype=np.float32)
    for k in range(h.shape[-1]):
        prod = A_f32[:, k] * np.float32(h[k])      # binary32 product, rounded once
        acc = acc + prod                            # binary32 sum, rounded once
    pre = acc + np.asarray(e_row, dtype=np.float32)
    return pre + np.asarray(c, dtype=np.float32)


def recurrent_update(A_f32, h, e_row, c):
    """h_new = tanh_p(recurrent_preact(A_f32, h, e_row, c)) (Fig. 13)."""
    return tanh_p(recurrent_preact(A_f32, h, e_row, c))


def log_normaliser(logit_bits):
    """ln sum_v exp(l_v) of one step's bf16 logits, in float64.

    The log normaliser of the draft distribution q(v) = exp(l_v - lse) that a
    Gumbel-max walk at T=1 samples from (Fig. 10, T=1).  Definition, with the
    largest logit factored out so no term overflows; math.fsum adds the terms
    with a single final rounding.
    """
    l = bf16_to_f32(np.asarray(logit_bits, dtype=np.uint16)).astype(np.float64)
    m = float(l.max())
    return m + math.log(math.fsum(np.exp(l - m).tolist()))


def walk(W, E, base, x0, *, wtype="int8", s_w=None, head="markov", A=None,
         c=None, h0=None, temperature=0, seed=0, step_offset=0,
         keep_logits=True, keep_z=False, keep_lse=False, fixed_latent=False):
    """Run the walk for every batch row.

    W: int8 [V, r] (wtype 'int8', with s_w float32 [V]) or bf16 bits uint16
    [V, r] (wtype 'bf16').  E: float32 [V, r].  base: bf16 bits [B, gamma, V].
    x0: int [B].  Recurrent head: A bf16 bits [r, r], c float32 [r], h0
    float32 [B, r].  temperature 0 (greedy) or 1 (Gumbel-max).

    fixed_latent: the probe of Fig. 13b -- every step uses the latent of step
    0 and the tokens do not feed back.

    Returns dict with 'tokens' int32 [B, gamma], 'logits' uint16 [B, gamma, V]
    (if keep_logits), 'z' float32 [B, gamma, V] (if keep_z; the value that
    is rounded to the logit), 'lse' float64 [B, gamma] (if keep_lse; the log
    normaliser of each step's logits), 'state' float32 [B, r] (recurrent).
    """
    if temperature not in (0, 1):
        raise ValueError("temperature must be 0 or 1")
    base = np.asarray(base, dtype=np.uint16)
    B, gamma, V = base.shape
    Vw, r = W.shape
    assert Vw == V and E.shape == (V, r)
    x_prev = np.asarray(x0, dtype=np.int64).copy()
    assert x_prev.shape == (B,) and np.all((x_prev >= 0) & (x_prev < V))
    W64 = np.asarray(W, dtype=np.float64) if wtype == "int8" else \
        bf16_to_f32(W).astype(np.float64)
    if head == "recurrent":
        A32 = bf16_to_f32(A)
        h = np.asarray(h0, dtype=np.float32).copy()
    tokens = np.zeros((B, gamma), dtype=np.int32)
    logits = np.zeros((B, gamma, V), dtype=np.uint16) if keep_logits else None
    zs = np.zeros((B, gamma, V), dtype=np.float32) if keep_z else None
    lse = np.zeros((B, gamma), dtype=np.float64) if keep_lse else None
    vidx = np.arange(V, dtype=np.int64)
    for t in range(gamma):
        if head == "markov":
            lat = E[x_prev]                                   # [B, r]
        elif t == 0 or not fixed_latent:
            for b in range(B):
                h[b] = recurrent_update(A32, h[b], E[x_prev[b]], c)
            lat = h
        if wtype == "int8":
            hi, lo, s_hi, s_lo = quant_hilo(lat)
            acc_hi, acc_lo = project_int8(W64, hi, lo)        # [B, V]
        for b in range(B):
            if wtype == "int8":
                lg, z = epilogue_int8(acc_hi[b], acc_lo[b], s_hi[b], s_lo[b], s_w, base[b, t])
            else:
                p = project_bf16(W64, bf16_rne(lat[b]))
                z = (p + bf16_to_f32(base[b, t])).astype(np.float32)
                lg = bf16_rne(z)
            score = bf16_to_f32(lg)
            if temperature == 1:
                score = (score + gumbel_noise(seed, b, step_offset + t, vidx)).astype(np.float32)
            x = select_token(score)
            tokens[b, t] = x
            if keep_logits:
                logits[b, t] = lg
            if keep_z:
                zs[b, t] = z
            if keep_lse:
                lse[b, t] = log_normaliser(lg)
        if not fixed_latent:
            x_prev = tokens[:, t].astype(np.int64)
    out = {"tokens": tokens, "logits": logits, "z": zs, "lse": lse}
    out["state"] = h if head == "recurrent" else None
    return out
