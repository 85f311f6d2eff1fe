"""Seeded synthetic inputs for the serial draft walk.

Shared by the oracle tests, the GPU parity tests and the benchmark.  Holds
none of the walk's arithmetic: it only draws arrays (and converts draws to
the storage formats int8 + per-row scale and bf16 with torch's CPU cast).

The pages benchmark released draft heads with a Qwen3 vocabulary (151,936)
and a 248k vocabulary at rank 256 (Weights That Stay, Figs. 3, 10, 13, 14);
those heads are not available, so seeded draws of the same shapes stand in:

  W source  Student-t(nu=4) [V, r] (heavy-tailed, like trained weights);
            int8: per-row absmax quantisation, s_w = fp32(max|t| / 127),
            W_q = clip(rint(t / s_w), -127, 127);  bf16: bf16(t)
  E         N(0, 1/r) fp32 [V, r]
  base      N(0, 2) rounded to bf16 [B, gamma, V]
  x0        uniform integers in [0, V) [B]
  A         N(0, 0.5/r) rounded to bf16 [r, r]  (recurrent head only)
  c         N(0, 0.1) fp32 [r];  h0  N(0, 1) fp32 [B, r]
Second parameters of N are variances.  One numpy PCG64 generator per call,
seeded with ``seed``; draw order W, E, base, x0, A, c, h0.
"""
import numpy as np

R = 256

# Named workloads (sizes of the pages' microbenchmarks).
CONFIGS = {
    0: dict(name="markov-int8-v8192-b1-g4", head="markov", wtype="int8", V=8192, B=1, gamma=4),
    1: dict(name="markov-int8-v151936-b1-g16", head="markov", wtype="int8", V=151936, B=1, gamma=16),
    2: dict(name="markov-int8-v151936-sweep", head="markov", wtype="int8", V=151936, B=16, gamma=16),
    3: dict(name="markov-bf16-v248320", head="markov", wtype="bf16", V=248320, B=1, gamma=16),
    4: dict(name="recurrent-int8-v151936-b1-g15", head="recurrent", wtype="int8", V=151936, B=1, gamma=15),
}


def _to_bf16_bits(x):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def make_inputs(V, r=R, B=1, gamma=16, *, wtype="int8", head="markov", seed=0,
                W_source=None):
    """Draw one workload.  Returns a dict of numpy arrays (host memory)."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed)))
    out = dict(V=V, r=r, B=B, gamma=gamma, wtype=wtype, head=head, seed=seed)
    t = rng.standard_t(4, size=(V, r)) if W_source is None else np.asarray(W_source, np.float64)
    if wtype == "int8":
        amax = np.max(np.abs(t), axis=1)
        s_w = (amax / 127.0).astype(np.float32)
        s_w = np.where(s_w == 0, np.float32(1.0), s_w).astype(np.float32)
        out["W"] = np.clip(np.rint(t / s_w.astype(np.float64)[:, None]), -127, 127).astype(np.int8)
        out["s_w"] = s_w
    else:
        out["W"] = _to_bf16_bits(t.astype(np.float32))
        out["s_w"] = None
    del t
    out["E"] = rng.normal(0.0, np.sqrt(1.0 / r), size=(V, r)).astype(np.float32)
    out["base"] = _to_bf16_bits(rng.normal(0.0, np.sqrt(2.0), size=(B, gamma, V)))
    out["x0"] = rng.integers(0, V, size=B).astype(np.int32)
    if head == "recurrent":
        out["A"] = _to_bf16_bits(rng.normal(0.0, np.sqrt(0.5 / r), size=(r, r)))
        out["c"] = rng.normal(0.0, np.sqrt(0.1), size=r).astype(np.float32)
        out["h0"] = rng.normal(0.0, 1.0, size=(B, r)).astype(np.float32)
    else:
        out["A"] = out["c"] = out["h0"] = None
    return out


def config_inputs(k, *, B=None, gamma=None, seed=0, V=None):
    """Inputs of named workload k, optionally with another B / gamma / V."""
    c = CONFIGS[k]
    return make_inputs(V or c["V"], R, B or c["B"], gamma or c["gamma"],
                       wtype=c["wtype"], head=c["head"], seed=seed)
