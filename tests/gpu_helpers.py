"""Host-side helpers of the GPU tests: move seeded inputs to the device, run
walks through the C ABI, and compare with the oracle."""
import numpy as np


def dev_inputs(d):
    import torch
    dev = torch.device("cuda", 0)
    out = {}
    if d["wtype"] == "int8":
        out["W"] = torch.from_numpy(np.ascontiguousarray(d["W"])).to(dev)
        out["w_scale"] = torch.from_numpy(d["s_w"]).to(dev)
    else:
        out["W"] = torch.from_numpy(d["W"].view(np.int16)).view(torch.bfloat16).to(dev)
        out["w_scale"] = None
    out["E"] = torch.from_numpy(d["E"]).to(dev)
    out["base"] = torch.from_numpy(d["base"].view(np.int16)).view(torch.bfloat16).to(dev)
    out["x0"] = torch.from_numpy(d["x0"].astype(np.int32)).to(dev)
    if d["head"] == "recurrent":
        out["A"] = torch.from_numpy(d["A"].view(np.int16)).view(torch.bfloat16).to(dev)
        out["c"] = torch.from_numpy(d["c"]).to(dev)
        out["h0"] = torch.from_numpy(d["h0"]).to(dev)
    else:
        out["A"] = out["c"] = out["h0"] = None
    return out


def make_head(d, t=None, **kw):
    from serial_draft_head_persistent_amd import Head
    t = t or dev_inputs(d)
    return Head(t["W"], t["E"], w_scale=t["w_scale"], A=t["A"], c=t["c"], head=d["head"], **kw), t


def run(head, t, *, base=None, x0=None, h0=None, temperature=0, seed=0, step_offset=0, exec="resident",
        logits=True, state=None, lse=False, fixed_latent=False, stress=False, winners=False):
    import torch
    base = t["base"] if base is None else base
    x0 = t["x0"] if x0 is None else x0
    h0 = t["h0"] if h0 is None else h0
    state = (head.head == "recurrent") if state is None else state
    o = head.walk(base, x0, h0=h0, temperature=temperature, seed=seed, step_offset=step_offset,
                  logits=logits, state=state, exec=exec, lse=lse, fixed_latent=fixed_latent,
                  stress=stress, winners=winners)
    torch.cuda.synchronize()
    err = head.error()
    assert err == "WTS_OK", err
    res = {"tokens": o["tokens"].cpu().numpy()}
    if logits:
        res["logits"] = o["logits"].view(torch.int16).cpu().numpy().view(np.uint16)
    if state:
        res["state"] = o["state"].cpu().numpy()
    if lse:
        res["lse"] = o["lse"].cpu().numpy()
    if winners:
        res["winners"] = o["winners"].cpu().numpy().view(np.uint64)
    return res


def oracle_walk(d, temperature=0, seed=0, step_offset=0, keep_z=False, base=None, x0=None, h0=None,
                keep_lse=False, fixed_latent=False):
    import oracle
    return oracle.walk(d["W"], d["E"], d["base"] if base is None else base,
                       d["x0"] if x0 is None else x0, wtype=d["wtype"], s_w=d["s_w"], head=d["head"],
                       A=d["A"], c=d["c"], h0=d["h0"] if h0 is None else h0,
                       temperature=temperature, seed=seed, step_offset=step_offset, keep_z=keep_z,
                       keep_lse=keep_lse, fixed_latent=fixed_latent)


# Log normaliser of the kernel: fp32 terms 2^(l log2 e - m) with one rounding
# each (plus the v_exp_f32 error of about 1 ulp), summed in fp32 over at most
# ~40 levels (per-lane running sums, 6 lane levels, waves, workgroups), then
# (m + log2 s) ln 2 in fp32.  Relative error of the sum <= ~60 * 2^-24 ~ 4e-6,
# i.e. an absolute error of about 4e-6 in lse, plus the final rounding of a
# value below 64 (< 4e-6).  The bar is 1e-5 * max(1, |lse|) (the values here
# are 5..40, so 5e-5..4e-4).
LSE_RTOL = 1e-5


def assert_lse_close(got_lse, logits_bits, what=""):
    """lse of every (b, t) against the float64 normaliser of the same logits."""
    from oracle.walk import log_normaliser
    B, gamma = got_lse.shape
    for b in range(B):
        for t in range(gamma):
            want = log_normaliser(logits_bits[b, t])
            err = abs(float(got_lse[b, t]) - want)
            assert err <= LSE_RTOL * max(1.0, abs(want)), f"{what}: lse b={b} t={t} gpu {got_lse[b, t]} want {want}"


def assert_exact(got, ref, what=""):
    """int8 path: tokens and bf16 logit bits identical."""
    tok_bad = np.argwhere(got["tokens"] != ref["tokens"])
    assert tok_bad.size == 0, f"{what}: token mismatch at {tok_bad[:5].tolist()}: " \
        f"gpu {got['tokens'][tuple(tok_bad[0])]} oracle {ref['tokens'][tuple(tok_bad[0])]}"
    if "logits" in got and ref.get("logits") is not None:
        bad = np.argwhere(got["logits"] != ref["logits"])
        assert bad.size == 0, f"{what}: {len(bad)} logit mismatches, first at {bad[:3].tolist()}"
    if "state" in got and ref.get("state") is not None:
        assert np.array_equal(got["state"], ref["state"]), f"{what}: final state differs"


def bf16_ulp(x):
    """Spacing of bf16 values at |x| (as float64)."""
    x = np.abs(np.asarray(x, np.float64))
    e = np.floor(np.log2(np.maximum(x, 2.0 ** -126)))
    return 2.0 ** (e - 7)


def assert_bf16_close(got, ref, what="", d=None, temperature=0, seed=0, step_offset=0, fixed_latent=False,
                      max_total=2):
    """bf16 W path: logits within 1e-2 relative (floor 1 in the denominator);
    tokens equal except where the oracle's own pre-rounding gap between its
    winner and the GPU's token is below max(1e-3 |z|, one bf16 ulp).

    After an accepted mismatch at step t the oracle is run again from step
    t + 1 for every row, starting from the GPU's tokens of step t (forced
    continuation; rows that agreed at t continue exactly as before), so the
    rest of the walk is still compared.  That needs the inputs `d` (and the
    walk's temperature, seed and step offset) and a Markov head; without `d`,
    or for a recurrent head, a row is not compared after its accepted
    mismatch.  At most one accepted mismatch per
    row and `max_total` per call.  Returns the number accepted."""
    from oracle.fp import bf16_to_f32
    B, gamma = ref["tokens"].shape
    accepted = 0
    per_row = np.zeros(B, np.int64)
    done = np.zeros(B, bool)          # rows no longer compared (no inputs to continue)
    cur = ref
    t0 = 0                            # step of cur's first column
    for t in range(gamma):
        forced = False
        for b in range(B):
            if done[b]:
                continue
            g = bf16_to_f32(got["logits"][b, t]).astype(np.float64)
            r = bf16_to_f32(cur["logits"][b, t - t0]).astype(np.float64)
            err = np.abs(g - r) / np.maximum(np.abs(r), 1.0)
            assert err.max() <= 1e-2, f"{what}: b={b} t={t} max rel err {err.max()}"
            xg, xr = int(got["tokens"][b, t]), int(cur["tokens"][b, t - t0])
            if xg != xr:
                z = cur["z"][b, t - t0].astype(np.float64)
                gap = z[xr] - z[xg]
                tol = max(1e-3 * abs(z[xr]), bf16_ulp(z[xr]))
                assert gap < tol, f"{what}: token b={b} t={t} gpu {xg} oracle {xr} gap {gap} > {tol}"
                accepted += 1
                per_row[b] += 1
                assert per_row[b] <= 1, f"{what}: a second accepted near-tie mismatch in row {b} (t={t})"
                if d is None or d["head"] == "recurrent":
                    # a recurrent continuation would need the hidden state after
                    # step t, which the walk does not expose per step
                    done[b] = True
                elif not fixed_latent:
                    forced = True
        if forced and t + 1 < gamma:
            import oracle
            x_next = got["tokens"][:, t].astype(np.int32)
            cur = oracle.walk(d["W"], d["E"], d["base"][:, t + 1:], x_next, wtype=d["wtype"], s_w=d["s_w"],
                              head=d["head"], A=d["A"], c=d["c"], h0=d["h0"], temperature=temperature, seed=seed,
                              step_offset=step_offset + t + 1, keep_z=True)
            t0 = t + 1
    assert accepted <= max_total, f"{what}: {accepted} accepted near-tie mismatches (bound {max_total})"
    return accepted
