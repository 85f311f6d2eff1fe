"""Benchmark of the serial draft walk on one MI355X.

Workload (the headline configuration): Markov head, int8 W with per-row
scales, V = 151,936, r = 256, B = 1, gamma = 16, greedy; W fully resident in
one persistent kernel.  One "step" of this benchmark is one complete walk
(gamma serial head steps) over one batch of synthetic input already resident
in HBM.

Prints one JSON line: microseconds per walk (lower is better), the per-step
cost and entry cost fitted over gamma in {1, 7, 16}, achieved W-read
bandwidth, the roofline of the dominant kernel, the CPU oracle on the host
cores, and side measurements (batch and temperature sweep, bf16 248k,
recurrent head, fused-streaming and step-wise execution).

    python bench.py [--steps K] [--warmup W] [--quick] [--no-cpu]
    python bench.py --profile-walk NAME   (one workload's walks only, for rocprofv3)

Roofline denominators are measured on the same device by wts_roofline()
(LDS and MFMA operand rates, shader clock, HBM and memory-side-cache stream
rates, the cross-workgroup selection round in isolation, VALU issue rate);
the published peaks are reported beside them.
"""
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
I8_PEAK_TOPS = 5000.0          # dense int8 MFMA, published (TOP/s)
BF16_PEAK_TFLOPS = 2500.0      # dense bf16 MFMA, published


# Workloads whose walks --profile-walk runs alone (name: (config, B, gamma,
# T, create kwargs)), for rocprofv3 kernel traces and counter passes.
PROFILE_WALKS = {
    "markov-int8-v151936-b1-g16": (1, 1, 16, 0, {}),
    "markov-bf16-v248320-b1-g16": (3, 1, 16, 0, {}),
    "markov-bf16-v248320-b16-g16": (3, 16, 16, 0, {}),
    "markov-int8-v151936-b16-g16-partial": (2, 16, 16, 0, {"resident_tiles": 2, "lds_tiles": 0}),
    "markov-int8-v151936-b16-g16-t1": (2, 16, 16, 1, {}),
}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--quick", action="store_true", help="headline only: no sweeps, no CPU baseline")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--profile", action="store_true",
                    help="only the timed headline walks (for rocprofv3 runs)")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="turn two rocprofv3 --pmc counter_collection.csv files (FETCH_SIZE, WRITE_SIZE) "
                         "of a --profile --copy-calib run into profiles/" + "walk_traffic.json and exit")
    ap.add_argument("--summarize-counters", metavar="CSV",
                    help="print the per-dispatch mean of every counter in a rocprofv3 --pmc "
                         "counter_collection.csv for the headline kernel, and exit")
    ap.add_argument("--profile-walk", choices=sorted(PROFILE_WALKS),
                    help="run only the timed walks of one workload (for rocprofv3 runs)")
    ap.add_argument("--copy-calib", action="store_true",
                    help="with --profile or --profile-walk: also run a plain 512 MiB device copy (known "
                         "bytes) so a counter run can scale FETCH_SIZE / WRITE_SIZE")
    ap.add_argument("--kernel", default=HEADLINE_KERNEL,
                    help="with --summarize-pmc / --summarize-counters: the kernel to summarize (another "
                         "kernel than the headline's is printed, not written to the traffic file)")
    return ap.parse_args()


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def timed_walks(head, t, n, warmup, **kw):
    """Total-event time of n back-to-back walks (ms per walk) and per-walk samples (us)."""
    import torch
    out = None
    for _ in range(warmup):
        out = head.walk(t["base"], t["x0"], h0=t.get("h0"), out=out, **kw)
    torch.cuda.synchronize()
    s = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(s)
    for _ in range(n):
        out = head.walk(t["base"], t["x0"], h0=t.get("h0"), out=out, **kw)
    e1.record(s)
    torch.cuda.synchronize()
    total_ms = e0.elapsed_time(e1)
    # per-walk distribution
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for a, b in evs:
        a.record(s)
        out = head.walk(t["base"], t["x0"], h0=t.get("h0"), out=out, **kw)
        b.record(s)
    torch.cuda.synchronize()
    us = np.array([a.elapsed_time(b) * 1e3 for a, b in evs])
    err = head.error()
    if err != "WTS_OK":
        raise RuntimeError(err)
    return total_ms / n, us


def cold_walks(head, t, n, flush_bytes=512 << 20, **kw):
    """Per-walk times (us) with the caches flushed before each walk: a write of
    flush_bytes (twice the 256 MB memory-side cache) lands between walks, so
    the entry's shard load and the base logits come from HBM."""
    import torch
    scratch = torch.empty(flush_bytes, dtype=torch.uint8, device=t["base"].device)
    s = torch.cuda.current_stream()
    out = head.walk(t["base"], t["x0"], h0=t.get("h0"), **kw)
    us = []
    for i in range(n):
        scratch.fill_(i & 0xFF)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(s)
        out = head.walk(t["base"], t["x0"], h0=t.get("h0"), out=out, **kw)
        b.record(s)
        b.synchronize()
        us.append(a.elapsed_time(b) * 1e3)
    del scratch
    err = head.error()
    if err != "WTS_OK":
        raise RuntimeError(err)
    return np.array(us)


SIMDS_PER_CU = 4
MFMA_OPS_I8 = 16 * 16 * 64 * 2     # one v_mfma_i32_16x16x64_i8
MFMA_B_BYTES = 64 * 16             # its B operand: 64 lanes x 16 bytes of W
# VALU instructions per Gumbel value of the T=1 noise: the noise loop of
# walk_kernel<0, 16, 0, 1, false, false> issues 338 VALU instructions per
# Philox4x32-10 call, which yields four values (one counter, four words).
NOISE_VALU_PER_VALUE = 338 / 4


def step_rooflines(plan, V, r, B, fit, rf):
    """Rooflines of the resident step (int8 W, Markov, B rows), against the
    denominators measured on this device (rf = wts_roofline()).

    Resident step, per SIMD: every W tile is an MFMA B operand read from
    registers or LDS; the busiest SIMD issues r/64 int8 MFMAs per tile of its
    share, at the measured MFMA rate.  On-chip operand rate, aggregate: the W
    bytes of one step against the measured rate at which all CUs' MFMAs take
    B operands (1 KiB per MFMA) and LDS delivers reads (the resident-bandwidth
    roofline: resident steps against aggregate on-chip read bandwidth).  Step floor: that bound plus one
    cross-workgroup selection round measured in isolation.  Entry: the shard's
    one-time load against the measured HBM rate."""
    G = rf["grid"]
    tiles_cu = -(-plan["tiles"] // plan["grid"])
    tiles_simd = -(-tiles_cu // SIMDS_PER_CU)
    mfma_simd = tiles_simd * (r // 64)
    mfma_rate_simd = rf["mfma_i8_TOPs"] * 1e12 / MFMA_OPS_I8 / (G * SIMDS_PER_CU)   # MFMA/s per SIMD
    bound_us = mfma_simd / mfma_rate_simd * 1e6
    slope, entry = fit["per_step_us"], max(fit["entry_us"], 1e-3)
    w_bytes = V * r
    w_lds = plan["lds_tiles"] * plan["waves"] * plan["grid"] * 16 * r
    w_reg = max(0, min(plan["resident_bytes"], w_bytes) - w_lds)
    operand_GBps = rf["mfma_i8_TOPs"] * 1e12 / MFMA_OPS_I8 * MFMA_B_BYTES / 1e9
    onchip_us = (w_reg / (operand_GBps * 1e9) + w_lds / (rf["lds_read_GBps"] * 1e9)) * 1e6
    floor_us = bound_us + rf["exchange_us"][0]
    useful_ops = 2.0 * 2 * V * r * B
    # the same W share projected with v_dot4_i32_i8 instead: each instruction
    # takes 4 W bytes per lane (256 B per wave) for one latent row, and hi and
    # lo need one each; two waves per SIMD at the measured cycles per wave
    # (the cross-lane sums of each row's partial products not counted)
    dot4_instr_simd = tiles_simd * 16 * r / 256 * 2 * B
    dot4_us = dot4_instr_simd * rf.get("dot4_2w_cycles", 0.0) / 2 / (rf["clock_MHz"] * 1e6) * 1e6
    return {
        "resident_step_roofline": {
            "bound": "mfma issue on the busiest SIMD, W operands on chip (measured MFMA rate)",
            "tiles_per_cu": tiles_cu, "mfma_per_simd_per_step": mfma_simd,
            "mfma_cycles_measured": round(rf["clock_MHz"] * 1e6 / mfma_rate_simd, 2),
            "bound_us": round(bound_us, 3), "frac": round(bound_us / slope, 4)},
        "onchip_operand_roofline": {
            "bound": "aggregate on-chip operand rate (MFMA B operands from registers, LDS reads), measured",
            "register_w_bytes": int(w_reg), "lds_w_bytes": int(w_lds),
            "operand_rate_GBps": round(operand_GBps, 0), "lds_read_GBps": round(rf["lds_read_GBps"], 0),
            "achieved_GBps": round(w_bytes / (slope * 1e-6) / 1e9, 0),
            "bound_us": round(onchip_us, 3), "frac": round(onchip_us / slope, 4)},
        "dot4_projection_bound": {
            "bound": "the busiest SIMD's W share through v_dot4_i32_i8 (measured issue rate), a lower bound",
            "dot4_per_simd_per_step": int(dot4_instr_simd),
            "dot4_cycles_per_wave_2w": round(rf.get("dot4_2w_cycles", 0.0), 2),
            "bound_us": round(dot4_us, 3), "vs_mfma_bound": round(dot4_us / bound_us, 2) if bound_us else None},
        "step_floor": {
            "bound": "resident-step bound + one selection round in isolation (both measured)",
            "exchange_round_us": round(rf["exchange_us"][0], 3), "floor_us": round(floor_us, 3),
            "frac": round(floor_us / slope, 4)},
        "useful_int8_ops": {"ops_per_step": int(useful_ops),
                            "achieved_TOPs": round(useful_ops / (slope * 1e-6) / 1e12, 1),
                            "peak_TOPs_published": I8_PEAK_TOPS, "peak_TOPs_measured": round(rf["mfma_i8_TOPs"], 0),
                            "frac_measured": round(useful_ops / (slope * 1e-6) / 1e12 / rf["mfma_i8_TOPs"], 4)},
        "entry_roofline": {"bound": "hbm", "bytes": int(V * r + 4 * V),
                           "achieved_GBps": round((V * r + 4 * V) / (entry * 1e-6) / 1e9, 1),
                           "peak_GBps_published": HBM_PEAK_GBS, "peak_GBps_measured": round(rf["hbm_read_GBps"], 0),
                           "frac_measured": round((V * r + 4 * V) / (entry * 1e-6) / 1e9 / rf["hbm_read_GBps"], 4)},
    }


def graph_walks(head, t, n, **kw):
    """Per-walk times (us) of one walk captured in a HIP graph and replayed n times."""
    import torch
    out = head.walk(t["base"], t["x0"], h0=t.get("h0"), **kw)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        head.walk(t["base"], t["x0"], h0=t.get("h0"), out=out, **kw)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        head.walk(t["base"], t["x0"], h0=t.get("h0"), out=out, **kw)
    for _ in range(5):
        g.replay()
    torch.cuda.synchronize()
    s = torch.cuda.current_stream()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for a, b in evs:
        a.record(s)
        g.replay()
        b.record(s)
    torch.cuda.synchronize()
    err = head.error()
    if err != "WTS_OK":
        raise RuntimeError(err)
    del g
    return np.array([a.elapsed_time(b) * 1e3 for a, b in evs])


def _stream_report(fit, plan, rf, phases=None):
    """Per-step streamed W bytes against the measured stream rates (HBM, and a
    128 MiB working set in the memory-side cache).  With the walk's phase
    times, also the rate within the projection phase, the part of the step in
    which the tiles stream (the gather and the exchange move no W)."""
    slope = fit["per_step_us"]
    gbps = plan["streamed_bytes"] / (slope * 1e-6) / 1e9
    out = {"per_step_us": round(slope, 3), "entry_us": round(fit["entry_us"], 2),
           "median_us_g16": round(fit["median_us"][-1], 2),
           "streamed_MB_per_step": round(plan["streamed_bytes"] / 1e6, 2),
           "resident_MB": round(plan["resident_bytes"] / 1e6, 1),
           "stream_GBps": round(gbps, 1),
           "frac_of_hbm_measured": round(gbps / rf["hbm_read_GBps"], 4),
           "frac_of_mall_measured": round(gbps / rf["mall_read_GBps"], 4)}
    if phases:
        proj = phases["project_epilogue_reduce_us"]
        g2 = plan["streamed_bytes"] / (proj * 1e-6) / 1e9
        out.update({"projection_phase_us": proj, "stream_GBps_in_projection": round(g2, 1),
                    "frac_of_hbm_measured_in_projection": round(g2 / rf["hbm_read_GBps"], 4)})
    return out


def walk_stats(us):
    return {"median_us": float(np.median(us)), "p10_us": float(np.percentile(us, 10)),
            "p90_us": float(np.percentile(us, 90))}


def fit_steps(head, d, t, gammas=(1, 7, 16), n=100, warmup=10, graph=False, **kw):
    """Least-squares line over complete walks of gamma steps: slope = per-step cost, intercept = entry.
    graph: each walk captured in a HIP graph and replayed."""
    med = []
    for g in gammas:
        tg = dict(t)
        tg["base"] = t["base"][:, :g].contiguous()
        us = graph_walks(head, tg, n, **kw) if graph else timed_walks(head, tg, n, warmup, **kw)[1]
        med.append(float(np.median(us)))
    A = np.vstack([np.array(gammas, float), np.ones(len(gammas))]).T
    slope, icpt = np.linalg.lstsq(A, np.array(med), rcond=None)[0]
    return {"gammas": list(gammas), "median_us": med, "per_step_us": float(slope), "entry_us": float(icpt)}


WALLCLOCK_MHZ = 100.0   # s_memrealtime rate on MI355X (hipDeviceAttributeWallClockRate)
COPY_BYTES = 512 << 20  # the --copy-calib copy
HEADLINE_KERNEL = "walk_kernel<0, 1, 0, 0, false, false>"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "walk_traffic.json")


def kernel_source_hash():
    """Hash of the kernel sources with comments and blank space removed, so
    that the committed counters stay attached to the code they measured."""
    import hashlib
    import re
    h = hashlib.sha256()
    for f in ("wts_kernels.hip", "wts_internal.h"):
        with open(os.path.join(ROOT, "serial_draft_head_persistent_amd", "csrc", f)) as fh:
            src = fh.read()
        src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
        src = re.sub(r"//[^\n]*", " ", src)
        h.update(" ".join(src.split()).encode())
    return h.hexdigest()


def summarize_pmc(fetch_csv, write_csv, kernel=HEADLINE_KERNEL):
    """Per-dispatch HBM bytes of one kernel (the headline's by default) from two
    counter runs, each scaled by what the same counter reads for a plain copy
    of known size."""
    import csv
    out = {}
    for name, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        rows = [r for r in csv.DictReader(open(path)) if r["Counter_Name"] == name]
        copies = [float(r["Counter_Value"]) for r in rows if "copyBuffer" in r["Kernel_Name"]]
        walk = [float(r["Counter_Value"]) for r in rows if kernel in r["Kernel_Name"]]
        calib_kib = max(copies)            # the 512 MiB copies are the largest copy dispatches
        factor = COPY_BYTES / (calib_kib * 1024.0)
        out[name] = {"walk_kib_per_dispatch": sum(walk) / len(walk), "dispatches": len(walk),
                     "copy_kib": calib_kib, "copy_bytes": COPY_BYTES, "scale": factor,
                     "walk_bytes_per_dispatch": sum(walk) / len(walk) * 1024.0 * factor}
    res = {"kernel": kernel, "source_sha256": kernel_source_hash(), "counters": out,
           "traffic_bytes_per_launch": out["FETCH_SIZE"]["walk_bytes_per_dispatch"]
           + out["WRITE_SIZE"]["walk_bytes_per_dispatch"]}
    if kernel == HEADLINE_KERNEL:
        res["workload"] = "markov-int8-v151936-r256-b1-g16-greedy"
        with open(TRAFFIC_FILE, "w") as fh:
            json.dump(res, fh, indent=1)
    print(json.dumps(res, indent=1))


def summarize_counters(path, kernel=HEADLINE_KERNEL):
    """Per-dispatch means of the counters of one --pmc pass over one kernel."""
    import csv
    vals = {}
    for r in csv.DictReader(open(path)):
        if kernel in r["Kernel_Name"]:
            vals.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    res = {"kernel": kernel, "source_sha256": kernel_source_hash(),
           "dispatches": max((len(v) for v in vals.values()), default=0),
           "per_dispatch_mean": {k: sum(v) / len(v) for k, v in sorted(vals.items())}}
    print(json.dumps(res, indent=1))


def committed_traffic():
    """Traffic of the headline kernel from the committed counter summary, or
    None if the kernel source changed since the counters were taken."""
    try:
        with open(TRAFFIC_FILE) as fh:
            t = json.load(fh)
    except (OSError, ValueError):
        return None
    if t.get("source_sha256") != kernel_source_hash():
        return None
    return t["traffic_bytes_per_launch"]


def breakdown(head, t, reps=20, **kw):
    """Per-step phase times from the kernel's wall-clock stamps (Fig. 13b analog)."""
    import torch
    out = None
    rows = []
    for _ in range(reps):
        out = head.walk(t["base"], t["x0"], h0=t.get("h0"), out=out, trace=True, **kw)
        torch.cuda.synchronize()
        rows.append(out["trace"].cpu().numpy().astype(np.float64) / WALLCLOCK_MHZ)
    tr = np.stack(rows)                       # [reps, gamma, grid, 4] in us
    lat = tr[..., 1] - tr[..., 0]
    proj = tr[..., 2] - tr[..., 1]
    exch = tr[..., 3] - tr[..., 2]
    step = tr[:, 1:, :, 0] - tr[:, :-1, :, 0]
    skew = tr[..., 2].max(axis=2) - tr[..., 2].min(axis=2)   # spread of local-winner-ready times
    med = lambda x: round(float(np.median(x)), 3)
    return {"latent_us": med(lat), "project_epilogue_reduce_us": med(proj), "exchange_us": med(exch),
            "step_us": med(step), "arrival_skew_us": med(skew),
            "exchange_us_p90": round(float(np.percentile(exch, 90)), 3)}


def cpu_baseline(d, budget_s=12.0):
    """The oracle (as it stands) on the host cores, on a bounded sample of the same workload."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        threads = 1
    walks, t0 = 0, time.perf_counter()
    while True:
        oracle.walk(d["W"], d["E"], d["base"], d["x0"], s_w=d["s_w"], keep_logits=False)
        walks += 1
        el = time.perf_counter() - t0
        if el >= budget_s or walks >= 400:
            break
    model = None
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"value": el / walks * 1e6, "unit": "us/walk", "cores": int(threads), "kind": "oracle",
            "os_cpu_count": os.cpu_count(), "cpu_model": model, "blas_threads": int(threads),
            "sample": f"{walks} complete walks of the headline workload (V=151936, B=1, gamma=16, greedy), "
                      f"{el:.1f} s; int8 dot products via fp64 BLAS on {threads} threads, epilogue "
                      f"single-threaded numpy"}


def main():
    args = parse()
    if args.summarize_pmc:
        summarize_pmc(*args.summarize_pmc, kernel=args.kernel)
        return
    if args.summarize_counters:
        summarize_counters(args.summarize_counters, kernel=args.kernel)
        return
    if args.gpus != 1:
        print(json.dumps({"error": "the walk runs on one GPU only; run with --gpus 1 "
                          "(the walk's vocabulary sharding over several GPUs is a design note, not built)"}))
        sys.exit(2)
    import torch
    import datagen
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from gpu_helpers import dev_inputs, make_head

    dev_name = torch.cuda.get_device_name(0)
    log("device", dev_name)
    if args.copy_calib:
        src = torch.ones(512 << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log("copy calibration: 3 x 536870912 bytes")
        del src, dst
    if args.profile_walk:
        cfg, B_, g_, T_, ckw = PROFILE_WALKS[args.profile_walk]
        dp = datagen.config_inputs(cfg, B=B_, gamma=g_)
        hp, tp = make_head(dp, **ckw)
        log("plan", hp.plan(B_, temperature=T_))
        m, u = timed_walks(hp, tp, args.steps, args.warmup, temperature=T_)
        print(json.dumps({"workload": args.profile_walk, "us_per_walk": m * 1e3,
                          "median_us": float(np.median(u)), "walks": args.steps}))
        hp.close()
        return
    import serial_draft_head_persistent_amd as wts
    rf = None
    if not args.profile:
        rf = wts.roofline(0)
        log("measured denominators", rf)
    t_gen = time.perf_counter()
    d = datagen.config_inputs(1)
    t = dev_inputs(d)
    log(f"inputs ready in {time.perf_counter() - t_gen:.1f} s")
    head, t = make_head(d, t)
    plan = head.plan(1)
    log("plan", plan)

    K, W = args.steps, args.warmup
    ms_per_walk, us = timed_walks(head, t, K, W)
    log(f"resident walk: {ms_per_walk * 1e3:.2f} us (mean over {K}), median {np.median(us):.2f} us")
    if args.profile:
        print(json.dumps({"metric": "us_per_walk", "value": ms_per_walk * 1e3}))
        return

    fit = fit_steps(head, d, t)
    log("fit", fit)
    V, r = d["V"], d["r"]
    w_bytes = V * r
    # algorithmic HBM bytes of one resident walk: one-time shard load of W and
    # its row scales, base logits, the gamma gathered latent rows (512 B +
    # scale), tokens out
    gamma, B = d["gamma"], d["B"]
    hbm_bytes = w_bytes + 4 * V + 2 * B * gamma * V + B * gamma * (512 + 4) + 4 * B * gamma
    achieved = hbm_bytes / (ms_per_walk * 1e-3) / 1e9
    traffic = committed_traffic()
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4),
                "peak_measured": round(rf["hbm_read_GBps"], 1),
                "frac_measured": round(achieved / rf["hbm_read_GBps"], 4),
                "traffic": None if traffic is None else round(traffic / (ms_per_walk * 1e-3) / 1e9, 1),
                "algorithmic_bytes_per_launch": int(hbm_bytes),
                "traffic_bytes_per_launch": None if traffic is None else int(traffic)}
    per_step = {
        "per_step_us": round(fit["per_step_us"], 3), "entry_us": round(fit["entry_us"], 3),
        "w_read_GBps_per_step": round(w_bytes / (fit["per_step_us"] * 1e-6) / 1e9, 1),
        "entry_w_load_GBps": round(w_bytes / (max(fit["entry_us"], 1e-3) * 1e-6) / 1e9, 1),
    }
    per_step.update(step_rooflines(plan, V, r, B, fit, rf))
    log("per-step rooflines", per_step)

    extras = {"walk": walk_stats(us), "fit_resident": fit, "plan": plan, "measured_denominators": rf}
    extras["walk_cold_cache"] = walk_stats(cold_walks(head, t, 50))
    log("cold-cache walks", extras["walk_cold_cache"])
    extras["breakdown_resident"] = breakdown(head, t)
    log("breakdown resident", extras["breakdown_resident"])
    extras["breakdown_stream"] = breakdown(head, t, exec="stream")
    log("breakdown stream", extras["breakdown_stream"])
    if not args.quick:
        for ex in ("stream", "stepwise"):
            extras[f"fit_{ex}"] = fit_steps(head, d, t, exec=ex)
            log(ex, extras[f"fit_{ex}"])
        # the guaranteed co-residency of a cooperative launch, at its cost
        hc, _ = make_head(d, t, cooperative=True)
        _, uc = timed_walks(hc, t, 100, 10)
        hc.close()
        extras["cooperative_launch"] = {"median_us": round(float(np.median(uc)), 2),
                                        "plain_launch_median_us": round(float(np.median(us)), 2)}
        log("cooperative", extras["cooperative_launch"])
        # Fig. 3b / Fig. 11: the step-wise baseline and the resident walk captured
        # once in a HIP graph and replayed (no launch gaps from the host)
        for ex in ("stepwise", "resident"):
            extras[f"fit_{ex}_graph"] = fit_steps(head, d, t, exec=ex, graph=True)
            log(ex, "graph", extras[f"fit_{ex}_graph"])
        # Fig. 13b analogue: walks with the step-0 latent held fixed; the
        # slope difference is what advancing the state costs per step
        fx = fit_steps(head, d, t, fixed_latent=True)
        extras["fit_fixed_latent"] = fx
        extras["advance_us_per_step"] = round(fit["per_step_us"] - fx["per_step_us"], 3)
        extras["breakdown_fixed_latent"] = breakdown(head, t, fixed_latent=True)
        log("fixed latent", fx, extras["breakdown_fixed_latent"])
        # verification-ready output: cost of the per-step log normaliser at T=1
        _, u0 = timed_walks(head, t, 100, 10, temperature=1, seed=0)
        _, u1 = timed_walks(head, t, 100, 10, temperature=1, seed=0, lse=True)
        extras["lse_t1"] = {"median_us_without": round(float(np.median(u0)), 2),
                            "median_us_with": round(float(np.median(u1)), 2)}
        log("lse", extras["lse_t1"])
        # Fig. 12 analog: placement of the shard between registers and LDS
        # (B=1, greedy); nreg register tiles per wave, the rest of the shard in LDS
        place = []
        for nreg in range(0, plan["reg_tiles"] + 1):
            hp, _ = make_head(d, t, resident_tiles=nreg)
            pp = hp.plan(1)
            fp = fit_steps(hp, d, t, n=50, warmup=5)
            place.append({"reg_tiles": pp["reg_tiles"], "lds_tiles": pp["lds_tiles"],
                          "stream_tiles": pp["stream_tiles"], "per_step_us": round(fp["per_step_us"], 3),
                          "entry_us": round(fp["entry_us"], 2)})
            hp.close()
            log("placement", place[-1])
        extras["placement_int8_v151936_b1"] = place
        # batch / temperature sweep on the same W (partial residency above B=4 is not needed here:
        # the shard stays fully on chip, registers then LDS)
        sweep = []
        for B_ in (1, 2, 4, 8, 16):
            dB = datagen.config_inputs(1, B=B_, gamma=16, seed=1)
            import torch as _t
            base = _t.from_numpy(dB["base"].view(np.int16)).view(_t.bfloat16).cuda()
            x0 = _t.from_numpy(dB["x0"]).cuda()
            for T in (0, 1):
                tb = {"base": base, "x0": x0}
                m, u = timed_walks(head, tb, 50, 5, temperature=T, seed=0)
                sweep.append({"B": B_, "gamma": 16, "T": T, "median_us": round(float(np.median(u)), 2),
                              "plan_reg_lds_stream": [head.plan(B_, temperature=T)[k]
                                                     for k in ("reg_tiles", "lds_tiles", "stream_tiles")],
                              "phases": breakdown(head, tb, reps=10, temperature=T, seed=0)})
            log("sweep B", B_, sweep[-2:])
        extras["sweep_markov_int8_v151936"] = sweep
        # T=1 Gumbel noise against its VALU bound: B x V values per step, each
        # NOISE_VALU_PER_VALUE wave64 instructions (64 values per instruction),
        # spread over every SIMD at the measured four-waves-per-SIMD issue rate
        noise = []
        for B_ in (1, 2, 4, 8, 16):
            m0 = next(x["median_us"] for x in sweep if x["B"] == B_ and x["T"] == 0)
            m1 = next(x["median_us"] for x in sweep if x["B"] == B_ and x["T"] == 1)
            instr = B_ * V * NOISE_VALU_PER_VALUE / 64
            cyc_simd = instr / (rf["grid"] * SIMDS_PER_CU) * rf["valu_indep_4w_cycles"] / 4
            bound_step = cyc_simd / rf["clock_MHz"]
            bound_walk = m0 + 16 * bound_step
            noise.append({"B": B_, "noise_valu_bound_us_per_step": round(bound_step, 3),
                          "noise_measured_us_per_step": round((m1 - m0) / 16, 3),
                          "greedy_plus_bound_us": round(bound_walk, 1), "t1_walk_us": m1,
                          "t1_over_bound": round(m1 / bound_walk, 3)})
        extras["noise_roofline_t1"] = noise
        log("noise roofline", noise)
        # streamed tiles (partial residency), int8: two register tiles per wave,
        # the rest streamed every step
        hp, _ = make_head(d, t, resident_tiles=2, lds_tiles=0)
        d16 = datagen.config_inputs(1, B=16, gamma=16, seed=1)
        t16 = {"base": torch.from_numpy(d16["base"].view(np.int16)).view(torch.bfloat16).cuda(),
               "x0": torch.from_numpy(d16["x0"]).cuda()}
        pp = hp.plan(16)
        fp = fit_steps(hp, d16, t16, n=50, warmup=5)
        extras["stream_int8_v151936_b16_partial"] = _stream_report(fp, pp, rf, breakdown(hp, t16, reps=10))
        log("stream int8 partial", extras["stream_int8_v151936_b16_partial"])
        hp.close()
        head.close()
        del t, t16
        torch.cuda.empty_cache()
        # bf16 W, V = 248,320 (partial residency)
        d3 = datagen.config_inputs(3, B=16, gamma=16)
        h3, t3 = make_head(d3)
        r3 = []
        for B_ in (1, 4, 16):
            tb = {"base": t3["base"][:B_].contiguous(), "x0": t3["x0"][:B_].contiguous()}
            m, u = timed_walks(h3, tb, 50, 5)
            p3 = h3.plan(B_)
            r3.append({"B": B_, "median_us": round(float(np.median(u)), 2),
                       "resident_MB": round(p3["resident_bytes"] / 1e6, 1),
                       "streamed_MB_per_step": round(p3["streamed_bytes"] / 1e6, 1),
                       "phases": breakdown(h3, tb, reps=10)})
        extras["markov_bf16_v248320"] = r3
        log("bf16 248k", r3)
        # the partially resident sixteen-row walk against the stream rates
        f3 = fit_steps(h3, d3, t3, n=50, warmup=5)
        extras["stream_bf16_v248320_b16"] = _stream_report(f3, h3.plan(16), rf, r3[-1]["phases"])
        log("stream bf16 248k B=16", extras["stream_bf16_v248320_b16"])
        h3.close()
        del t3, d3
        torch.cuda.empty_cache()
        # other residency points: bf16 W at V=151,936 and int8 W at V=248,320, both on chip
        for name, V_, wt in (("markov_bf16_v151936", 151936, "bf16"), ("markov_int8_v248320", 248320, "int8")):
            dx = datagen.make_inputs(V_, 256, 1, 16, wtype=wt, seed=0)
            hx, tx = make_head(dx)
            px = hx.plan(1)
            fx = fit_steps(hx, dx, tx, n=50, warmup=5)
            extras[name] = {"per_step_us": round(fx["per_step_us"], 3), "entry_us": round(fx["entry_us"], 2),
                            "median_us_g16": round(fx["median_us"][-1], 2),
                            "resident_MB": round(px["resident_bytes"] / 1e6, 1),
                            "streamed_MB_per_step": round(px["streamed_bytes"] / 1e6, 1)}
            log(name, extras[name])
            hx.close()
            del tx, dx
            torch.cuda.empty_cache()
        # recurrent head, 15 steps
        d4 = datagen.config_inputs(4)
        h4, t4 = make_head(d4)
        m, u = timed_walks(h4, t4, 100, 10)
        extras["recurrent_int8_v151936_g15"] = walk_stats(u)
        log("recurrent", extras["recurrent_int8_v151936_g15"])
        h4.close()
        del t4, d4

    cpu = None
    if not (args.quick or args.no_cpu):
        cpu = cpu_baseline(d)
        log("cpu", cpu)

    line = {
        "metric": "us per gamma=16 draft walk (V=151936, r=256, B=1, int8 W resident, greedy)",
        "value": round(ms_per_walk * 1e3, 3),
        "unit": "us/walk",
        "n_gpus": 1, "steps": K, "warmup": W,
        "ms_per_step": round(ms_per_walk, 6),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "i8",
        "data": "synthetic (seeded Student-t(4) int8 W, N(0,1/256) E, N(0,2) bf16 base)",
        "config": {"workload": "markov-int8-v151936-r256-b1-g16-greedy", "V": V, "r": r, "B": 1,
                   "gamma": 16, "temperature": 0, "residency": "full",
                   "device": dev_name},
        "per_step": per_step,
        "roofline": roofline,
        "cpu_baseline": cpu,
        "extras": extras,
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
