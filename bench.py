#!/usr/bin/env python3
"""Throughput of the low-bit GEMM path on one MI355X.

Default workload (one step): the dense W4A16 layer with asymmetric uint4
weights (group 128, bf16 scales, 4-bit zero points), N=14336, K=4096, run at
every M of the sweep {1, 16, 128, 1024, 4096}.  value = total algorithmic
flops of the step / step time (TFLOP/s).  Weights rotate through enough
distinct copies (>= 2 x 256 MB) that the 256 MB last-level cache cannot serve
them; activations are resident in HBM before the timed region starts.

The same line carries the MoE half of the metric under "moe": the grouped
GEMMs of the 256-expert top-8 MoE layer with symmetric INT4 weights and bf16
rows at T = 64, 1024, 8192, and with MXFP4 weights and per-token FP8 rows at
T = 16384 (TFLOP/s, weight GB/s and roofline fraction per T), each checked
against the oracle on sampled pairs in its own cpu_baseline.

    python bench.py [--gpus 1] [--steps K] [--warmup W]
        [--workload dense_w4a16|dense_w4a8|dense_w4a4|moe_w4a16|moe_w4a8|moe_w4a16_mxfp4|moe_w4a16_mxint4|shards|readfloor]

One JSON line is printed (rank 0).
"""
import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "W4A16 GEMM TFLOP/s & weight-HBM GB/s vs M; MoE grouped-GEMM TFLOP/s"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # dense bf16 MFMA
FP8_PEAK_TFLOPS = 5000.0       # dense fp8 MFMA
FP4_PEAK_TFLOPS = 10100.0      # dense fp4 (and fp6) MFMA
LLC_BYTES = 256 * 2 ** 20      # last-level (Infinity) cache


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--workload", default="dense_w4a16",
                   choices=["dense_w4a16", "dense_w4a8", "dense_w4a4", "moe_w4a16", "moe_w4a8", "moe_w4a16_mxfp4",
                            "moe_w4a16_mxint4", "shards", "readfloor"])
    p.add_argument("--reps", type=int, default=30, help="launches per M for per-kernel timing")
    p.add_argument("--no-cpu", action="store_true", help="skip the oracle (cpu_baseline) legs")
    p.add_argument("--no-moe", action="store_true",
                   help="default workload: skip the MoE half of the metric (grouped GEMM figures)")
    p.add_argument("--counters-run", action="store_true",
                   help="launches only, for rocprofv3 --pmc: each M of the dense sweep 3 times "
                        "between marker kernels, then a 512 MiB copy for calibration")
    p.add_argument("--ingest-counters", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                   help="turn the FETCH_SIZE and WRITE_SIZE csv output of two --counters-run "
                        "passes into profiles/traffic.json (no GPU needed)")
    return p.parse_args()


def weight_bytes(n, k, fmt):
    """Algorithmic bytes of one layer's weights in the standard format: 4-bit
    codes plus one scale per group (bf16 per 128 for the INT4 formats, one
    E8M0 byte per 32 for MXFP4 and MXINT4) and, for uint4, one 4-bit zero point per
    group (the pages' 66 bytes per 128 weights, 66.5 with the zero point)."""
    if fmt in ("mxfp4", "mxint4"):
        return n * k / 2 + n * (k // 32)
    extra = 0.5 if fmt == "uint4_zp" else 0.0
    return n * k / 2 + n * (k // 128) * (2 + extra)


def kernel_of(plan):
    """Kernel that carries a dense launch, from its plan string."""
    if " stream " in plan:
        return "k_gemm_stream"
    if "256x256" in plan:
        return "k_gemm_big"
    if "128x64" in plan:
        return "k_gemm_mid"
    return "k_gemm_mid_mx" if "64x128" in plan else "k_gemm_tile"


def src_hash():
    h = hashlib.sha256()
    d = os.path.join(ROOT, "quantized_gemm_int4_amd", "csrc")
    for f in sorted(os.listdir(d)):
        with open(os.path.join(d, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def traffic_for(workload, ms):
    """Mean HBM bytes (read + written) per launch over the given M values, as
    measured with rocprofv3 FETCH_SIZE / WRITE_SIZE counters for this exact
    kernel source (profiles/traffic.json), or None if absent or stale."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    e = t.get(workload)
    if not e or e.get("src_hash") != src_hash():
        return None
    per_m = e.get("bytes_per_launch_by_M", {})
    if not all(str(m) in per_m for m in ms):
        return None
    return round(float(np.mean([per_m[str(m)] for m in ms])), 1)


def capture(torch, fn):
    """Run fn once eagerly on a side stream (warm-up, lazy init), then capture
    it into a HIP graph (torch.cuda.CUDAGraph).  The library launches on the
    current stream, so every kernel of fn is recorded; fn allocates nothing."""
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


class Timer:
    """HIP events on the current stream (the stream the library launches on)."""

    def __init__(self, torch):
        self.torch = torch
        self.a = torch.cuda.Event(enable_timing=True)
        self.b = torch.cuda.Event(enable_timing=True)

    def start(self):
        self.a.record()

    def stop_ms(self):
        self.b.record()
        self.b.synchronize()
        return self.a.elapsed_time(self.b)


# ============================================================================ dense

def wfmt_of(fmt):
    """Weight format of a bench format ("mxfp4" = W4A8, "mxfp4_a4" = W4A4)."""
    return "mxfp4" if fmt.startswith("mxfp4") else fmt


def dense_setup(torch, hm, synthetic, fmt, n, k, ms):
    wf = wfmt_of(fmt)
    codes, scales, zeros = synthetic.random_std_format(wf, 1, n, k, seed=1)
    dev = torch.device("cuda:0")
    d = hm.wdesc(wf, n, k)
    c = torch.from_numpy(codes).to(dev)
    s = torch.from_numpy(scales.view(np.int16) if wf != "mxfp4" else scales).to(dev)
    z = torch.from_numpy(zeros).to(dev) if zeros is not None else None
    w0 = hm.hm_transform(d, c, s, z)
    copies = max(2, int(np.ceil(2 * LLC_BYTES / w0.numel())) + 1)
    ws = [w0] + [w0.clone() for _ in range(copies - 1)]
    xs = {}
    for m in ms:
        xb = synthetic.activations(2 if wf != "mxfp4" else 3, m, k, index=m,
                                   outliers=0.01 if wf == "mxfp4" else 0.0)
        x = torch.from_numpy(xb.view(np.int16)).view(torch.bfloat16).to(dev)
        if fmt == "mxfp4":
            x8, sc = hm.hm_quant_fp8_rows(x)
            xs[m] = (x, x8, sc)
        elif fmt == "mxfp4_a4":
            x4, sc = hm.hm_quant_mxfp4_rows(x)
            xs[m] = (x, x4, sc)
        else:
            xs[m] = (x, None, None)
    ys = {m: torch.empty(m, n, dtype=torch.bfloat16, device=dev) for m in ms}
    wsz = max(hm.hm_gemm_workspace_size(d, afmt_of(fmt), m) for m in ms)
    work = torch.empty(max(wsz, 256), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()
    return dict(desc=d, codes=codes, scales=scales, zeros=zeros, w=ws, x=xs, y=ys, work=work,
                copies=copies, wbytes=w0.numel())


def afmt_of(fmt):
    return {"mxfp4": 1, "mxfp4_a4": 2}.get(fmt, 0)


def dense_call(hm, S, m, i, fmt):
    x, x8, sc = S["x"][m]
    w = S["w"][i % S["copies"]]
    if fmt == "mxfp4":
        # per-token FP8 quantization is part of the W4A8 step
        hm.hm_quant_fp8_rows(x, x8, sc)
        hm.hm_gemm(S["desc"], w, x8, sc, y=S["y"][m], ws=S["work"])
    elif fmt == "mxfp4_a4":
        # and the MXFP4 quantization of the rows part of the W4A4 step
        hm.hm_quant_mxfp4_rows(x, x8, sc)
        hm.hm_gemm(S["desc"], w, x8, sc, y=S["y"][m], ws=S["work"])
    else:
        hm.hm_gemm(S["desc"], w, x, y=S["y"][m], ws=S["work"])


def run_dense(args, fmt):
    import torch
    import quantized_gemm_int4_amd as hm
    import synthetic

    if fmt == "mxfp4":
        n, k, ms = 7168, 2048, [16, 256, 4096]
        peak = FP8_PEAK_TFLOPS
        afmt = 1
        wl = "dense W4A8-MXFP4 (E2M1 + E8M0/32, per-token FP8 E4M3) N=7168 K=2048 M={16,256,4096}"
    elif fmt == "mxfp4_a4":
        n, k, ms = 7168, 2048, [16, 256, 4096]
        peak = FP4_PEAK_TFLOPS
        afmt = 2
        wl = "dense W4A4-MXFP4 (E2M1 + E8M0/32 weights and rows) N=7168 K=2048 M={16,256,4096}"
    else:
        n, k, ms = 14336, 4096, [1, 16, 128, 1024, 4096]
        peak = BF16_PEAK_TFLOPS
        afmt = 0
        wl = "dense W4A16 asym uint4 G128 (bf16 scale + 4-bit zero) N=14336 K=4096 M={1,16,128,1024,4096}"
    S = dense_setup(torch, hm, synthetic, fmt, n, k, ms)
    alg_w = weight_bytes(n, k, fmt)              # algorithmic weight bytes (standard format)
    tm = Timer(torch)

    ctr = [0]

    def steps(nsteps):
        def fn():
            for _ in range(nsteps):
                for m in ms:
                    dense_call(hm, S, m, ctr[0], fmt)
                    ctr[0] += 1
        return fn

    # ---- eager launches (host launch overhead included), for reference
    steps(args.warmup)()
    torch.cuda.synchronize()
    tm.start()
    steps(args.steps)()
    eager_ms_step = tm.stop_ms() / args.steps

    # ---- the contract's timed region: K steps (one pass of the M sweep each),
    # launched as one HIP graph replay after W warm-up steps (also a replay)
    g_warm = capture(torch, steps(max(args.warmup, 1)))
    g_steps = capture(torch, steps(args.steps))
    g_warm.replay()
    torch.cuda.synchronize()
    tm.start()
    g_steps.replay()
    ms_total = tm.stop_ms()
    torch.cuda.synchronize()
    ms_step = ms_total / args.steps
    flops_step = sum(2.0 * m * n * k for m in ms)
    value = flops_step / (ms_step * 1e-3) / 1e12

    # ---- per-M timing: a graph of `reps` back-to-back calls, rotating weights
    sweep = []
    for m in ms:
        def reps_fn(m=m):
            for _ in range(args.reps):
                dense_call(hm, S, m, ctr[0], fmt)
                ctr[0] += 1
        g = capture(torch, reps_fn)
        g.replay()
        torch.cuda.synchronize()
        tm.start()
        g.replay()
        us = tm.stop_ms() * 1e3 / args.reps
        del g
        fl = 2.0 * m * n * k
        xbytes = {"mxfp4": m * k + 4 * m, "mxfp4_a4": m * k // 2 + m * k // 32}.get(fmt, m * k * 2)
        ybytes = m * n * 2
        t_roof = max((alg_w + xbytes + ybytes) / (HBM_PEAK_GBS * 1e9), fl / (peak * 1e12))
        sweep.append(dict(M=m, us=round(us, 3), tflops=round(fl / us / 1e6, 3),
                          weight_GBps=round(alg_w / us / 1e3, 1),
                          all_bytes_GBps=round((alg_w + xbytes + ybytes) / us / 1e3, 1),
                          roofline_frac=round(t_roof / (us * 1e-6), 4),
                          plan=hm.hm_gemm_plan(S["desc"], afmt, m)))

    # ---- roofline of the dominant kernel: the one with most launch time per
    # step.  achieved = its algorithmic flops (MFMA-bound, 2*M*N*K per launch)
    # or weight bytes (HBM-bound) summed over its launches, divided by their
    # summed launch times measured above.
    by_kernel = {}
    for s_ in sweep:
        by_kernel.setdefault(kernel_of(s_["plan"]), []).append(s_)
    dom = max(by_kernel, key=lambda kn: sum(s_["us"] for s_ in by_kernel[kn]))
    runs = by_kernel[dom]
    us_sum = sum(s_["us"] for s_ in runs)
    if dom == "k_gemm_stream":
        achieved = alg_w * len(runs) / (us_sum * 1e-6) / 1e9
        roof = dict(bound="hbm", kernel=dom, achieved=round(achieved, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                    frac=round(achieved / HBM_PEAK_GBS, 4),
                    per_launch=f"{alg_w} algorithmic weight bytes per launch, M={[s_['M'] for s_ in runs]}")
    else:
        achieved = sum(2.0 * s_["M"] * n * k for s_ in runs) / (us_sum * 1e-6) / 1e12
        roof = dict(bound="mfma", kernel=dom, achieved=round(achieved, 2), peak=peak, unit="TFLOP/s",
                    frac=round(achieved / peak, 4),
                    per_launch=f"2*M*N*K flops per launch, M={[s_['M'] for s_ in runs]}")
    roof["traffic"] = traffic_for(f"dense_{fmt}", [s_["M"] for s_ in runs])
    roof["traffic_unit"] = "bytes per launch (HBM read + write)"

    cpu = None if args.no_cpu else cpu_dense(S, fmt, n, k, ms, hm, torch)
    out = dict(metric=METRIC, value=round(value, 3), unit="TFLOP/s", n_gpus=1, steps=args.steps,
               warmup=args.warmup, ms_per_step=round(ms_step, 4), higher_is_better=True,
               scaling="weak", vs_baseline=None, dtype={"mxfp4": "fp8", "mxfp4_a4": "fp4"}.get(fmt, "bf16"),
               data="synthetic", timing="HIP graph replay of the K steps (eager launch: "
               f"{eager_ms_step:.4f} ms/step)",
               config=dict(workload=wl, weight_copies=S["copies"],
                           weight_bytes_per_copy=S["wbytes"], algorithmic_weight_bytes=alg_w),
               sweep=sweep, roofline=roof, cpu_baseline=cpu)
    if fmt == "uint4_zp" and not args.no_moe:
        # the MoE half of the metric: the grouped GEMMs of the W4A16 MoE layer
        # at every token count and of the W4A8-MXFP4 layer at T = 16384
        del S
        torch.cuda.empty_cache()
        out["moe"] = moe_half(args)
    return out


def moe_half(args):
    import torch
    res = {}
    cpus = []
    for key, fmt, a8, ts in (("w4a16_int4sym", "int4_sym", False, [64, 1024, 8192]),
                             ("w4a8_mxfp4", "mxfp4", True, [16384])):
        per_t, state = moe_measure(args, fmt, a8, ts, cpu_sample=not args.no_cpu)
        name = "W4A8-MXFP4 (E2M1 + E8M0/32, per-token FP8 E4M3)" if a8 else "W4A16 int4-sym G128 (bf16 scales)"
        res[key] = dict(workload=f"MoE {name}, 256 experts top-8 Zipf(1.1) router, gate_up N=4096 K=7168 + "
                                 f"down N=7168 K=2048, T={ts}; one call = expert sort + gate_up + down",
                        **moe_summary(per_t, a8, False))
        if not args.no_cpu:
            cpus.append((key, cpu_moe(state, budget_s=10.0)))
        del state
        torch.cuda.empty_cache()
    if cpus:
        flops_s = [c["value"] for _, c in cpus]
        res["cpu_baseline"] = dict(value=round(float(np.mean(flops_s)), 6), unit="TFLOP/s", cores=cpu_threads(),
                                   kind="oracle", host_cpus=os.cpu_count(),
                                   sample="; ".join(f"{k}: {c['sample']}" for k, c in cpus),
                                   parity_ok=all(c["parity_ok"] for _, c in cpus),
                                   parity_worst_ratio=max(c["parity_worst_ratio"] for _, c in cpus),
                                   per_workload={k: c for k, c in cpus})
    return res


def cpu_dense(S, fmt, n, k, ms, hm, torch):
    """The oracle (plain NumPy fp64) timed on the host on a bounded sample of the
    same workload: exact dequantization of the layer's weights, then the fp64
    GEMM and the |x||w| bound for every M of the sweep, rows capped at 512 per M.
    Also compares sampled GPU outputs with it."""
    from threadpoolctl import threadpool_info
    from oracle import codecs, gemm, quant
    import synthetic

    t0 = time.perf_counter()
    what = quant.dequant(wfmt_of(fmt), S["codes"][0], S["scales"][0],
                         S["zeros"][0] if S["zeros"] is not None else None).astype(np.float64)
    flops = 0.0
    worst = 0.0
    ok = True
    for m in ms:
        rows = min(m, 512)
        xb = synthetic.activations(2 if fmt == "uint4_zp" else 3, m, k, index=m,
                                   outliers=0.01 if fmt != "uint4_zp" else 0.0)[:rows]
        if fmt == "mxfp4":
            c, s = quant.quant_fp8_rows(xb)
            xh = quant.fp8_rows_dequant(c, s)
        elif fmt == "mxfp4_a4":
            c, s = quant.quant_mxfp4_rows(xb)
            xh = quant.mxfp4_rows_dequant(c, s)
        else:
            xh = codecs.bf16_value(xb).astype(np.float64)
        y, b = gemm.gemm_ref(xh, what)
        flops += 2.0 * rows * n * k
        # parity of the last GPU output for this M (same weights in every copy)
        yg = S["y"][m][:rows].view(torch.int16).cpu().numpy().view(np.uint16)
        r = gemm.check(yg, y, b)
        ok = ok and r["ok"]
        worst = max(worst, r["worst_ratio"])
    dt = time.perf_counter() - t0
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    return dict(value=round(flops / dt / 1e12, 6), unit="TFLOP/s", cores=int(threads), kind="oracle",
                sample=f"dequant of the full {n}x{k} weight + fp64 GEMM and bound at M={ms} "
                       f"(rows capped at 512 per M); {dt:.2f} s",
                host_cpus=os.cpu_count(), parity_ok=bool(ok), parity_worst_ratio=round(worst, 4))


# ============================================================================ MoE

def run_shards(args):
    """One rank's share of the dense W4A16 layer (N=14336, K=4096) under
    8-way tensor parallelism, on this one GPU: the column shard N=1792, K=4096
    (each rank a slice of the outputs; no exchange, or one all-gather) and the
    row shard N=14336, K=512 (each rank a slice of K; one all-reduce of the
    output).  The collectives are not run; the figures are the GEMM a rank
    would launch, per M of the sweep."""
    import torch
    import quantized_gemm_int4_amd as hm
    import synthetic

    ms = [1, 16, 128, 1024, 4096]
    tm = Timer(torch)
    ctr = [0]
    shapes = []
    tot_fl, tot_ms = 0.0, 0.0
    for label, n, k in (("tp8 column shard", 1792, 4096), ("tp8 row shard", 14336, 512)):
        S = dense_setup(torch, hm, synthetic, "uint4_zp", n, k, ms)
        alg_w = weight_bytes(n, k, "uint4_zp")
        per_m = []
        for m in ms:
            def reps_fn(m=m):
                for _ in range(args.reps):
                    dense_call(hm, S, m, ctr[0], "uint4_zp")
                    ctr[0] += 1
            g = capture(torch, reps_fn)
            g.replay()
            torch.cuda.synchronize()
            tm.start()
            g.replay()
            us = tm.stop_ms() * 1e3 / args.reps
            del g
            fl = 2.0 * m * n * k
            byts = alg_w + m * k * 2 + m * n * 2
            t_roof = max(byts / (HBM_PEAK_GBS * 1e9), fl / (BF16_PEAK_TFLOPS * 1e12))
            per_m.append(dict(M=m, us=round(us, 3), tflops=round(fl / us / 1e6, 3),
                              weight_GBps=round(alg_w / us / 1e3, 1), roofline_frac=round(t_roof / (us * 1e-6), 4),
                              plan=hm.hm_gemm_plan(S["desc"], 0, m)))
            tot_fl += fl
            tot_ms += us * 1e-3
        shapes.append(dict(shard=label, N=n, K=k, sweep=per_m))
        del S
        torch.cuda.empty_cache()
    return dict(metric=METRIC, value=round(tot_fl / (tot_ms * 1e-3) / 1e12, 3), unit="TFLOP/s", n_gpus=1,
                steps=args.reps, warmup=args.warmup, ms_per_step=round(tot_ms, 4), higher_is_better=True,
                scaling="weak", vs_baseline=None, dtype="bf16", data="synthetic",
                config=dict(workload="one rank's GEMM of the dense W4A16 uint4 layer N=14336 K=4096 under 8-way "
                                     "tensor parallelism (column shard N=1792 K=4096, row shard N=14336 K=512), "
                                     "M={1,16,128,1024,4096}; collectives not run"),
                shards=shapes, roofline=None, cpu_baseline=None)


MOE_E, MOE_TOPK, MOE_H, MOE_I = 256, 8, 7168, 2048


def moe_measure(args, fmt, a8, ts, cpu_sample=False):
    """The grouped GEMMs of one MoE layer (256 experts, top-8 Zipf(1.1)
    routing, gate_up N=4096 K=7168, down N=7168 K=2048) at each token count
    of ts.  One step = expert sort + gate_up + down grouped GEMMs (+ the
    per-token FP8 quantization of both inputs for FP8 rows), timed as HIP
    graph replays.  Weights are random standard-format codes drawn on the
    device; activations N(0,1) bf16 (down: an independent [P, 2048] input).
    Returns (per-T figures, state the oracle leg needs)."""
    import torch
    import quantized_gemm_int4_amd as hm
    import synthetic

    dev = torch.device("cuda:0")
    E, topk, H, I = MOE_E, MOE_TOPK, MOE_H, MOE_I

    def weights(n, k, seed, gated=False):
        codes, sc, zeros = synthetic.random_std_format_dev(fmt, E, n, k, seed)
        d = hm.wdesc(fmt, n, k, E)
        wg = hm.hm_transform(d, codes, sc, zeros, gated=True) if gated else None
        return d, hm.hm_transform(d, codes, sc, zeros), (codes, sc), wg

    d_gu, w_gu, std_gu, w_gu_gated = weights(2 * I, H, 5, gated=True)
    d_dn, w_dn, std_dn, _ = weights(H, I, 6)
    afmt = 1 if a8 else 0
    per_t = []
    keep = []
    tm = Timer(torch)
    for t in ts:
        ids, rw = synthetic.router_topk(5 if a8 else 4, t, E, topk)
        P = t * topk
        ids_d = torch.from_numpy(ids).to(dev)
        x = synthetic.activations_dev(10 + t, t, H)
        a2 = synthetic.activations_dev(20 + t, P, I)
        y1 = torch.empty(P, 2 * I, dtype=torch.bfloat16, device=dev)
        y2 = torch.empty(P, H, dtype=torch.bfloat16, device=dev)
        cnt = torch.empty(E, dtype=torch.int32, device=dev)
        off = torch.empty(E + 1, dtype=torch.int32, device=dev)
        sp = torch.empty(P, dtype=torch.int32, device=dev)
        sws = torch.empty(max(hm.hm_moe_sort_workspace_size(t, topk, E), 4), dtype=torch.uint8, device=dev)
        ws1 = torch.empty(hm.hm_moe_gemm_workspace_size(d_gu, afmt, t, topk), dtype=torch.uint8, device=dev)
        ws2 = torch.empty(hm.hm_moe_gemm_workspace_size(d_dn, afmt, t, topk), dtype=torch.uint8, device=dev)
        rw_d = torch.from_numpy(rw).to(dev)
        hbuf = torch.empty(P, I, dtype=torch.bfloat16, device=dev)
        out = torch.empty(t, H, dtype=torch.bfloat16, device=dev)
        x8 = xs = a8b = as_ = None
        if a8:
            x8 = torch.empty(t, H, dtype=torch.uint8, device=dev)
            xs = torch.empty(t, dtype=torch.float32, device=dev)
            a8b = torch.empty(P, I, dtype=torch.uint8, device=dev)
            as_ = torch.empty(P, dtype=torch.float32, device=dev)

        def step():
            hm.hm_moe_sort(ids_d, E, cnt, off, sp, ws=sws)
            if a8:
                hm.hm_quant_fp8_rows(x, x8, xs)
                hm.hm_moe_gemm(d_gu, w_gu, x8, off, sp, t, topk, 0, a_scales=xs, y=y1, ws=ws1)
                hm.hm_quant_fp8_rows(a2, a8b, as_)
                hm.hm_moe_gemm(d_dn, w_dn, a8b, off, sp, t, topk, 1, a_scales=as_, y=y2, ws=ws2)
            else:
                hm.hm_moe_gemm(d_gu, w_gu, x, off, sp, t, topk, 0, y=y1, ws=ws1)
                hm.hm_moe_gemm(d_dn, w_dn, a2, off, sp, t, topk, 1, y=y2, ws=ws2)

        def block():
            # the whole MoE feed-forward block: sort, gate_up with the SiLU
            # product in its epilogue (gated layout), [FP8 rows of h], down on
            # its output, weighted combine back to token order
            hm.hm_moe_sort(ids_d, E, cnt, off, sp, ws=sws)
            if a8:
                hm.hm_quant_fp8_rows(x, x8, xs)
                hm.hm_moe_gemm(d_gu, w_gu_gated, x8, off, sp, t, topk, 0, a_scales=xs, y=hbuf, ws=ws1, gated=True)
                hm.hm_quant_fp8_rows(hbuf, a8b, as_)
                hm.hm_moe_gemm(d_dn, w_dn, a8b, off, sp, t, topk, 1, a_scales=as_, y=y2, ws=ws2)
            else:
                hm.hm_moe_gemm(d_gu, w_gu_gated, x, off, sp, t, topk, 0, y=hbuf, ws=ws1, gated=True)
                hm.hm_moe_gemm(d_dn, w_dn, hbuf, off, sp, t, topk, 1, y=y2, ws=ws2)
            hm.hm_moe_combine(y2, rw_d, topk, out)

        def block_two_step():
            # the same block with the SiLU product as a pass of its own over
            # the bf16 gate_up output (fused with the FP8 rows for W4A8)
            hm.hm_moe_sort(ids_d, E, cnt, off, sp, ws=sws)
            if a8:
                hm.hm_quant_fp8_rows(x, x8, xs)
                hm.hm_moe_gemm(d_gu, w_gu, x8, off, sp, t, topk, 0, a_scales=xs, y=y1, ws=ws1)
                hm.hm_silu_mul_fp8(y1, a8b, as_)
                hm.hm_moe_gemm(d_dn, w_dn, a8b, off, sp, t, topk, 1, a_scales=as_, y=y2, ws=ws2)
            else:
                hm.hm_moe_gemm(d_gu, w_gu, x, off, sp, t, topk, 0, y=y1, ws=ws1)
                hm.hm_silu_mul(y1, hbuf)
                hm.hm_moe_gemm(d_dn, w_dn, hbuf, off, sp, t, topk, 1, y=y2, ws=ws2)
            hm.hm_moe_combine(y2, rw_d, topk, out)

        def nsteps(k, fn1=step):
            def fn():
                for _ in range(k):
                    fn1()
            return fn

        def timed(fn1, k):
            g_warm = capture(torch, nsteps(max(args.warmup, 1), fn1))
            g_steps = capture(torch, nsteps(k, fn1))
            g_warm.replay()
            torch.cuda.synchronize()
            tm.start()
            g_steps.replay()
            ms = tm.stop_ms() / k
            del g_warm, g_steps
            return ms
        msteps = max(2, min(args.steps, 10))
        block_ms = timed(block, msteps)
        block2_ms = timed(block_two_step, msteps)
        reps = max(args.reps, 1)
        if a8:
            silu_ms = timed(lambda: hm.hm_silu_mul_fp8(y1, a8b, as_), reps)
        else:
            silu_ms = timed(lambda: hm.hm_silu_mul(y1, hbuf), reps)
        comb_ms = timed(lambda: hm.hm_moe_combine(y2, rw_d, topk, out), reps)
        sort_ms = timed(lambda: hm.hm_moe_sort(ids_d, E, cnt, off, sp, ws=sws), reps)
        ms_t = timed(step, msteps)          # last: y1, y2 of the step stay for the oracle leg
        # read gate | up, write h (bf16; FP8 codes + a row scale for FP8 rows)
        silu_b = P * (2 * I) * 2 + (P * I + 4 * P if a8 else P * I * 2)
        comb_b = P * H * 2 + t * H * 2 + P * 4             # read pair rows and weights, write tokens
        counts = np.bincount(ids.ravel(), minlength=E)
        act = int((counts > 0).sum())
        fl = 2.0 * P * (2 * I) * H + 2.0 * P * H * I
        wb = act * (weight_bytes(2 * I, H, fmt) + weight_bytes(H, I, fmt))
        peak = FP8_PEAK_TFLOPS if a8 else BF16_PEAK_TFLOPS
        t_roof = max(wb / (HBM_PEAK_GBS * 1e9), fl / (peak * 1e12))
        bound = "mfma" if fl / (peak * 1e12) >= wb / (HBM_PEAK_GBS * 1e9) else "hbm"
        per_t.append(dict(T=t, ms=round(ms_t, 4), tflops=round(fl / ms_t / 1e9, 3),
                          weight_GBps=round(wb / ms_t / 1e6, 1), active_experts=act,
                          max_rows=int(counts.max()), roofline_frac=round(t_roof / (ms_t * 1e-3), 4),
                          bound=bound, flops=fl, weight_bytes=wb, block_ms=round(block_ms, 4),
                          block_two_step_ms=round(block2_ms, 4),
                          silu_mul=dict(us=round(silu_ms * 1e3, 2), GBps=round(silu_b / silu_ms / 1e6, 1),
                                        hbm_frac=round(silu_b / silu_ms / 1e6 / HBM_PEAK_GBS, 4)),
                          combine=dict(us=round(comb_ms * 1e3, 2), GBps=round(comb_b / comb_ms / 1e6, 1),
                                       hbm_frac=round(comb_b / comb_ms / 1e6 / HBM_PEAK_GBS, 4)),
                          sort_us=round(sort_ms * 1e3, 2),
                          plan_gate_up=hm.hm_moe_gemm_plan(d_gu, afmt, t, topk, 0)))
        if cpu_sample:
            keep.append(dict(t=t, ids=ids, x=x, a2=a2, y1=y1, y2=y2))
    state = dict(fmt=fmt, a8=a8, std_gu=std_gu, std_dn=std_dn, keep=keep)
    return per_t, state


def moe_roofline(per_t, a8, f4=False):
    """Roofline of the dominant part of the MoE step: the token count with the
    most time; one launch = one step (expert sort, gate_up and down grouped
    GEMMs), its bound the binding one at that token count."""
    r = max(per_t, key=lambda e: e["ms"])
    peak = FP8_PEAK_TFLOPS if a8 else BF16_PEAK_TFLOPS
    # MX weights with bf16 rows run grouped streaming and 128-row units only
    kern = ("hm_moe_gemm (grouped k_gemm_tile/mid + k_gemm_stream)" if f4 else
            "hm_moe_gemm (grouped k_gemm_big + k_gemm_mid/tile + k_gemm_stream)")
    if r["bound"] == "mfma":
        a = r["flops"] / (r["ms"] * 1e-3) / 1e12
        return dict(bound="mfma", kernel=kern,
                    achieved=round(a, 2), peak=peak, unit="TFLOP/s", frac=round(a / peak, 4),
                    per_launch=f"2*P*N*K flops of gate_up + down at T={r['T']}", traffic=None)
    a = r["weight_bytes"] / (r["ms"] * 1e-3) / 1e9
    return dict(bound="hbm", kernel=kern,
                achieved=round(a, 1), peak=HBM_PEAK_GBS, unit="GB/s", frac=round(a / HBM_PEAK_GBS, 4),
                per_launch=f"weight bytes of the active experts at T={r['T']}", traffic=None)


def moe_sample_pairs(ids, rng, per_chunk=2, experts_per_bucket=2):
    """Pairs to check: some of every 256-row chunk of the largest expert
    (including its last, partial chunk) and of a few experts in each
    row-count bucket, so every unit kind of the schedule is sampled."""
    flat = ids.ravel()
    order = np.argsort(flat, kind="stable")
    counts = np.bincount(flat, minlength=MOE_E)
    starts = np.concatenate([[0], np.cumsum(counts)])
    picks = []
    big = int(np.argmax(counts))
    seg = order[starts[big]:starts[big + 1]]
    for c0 in range(0, seg.size, 256):
        ch = seg[c0:c0 + 256]
        picks += [ch[0], ch[-1]] + list(rng.choice(ch, min(per_chunk, ch.size), replace=False))
    for lo, hi in [(1, 16), (17, 64), (65, 128), (129, 256), (257, 1 << 30)]:
        es = [e for e in range(MOE_E) if lo <= counts[e] <= hi and e != big]
        for e in (rng.choice(es, min(experts_per_bucket, len(es)), replace=False) if es else []):
            seg = order[starts[e]:starts[e + 1]]
            picks += [seg[0], seg[-1]]
    return np.unique(np.array(picks, dtype=np.int64))


def cpu_moe(state, budget_s=20.0):
    """The oracle (plain NumPy fp64) on sampled pairs of the timed MoE calls:
    exact dequantization of each sampled expert's weights, the fp64 GEMM of
    its sampled rows and the |x||w| bound, for gate_up and down; checks the
    GPU outputs of those pairs.  Stops adding token counts once `budget_s`
    seconds of oracle time are used."""
    import torch
    from oracle import codecs, gemm, quant

    fmt, a8 = state["fmt"], state["a8"]
    t0 = time.perf_counter()
    flops, worst, ok, npairs, nexp, desc = 0.0, 0.0, True, 0, 0, []
    rng = np.random.default_rng(3)
    for kp in state["keep"]:
        if time.perf_counter() - t0 > budget_s:
            break
        ids = kp["ids"]
        flat = ids.ravel()
        pairs = moe_sample_pairs(ids, rng)
        for proj, std, a, y, n, k, rows_are_pairs in (
                ("gate_up", state["std_gu"], kp["x"], kp["y1"], 2 * MOE_I, MOE_H, False),
                ("down", state["std_dn"], kp["a2"], kp["y2"], MOE_H, MOE_I, True)):
            arows = pairs if rows_are_pairs else pairs // MOE_TOPK
            ab = a[torch.from_numpy(arows).to(a.device)].view(torch.int16).cpu().numpy().view(np.uint16)
            if a8:
                c8, s8 = quant.quant_fp8_rows(ab)
                xh = quant.fp8_rows_dequant(c8, s8)
            else:
                xh = codecs.bf16_value(ab).astype(np.float64)
            yg = y[torch.from_numpy(pairs).to(y.device)].view(torch.int16).cpu().numpy().view(np.uint16)
            yref = np.zeros((pairs.size, n))
            bnd = np.zeros((pairs.size, n))
            for e in np.unique(flat[pairs]):
                sel = np.nonzero(flat[pairs] == e)[0]
                c = std[0][int(e)].cpu().numpy()
                sc = std[1][int(e)].cpu().numpy()
                what = quant.dequant(fmt, c, sc if fmt in quant.MX_FORMATS else sc.view(np.uint16)).astype(np.float64)
                yref[sel], bnd[sel] = gemm.gemm_ref(xh[sel], what, bound_dtype=np.float32)
                flops += 2.0 * sel.size * n * k
                nexp += 1
            r = gemm.check(yg, yref, bnd)
            ok = ok and r["ok"]
            worst = max(worst, r["worst_ratio"])
            npairs += pairs.size
        desc.append(kp["t"])
    dt = time.perf_counter() - t0
    return dict(value=round(flops / dt / 1e12, 6), unit="TFLOP/s", kind="oracle",
                sample=f"{npairs} sampled (pair, projection) rows at T={desc} (every 256-row chunk of the "
                       f"largest expert and experts of every row-count bucket), {nexp} expert dequantizations "
                       f"+ fp64 GEMM and bound; {dt:.2f} s",
                parity_ok=bool(ok), parity_worst_ratio=round(worst, 4))


def moe_summary(per_t, a8, f4):
    return dict(per_T=[{k: v for k, v in e.items() if k not in ("flops", "weight_bytes")} for e in per_t],
                roofline=moe_roofline(per_t, a8, f4))


def run_moe(args, fmt, a8):
    """a8: FP8 rows (W4A8-MXFP4); otherwise bf16 rows with any weight format."""
    ts = [16384] if a8 else [64, 1024, 8192]
    per_t, state = moe_measure(args, fmt, a8, ts, cpu_sample=not args.no_cpu)
    step_ms = sum(e["ms"] for e in per_t)
    step_fl = sum(e["flops"] for e in per_t)
    name = "W4A8-MXFP4" if a8 else {"mxfp4": "W4A16-MXFP4 (E2M1 + E8M0/32, bf16 rows)",
                                     "mxint4": "W4A16-MXINT4 (1.2 fixed-point INT4 + E8M0/32, bf16 rows)"}.get(
                                         fmt, "W4A16 int4-sym G128")
    wl = (f"MoE {name} 256 experts top-8 "
          f"Zipf(1.1) router, gate_up N=4096 K=7168 + down N=7168 K=2048, T={ts}, sort included; "
          f"block_ms: the whole block with the SiLU product in the gate_up epilogue (gated layout), "
          f"the down GEMM on its output and the weighted combine; block_two_step_ms: the same with the "
          f"SiLU product as a pass of its own")
    cpu = None if args.no_cpu else cpu_moe(state)
    if cpu:
        cpu.update(cores=cpu_threads(), host_cpus=os.cpu_count())
    return dict(metric=METRIC, value=round(step_fl / (step_ms * 1e-3) / 1e12, 3), unit="TFLOP/s",
                n_gpus=1, steps=args.steps, warmup=args.warmup, ms_per_step=round(step_ms, 4),
                higher_is_better=True, scaling="weak", vs_baseline=None,
                dtype="fp8" if a8 else "bf16", data="synthetic",
                config=dict(workload=wl), per_T=moe_summary(per_t, a8, fmt in ("mxfp4", "mxint4") and not a8)["per_T"],
                roofline=moe_roofline(per_t, a8, fmt in ("mxfp4", "mxint4") and not a8),
                cpu_baseline=cpu)


def run_readfloor(args):
    """Plain-read floor of the decode shape: hm_read_probe reads the dense
    layer's weight bytes (N=14336, K=4096, uint4 + zero point: 30.5 MB) once
    per call with 16-byte loads, rotating over copies that exceed the
    last-level cache, timed like the GEMM (graph of back-to-back calls)."""
    import torch
    import quantized_gemm_int4_amd as hm
    nbytes = int(weight_bytes(14336, 4096, "uint4_zp"))
    copies = int(np.ceil(2 * LLC_BYTES / nbytes)) + 1
    bufs = [torch.empty(nbytes, dtype=torch.uint8, device="cuda:0").fill_(1) for _ in range(copies)]
    tm = Timer(torch)
    ctr = [0]
    res = []
    for blocks, unroll in ((1024, 2), (2048, 4), (2048, 8), (4096, 2)):
        out = torch.empty(blocks, dtype=torch.int32, device="cuda:0")

        def fn(blocks=blocks, unroll=unroll, out=out):
            for _ in range(args.reps):
                hm.hm_read_probe(bufs[ctr[0] % copies], blocks, unroll, out)
                ctr[0] += 1
        g = capture(torch, fn)
        g.replay()
        torch.cuda.synchronize()
        tm.start()
        g.replay()
        us = tm.stop_ms() * 1e3 / args.reps
        res.append(dict(blocks=blocks, unroll=unroll, us=round(us, 3), GBps=round(nbytes / us / 1e3, 1),
                        hbm_frac=round(nbytes / us / 1e3 / HBM_PEAK_GBS, 4)))
    best = min(res, key=lambda r: r["us"])
    return dict(metric="plain-read floor GB/s", value=best["GBps"], unit="GB/s", n_gpus=1, steps=args.reps,
                warmup=1, ms_per_step=round(best["us"] / 1e3, 5), higher_is_better=True, scaling="weak",
                vs_baseline=None, dtype="u8", data="synthetic",
                config=dict(workload=f"hm_read_probe over {nbytes} bytes (the dense W4A16 layer's weights), "
                                     f"{copies} rotating copies"), shapes=res, roofline=None, cpu_baseline=None)


def cpu_threads():
    from threadpoolctl import threadpool_info
    return int(max([p.get("num_threads", 1) for p in threadpool_info()] or [1]))


def counters_run(fmt):
    """Launches only (no timing), for two rocprofv3 --pmc passes (FETCH_SIZE,
    then WRITE_SIZE): each M of the dense sweep 3 times on rotating weight
    copies, a marker fill kernel after each M, then a 512 MiB device copy
    whose known traffic calibrates the counters."""
    import torch
    import quantized_gemm_int4_amd as hm
    import synthetic
    n, k, ms = (7168, 2048, [16, 256, 4096]) if fmt == "mxfp4" else (14336, 4096, [1, 16, 128, 1024, 4096])
    S = dense_setup(torch, hm, synthetic, fmt, n, k, ms)
    marker = torch.empty(64, dtype=torch.int32, device="cuda:0")
    i = 0
    # warm-up sweep (lazy initialization, write-back of the weight copies just
    # made), closed by a marker; the ingest step skips this first group
    for m in ms:
        dense_call(hm, S, m, i, fmt)
        i += 1
    torch.cuda.synchronize()
    marker.fill_(0)
    for m in ms:
        for _ in range(3):
            dense_call(hm, S, m, i, fmt)
            i += 1
        marker.fill_(m)
    torch.cuda.synchronize()
    src = torch.empty(512 * 2 ** 20, dtype=torch.uint8, device="cuda:0").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps(dict(counters_run=fmt, M=ms, plans=[hm.hm_gemm_plan(S["desc"], 1 if fmt == "mxfp4" else 0, m)
                                                        for m in ms])), flush=True)


def ingest_counters(fetch_dir, write_dir):
    """Per-launch HBM bytes of the dense sweep from two counters-run passes.
    Dispatches between consecutive marker fills belong to one M (3 launches;
    the W4A8 launches include the FP8 activation quantization); the group
    before the first marker is the warm-up sweep and is skipped.  The counters
    are scaled by the factor that makes the 512 MiB copy read (FETCH_SIZE) and
    write (WRITE_SIZE) exactly 512 MiB."""
    import csv
    import glob

    def load(d, counter):
        f = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)[0]
        rows = [r for r in csv.DictReader(open(f)) if r["Counter_Name"] == counter]
        rows.sort(key=lambda r: int(r["Dispatch_Id"]))
        return rows

    out = {}
    for d, counter in ((fetch_dir, "FETCH_SIZE"), (write_dir, "WRITE_SIZE")):
        rows = load(d, counter)
        marks = [i for i, r in enumerate(rows) if "FillFunctor<int>" in r["Kernel_Name"]]
        # the calibration copies are the copy dispatches after the last marker
        copy = [float(r["Counter_Value"]) for r in rows[marks[-1] + 1:] if "copy" in r["Kernel_Name"].lower()]
        calib = (512 * 2 ** 20 / 1024) / float(np.median(copy))       # counters are KiB
        groups, cur = [], []
        for r in rows[:marks[-1] + 1]:
            name = r["Kernel_Name"]
            if "FillFunctor<int>" in name:
                groups.append(cur)
                cur = []
            elif "hm::" in name:
                cur.append(float(r["Counter_Value"]) * 1024 * calib)
        out[counter] = dict(calib=calib, per_group=[sum(g) / 3.0 for g in groups[1:]],
                            copy_kib=float(np.median(copy)))
    return out


def main():
    args = parse()
    if args.ingest_counters:
        fmt = "mxfp4" if args.workload == "dense_w4a8" else "uint4_zp"
        ms = [16, 256, 4096] if fmt == "mxfp4" else [1, 16, 128, 1024, 4096]
        res = ingest_counters(*args.ingest_counters)
        fetch, write = res["FETCH_SIZE"]["per_group"], res["WRITE_SIZE"]["per_group"]
        if len(fetch) != len(ms) or len(write) != len(ms):
            sys.exit(f"expected {len(ms)} marker-separated groups, got {len(fetch)} / {len(write)}")
        path = os.path.join(ROOT, "profiles", "traffic.json")
        t = json.load(open(path)) if os.path.exists(path) else {}
        t[f"dense_{fmt}"] = dict(
            src_hash=src_hash(),
            bytes_per_launch_by_M={str(m): round(f + w, 1) for m, f, w in zip(ms, fetch, write)},
            fetch_bytes_by_M={str(m): round(f, 1) for m, f in zip(ms, fetch)},
            write_bytes_by_M={str(m): round(w, 1) for m, w in zip(ms, write)},
            calibration=dict(fetch=round(res["FETCH_SIZE"]["calib"], 4), write=round(res["WRITE_SIZE"]["calib"], 4),
                             reference="512 MiB device copy, known read and write bytes"),
            command=f"rocprofv3 --pmc FETCH_SIZE (then WRITE_SIZE) --output-format csv -- "
                    f"python3 bench.py --workload {args.workload} --counters-run")
        with open(path, "w") as f:
            json.dump(t, f, indent=1, sort_keys=True)
        print(json.dumps(t[f"dense_{fmt}"]))
        return
    if args.counters_run:
        counters_run("mxfp4" if args.workload == "dense_w4a8" else "uint4_zp")
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); this build has no "
              "multi-GPU path", file=sys.stderr)
        sys.exit(2)
    if args.workload == "shards":
        out = run_shards(args)
    elif args.workload == "readfloor":
        out = run_readfloor(args)
    elif args.workload.startswith("dense"):
        out = run_dense(args, {"dense_w4a8": "mxfp4", "dense_w4a4": "mxfp4_a4"}.get(args.workload, "uint4_zp"))
    else:
        fmt = {"moe_w4a16": "int4_sym", "moe_w4a16_mxint4": "mxint4"}.get(args.workload, "mxfp4")
        out = run_moe(args, fmt, args.workload == "moe_w4a8")
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
