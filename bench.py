#!/usr/bin/env python3
"""Throughput of the low-bit GEMM path on one MI355X.

Default workload (one step): the dense W4A16 layer with asymmetric uint4
weights (group 128, bf16 scales, 4-bit zero points), N=14336, K=4096, run at
every M of the sweep {1, 16, 128, 1024, 4096}.  value = total algorithmic
flops of the step / step time (TFLOP/s).  Weights rotate through enough
distinct copies (>= 2 x 256 MB) that the 256 MB last-level cache cannot serve
them; activations are resident in HBM before the timed region starts.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload dense_w4a16|dense_w4a8|moe_w4a16|moe_w4a8]

One JSON line is printed (rank 0).  Extra workloads exist for measurement; the
default line is the dense W4A16 sweep.
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
LLC_BYTES = 256 * 2 ** 20      # last-level (Infinity) cache


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--workload", default="dense_w4a16",
                   choices=["dense_w4a16", "dense_w4a8", "moe_w4a16", "moe_w4a8"])
    p.add_argument("--reps", type=int, default=30, help="launches per M for per-kernel timing")
    p.add_argument("--no-cpu", action="store_true", help="skip the oracle (cpu_baseline) leg")
    return p.parse_args()


def src_hash():
    h = hashlib.sha256()
    d = os.path.join(ROOT, "quantized_gemm_int4_amd", "csrc")
    for f in sorted(os.listdir(d)):
        with open(os.path.join(d, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def traffic_for(kernel_key):
    """HBM bytes per launch measured with rocprofv3 counters for this exact
    kernel source (profiles/traffic.json), or None if absent or stale."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    e = t.get(kernel_key)
    if not e or e.get("src_hash") != src_hash():
        return None
    return e.get("bytes_per_launch")


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

def dense_setup(torch, hm, synthetic, fmt, n, k, ms):
    codes, scales, zeros = synthetic.random_std_format(fmt, 1, n, k, seed=1)
    dev = torch.device("cuda:0")
    d = hm.wdesc(fmt, n, k)
    c = torch.from_numpy(codes).to(dev)
    s = torch.from_numpy(scales.view(np.int16) if fmt != "mxfp4" else scales).to(dev)
    z = torch.from_numpy(zeros).to(dev) if zeros is not None else None
    w0 = hm.hm_transform(d, c, s, z)
    copies = max(2, int(np.ceil(2 * LLC_BYTES / w0.numel())) + 1)
    ws = [w0] + [w0.clone() for _ in range(copies - 1)]
    xs = {}
    for m in ms:
        xb = synthetic.activations(2 if fmt != "mxfp4" else 3, m, k, index=m,
                                   outliers=0.01 if fmt == "mxfp4" else 0.0)
        x = torch.from_numpy(xb.view(np.int16)).view(torch.bfloat16).to(dev)
        if fmt == "mxfp4":
            x8, sc = hm.hm_quant_fp8_rows(x)
            xs[m] = (x, x8, sc)
        else:
            xs[m] = (x, None, None)
    ys = {m: torch.empty(m, n, dtype=torch.bfloat16, device=dev) for m in ms}
    wsz = max(hm.hm_gemm_workspace_size(d, 1 if fmt == "mxfp4" else 0, m) for m in ms)
    work = torch.empty(max(wsz, 256), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()
    return dict(desc=d, codes=codes, scales=scales, zeros=zeros, w=ws, x=xs, y=ys, work=work,
                copies=copies, wbytes=w0.numel())


def dense_call(hm, S, m, i, fmt):
    x, x8, sc = S["x"][m]
    w = S["w"][i % S["copies"]]
    if fmt == "mxfp4":
        # per-token FP8 quantization is part of the W4A8 step
        hm.hm_quant_fp8_rows(x, x8, sc)
        hm.hm_gemm(S["desc"], w, x8, sc, y=S["y"][m], ws=S["work"])
    else:
        hm.hm_gemm(S["desc"], w, x, y=S["y"][m], ws=S["work"])


def run_dense(args, fmt):
    import torch
    import quantized_gemm_int4_amd as hm
    import synthetic
    from oracle import quant as oq  # noqa: F401  (only the cpu_baseline leg below uses the oracle)

    if fmt == "mxfp4":
        n, k, ms = 7168, 2048, [16, 256, 4096]
        peak = FP8_PEAK_TFLOPS
        afmt = 1
        wl = "dense W4A8-MXFP4 (E2M1 + E8M0/32, per-token FP8 E4M3) N=7168 K=2048 M={16,256,4096}"
    else:
        n, k, ms = 14336, 4096, [1, 16, 128, 1024, 4096]
        peak = BF16_PEAK_TFLOPS
        afmt = 0
        wl = "dense W4A16 asym uint4 G128 (bf16 scale + 4-bit zero) N=14336 K=4096 M={1,16,128,1024,4096}"
    S = dense_setup(torch, hm, synthetic, fmt, n, k, ms)
    alg_w = oq.storage_bytes(n, k, fmt)          # algorithmic weight bytes (standard format)
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
        xbytes = m * k * (1 if fmt == "mxfp4" else 2) + (4 * m if fmt == "mxfp4" else 0)
        ybytes = m * n * 2
        t_roof = max((alg_w + xbytes + ybytes) / (HBM_PEAK_GBS * 1e9), fl / (peak * 1e12))
        sweep.append(dict(M=m, us=round(us, 3), tflops=round(fl / us / 1e6, 3),
                          weight_GBps=round(alg_w / us / 1e3, 1),
                          all_bytes_GBps=round((alg_w + xbytes + ybytes) / us / 1e3, 1),
                          roofline_frac=round(t_roof / (us * 1e-6), 4),
                          plan=hm.hm_gemm_plan(S["desc"], afmt, m)))

    # ---- roofline of the dominant kernel (the one with most time per step)
    tile_ms = [s for s in sweep if "tile" in s["plan"]]
    stream_ms = [s for s in sweep if "stream" in s["plan"]]
    if sum(s["us"] for s in tile_ms) >= sum(s["us"] for s in stream_ms):
        fl_avg = np.mean([2.0 * s["M"] * n * k for s in tile_ms])
        us_avg = np.mean([s["us"] for s in tile_ms])
        achieved = fl_avg / (us_avg * 1e-6) / 1e12
        roof = dict(bound="mfma", kernel="k_gemm_tile", achieved=round(achieved, 2), peak=peak,
                    unit="TFLOP/s", frac=round(achieved / peak, 4),
                    per_launch=f"mean over M={[s['M'] for s in tile_ms]} of 2*M*N*K flops",
                    traffic=traffic_for(f"tile_{fmt}"))
    else:
        by_avg = np.mean([alg_w for _ in stream_ms])
        us_avg = np.mean([s["us"] for s in stream_ms])
        achieved = by_avg / (us_avg * 1e-6) / 1e9
        roof = dict(bound="hbm", kernel="k_gemm_stream", achieved=round(achieved, 1),
                    peak=HBM_PEAK_GBS, unit="GB/s", frac=round(achieved / HBM_PEAK_GBS, 4),
                    traffic=traffic_for(f"stream_{fmt}"))

    cpu = None if args.no_cpu else cpu_dense(S, fmt, n, k, ms, hm, torch)
    out = dict(metric=METRIC, value=round(value, 3), unit="TFLOP/s", n_gpus=1, steps=args.steps,
               warmup=args.warmup, ms_per_step=round(ms_step, 4), higher_is_better=True,
               scaling="weak", vs_baseline=None, dtype="fp8" if fmt == "mxfp4" else "bf16",
               data="synthetic", timing="HIP graph replay of the K steps (eager launch: "
               f"{eager_ms_step:.4f} ms/step)",
               config=dict(workload=wl, weight_copies=S["copies"],
                           weight_bytes_per_copy=S["wbytes"], algorithmic_weight_bytes=alg_w),
               sweep=sweep, roofline=roof, cpu_baseline=cpu)
    return out


def cpu_dense(S, fmt, n, k, ms, hm, torch):
    """The oracle (plain NumPy fp64) timed on the host on a bounded sample of the
    same workload: exact dequantization of the layer's weights, then the fp64
    GEMM and the |x||w| bound for every M of the sweep, rows capped at 512 per M.
    Also compares sampled GPU outputs with it."""
    from threadpoolctl import threadpool_info
    from oracle import codecs, gemm, quant
    import synthetic

    t0 = time.perf_counter()
    what = quant.dequant(fmt, S["codes"][0], S["scales"][0],
                         S["zeros"][0] if S["zeros"] is not None else None).astype(np.float64)
    flops = 0.0
    worst = 0.0
    ok = True
    for m in ms:
        rows = min(m, 512)
        xb = synthetic.activations(2 if fmt != "mxfp4" else 3, m, k, index=m,
                                   outliers=0.01 if fmt == "mxfp4" else 0.0)[:rows]
        if fmt == "mxfp4":
            c, s = quant.quant_fp8_rows(xb)
            xh = quant.fp8_rows_dequant(c, s)
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

def run_moe(args, fmt):
    import torch
    import quantized_gemm_int4_amd as hm
    import synthetic
    from oracle import quant as oq

    dev = torch.device("cuda:0")
    E, topk, H, I = 256, 8, 7168, 2048
    ts = [16384] if fmt == "mxfp4" else [64, 1024, 8192]
    g = torch.Generator(device="cuda")
    g.manual_seed(5)

    def weights(n, k):
        codes = torch.randint(0, 256, (E, n, k // 2), dtype=torch.uint8, device=dev, generator=g)
        if fmt == "mxfp4":
            sc = torch.randint(118, 122, (E, n, k // 32), dtype=torch.uint8, device=dev, generator=g)
        else:
            sc = (0x3B00 + torch.randint(0, 0x100, (E, n, k // 128), device=dev, generator=g)).to(torch.int16)
        d = hm.wdesc(fmt, n, k, E)
        w = hm.hm_transform(d, codes, sc, None)
        del codes, sc
        return d, w

    d_gu, w_gu = weights(2 * I, H)
    d_dn, w_dn = weights(H, I)
    afmt = 1 if fmt == "mxfp4" else 0
    per_t = []
    tm = Timer(torch)
    step_ms = 0.0
    step_fl = 0.0
    for t in ts:
        ids, _ = synthetic.router_topk(4 if fmt != "mxfp4" else 5, t, E, topk)
        P = t * topk
        ids_d = torch.from_numpy(ids).to(dev)
        x = torch.from_numpy(synthetic.activations(4, t, H, index=t).view(np.int16)).view(torch.bfloat16).to(dev)
        a2 = torch.from_numpy(synthetic.activations(4, P, I, index=t, role=synthetic.ROLE_DOWN)
                              .view(np.int16)).view(torch.bfloat16).to(dev)
        y1 = torch.empty(P, 2 * I, dtype=torch.bfloat16, device=dev)
        y2 = torch.empty(P, H, dtype=torch.bfloat16, device=dev)
        cnt = torch.empty(E, dtype=torch.int32, device=dev)
        off = torch.empty(E + 1, dtype=torch.int32, device=dev)
        sp = torch.empty(P, dtype=torch.int32, device=dev)
        ws1 = torch.empty(hm.hm_moe_gemm_workspace_size(d_gu, afmt, t, topk), dtype=torch.uint8, device=dev)
        ws2 = torch.empty(hm.hm_moe_gemm_workspace_size(d_dn, afmt, t, topk), dtype=torch.uint8, device=dev)
        if fmt == "mxfp4":
            x8 = torch.empty(t, H, dtype=torch.uint8, device=dev)
            xs = torch.empty(t, dtype=torch.float32, device=dev)
            a8 = torch.empty(P, I, dtype=torch.uint8, device=dev)
            as_ = torch.empty(P, dtype=torch.float32, device=dev)

        def step():
            hm.hm_moe_sort(ids_d, E, cnt, off, sp)
            if fmt == "mxfp4":
                hm.hm_quant_fp8_rows(x, x8, xs)
                hm.hm_moe_gemm(d_gu, w_gu, x8, off, sp, t, topk, 0, a_row_scale=xs, y=y1, ws=ws1)
                hm.hm_quant_fp8_rows(a2, a8, as_)
                hm.hm_moe_gemm(d_dn, w_dn, a8, off, sp, t, topk, 1, a_row_scale=as_, y=y2, ws=ws2)
            else:
                hm.hm_moe_gemm(d_gu, w_gu, x, off, sp, t, topk, 0, y=y1, ws=ws1)
                hm.hm_moe_gemm(d_dn, w_dn, a2, off, sp, t, topk, 1, y=y2, ws=ws2)

        def nsteps(k):
            def fn():
                for _ in range(k):
                    step()
            return fn
        g_warm = capture(torch, nsteps(max(args.warmup, 1)))
        g_steps = capture(torch, nsteps(args.steps))
        g_warm.replay()
        torch.cuda.synchronize()
        tm.start()
        g_steps.replay()
        ms_t = tm.stop_ms() / args.steps
        del g_warm, g_steps
        counts = np.bincount(ids.ravel(), minlength=E)
        act = int((counts > 0).sum())
        fl = 2.0 * P * (2 * I) * H + 2.0 * P * H * I
        wb = act * (oq.storage_bytes(2 * I, H, fmt) + oq.storage_bytes(H, I, fmt))
        peak = FP8_PEAK_TFLOPS if fmt == "mxfp4" else BF16_PEAK_TFLOPS
        t_roof = max(wb / (HBM_PEAK_GBS * 1e9), fl / (peak * 1e12))
        per_t.append(dict(T=t, ms=round(ms_t, 4), tflops=round(fl / ms_t / 1e9, 3),
                          weight_GBps=round(wb / ms_t / 1e6, 1), active_experts=act,
                          max_rows=int(counts.max()), roofline_frac=round(t_roof / (ms_t * 1e-3), 4)))
        step_ms += ms_t
        step_fl += fl
    wl = (f"MoE {'W4A8-MXFP4' if fmt == 'mxfp4' else 'W4A16 int4-sym G128'} 256 experts top-8 "
          f"Zipf(1.1) router, gate_up N=4096 K=7168 + down N=7168 K=2048, T={ts}, sort included")
    return dict(metric=METRIC, value=round(step_fl / (step_ms * 1e-3) / 1e12, 3), unit="TFLOP/s",
                n_gpus=1, steps=args.steps, warmup=args.warmup, ms_per_step=round(step_ms, 4),
                higher_is_better=True, scaling="weak", vs_baseline=None,
                dtype="fp8" if fmt == "mxfp4" else "bf16", data="synthetic",
                config=dict(workload=wl), per_T=per_t, roofline=None, cpu_baseline=None)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); this build has no "
              "multi-GPU path", file=sys.stderr)
        sys.exit(2)
    if args.workload.startswith("dense"):
        out = run_dense(args, "mxfp4" if args.workload == "dense_w4a8" else "uint4_zp")
    else:
        out = run_moe(args, "mxfp4" if args.workload == "moe_w4a8" else "int4_sym")
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
