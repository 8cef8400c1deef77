"""GPU parity of the grouped GEMM at the MoE workload sizes: 256 experts,
top-8 Zipf-skewed routing, gate_up N=4096 K=7168 and down N=7168 K=2048, at
every token count of the W4A16 workload (T = 64, 1024, 8192) and of the
W4A8-MXFP4 workload (T = 16384), plus the MX formats with bf16 rows.

Per-expert M follows the routing load (ywsung.com note "How vLLM Humming
computes 4 bits", section on one token vs many tokens), so one call mixes
every unit kind of the schedule.  The pairs checked are drawn from all of
them: a few pairs of every 256-row chunk of the two largest experts
(including each last, partial chunk), and the first, last and two random
pairs of up to three experts in each row-count bucket 1-16, 17-64, 65-128,
129-256 and above.  Each sampled output row is compared element by element
with the oracle's fp64 GEMM of the exact dequantized expert weights, under
the acceptance rule (normwise 5e-3, element-wise 4e-3 * sum |x w| + 1 ulp).
Weights are random standard-format codes and activations N(0, 1) (1% x20
outliers for FP8 rows), drawn on the device from seeded generators."""
import numpy as np
import pytest
import torch

import synthetic
from oracle import codecs, gemm, moe, quant
from gpu_util import bits_of, to_dev

pytestmark = pytest.mark.gpu

E, TOPK, H, I = 256, 8, 7168, 2048
BUCKETS = [(1, 16), (17, 64), (65, 128), (129, 256), (257, 1 << 30)]


def sample_pairs(ids, seed):
    """Pair ids to check, drawn from every unit kind (see the module notes)."""
    counts, offsets, sp = moe.moe_sort_ref(ids, E)
    r = np.random.default_rng(seed)
    picks = []
    for e in np.argsort(-counts, kind="stable")[:2]:
        seg = sp[offsets[e]:offsets[e + 1]]
        for c0 in range(0, seg.size, 256):
            chunk = seg[c0:c0 + 256]
            picks += [chunk[0], chunk[-1]] + list(r.choice(chunk, min(2, chunk.size), replace=False))
    for lo, hi in BUCKETS:
        es = [e for e in range(E) if lo <= counts[e] <= hi]
        for e in (r.choice(es, min(3, len(es)), replace=False) if es else []):
            seg = sp[offsets[e]:offsets[e + 1]]
            picks += [seg[0], seg[-1]] + list(r.choice(seg, min(2, seg.size), replace=False))
    return np.unique(np.array(picks, dtype=np.int64))


def host_std(fmt, codes, scales, zeros, e):
    c = codes[e].cpu().numpy()
    s = scales[e].cpu().numpy()
    s = s if fmt in quant.MX_FORMATS else s.view(np.uint16)
    z = zeros[e].cpu().numpy() if zeros is not None else None
    return c, s, z


CASES = [("int4_sym", False, 64, "gate_up"), ("int4_sym", False, 64, "down"),
         ("int4_sym", False, 1024, "gate_up"), ("int4_sym", False, 1024, "down"),
         ("int4_sym", False, 8192, "gate_up"), ("int4_sym", False, 8192, "down"),
         ("mxfp4", True, 16384, "gate_up"), ("mxfp4", True, 16384, "down"),
         ("mxfp4", False, 8192, "gate_up"), ("mxfp4", False, 1024, "down"),
         ("mxint4", False, 8192, "gate_up"), ("mxint4", False, 1024, "down")]


@pytest.mark.parametrize("fmt,a8,t,proj", CASES)
def test_moe_workload_parity(fmt, a8, t, proj):
    import quantized_gemm_int4_amd as hm
    n, k = (2 * I, H) if proj == "gate_up" else (H, I)
    rows_are_pairs = 0 if proj == "gate_up" else 1
    seed = 1000 + t + (7 if proj == "down" else 0) + (3 if a8 else 0)
    print(f"[moe parity] {fmt} a8={a8} T={t} {proj} n={n} k={k}", flush=True)
    codes, scales, zeros = synthetic.random_std_format_dev(fmt, E, n, k, seed)
    d = hm.wdesc(fmt, n, k, E)
    w = hm.hm_transform(d, codes, scales, zeros)
    ids, _ = synthetic.router_topk(5 if a8 else 4, t, E, TOPK)
    P = t * TOPK
    a = synthetic.activations_dev(seed, P if rows_are_pairs else t, k, outliers=0.01 if a8 else 0.0)
    _, off, sp = hm.hm_moe_sort(to_dev(ids), E)
    if a8:
        a8b, asc = hm.hm_quant_fp8_rows(a)
        y = hm.hm_moe_gemm(d, w, a8b, off, sp, t, TOPK, rows_are_pairs, a_scales=asc)
    else:
        y = hm.hm_moe_gemm(d, w, a, off, sp, t, TOPK, rows_are_pairs)
    torch.cuda.synchronize()
    pairs = sample_pairs(ids, seed)
    arows = pairs if rows_are_pairs else pairs // TOPK
    ab = a[torch.from_numpy(arows).to(a.device)].view(torch.int16).cpu().numpy().view(np.uint16)
    if a8:
        c8, s8 = quant.quant_fp8_rows(ab)                     # per-row quantization: rows independent
        xh_rows = quant.fp8_rows_dequant(c8, s8)
    else:
        xh_rows = codecs.bf16_value(ab).astype(np.float64)
    # moe_gemm_ref indexes activation rows by pair (down) or token (gate_up):
    # give it a compact matrix whose row of each sampled pair is its own row
    flat = ids.ravel()
    yref = np.zeros((pairs.size, n))
    bnd = np.zeros((pairs.size, n))
    for e in np.unique(flat[pairs]):
        sel = np.nonzero(flat[pairs] == e)[0]
        what = quant.dequant(fmt, *host_std(fmt, codes, scales, zeros, int(e))).astype(np.float64)
        ye, be = gemm.gemm_ref(xh_rows[sel], what, bound_dtype=np.float32)
        yref[sel] = ye
        bnd[sel] = be
    yb = bits_of(y)[pairs]
    res = gemm.check(yb, yref, bnd)
    counts = np.bincount(flat, minlength=E)
    print(f"[moe parity] {pairs.size} pairs from {np.unique(flat[pairs]).size} experts "
          f"(max rows {counts.max()}): {res}", flush=True)
    assert res["ok"], res
