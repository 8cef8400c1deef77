"""GPU parity for the MoE block steps around the grouped GEMMs: the SiLU-gated
product and the top-k weighted combine against the oracle's fp64 definitions
(element-wise, one bf16 ulp, plus the fp32 summation bound for the combine),
on both the 16-byte-chunk and the per-element kernels, special values, the
workload's shapes, and the whole block chained through the library."""
import numpy as np
import pytest
import torch

import synthetic
from oracle import codecs, gemm, moe, quant
from gpu_util import bf16_to_dev, bits_of, quantize_experts, std_to_dev, to_dev

pytestmark = pytest.mark.gpu


def _bf16_bits(x):
    return codecs.bf16_rne_bits(np.asarray(x, dtype=np.float32))


def _combine_extra(w, b, topk):
    # fp32 fused multiply-adds over topk terms: |error| <= topk 2^-24 sum_j |w y| (first order),
    # taken twice for the second-order terms
    return topk * 2.0 ** -23 * b


@pytest.mark.parametrize("rows,d", [(1, 8), (37, 2048), (300, 64), (5, 13), (64, 1001)])
def test_silu_mul_parity(rows, d):
    import quantized_gemm_int4_amd as hm
    r = np.random.default_rng(rows * 7 + d)
    gu = r.normal(0, 3, size=(rows, 2 * d))
    flat = gu.reshape(-1)
    special = [0.0, -0.0, 100.0, -100.0, -90.0, 88.5, 1e-30, -1e-38, 6.0, -87.5, -79.9, -150.0, -80.5]
    flat[: min(flat.size, len(special))] = special[: min(flat.size, len(special))]
    bits = _bf16_bits(gu)
    h = hm.hm_silu_mul(bf16_to_dev(bits))
    torch.cuda.synchronize()
    ref = moe.silu_mul_ref(codecs.bf16_value(bits).astype(np.float64), d)
    res = gemm.check_elementwise(bits_of(h), ref)
    assert res["ok"], res


def test_silu_mul_rows_zero_and_workload_rows():
    """rows = 0 is a no-op; the gate_up output of the T = 1024 workload (8192
    pairs x 4096 columns) is checked on 256 sampled rows."""
    import quantized_gemm_int4_amd as hm
    h = hm.hm_silu_mul(torch.empty(0, 16, dtype=torch.bfloat16, device="cuda"))
    assert h.shape == (0, 8)
    P, d = 8192, 2048
    g = torch.Generator(device="cuda")
    g.manual_seed(3)
    gu = (torch.randn(P, 2 * d, device="cuda", generator=g) * 2).to(torch.bfloat16)
    h = hm.hm_silu_mul(gu)
    torch.cuda.synchronize()
    rows = np.random.default_rng(0).choice(P, 256, replace=False)
    gb = bits_of(gu)[rows]
    ref = moe.silu_mul_ref(codecs.bf16_value(gb).astype(np.float64), d)
    res = gemm.check_elementwise(bits_of(h)[rows], ref)
    assert res["ok"], res


@pytest.mark.parametrize("rows,d", [(1, 8), (37, 2048), (300, 64), (3, 2056), (9, 4104), (2, 8192), (64, 1000)])
def test_silu_mul_fp8_equals_two_steps(rows, d):
    """The fused pass gives exactly the bytes and scales of the SiLU product
    followed by the per-token FP8 quantization of its bf16 output, and both
    match the oracle's quantization of the oracle's product where the bf16
    product agrees (it is within one ulp of it by the parity above)."""
    import quantized_gemm_int4_amd as hm
    r = np.random.default_rng(rows * 13 + d)
    gu = r.normal(0, 3, size=(rows, 2 * d))
    flat = gu.reshape(-1)
    special = [0.0, -0.0, 100.0, -100.0, -90.0, 88.5, 1e-30, -1e-38, 6.0, -87.5, -79.9, -150.0, -80.5]
    flat[: min(flat.size, len(special))] = special[: min(flat.size, len(special))]
    if rows > 2:
        gu[1] = 0.0                                   # an all-zero row: scale 0, codes 0
    bits = _bf16_bits(gu)
    x = bf16_to_dev(bits)
    h8, hs = hm.hm_silu_mul_fp8(x)
    h = hm.hm_silu_mul(x)
    c2, s2 = hm.hm_quant_fp8_rows(h)
    torch.cuda.synchronize()
    assert np.array_equal(h8.cpu().numpy(), c2.cpu().numpy())
    assert np.array_equal(hs.cpu().numpy().view(np.uint32), s2.cpu().numpy().view(np.uint32))
    c_ref, s_ref = quant.quant_fp8_rows(bits_of(h))
    assert np.array_equal(h8.cpu().numpy(), c_ref)
    assert np.array_equal(hs.cpu().numpy().view(np.uint32), np.asarray(s_ref, np.float32).view(np.uint32))


# (amax, h values) as bf16 bits where h * fl(1/s), s = fl(amax / 448), rounds
# to another E4M3 code than the correctly rounded h / s (found by a search
# over bf16 values with a float32 model of that product)
_RECIP_CASES = [(0x3fc4, [0x3f2f, 0x3f4b, 0x3faf]), (0x3fcc, [0x3f19, 0x3f99]), (0x3fd0, [0x3f1c, 0x3f9c]),
                (0x3ff8, [0x3f3a, 0x3fba]), (0x3f8a, [0x3ecf, 0x3f4f]), (0x3f98, [0x3f64]), (0x3fa6, [0x3f79])]


def test_silu_mul_fp8_quotients_near_e4m3_midpoints():
    """Rows where a multiply by the reciprocal of the row scale would give a
    different code than the correctly rounded quotient: the fused pass must
    give the quotient's code (that of the two-step path and the oracle).
    gate = 64 gives silu = 64 exactly, so h = 64 u exactly."""
    import quantized_gemm_int4_amd as hm
    d = 64
    h = np.zeros((len(_RECIP_CASES), d), dtype=np.float32)
    for r, (amax, hv) in enumerate(_RECIP_CASES):
        v = codecs.bf16_value(np.array([amax] + hv + hv, dtype=np.uint16)).astype(np.float32)
        v[1 + len(hv):] *= -1.0
        h[r, :v.size] = v
        s = np.float32(v[0]) / np.float32(448.0)
        fast = codecs.e4m3_rne_sat(v * (np.float32(1.0) / s))
        exact = codecs.e4m3_rne_sat(v / s)
        assert (fast != exact).any()                  # the case does separate the two
    gu = np.concatenate([np.full_like(h, 64.0), h / np.float32(64.0)], axis=1)
    bits = _bf16_bits(gu)
    x = bf16_to_dev(bits)
    h8, hs = hm.hm_silu_mul_fp8(x)
    hh = hm.hm_silu_mul(x)
    c2, s2 = hm.hm_quant_fp8_rows(hh)
    torch.cuda.synchronize()
    assert np.array_equal(bits_of(hh), _bf16_bits(h))          # h is what was planned
    assert np.array_equal(h8.cpu().numpy(), c2.cpu().numpy())
    assert np.array_equal(hs.cpu().numpy(), s2.cpu().numpy())
    c_ref, s_ref = quant.quant_fp8_rows(bits_of(hh))
    assert np.array_equal(h8.cpu().numpy(), c_ref)


def test_silu_mul_fp8_rows_zero_and_shape_errors():
    import quantized_gemm_int4_amd as hm
    h8, hs = hm.hm_silu_mul_fp8(torch.empty(0, 16, dtype=torch.bfloat16, device="cuda"))
    assert h8.shape == (0, 8) and hs.shape == (0,)
    for d in (12, 8200):
        with pytest.raises(hm.HmError):
            hm.hm_silu_mul_fp8(torch.zeros(2, 2 * d, dtype=torch.bfloat16, device="cuda"))


@pytest.mark.parametrize("t,topk,n", [(1, 1, 8), (50, 8, 7168), (33, 2, 24), (7, 3, 13), (16, 8, 1001)])
def test_combine_parity(t, topk, n):
    import quantized_gemm_int4_amd as hm
    r = np.random.default_rng(t * 31 + topk * 7 + n)
    y = r.normal(0, 2, size=(t * topk, n))
    ybits = _bf16_bits(y)
    if topk == 8:
        _, w = synthetic.router_topk(4, t, 256, 8)          # the workload's softmax weights
    else:
        w = r.random((t, topk)).astype(np.float32)
    out = hm.hm_moe_combine(bf16_to_dev(ybits), to_dev(w), topk)
    torch.cuda.synchronize()
    ref, b = moe.combine_ref(codecs.bf16_value(ybits).astype(np.float64), w.astype(np.float64), topk)
    res = gemm.check_elementwise(bits_of(out), ref, _combine_extra(w, b, topk))
    assert res["ok"], res


def test_combine_one_hot_weights_gather_exactly():
    """One-hot weights pick one pair's row: the output equals it bit for bit."""
    import quantized_gemm_int4_amd as hm
    t, topk, n = 40, 8, 264
    r = np.random.default_rng(9)
    ybits = _bf16_bits(r.normal(size=(t * topk, n)))
    pick = r.integers(0, topk, t)
    w = np.zeros((t, topk), dtype=np.float32)
    w[np.arange(t), pick] = 1.0
    out = bits_of(hm.hm_moe_combine(bf16_to_dev(ybits), to_dev(w), topk))
    assert np.array_equal(out, ybits[np.arange(t) * topk + pick])


@pytest.mark.parametrize("fmt", [quant.FMT_INT4_SYM, quant.FMT_MXFP4])
def test_moe_block_chained(fmt):
    """Sort, gate_up (n = 2d), SiLU product, [FP8 rows], down, combine, all
    through the library on a small routed batch; every step is compared with
    the oracle applied to the previous step's GPU output."""
    import quantized_gemm_int4_amd as hm
    t, topk, E, H, d = 48, 2, 6, 256, 128
    ids, w = synthetic.router_topk(6, t, E, topk)
    wg = [synthetic.weights(16, 2 * d, H, index=e) for e in range(E)]
    wd = [synthetic.weights(16, H, d, index=100 + e) for e in range(E)]
    cg, sg, zg, what_g = quantize_experts(fmt, wg)
    cd, sd, zd, what_d = quantize_experts(fmt, wd)
    dg, dd = hm.wdesc(fmt, 2 * d, H, E), hm.wdesc(fmt, H, d, E)
    w_g = hm.hm_transform(dg, *std_to_dev(fmt, cg, sg, zg))
    w_d = hm.hm_transform(dd, *std_to_dev(fmt, cd, sd, zd))
    xb = synthetic.activations(16, t, H, index=1)
    _, off, sp = hm.hm_moe_sort(to_dev(ids), E)
    x = bf16_to_dev(xb)
    a8 = fmt == quant.FMT_MXFP4
    if a8:
        x8, xs = hm.hm_quant_fp8_rows(x)
        y1 = hm.hm_moe_gemm(dg, w_g, x8, off, sp, t, topk, 0, a_scales=xs)
    else:
        y1 = hm.hm_moe_gemm(dg, w_g, x, off, sp, t, topk, 0)
    h = hm.hm_silu_mul(y1)
    if a8:
        h8, hs = hm.hm_silu_mul_fp8(y1)
        y2 = hm.hm_moe_gemm(dd, w_d, h8, off, sp, t, topk, 1, a_scales=hs)
    else:
        y2 = hm.hm_moe_gemm(dd, w_d, h, off, sp, t, topk, 1)
    out = hm.hm_moe_combine(y2, to_dev(w), topk)
    torch.cuda.synchronize()

    def xhat(bits_dev_bf16):
        b = bits_of(bits_dev_bf16)
        if not a8:
            return codecs.bf16_value(b).astype(np.float64)
        c, s = quant.quant_fp8_rows(b)
        return quant.fp8_rows_dequant(c, s)

    yr, bb, _ = moe.moe_gemm_ref(xhat(x), False, topk, ids, lambda e: what_g[e].astype(np.float64), 2 * d)
    assert gemm.check(bits_of(y1), yr, bb)["ok"]
    y1v = codecs.bf16_value(bits_of(y1)).astype(np.float64)
    assert gemm.check_elementwise(bits_of(h), moe.silu_mul_ref(y1v, d))["ok"]
    yr, bb, _ = moe.moe_gemm_ref(xhat(h), True, topk, ids, lambda e: what_d[e].astype(np.float64), H)
    assert gemm.check(bits_of(y2), yr, bb)["ok"]
    y2v = codecs.bf16_value(bits_of(y2)).astype(np.float64)
    ref, b = moe.combine_ref(y2v, w.astype(np.float64), topk)
    assert gemm.check_elementwise(bits_of(out), ref, _combine_extra(w, b, topk))["ok"]
