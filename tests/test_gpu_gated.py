"""GPU parity of the gate_up grouped GEMM with the gated activation in its
epilogue (hm_transform_gated + hm_moe_gemm_gated):
  * the gated layout is byte-exact against the oracle's layout of the rows
    in the gated order, for every weight format;
  * h is bit for bit hm_moe_gemm on the plain layout followed by
    hm_silu_mul, on every unit kind (streaming, 128-row tile units on
    either kernel, 256-row units) and activation format;
  * h matches the oracle: the fp64 gate_up product of the exact
    dequantized weights, through silu(gate) * up, within the GEMM's
    element-wise acceptance bound carried through the product
    (oracle.moe.silu_mul_bound) plus one bf16 ulp."""
import numpy as np
import pytest
import torch

import synthetic
from oracle import codecs, gemm, layout, moe, quant
from gpu_util import bf16_to_dev, bits_of, quantize_experts, std_to_dev, to_dev

pytestmark = pytest.mark.gpu

ALL = quant.FORMATS + (quant.FMT_MXINT4, quant.FMT_UINT3_ZP, quant.FMT_UINT2_ZP, quant.FMT_INT8_SYM)


def _perm_rows(a, p):
    return None if a is None else np.ascontiguousarray(a[:, p])


@pytest.mark.parametrize("fmt", ALL)
def test_gated_transform_byte_exact(fmt):
    import quantized_gemm_int4_amd as hm
    E, N, K = 2, 96, 256
    ws = [synthetic.weights(31, N, K, index=e) for e in range(E)]
    codes, scales, zeros, _ = quantize_experts(fmt, ws)
    d = hm.wdesc(fmt, N, K, E)
    w = hm.hm_transform(d, *std_to_dev(fmt, codes, scales, zeros), gated=True)
    torch.cuda.synchronize()
    p = layout.gated_rows(N)
    ref = layout.transform_ref(fmt, _perm_rows(codes, p), _perm_rows(scales, p), _perm_rows(zeros, p))
    assert np.array_equal(w.cpu().numpy(), ref)


def test_gated_shape_and_tuning_errors():
    import quantized_gemm_int4_amd as hm
    d = hm.wdesc(quant.FMT_INT4_SYM, 48, 128, 4)              # n not a multiple of 32
    c = torch.zeros(4, 48, 64, dtype=torch.uint8, device="cuda")
    s = torch.zeros(4, 48, 1, dtype=torch.int16, device="cuda")
    with pytest.raises(hm.HmError):
        hm.hm_transform(d, c, s, gated=True)
    with pytest.raises(hm.HmError):
        hm.hm_moe_gemm_plan(d, 0, 16, 2, 0, gated=True)
    d = hm.wdesc(quant.FMT_INT4_SYM, 64, 128, 4)
    assert "gated" in hm.hm_moe_gemm_plan(d, 0, 16, 2, 0, gated=True)
    assert "nbw=2" in hm.hm_moe_gemm_plan(d, 0, 16, 2, 0, gated=True)
    with pytest.raises(hm.HmError):
        hm.hm_moe_gemm_plan(d, 0, 16, 2, 0, tuning=dict(moe_stream_nbw=1), gated=True)


def _ids(t, topk, E, seed):
    """Skewed routing: expert 0 takes two 256-row units, expert 1 one, expert
    2 a 128-row unit (65..128 rows), the rest stream."""
    r = np.random.default_rng(seed)
    p = np.array([60.0, 20.0, 6.0] + [1.0] * (E - 3))
    p /= p.sum()
    return np.stack([r.choice(E, topk, replace=False, p=p) for _ in range(t)]).astype(np.int32)


def _acts(afmt, xb):
    """Device activations (+ scales) and the values the kernel multiplies."""
    import quantized_gemm_int4_amd as hm
    x = bf16_to_dev(xb)
    if afmt == "fp8":
        x8, s = hm.hm_quant_fp8_rows(x)
        c, sc = quant.quant_fp8_rows(xb)
        return x8, s, quant.fp8_rows_dequant(c, sc)
    if afmt == "mxfp4":
        c4, s4 = hm.hm_quant_mxfp4_rows(x)
        c, sc = quant.quant_mxfp4_rows(xb)
        return c4, s4, quant.mxfp4_rows_dequant(c, sc)
    return x, None, codecs.bf16_value(xb).astype(np.float64)


CASES = [(quant.FMT_INT4_SYM, "bf16"), (quant.FMT_UINT4_ZP, "bf16"), (quant.FMT_MXFP4, "fp8"),
         (quant.FMT_MXFP4, "bf16"), (quant.FMT_MXINT4, "bf16"), (quant.FMT_UINT3_ZP, "bf16"),
         (quant.FMT_INT8_SYM, "bf16"), (quant.FMT_MXFP4, "mxfp4")]


@pytest.mark.parametrize("fmt,afmt", CASES)
@pytest.mark.parametrize("tiles", [0, 1, 2])
@pytest.mark.parametrize("rows_are_pairs", [0, 1])
def test_gated_moe_equals_two_steps_and_oracle(fmt, afmt, tiles, rows_are_pairs):
    """tiles: 0 default unit kernels, 1 the 128-row tile kernel for the
    up-to-128-row units (where the format has it), 2 the 128 x 128 kernel."""
    import quantized_gemm_int4_amd as hm
    t, topk, E, dff, k = 400, 2, 8, 128, 384
    n = 2 * dff
    ids = _ids(t, topk, E, 3)
    counts = np.bincount(ids.ravel(), minlength=E)
    assert counts[0] > 256 + 96 and 64 < counts[2] <= 128
    ws = [synthetic.weights(17, n, k, index=e) for e in range(E)]
    codes, scales, zeros, what = quantize_experts(fmt, ws)
    d = hm.wdesc(fmt, n, k, E)
    w_plain = hm.hm_transform(d, *std_to_dev(fmt, codes, scales, zeros))
    w_gated = hm.hm_transform(d, *std_to_dev(fmt, codes, scales, zeros), gated=True)
    P = t * topk
    rows = P if rows_are_pairs else t
    xb = synthetic.activations(17, rows, k, index=5)
    a, a_s, xh = _acts(afmt, xb)
    _, off, sp = hm.hm_moe_sort(to_dev(ids), E)
    afmt_code = hm._afmt(a, a_s)
    tuning = dict(moe_stream_nbw=2)
    if tiles:
        tuning["moe_tile"] = tiles
    try:
        hm.hm_moe_gemm_plan(d, afmt_code, t, topk, rows_are_pairs, tuning=tuning)
    except hm.HmError:
        pytest.skip("this format has no such tile kernel")
    y = hm.hm_moe_gemm(d, w_plain, a, off, sp, t, topk, rows_are_pairs, a_scales=a_s, tuning=tuning)
    h2 = hm.hm_silu_mul(y)
    h = hm.hm_moe_gemm(d, w_gated, a, off, sp, t, topk, rows_are_pairs, a_scales=a_s, tuning=tuning,
                       gated=True)
    torch.cuda.synchronize()
    assert h.shape == (P, dff)
    assert np.array_equal(bits_of(h), bits_of(h2))
    yref, b, _ = moe.moe_gemm_ref(xh, bool(rows_are_pairs), topk, ids, lambda e: what[e].astype(np.float64), n)
    assert gemm.check(bits_of(y), yref, b)["ok"]
    e_y = gemm.ELEM_TOL * b + codecs.ulp_bf16(yref)          # the GEMM's element-wise acceptance
    bound = moe.silu_mul_bound(yref[:, :dff], yref[:, dff:], e_y[:, :dff], e_y[:, dff:])
    res = gemm.check_elementwise(bits_of(h), moe.silu_mul_ref(yref, dff), bound)
    assert res["ok"], res


def test_gated_moe_workload_shape_sampled():
    """The workload's gate_up (256 experts top-8, n = 4096, k = 7168) at
    T = 64 and 1024 with INT4 weights: bit-exact against the two-step path
    on every row."""
    import quantized_gemm_int4_amd as hm
    E, topk, n, k = 256, 8, 4096, 7168
    codes, sc, zeros = synthetic.random_std_format_dev(quant.FMT_INT4_SYM, E, n, k, 9)
    d = hm.wdesc(quant.FMT_INT4_SYM, n, k, E)
    w_plain = hm.hm_transform(d, codes, sc, zeros)
    w_gated = hm.hm_transform(d, codes, sc, zeros, gated=True)
    for t in (64, 1024):
        ids, _ = synthetic.router_topk(4, t, E, topk)
        x = synthetic.activations_dev(30 + t, t, k)
        _, off, sp = hm.hm_moe_sort(to_dev(ids), E)
        tuning = dict(moe_stream_nbw=2)
        y = hm.hm_moe_gemm(d, w_plain, x, off, sp, t, topk, 0, tuning=tuning)
        h2 = hm.hm_silu_mul(y)
        h = hm.hm_moe_gemm(d, w_gated, x, off, sp, t, topk, 0, tuning=tuning, gated=True)
        torch.cuda.synchronize()
        assert torch.equal(h.view(torch.int16), h2.view(torch.int16))


def test_gated_moe_workload_w4a8_t1024():
    """The W4A8 gate_up (MXFP4 weights, FP8 rows) at T = 1024: bit-exact
    against the two-step path on every row (streaming, 64 x 128 and 256-row
    units all take part)."""
    import quantized_gemm_int4_amd as hm
    E, topk, n, k, t = 256, 8, 4096, 7168, 1024
    codes, sc, zeros = synthetic.random_std_format_dev(quant.FMT_MXFP4, E, n, k, 10)
    d = hm.wdesc(quant.FMT_MXFP4, n, k, E)
    w_plain = hm.hm_transform(d, codes, sc, zeros)
    w_gated = hm.hm_transform(d, codes, sc, zeros, gated=True)
    ids, _ = synthetic.router_topk(5, t, E, topk)
    x8, xs = hm.hm_quant_fp8_rows(synthetic.activations_dev(40, t, k))
    _, off, sp = hm.hm_moe_sort(to_dev(ids), E)
    tuning = dict(moe_stream_nbw=2)
    plan = hm.hm_moe_gemm_plan(d, 1, t, topk, 0, tuning, gated=True)
    assert "k_gemm_big" in plan and "k_gemm_mid_mx" in plan, plan
    y = hm.hm_moe_gemm(d, w_plain, x8, off, sp, t, topk, 0, a_scales=xs, tuning=tuning)
    h2 = hm.hm_silu_mul(y)
    h = hm.hm_moe_gemm(d, w_gated, x8, off, sp, t, topk, 0, a_scales=xs, tuning=tuning, gated=True)
    torch.cuda.synchronize()
    assert torch.equal(h.view(torch.int16), h2.view(torch.int16))
