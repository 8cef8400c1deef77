"""GPU parity for W4A4 (the pages list 4-bit weights with 4-bit activations
among the GEMM types: cocoloop.cn news item, format list): MXFP4 weights and
MXFP4 activation rows, both E2M1 with an E8M0 scale per 32 values, on the
scaled fp4 x fp4 MFMA.  The activation quantizer is bit-exact against the
oracle's OCP MX rule; the GEMM matches the fp64 GEMM of the exactly
dequantized operands under the acceptance rule."""
import numpy as np
import pytest
import torch

import synthetic
from oracle import codecs, gemm, moe, quant
from gpu_util import bf16_to_dev, bits_of, quantize_experts, std_to_dev, to_dev

pytestmark = pytest.mark.gpu


def _rows(m, k, seed):
    """bf16 rows with the workload's outliers plus zeros, tiny, huge and tie values."""
    xb = synthetic.activations(40, m, k, index=seed, outliers=0.01)
    r = np.random.default_rng(seed)
    if m > 2 and k >= 64:
        xb[0, :32] = 0                                          # a zero block
        xb[1, :32] = synthetic.to_bf16_bits(np.float32(2.0 ** -130) * np.arange(32, dtype=np.float32))[None]
        xb[2, :32] = synthetic.to_bf16_bits(np.array([6, -0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0] * 4,
                                                     dtype=np.float32) * np.float32(2.0 ** 100))[None]
    return xb


@pytest.mark.parametrize("m,k", [(1, 32), (3, 96), (5, 128), (64, 7168), (300, 2048)])
def test_quant_mxfp4_rows_bit_exact(m, k):
    import quantized_gemm_int4_amd as hm
    xb = _rows(m, k, m + k)
    codes, scales = hm.hm_quant_mxfp4_rows(bf16_to_dev(xb))
    torch.cuda.synchronize()
    rc, rs = quant.quant_mxfp4_rows(xb)
    assert np.array_equal(scales.cpu().numpy(), rs)
    assert np.array_equal(codes.cpu().numpy(), rc)


class Layer:
    def __init__(self, n, k, seed=0):
        import quantized_gemm_int4_amd as hm
        codes, scales, _, what = quantize_experts(quant.FMT_MXFP4, [synthetic.weights(41, n, k, index=seed)])
        self.what = what[0].astype(np.float64)
        self.desc = hm.wdesc("mxfp4", n, k)
        self.w = hm.hm_transform(self.desc, *std_to_dev(quant.FMT_MXFP4, codes, scales, None))

    def check(self, xb, rows=None, tuning=None):
        import quantized_gemm_int4_amd as hm
        c, s = hm.hm_quant_mxfp4_rows(bf16_to_dev(xb))
        y = hm.hm_gemm(self.desc, self.w, c, s, tuning=tuning)
        torch.cuda.synchronize()
        assert "w4a4-mxfp4" in hm.hm_gemm_plan(self.desc, hm.HM_A_MXFP4, xb.shape[0], tuning)
        yb = bits_of(y)
        rc, rs = quant.quant_mxfp4_rows(xb if rows is None else xb[rows])
        xh = quant.mxfp4_rows_dequant(rc, rs)
        if rows is not None:
            yb = yb[rows]
        yref, b = gemm.gemm_ref(xh, self.what, bound_dtype=np.float32 if xh.shape[0] > 512 else np.float64)
        res = gemm.check(yb, yref, b)
        assert res["ok"], res
        return res


@pytest.mark.parametrize("n,k", [(200, 384), (37, 128), (1000, 1152)])
@pytest.mark.parametrize("m", [1, 7, 16, 17, 32, 33, 100, 129, 257, 513, 700])
def test_w4a4_ragged_default_path(n, k, m):
    Layer(n, k, seed=n + k).check(_rows(m, k, m))


@pytest.mark.parametrize("m,path", [(1, 4), (40, 4), (200, 1), (7, 1), (1, 3), (300, 3), (600, 3)])
def test_w4a4_forced_paths(m, path):
    Layer(264, 640, seed=3).check(_rows(m, 640, m), tuning=dict(path=path))


@pytest.mark.parametrize("ks,nbw,splits", [(1, 1, 1), (2, 2, 1), (4, 1, 3)])
def test_w4a4_stream_shapes(ks, nbw, splits):
    Layer(216, 1152, seed=ks).check(_rows(20, 1152, 20), tuning=dict(path=1, stream_ks=ks, stream_nbw=nbw,
                                                                      stream_splits=splits))


@pytest.fixture(scope="module")
def wide():
    return Layer(7168, 2048, seed=9)


@pytest.mark.parametrize("m", [16, 256])
def test_w4a4_workload_shape(wide, m):
    """The W4A8-MXFP4 workload's weight shape (N = 7168, K = 2048) with MXFP4 rows."""
    wide.check(_rows(m, 2048, m))


def test_w4a4_workload_shape_m4096_sampled(wide):
    rows = np.concatenate([np.random.default_rng(4).choice(4096, 60, replace=False), [0, 1, 2, 127, 4095]])
    wide.check(_rows(4096, 2048, 4096), rows=rows)


def test_w4a4_rejects_other_kernels_and_weights():
    import quantized_gemm_int4_amd as hm
    d = hm.wdesc("mxfp4", 7168, 2048)
    with pytest.raises(hm.HmError) as e:
        hm.hm_gemm_plan(d, hm.HM_A_MXFP4, 256, dict(path=2))
    assert e.value.code == 8
    assert "256x256" in hm.hm_gemm_plan(d, hm.HM_A_MXFP4, 256, dict(path=3))
    assert "256x256" in hm.hm_gemm_plan(d, hm.HM_A_MXFP4, 4096)
    assert "fp4xfp4" in hm.hm_gemm_plan(d, hm.HM_A_MXFP4, 4096)
    with pytest.raises(hm.HmError) as e:
        hm.hm_gemm_plan(hm.wdesc("int4_sym", 256, 512), hm.HM_A_MXFP4, 16)
    assert e.value.code == 4


@pytest.mark.parametrize("rows_are_pairs", [0, 1])
@pytest.mark.parametrize("big", [0, -1])
def test_w4a4_grouped_mixed_units(rows_are_pairs, big):
    """A grouped W4A4 call: small experts on streaming units, large ones on
    256-row units (big = 0, the default) and on 128-row units of the 128 x
    128 kernel (big = -1: no 256-row units)."""
    import quantized_gemm_int4_amd as hm
    t, topk, E, n, k = 150, 2, 8, 208, 384
    r = np.random.default_rng(1)
    p = np.array([40.0, 20.0] + [1.0] * (E - 2))
    p /= p.sum()
    ids = np.stack([r.choice(E, topk, replace=False, p=p) for _ in range(t)]).astype(np.int32)
    codes, scales, _, what = quantize_experts(quant.FMT_MXFP4, [synthetic.weights(42, n, k, index=e) for e in range(E)])
    d = hm.wdesc("mxfp4", n, k, E)
    w = hm.hm_transform(d, *std_to_dev(quant.FMT_MXFP4, codes, scales, None))
    xb = _rows(t * topk if rows_are_pairs else t, k, 5)
    c, s = hm.hm_quant_mxfp4_rows(bf16_to_dev(xb))
    _, off, sp = hm.hm_moe_sort(to_dev(ids), E)
    tuning = dict(moe_big_min=big) if big else None
    plan = hm.hm_moe_gemm_plan(d, hm.HM_A_MXFP4, t, topk, rows_are_pairs, tuning)
    assert "k_gemm_tile" in plan, plan
    assert ("big(256 rows)=none" in plan) == (big == -1), plan
    counts = np.bincount(ids.ravel(), minlength=E)
    assert counts.max() >= 97                                # a 256-row unit by default
    y = hm.hm_moe_gemm(d, w, c, off, sp, t, topk, rows_are_pairs, a_scales=s, tuning=tuning)
    torch.cuda.synchronize()
    rc, rs = quant.quant_mxfp4_rows(xb)
    yref, b, _ = moe.moe_gemm_ref(quant.mxfp4_rows_dequant(rc, rs), bool(rows_are_pairs), topk, ids,
                                  lambda e: what[e].astype(np.float64), n)
    res = gemm.check(bits_of(y), yref, b)
    assert res["ok"], res


@pytest.mark.parametrize("t,proj", [(1024, "gate_up"), (1024, "down")])
def test_w4a4_moe_workload_size_sampled(t, proj):
    """256 experts, top-8 routing, gate_up N=4096 K=7168 / down N=7168 K=2048
    with MXFP4 rows: the largest expert runs 256-row units; every 256-row
    chunk of it (the partial last one included) and a few rows of the three
    smallest experts (streaming units) are checked."""
    import quantized_gemm_int4_amd as hm
    E, topk = 256, 8
    n, k = (4096, 7168) if proj == "gate_up" else (7168, 2048)
    rows_are_pairs = 0 if proj == "gate_up" else 1
    g = torch.Generator(device="cuda")
    g.manual_seed(21)
    codes = torch.randint(0, 256, (E, n, k // 2), dtype=torch.uint8, device="cuda", generator=g)
    scales = torch.randint(118, 122, (E, n, k // 32), dtype=torch.uint8, device="cuda", generator=g)
    d = hm.wdesc("mxfp4", n, k, E)
    w = hm.hm_transform(d, codes, scales, None)
    ids, _ = synthetic.router_topk(6, t, E, topk)
    xb = _rows(t * topk if rows_are_pairs else t, k, 8)
    c, s = hm.hm_quant_mxfp4_rows(bf16_to_dev(xb))
    _, off, sp = hm.hm_moe_sort(to_dev(ids), E)
    assert "k_gemm_big" in hm.hm_moe_gemm_plan(d, hm.HM_A_MXFP4, t, topk, rows_are_pairs)
    y = hm.hm_moe_gemm(d, w, c, off, sp, t, topk, rows_are_pairs, a_scales=s)
    torch.cuda.synchronize()
    counts = np.bincount(ids.ravel(), minlength=E)
    flat = ids.ravel()
    big = int(np.argmax(counts))
    assert counts[big] > 256
    seg = np.nonzero(flat == big)[0]                  # the expert's pairs in sorted (stable) order
    pick = [seg[i] for i in range(0, seg.size, 256)] + [seg[min(i + 255, seg.size - 1)] for i in range(0, seg.size, 256)]
    small = [e for e in np.argsort(counts) if counts[e] > 0][:3]
    pairs = np.unique(np.concatenate([np.array(pick)] + [np.nonzero(flat == e)[0][:4] for e in small]))
    cache = {}

    def what(e):
        if e not in cache:
            cache[e] = quant.dequant("mxfp4", codes[e].cpu().numpy(), scales[e].cpu().numpy(), None).astype(np.float64)
        return cache[e]

    rc, rs = quant.quant_mxfp4_rows(xb)
    yref, b, _ = moe.moe_gemm_ref(quant.mxfp4_rows_dequant(rc, rs), bool(rows_are_pairs), topk, ids, what, n,
                                  pairs=pairs)
    res = gemm.check(bits_of(y)[pairs], yref, b)
    assert res["ok"], res
