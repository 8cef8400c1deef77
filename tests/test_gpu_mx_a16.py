"""GPU parity for MX weights with bf16 activation rows: MXFP4 (the MXFP4
W4A16 pair the pages report for MoE layers) and MXINT4 (1.2 fixed-point
INT4 elements): the codes are scaled by their E8M0 block scale to bf16
inside the kernels and multiplied on the bf16 MFMA.

The oracle is the same fp64 GEMM of the exactly dequantized weights as for
the other pairs, with the bf16 values of X; the dequantization itself is
checked bit for bit through unit activation rows (every output is then one
weight)."""
import numpy as np
import pytest
import torch

import synthetic
from oracle import codecs, gemm, moe, quant
from gpu_util import bf16_to_dev, bits_of, quantize_experts, std_to_dev, to_dev

pytestmark = pytest.mark.gpu

MX = quant.FMT_MXFP4
MXS = [quant.FMT_MXFP4, quant.FMT_MXINT4]


def _bf16_one_rows(k, cols):
    """bf16 patterns of rows e_c (1.0 at column c, zeros elsewhere)."""
    x = np.zeros((len(cols), k), dtype=np.uint16)
    x[np.arange(len(cols)), cols] = 0x3F80
    return x


@pytest.mark.parametrize("fmt", MXS)
@pytest.mark.parametrize("m,force", [(32, None), (7, None), (256, None), (256, 4), (200, 1), (256, 3), (100, 3)])
def test_dequant_through_unit_rows(fmt, m, force):
    """y[i, n] = w_hat[n, c_i] exactly: all 16 E2M1 codes under scale bytes
    from 0 (products down to 2^-128, subnormal in fp32 and bf16) to 252
    (largest 6 * 2^125, the last byte whose products stay below 2^128), on the
    streaming (m <= 32, or forced), 128 x 64 (default above 32 rows), 128 x
    128 and 256 x 256 (forced) kernels."""
    import quantized_gemm_int4_amd as hm
    n, k = 40, 256
    r = np.random.default_rng(11)
    codes = r.integers(0, 256, (n, k // 2), dtype=np.uint8)
    ebytes = [0, 1, 2, 3, 4, 60, 100, 119, 120, 126, 127, 128, 140, 200, 250, 252]
    if fmt == quant.FMT_MXINT4:
        ebytes.append(253)                       # |w| <= 2 * 2^126
    scales = r.choice(np.array(ebytes, dtype=np.uint8), (n, k // 32)).astype(np.uint8)
    what = quant.dequant(fmt, codes, scales, None).astype(np.float64)
    d = hm.wdesc(fmt, n, k)
    w = hm.hm_transform(d, *std_to_dev(fmt, codes[None], scales[None], None))
    cols = r.permutation(k)[:m] if m <= k else None
    xb = _bf16_one_rows(k, cols)
    y = hm.hm_gemm(d, w, bf16_to_dev(xb), tuning=None if force is None else dict(path=force))
    torch.cuda.synchronize()
    got = codecs.bf16_value(bits_of(y)).astype(np.float64)
    want = what[:, cols].T
    bad = np.argwhere(got != want)
    assert bad.size == 0, (bad[:5], got[tuple(bad[0])], want[tuple(bad[0])])


class MxLayer:
    def __init__(self, n, k, cfg=3, wseed=0, fmt=MX):
        import quantized_gemm_int4_amd as hm
        codes, scales, _, what = quantize_experts(fmt, [synthetic.weights(cfg, n, k, index=wseed)])
        self.what = what[0].astype(np.float64)
        self.desc = hm.wdesc(fmt, n, k)
        self.w = hm.hm_transform(self.desc, *std_to_dev(fmt, codes, scales, None))

    def check(self, xb, rows=None, tuning=None):
        import quantized_gemm_int4_amd as hm
        y = hm.hm_gemm(self.desc, self.w, bf16_to_dev(xb), tuning=tuning)
        torch.cuda.synchronize()
        yb = bits_of(y)
        xh = codecs.bf16_value(xb).astype(np.float64)
        if rows is not None:
            xh, yb = xh[rows], yb[rows]
        yref, b = gemm.gemm_ref(xh, self.what, bound_dtype=np.float32 if xh.shape[0] > 512 else np.float64)
        res = gemm.check(yb, yref, b)
        assert res["ok"], res
        return res


@pytest.mark.parametrize("fmt", MXS)
@pytest.mark.parametrize("n,k", [(200, 384), (37, 128), (1000, 1152)])
@pytest.mark.parametrize("m", [1, 7, 16, 17, 32, 33, 100, 129, 257, 513, 700])
def test_ragged_default_path(fmt, n, k, m):
    MxLayer(n, k, cfg=7, wseed=n + k, fmt=fmt).check(synthetic.activations(7, m, k, index=m, outliers=0.01))


@pytest.mark.parametrize("m,force", [(64, 1), (256, 1), (1, 4), (17, 4), (100, 4), (300, 4), (300, 2), (1, 2),
                                     (1, 3), (300, 3), (600, 3)])
@pytest.mark.parametrize("fmt", MXS)
def test_forced_paths(fmt, m, force):
    MxLayer(264, 640, cfg=7, wseed=5, fmt=fmt).check(synthetic.activations(7, m, 640, index=m, outliers=0.01),
                                                     tuning=dict(path=force))


@pytest.fixture(scope="module", params=MXS)
def wide(request):
    return MxLayer(7168, 2048, cfg=3, fmt=request.param)


@pytest.mark.parametrize("m", [1, 16, 256])
def test_w4a8_shape_full(wide, m):
    """The MXFP4 workload's weight shape (N = 7168, K = 2048) with bf16 rows."""
    wide.check(synthetic.activations(3, m, 2048, index=m, outliers=0.01))


def test_w4a8_shape_m4096_sampled_rows(wide):
    rows = np.random.default_rng(2).choice(4096, 96, replace=False)
    rows = np.concatenate([rows, [0, 127, 128, 4095]])
    wide.check(synthetic.activations(3, 4096, 2048, index=4096, outliers=0.01), rows=rows)


def _skewed_ids(t, topk, E, seed):
    r = np.random.default_rng(seed)
    p = np.array([40.0, 20.0] + [1.0] * (E - 2))
    p /= p.sum()
    return np.stack([r.choice(E, topk, replace=False, p=p) for _ in range(t)]).astype(np.int32)


@pytest.mark.parametrize("fmt", MXS)
@pytest.mark.parametrize("rows_are_pairs", [0, 1])
@pytest.mark.parametrize("mid", [1, 0])
def test_moe_mixed_units(fmt, rows_are_pairs, mid):
    """Streaming units (small experts), 128-row tile units and 256-row units
    in one grouped call; the tile units on the 128 x 64 kernel
    (mid=1, the default) or the 128 x 128 one."""
    import quantized_gemm_int4_amd as hm
    _moe_mixed(hm, rows_are_pairs, fmt, dict(moe_tile=1 if mid else 2))


def _moe_mixed(hm, rows_are_pairs, fmt, tuning):
    t, topk, E, n, k = 150, 2, 8, 208, 384
    ids = _skewed_ids(t, topk, E, 1)
    counts = np.bincount(ids.ravel(), minlength=E)
    assert counts.max() > 128 and (counts[counts > 0] <= 32).any()
    ws = [synthetic.weights(12, n, k, index=100 + e) for e in range(E)]
    codes, scales, _, what = quantize_experts(fmt, ws)
    d = hm.wdesc(fmt, n, k, E)
    w = hm.hm_transform(d, *std_to_dev(fmt, codes, scales, None))
    xb = synthetic.activations(12, t * topk if rows_are_pairs else t, k, index=1, outliers=0.01)
    _, off, sp = hm.hm_moe_sort(to_dev(ids), E)
    y = hm.hm_moe_gemm(d, w, bf16_to_dev(xb), off, sp, t, topk, rows_are_pairs, tuning=tuning)
    torch.cuda.synchronize()
    yref, b, _ = moe.moe_gemm_ref(codecs.bf16_value(xb).astype(np.float64), bool(rows_are_pairs), topk, ids,
                                  lambda e: what[e].astype(np.float64), n)
    res = gemm.check(bits_of(y), yref, b)
    assert res["ok"], res


@pytest.mark.parametrize("fmt", MXS)
@pytest.mark.parametrize("t,proj", [(64, "gate_up"), (1024, "down")])
def test_moe_workload_size_sampled(fmt, t, proj):
    """256 experts, top-8 routing, gate_up N=4096 K=7168 / down N=7168 K=2048,
    bf16 rows, checked on pairs of the largest and a few small experts."""
    import quantized_gemm_int4_amd as hm
    E, topk = 256, 8
    n, k = (4096, 7168) if proj == "gate_up" else (7168, 2048)
    rows_are_pairs = 0 if proj == "gate_up" else 1
    g = torch.Generator(device="cuda")
    g.manual_seed(9)
    codes = torch.randint(0, 256, (E, n, k // 2), dtype=torch.uint8, device="cuda", generator=g)
    scales = torch.randint(118, 122, (E, n, k // 32), dtype=torch.uint8, device="cuda", generator=g)
    d = hm.wdesc(fmt, n, k, E)
    w = hm.hm_transform(d, codes, scales, None)
    ids, _ = synthetic.router_topk(6, t, E, topk)
    xb = synthetic.activations(14, t * topk if rows_are_pairs else t, k, outliers=0.01)
    _, off, sp = hm.hm_moe_sort(to_dev(ids), E)
    y = hm.hm_moe_gemm(d, w, bf16_to_dev(xb), off, sp, t, topk, rows_are_pairs)
    torch.cuda.synchronize()
    counts = np.bincount(ids.ravel(), minlength=E)
    flat = ids.ravel()
    big = int(np.argmax(counts))
    small = [e for e in np.argsort(counts) if counts[e] > 0][:3]
    r = np.random.default_rng(0)
    pairs = np.concatenate([r.choice(np.nonzero(flat == big)[0], min(24, counts[big]), replace=False)] +
                           [np.nonzero(flat == e)[0][:4] for e in small])
    cache = {}

    def what(e):
        if e not in cache:
            cache[e] = quant.dequant(fmt, codes[e].cpu().numpy(), scales[e].cpu().numpy(), None).astype(np.float64)
        return cache[e]

    yref, b, _ = moe.moe_gemm_ref(codecs.bf16_value(xb).astype(np.float64), bool(rows_are_pairs), topk, ids,
                                  what, n, pairs=pairs)
    res = gemm.check(bits_of(y)[pairs], yref, b)
    assert res["ok"], res
