"""GPU parity for symmetric INT8 weights with bf16 rows (W8A16; the pages
list INT1..INT8 weight formats: cocoloop.cn news item, format list): 2 KiB
device tiles, the streaming kernel feeding the exact bytes to the bf16 MFMA
and the 128 x 128 kernel multiplying bf16 s * q, checked against the oracle's
fp64 GEMM of the exact dequantized weights under the acceptance rule."""
import numpy as np
import pytest
import torch

import synthetic
from oracle import codecs, gemm, moe, quant
from gpu_util import bf16_to_dev, bits_of, quantize_experts, std_to_dev, to_dev

pytestmark = pytest.mark.gpu
F = quant.FMT_INT8_SYM


def _layer(n, k, seed):
    import quantized_gemm_int4_amd as hm
    codes, scales, _, what = quantize_experts(F, [synthetic.weights(60, n, k, index=seed)])
    d = hm.wdesc(F, n, k)
    return d, hm.hm_transform(d, *std_to_dev(F, codes, scales, None)), what[0].astype(np.float64)


def _check(d, w, what, xb, tuning=None, rows=None):
    import quantized_gemm_int4_amd as hm
    y = hm.hm_gemm(d, w, bf16_to_dev(xb), tuning=tuning)
    torch.cuda.synchronize()
    assert hm.hm_gemm_plan(d, 0, xb.shape[0], tuning).startswith("w8a16-int8sym")
    yb = bits_of(y)
    xh = codecs.bf16_value(xb).astype(np.float64)
    if rows is not None:
        yb, xh = yb[rows], xh[rows]
    yref, b = gemm.gemm_ref(xh, what, bound_dtype=np.float32 if xh.shape[0] > 512 else np.float64)
    res = gemm.check(yb, yref, b)
    assert res["ok"], res


@pytest.mark.parametrize("n,k", [(200, 384), (37, 128), (1000, 1152)])
@pytest.mark.parametrize("m", [1, 7, 16, 17, 32, 33, 100, 257, 700])
def test_int8_ragged_default_path(n, k, m):
    d, w, what = _layer(n, k, n + k)
    _check(d, w, what, synthetic.activations(60, m, k, index=m))


@pytest.mark.parametrize("m,tuning", [(1, dict(path=4)), (40, dict(path=4)), (200, dict(path=1)),
                                      (16, dict(path=1, stream_ks=1, stream_nbw=2, stream_splits=3)),
                                      (16, dict(path=1, stream_waves=8, stream_ks=8, stream_nbw=1)),
                                      (32, dict(path=1, stream_ks=4, stream_nbw=1)),
                                      (1, dict(path=3)), (300, dict(path=3)), (600, dict(path=3))])
def test_int8_forced_paths(m, tuning):
    d, w, what = _layer(264, 1152, 4)
    _check(d, w, what, synthetic.activations(60, m, 1152, index=m), tuning)


def test_int8_one_hot_exact():
    """One nonzero byte per row with a power-of-two scale: every path
    reproduces the scaled column gather bit for bit."""
    import quantized_gemm_int4_amd as hm
    n, k = 96, 512
    ks = np.random.default_rng(3).integers(0, k, size=n)
    q = np.zeros((n, k), dtype=np.int8)
    q[np.arange(n), ks] = -77
    scales = np.full((1, n, k // 128), 0x3E00, dtype=np.uint16)     # bf16 0.125
    d = hm.wdesc(F, n, k)
    w = hm.hm_transform(d, *std_to_dev(F, q.view(np.uint8)[None], scales, None))
    for m, path in [(3, 1), (40, 4), (1, 1), (40, 3), (300, 3)]:
        xb = synthetic.activations(61, m, k, index=m)
        y = bits_of(hm.hm_gemm(d, w, bf16_to_dev(xb), tuning=dict(path=path)))
        x = codecs.bf16_value(xb).astype(np.float64)
        want = codecs.bf16_rne_bits((x[:, ks] * (-77 * 0.125)).astype(np.float32))
        assert np.array_equal(y, want), (m, path)


def test_int8_full_layer():
    """The dense FFN up-projection shape (N = 14336, K = 4096): M = 1, 16, and
    sampled rows of M = 1024 and of M = 4096 (256 x 256 tiles)."""
    d, w, what = _layer(14336, 4096, 9)
    for m in (1, 16):
        _check(d, w, what, synthetic.activations(62, m, 4096, index=m))
    for m in (1024, 4096):
        rows = np.concatenate([np.random.default_rng(m).choice(m, 40, replace=False), [0, m - 1]])
        _check(d, w, what, synthetic.activations(62, m, 4096, index=m), rows=rows)


def test_int8_grouped():
    import quantized_gemm_int4_amd as hm
    t, topk, E, n, k = 300, 2, 6, 208, 640
    r = np.random.default_rng(2)
    p = np.array([40.0, 20.0] + [1.0] * (E - 2))
    p /= p.sum()
    ids = np.stack([r.choice(E, topk, replace=False, p=p) for _ in range(t)]).astype(np.int32)
    codes, scales, _, what = quantize_experts(F, [synthetic.weights(63, n, k, index=e) for e in range(E)])
    d = hm.wdesc(F, n, k, E)
    w = hm.hm_transform(d, *std_to_dev(F, codes, scales, None))
    plan = hm.hm_moe_gemm_plan(d, 0, t, topk, 0)
    assert "k_gemm_tile" in plan and "k_gemm_big" in plan, plan
    xb = synthetic.activations(63, t, k)
    _, off, sp = hm.hm_moe_sort(to_dev(ids), E)
    y = hm.hm_moe_gemm(d, w, bf16_to_dev(xb), off, sp, t, topk, 0)
    torch.cuda.synchronize()
    yref, b, _ = moe.moe_gemm_ref(codecs.bf16_value(xb).astype(np.float64), False, topk, ids,
                                  lambda e: what[e].astype(np.float64), n)
    res = gemm.check(bits_of(y), yref, b)
    assert res["ok"], res
