"""GPU parity for the 3- and 2-bit zero-point weight formats (the pages list
INT1..INT8 weights and name GPTQ INT3 as a compatibility case: cocoloop.cn
news item, format list and deployer section).  hm_transform widens their
codes and zero points into the 4-bit zero-point device layout, so every
W4A16 kernel runs them; the results must match the oracle's fp64 GEMM of the
exactly dequantized weights under the acceptance rule."""
import numpy as np
import pytest
import torch

import synthetic
from oracle import codecs, gemm, moe, quant
from gpu_util import bf16_to_dev, bits_of, quantize_experts, std_to_dev, to_dev

pytestmark = pytest.mark.gpu
NARROW = [quant.FMT_UINT3_ZP, quant.FMT_UINT2_ZP]


def _check(fmt, n, k, m, tuning=None, seed=0):
    import quantized_gemm_int4_amd as hm
    codes, scales, zeros, what = quantize_experts(fmt, [synthetic.weights(50, n, k, index=seed)])
    d = hm.wdesc(fmt, n, k)
    w = hm.hm_transform(d, *std_to_dev(fmt, codes, scales, zeros))
    xb = synthetic.activations(50, m, k, index=m + seed)
    y = hm.hm_gemm(d, w, bf16_to_dev(xb), tuning=tuning)
    torch.cuda.synchronize()
    assert hm.hm_gemm_plan(d, 0, m, tuning).startswith("w3a16" if fmt == quant.FMT_UINT3_ZP else "w2a16")
    yref, b = gemm.gemm_ref(codecs.bf16_value(xb).astype(np.float64), what[0].astype(np.float64))
    res = gemm.check(bits_of(y), yref, b)
    assert res["ok"], res


@pytest.mark.parametrize("fmt", NARROW)
@pytest.mark.parametrize("m", [1, 16, 33, 200, 600])
def test_narrow_default_paths(fmt, m):
    _check(fmt, 520, 640, m)


@pytest.mark.parametrize("fmt", NARROW)
@pytest.mark.parametrize("path", [1, 2, 3, 4])
def test_narrow_forced_paths(fmt, path):
    _check(fmt, 328, 1152, 40, tuning=dict(path=path), seed=path)


@pytest.mark.parametrize("fmt", NARROW)
def test_narrow_full_layer_decode(fmt):
    """The dense FFN up-projection shape (N = 14336, K = 4096) at M = 16."""
    _check(fmt, 14336, 4096, 16, seed=3)


@pytest.mark.parametrize("fmt", NARROW)
def test_narrow_grouped(fmt):
    import quantized_gemm_int4_amd as hm
    t, topk, E, n, k = 300, 2, 6, 208, 640
    r = np.random.default_rng(2)
    p = np.array([40.0, 20.0] + [1.0] * (E - 2))
    p /= p.sum()
    ids = np.stack([r.choice(E, topk, replace=False, p=p) for _ in range(t)]).astype(np.int32)
    codes, scales, zeros, what = quantize_experts(fmt, [synthetic.weights(51, n, k, index=e) for e in range(E)])
    d = hm.wdesc(fmt, n, k, E)
    w = hm.hm_transform(d, *std_to_dev(fmt, codes, scales, zeros))
    xb = synthetic.activations(51, t, k)
    _, off, sp = hm.hm_moe_sort(to_dev(ids), E)
    y = hm.hm_moe_gemm(d, w, bf16_to_dev(xb), off, sp, t, topk, 0)
    torch.cuda.synchronize()
    yref, b, _ = moe.moe_gemm_ref(codecs.bf16_value(xb).astype(np.float64), False, topk, ids,
                                  lambda e: what[e].astype(np.float64), n)
    res = gemm.check(bits_of(y), yref, b)
    assert res["ok"], res
