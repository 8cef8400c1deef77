"""The allocation-free grouped GEMM (hm_moe_gemm_static, for callers that
cannot allocate device memory) returns exactly what hm_moe_gemm returns with
a caller workspace, on two calls in a row, the second with a smaller input
(so stale work lists of the first call in the shared static array must not
leak into the second), for bf16 and FP8 rows."""
import numpy as np
import pytest
import torch

import synthetic
from gpu_util import bf16_to_dev, quantize_experts, std_to_dev, to_dev
from oracle import quant

pytestmark = pytest.mark.gpu


def _ids(t, topk, E, seed):
    r = np.random.default_rng(seed)
    p = np.array([40.0, 20.0] + [1.0] * (E - 2))
    p /= p.sum()
    return np.stack([r.choice(E, topk, replace=False, p=p) for _ in range(t)]).astype(np.int32)


@pytest.mark.parametrize("fmt,a8", [(quant.FMT_INT4_SYM, False), (quant.FMT_UINT4_ZP, False), (quant.FMT_MXFP4, True)])
def test_static_matches_workspace_variant(fmt, a8):
    import quantized_gemm_int4_amd as hm
    E, n, k, topk = 8, 208, 640, 2
    codes, scales, zeros, _ = quantize_experts(fmt, [synthetic.weights(30, n, k, index=e) for e in range(E)])
    d = hm.wdesc(fmt, n, k, E)
    w = hm.hm_transform(d, *std_to_dev(fmt, codes, scales, zeros))
    for call, (t, rows_are_pairs, seed) in enumerate([(600, 0, 1), (37, 1, 2)]):
        ids = _ids(t, topk, E, seed)
        _, off, sp = hm.hm_moe_sort(to_dev(ids), E)
        a = bf16_to_dev(synthetic.activations(30, t * topk if rows_are_pairs else t, k, index=call))
        sc = None
        if a8:
            a, sc = hm.hm_quant_fp8_rows(a)
        y_ref = hm.hm_moe_gemm(d, w, a, off, sp, t, topk, rows_are_pairs, a_scales=sc)
        y = torch.full_like(y_ref, 7.0)
        hm.hm_moe_gemm_static(d, w, a, off, sp, t, topk, rows_are_pairs, a_scales=sc, y=y)
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), y_ref.view(torch.int16)), (fmt, call)
