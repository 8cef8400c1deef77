"""GPU parity: the repack is byte-exact against the oracle's implementation of
the documented device layout, and the device dequantization is bit-exact
against the oracle's exact dequantization."""
import numpy as np
import pytest
import torch

import synthetic
from oracle import layout, quant
from gpu_util import std_to_dev, quantize_experts

pytestmark = pytest.mark.gpu

SHAPES = [(1, 16, 128), (2, 37, 256), (1, 5, 640), (3, 100, 384)]


def _random_std(fmt, E, N, K, seed):
    r = np.random.default_rng(seed)
    bits = 8 if fmt == quant.FMT_INT8_SYM else quant.NARROW_ZP.get(fmt, 4)
    codes = r.integers(0, 256, size=(E, N, K * bits // 8), dtype=np.uint8)
    if fmt in quant.MX_FORMATS:
        scales = r.integers(0, 256, size=(E, N, K // 32), dtype=np.uint8)   # every byte, NaN (255) included
        scales.reshape(-1)[:4] = [252, 253, 254, 255]          # the top bytes on every shape
    else:
        # finite bf16 patterns of both signs (|s| < 2^119 so s*15 stays finite),
        # including subnormals and zero
        scales = r.integers(0, 0x7B00, size=(E, N, K // 128)).astype(np.uint16)
        scales |= (r.integers(0, 2, size=scales.shape) << 15).astype(np.uint16)
    # zero-point bytes: random high bits too (only the code width's low bits count)
    zeros = (r.integers(0, 256, size=(E, N, K // 128), dtype=np.uint8)
             if fmt in (quant.FMT_UINT4_ZP,) + tuple(quant.NARROW_ZP) else None)
    return codes, scales, zeros


ALL = quant.FORMATS + (quant.FMT_MXINT4, quant.FMT_UINT3_ZP, quant.FMT_UINT2_ZP, quant.FMT_INT8_SYM)


@pytest.mark.parametrize("fmt", ALL)
@pytest.mark.parametrize("E,N,K", SHAPES)
def test_transform_byte_exact(fmt, E, N, K):
    import quantized_gemm_int4_amd as hm
    codes, scales, zeros = _random_std(fmt, E, N, K, 5)
    d = hm.wdesc(fmt, N, K, E)
    c, s, z = std_to_dev(fmt, codes, scales, zeros)
    w = hm.hm_transform(d, c, s, z)
    torch.cuda.synchronize()
    ref = layout.transform_ref(fmt, codes, scales, zeros)
    assert np.array_equal(w.cpu().numpy(), ref)


@pytest.mark.parametrize("fmt", ALL)
@pytest.mark.parametrize("E,N,K", SHAPES)
def test_dequant_bit_exact(fmt, E, N, K):
    import quantized_gemm_int4_amd as hm
    codes, scales, zeros = _random_std(fmt, E, N, K, 6)
    d = hm.wdesc(fmt, N, K, E)
    w = hm.hm_transform(d, *std_to_dev(fmt, codes, scales, zeros))
    for e in range(E):
        out = hm.hm_dequant(d, w, e).cpu().numpy()
        with np.errstate(over="ignore", invalid="ignore"):
            ref = quant.dequant(fmt, codes[e], scales[e], zeros[e] if zeros is not None else None)
        # bit for bit, except that a NaN (E8M0 byte 255) only has to be a NaN
        nan = np.isnan(ref)
        assert np.array_equal(np.isnan(out), nan), f"expert {e}"
        assert np.array_equal(out.view(np.uint32)[~nan], ref.view(np.uint32)[~nan]), f"expert {e}"
    if fmt in quant.MX_FORMATS:
        assert (scales == 255).any() and (scales >= 253).any()


@pytest.mark.parametrize("fmt", ALL)
def test_dequant_full_size_quantized(fmt):
    """Quantized N(0,0.02) weights at the dense FFN up-projection size."""
    import quantized_gemm_int4_amd as hm
    N, K = (7168, 2048) if fmt in quant.MX_FORMATS else (14336, 4096)
    wf = synthetic.weights(2, N, K)
    codes, scales, zeros, what = quantize_experts(fmt, [wf])
    d = hm.wdesc(fmt, N, K)
    w = hm.hm_transform(d, *std_to_dev(fmt, codes, scales, zeros))
    out = hm.hm_dequant(d, w, 0).cpu().numpy()
    assert np.array_equal(out.view(np.uint32), what[0].view(np.uint32))
