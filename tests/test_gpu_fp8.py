"""GPU parity: per-token FP8 quantization is bit-exact (codes and fp32 scales)
against the oracle."""
import numpy as np
import pytest
import torch

import synthetic
from oracle import quant
from gpu_util import bf16_to_dev

pytestmark = pytest.mark.gpu


def _rows(m, k, seed):
    r = np.random.default_rng(seed)
    x = r.normal(0, 1, size=(m, k)).astype(np.float32)
    # spread magnitudes over many binades so subnormal E4M3 codes appear
    x *= np.exp2(r.integers(-12, 4, size=(m, 1))).astype(np.float32)
    x *= np.exp2(r.integers(-10, 1, size=(m, k))).astype(np.float32)
    x[0] = 0.0                                     # zero row
    if m > 2:
        x[1, :] = -0.0
        x[2, min(3, k - 1)] = 1e4                    # one dominant outlier
    return synthetic.to_bf16_bits(x)


@pytest.mark.parametrize("m,k", [(1, 128), (7, 2048), (33, 100), (300, 7168), (5, 1)])
def test_fp8_rows_bit_exact(m, k):
    import quantized_gemm_int4_amd as hm
    xb = _rows(m, k, m * 1000 + k)
    x8, s = hm.hm_quant_fp8_rows(bf16_to_dev(xb))
    torch.cuda.synchronize()
    rc, rs = quant.quant_fp8_rows(xb)
    assert np.array_equal(s.cpu().numpy().view(np.uint32), rs.view(np.uint32))
    assert np.array_equal(x8.cpu().numpy(), rc)


@pytest.mark.parametrize("m,k", [(5, 8), (9, 512), (6, 520), (4, 1032), (3, 4096), (2, 4104), (2, 8192),
                                 (3, 8200), (262149, 8)])
def test_fp8_rows_every_row_length_class(m, k):
    """Each register-chunk count of the wave-per-row kernel (k up to 512,
    1024, 2048, 4096, 8192, full and ragged), the two-pass kernel above 8192,
    row counts that leave a block's waves idle, and more rows than the grid
    holds (grid-stride loop)."""
    import quantized_gemm_int4_amd as hm
    xb = _rows(m, k, m + 7 * k)
    x8, s = hm.hm_quant_fp8_rows(bf16_to_dev(xb))
    torch.cuda.synchronize()
    rc, rs = quant.quant_fp8_rows(xb)
    assert np.array_equal(s.cpu().numpy().view(np.uint32), rs.view(np.uint32))
    assert np.array_equal(x8.cpu().numpy(), rc)


def test_fp8_rows_extreme_scales():
    """Rows whose scale falls outside the reciprocal path's range (amax about
    2^-100 and 2^115: the IEEE division) next to rows inside it, with bf16
    subnormal elements and -0 in a normal row, all bit-exact."""
    import quantized_gemm_int4_amd as hm
    r = np.random.default_rng(5)
    x = r.normal(0, 1, size=(8, 1024)).astype(np.float32)
    x[0] *= np.float32(2.0 ** -100)
    x[1] *= np.float32(2.0 ** -92)
    x[2] *= np.float32(2.0 ** 100)
    x[3] *= np.float32(2.0 ** 115)
    x[4, :64] = np.float32(2.0 ** -130) * r.integers(-64, 64, size=64)     # bf16 subnormals
    x[4, 64:70] = -0.0
    x[5] = 0.0
    x[5, 17] = -1.0                                                          # one nonzero, negative
    x[6] = np.float32(2.0 ** -20) * r.normal(0, 1, size=1024)
    x[6, 3] = 1.0                                                            # others far below the amax
    xb = synthetic.to_bf16_bits(x)
    x8, s = hm.hm_quant_fp8_rows(bf16_to_dev(xb))
    torch.cuda.synchronize()
    rc, rs = quant.quant_fp8_rows(xb)
    assert np.array_equal(s.cpu().numpy().view(np.uint32), rs.view(np.uint32))
    assert np.array_equal(x8.cpu().numpy(), rc)


def test_fp8_rows_workload_outliers():
    import quantized_gemm_int4_amd as hm
    xb = synthetic.activations(3, 256, 2048, outliers=0.01)
    x8, s = hm.hm_quant_fp8_rows(bf16_to_dev(xb))
    rc, rs = quant.quant_fp8_rows(xb)
    assert np.array_equal(s.cpu().numpy().view(np.uint32), rs.view(np.uint32))
    assert np.array_equal(x8.cpu().numpy(), rc)
