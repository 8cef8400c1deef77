"""CPU oracle for the low-bit GEMM path: plain, slow, obviously correct.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import anything from this package.  The
product path (the HIP library and its Python binding) never imports, links or
calls it, and this package imports nothing from the product.

What it computes, and where each piece comes from (pages are cited by site,
title and section; the pages are the only specification):

* ``codecs``  -- bit-level number formats: bf16, OCP E4M3 (fp8), E2M1 (fp4),
  E8M0 (power-of-two block scale).
* ``quant``   -- the weight quantizers (symmetric INT4, asymmetric uint4 with a
  zero point, MXFP4, MXINT4), nibble packing, exact dequantization, per-token
  FP8 activation quantization, storage accounting.
* ``gemm``    -- Y = X_hat . W_hat^T in fp64, its error bound sum_k |x w|, the
  acceptance check, and the element-wise check of the MoE block steps.
* ``moe``     -- expert sort/offsets, the per-expert (grouped) GEMM, and the
  MoE block steps around it (SiLU-gated product, top-k weighted combine).
* ``layout``  -- an independent implementation of the library's documented
  device weight layout, used to check the repack byte for byte.

Everything is NumPy, float64 unless the pages or the format fix a precision.
Numbers are processed in the order the definitions state; a BLAS matmul is the
only library primitive used for the contraction.
"""
from . import codecs, quant, gemm, moe, layout  # noqa: F401
