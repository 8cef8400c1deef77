"""GPU checks of the measurement helpers: the autotuner picks a valid tuning
whose output agrees with the oracle, and the plain-read probe reads every
byte (the xor of its per-block words equals the xor of the buffer's words)."""
import numpy as np
import pytest
import torch

import synthetic
from oracle import codecs, gemm, quant
from gpu_util import bf16_to_dev, bits_of, quantize_experts, std_to_dev

pytestmark = pytest.mark.gpu


def test_tune_dense_small_and_parity():
    import quantized_gemm_int4_amd as hm
    from quantized_gemm_int4_amd import tune
    n, k = 1000, 1152
    codes, scales, zeros, what = quantize_experts(quant.FMT_UINT4_ZP, [synthetic.weights(20, n, k)])
    d = hm.wdesc("uint4_zp", n, k)
    w = hm.hm_transform(d, *std_to_dev(quant.FMT_UINT4_ZP, codes, scales, zeros))
    xb = synthetic.activations(20, 40, k)
    x = bf16_to_dev(xb)
    tab = tune.tune_dense(d, [w, w.clone()], x, [1, 17, 40], reps=3)
    for m in (1, 17, 40):
        tn = tab.lookup(d, 0, m)
        y = hm.hm_gemm(d, w, x[:m], tuning=tn)
        torch.cuda.synchronize()
        yref, b = gemm.gemm_ref(codecs.bf16_value(xb[:m]).astype(np.float64), what[0].astype(np.float64))
        res = gemm.check(bits_of(y), yref, b)
        assert res["ok"], (m, tn, res)
        e = tab.entries[tune._key(d, 0)][str(m)]
        assert e["us"] <= e["default_us"] + 1e-9


@pytest.mark.parametrize("nbytes,blocks,unroll", [(16, 1, 1), (4096, 3, 2), (1 << 20, 64, 4), ((1 << 22) + 48, 1000, 8)])
def test_read_probe_reads_every_word(nbytes, blocks, unroll):
    import quantized_gemm_int4_amd as hm
    r = np.random.default_rng(nbytes)
    host = r.integers(0, 2 ** 32, size=nbytes // 4, dtype=np.uint64).astype(np.uint32)
    buf = torch.from_numpy(host.view(np.int32)).cuda()
    out = hm.hm_read_probe(buf, blocks, unroll)
    got = np.bitwise_xor.reduce(out.cpu().numpy().view(np.uint32))
    assert got == np.bitwise_xor.reduce(host)
