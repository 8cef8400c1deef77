"""Pins for the oracle's dense GEMM, bound and acceptance check: closed forms
(one-hot weights, all-ones weights), a brute-force triple loop, and planted
mistakes in an oracle copy that the check must reject."""
import numpy as np

from oracle import codecs, gemm, quant
from synthetic import to_bf16_bits


def _xbf16(m, k, seed):
    return codecs.bf16_value(to_bf16_bits(np.random.default_rng(seed).normal(0, 1, (m, k)).astype(np.float32)))


def test_one_hot_weights_gather_columns_exactly():
    m, n, k = 5, 24, 256
    x = _xbf16(m, k, 1).astype(np.float64)
    ks = np.random.default_rng(2).integers(0, k, size=n)
    q = np.zeros((n, k), dtype=np.int64)
    q[np.arange(n), ks] = 1
    sbits = np.full((n, k // 128), 0x3E80, dtype=np.uint16)   # bf16 0.25 (power of two)
    w = quant.dequant(quant.FMT_INT4_SYM, quant.pack_nibbles(q), sbits)
    y, b = gemm.gemm_ref(x, w)
    assert np.array_equal(y, x[:, ks] * 0.25)
    # exact in bf16 as well: a bf16 times a power of two
    yb = codecs.bf16_rne_bits(y.astype(np.float32))
    assert gemm.check(yb, y, b)["ok"]


def test_all_ones_codes_give_row_sums():
    m, n, k = 3, 4, 128
    x = _xbf16(m, k, 3).astype(np.float64)
    u = np.ones((n, k), dtype=np.int64)
    sbits = np.full((n, 1), 0x3F80, dtype=np.uint16)          # s = 1
    z = np.zeros((n, 1), dtype=np.uint8)
    w = quant.dequant(quant.FMT_UINT4_ZP, quant.pack_nibbles(u), sbits, z)
    y, _ = gemm.gemm_ref(x, w)
    for j in range(n):
        assert np.allclose(y[:, j], [sum(row) for row in x], rtol=0, atol=1e-12)


def test_brute_force_triple_loop():
    r = np.random.default_rng(4)
    m, n, k = 3, 5, 7
    x = r.normal(size=(m, k))
    w = r.normal(size=(n, k))
    y, b = gemm.gemm_ref(x, w)
    for i in range(m):
        for j in range(n):
            acc = 0.0
            bb = 0.0
            for kk in range(k):
                acc += x[i, kk] * w[j, kk]
                bb += abs(x[i, kk] * w[j, kk])
            assert abs(acc - y[i, j]) < 1e-12 and abs(bb - b[i, j]) < 1e-12


def _setup(seed=5, m=4, n=32, k=256):
    x = _xbf16(m, k, seed).astype(np.float64)
    w = np.random.default_rng(seed + 1).normal(0, 0.02, (n, k)).astype(np.float32)
    st = quant.quantize(quant.FMT_INT4_SYM, w)
    wq = quant.dequant(quant.FMT_INT4_SYM, st["codes"], st["scales"]).astype(np.float64)
    return x, wq


def test_check_accepts_correct_bf16_result():
    x, wq = _setup()
    y, b = gemm.gemm_ref(x, wq)
    assert gemm.check(codecs.bf16_rne_bits(y.astype(np.float32)), y, b)["ok"]


def test_check_rejects_planted_mistakes():
    """Plant the plausible slips in a copy of the reference and check that the
    acceptance rule rejects each: a dropped K term, a sign flip, a transposed
    (shifted) operand, a wrong scale group and an off-by-one column."""
    x, wq = _setup()
    y, b = gemm.gemm_ref(x, wq)
    bad = {
        "dropped_term": x[:, 1:] @ wq[:, 1:].T,
        "sign": -y,
        "shifted_k": x @ np.roll(wq, 1, axis=1).T,
        "scale_group": x @ np.concatenate([wq[:, :128] * 2, wq[:, 128:]], axis=1).T,
        "column_shift": np.roll(y, 1, axis=1),
    }
    for name, yb in bad.items():
        res = gemm.check(codecs.bf16_rne_bits(yb.astype(np.float32)), y, b)
        assert not res["ok"], name


def test_check_zero_rows_need_exact_zero():
    y = np.zeros((1, 4))
    b = np.zeros((1, 4))
    assert gemm.check(np.zeros((1, 4), np.uint16), y, b)["ok"]
    assert not gemm.check(np.array([[0, 0, 0x3F80, 0]], np.uint16), y, b)["ok"]
