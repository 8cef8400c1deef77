"""Pins for the oracle's quantizers, packing, dequantization and FP8 rows:
the pages' worked examples, brute-force nearest-code searches on small inputs,
and invariants."""
import numpy as np
import pytest
import torch

from conftest import read_golden
from oracle import codecs, quant

G = read_golden("worked_examples.txt")


def test_worked_example_int4():
    ex = G["int4_example"]
    q = quant.quant_int4_sym_fixed_scale(np.array([ex["w"]]), ex["s"])
    assert q[0] == ex["q"]
    assert abs(q[0] * ex["s"] - ex["restored"]) < 1e-15
    lo, hi = G["int4_range"]["lo"], G["int4_range"]["hi"]
    # out-of-range values are limited (clamped) to the signed 4-bit range
    q2 = quant.quant_int4_sym_fixed_scale(np.array([0.9, -0.9, 100.0, -100.0]), 0.1)
    assert list(q2) == [hi, lo, hi, lo]


def test_worked_example_dot():
    ex = G["dot_example"]
    w = np.array(ex["w"])
    x = np.array(ex["x"])
    assert abs(w @ x - ex["exact"]) < 1e-15
    q = quant.quant_int4_sym_fixed_scale(w, 0.1)
    assert list(q) == [3, -1]
    wq = q * 0.1
    assert np.allclose(wq, ex["wq"], atol=1e-15)
    assert abs(wq @ x - ex["quantized"]) < 1e-15


def test_worked_example_storage():
    ex = G["storage_example"]
    g = int(ex["group"])
    assert quant.storage_bytes(1, g, quant.FMT_INT4_SYM) == ex["bytes"]
    assert quant.bits_per_value(quant.FMT_INT4_SYM) == ex["bits_per_value"]
    # same formula, extended: packed 4-bit zero point, and MX (8-bit scale per 32)
    assert quant.bits_per_value(quant.FMT_UINT4_ZP) == 4.15625
    assert quant.bits_per_value(quant.FMT_MXFP4) == 4.25
    # the dense FFN up-projection weight in the asymmetric format
    assert quant.storage_bytes(14336, 4096, quant.FMT_UINT4_ZP) == 30507008


def _brute_nearest(t, cands):
    """nearest candidate value to t; ties to the even candidate value"""
    d = np.abs(cands - t)
    best = cands[d == d.min()]
    if len(best) == 1:
        return best[0]
    ev = [b for b in best if int(b) % 2 == 0]
    return ev[0]


def test_int4_sym_brute_force():
    r = np.random.default_rng(10)
    w = r.normal(0, 0.02, size=(6, 256)).astype(np.float32)
    w[0, :128] = 0.0                      # an all-zero group
    w[1, :128] = 0.003                    # a constant group
    q, sbits = quant.quant_int4_sym(w)
    s = codecs.bf16_value(sbits).astype(np.float64)
    cands = np.arange(-8, 8, dtype=np.float64)
    for n in range(w.shape[0]):
        for g in range(2):
            amax = np.abs(w[n, g * 128:(g + 1) * 128]).max()
            # scale: bf16 of the fp32 quotient amax/7 (torch conversions as the reference)
            s32 = torch.tensor(float(amax), dtype=torch.float32) / 7.0
            assert sbits[n, g] == s32.to(torch.bfloat16).view(torch.int16).item() & 0xFFFF
            for k in range(g * 128, (g + 1) * 128):
                if s[n, g] == 0:
                    assert q[n, k] == 0
                else:
                    assert q[n, k] == _brute_nearest(float(w[n, k]) / s[n, g], cands)
    assert q.min() >= -8 and q.max() <= 7
    assert (q[0, :128] == 0).all() and s[0, 0] == 0


def test_int4_sym_error_bound():
    w = np.random.default_rng(11).normal(0, 0.02, size=(64, 1024)).astype(np.float32)
    q, sbits = quant.quant_int4_sym(w)
    wq = quant.dequant(quant.FMT_INT4_SYM, quant.pack_nibbles(q), sbits).astype(np.float64)
    s = np.repeat(codecs.bf16_value(sbits).astype(np.float64), 128, axis=1)
    # with the scale from amax/7 the clamp never binds, so |w - w_hat| <= s/2
    assert (np.abs(w - wq) <= s / 2 + 1e-12).all()


def test_uint4_zp_brute_force_and_invariants():
    r = np.random.default_rng(12)
    w = r.normal(0, 0.02, size=(5, 256)).astype(np.float32)
    w[2, 128:] = 0.01                     # constant group -> s = 0
    w[3, :128] = np.abs(w[3, :128]) + 0.05  # all positive -> z clamps at 0
    u, sbits, z = quant.quant_uint4_zp(w)
    s = codecs.bf16_value(sbits).astype(np.float64)
    assert u.max() <= 15 and z.max() <= 15
    for n in range(w.shape[0]):
        for g in range(2):
            blk = w[n, g * 128:(g + 1) * 128].astype(np.float64)
            if s[n, g] == 0:
                assert z[n, g] == 0 and (u[n, g * 128:(g + 1) * 128] == 0).all()
                continue
            zz = min(max(_brute_nearest(-blk.min() / s[n, g], np.arange(-64, 64.0)), 0), 15)
            assert z[n, g] == zz
            for i, wk in enumerate(blk):
                t = wk / s[n, g]
                v = _brute_nearest(t, np.arange(-64, 64.0)) + zz
                assert u[n, g * 128 + i] == min(max(v, 0), 15)
    wq = quant.dequant(quant.FMT_UINT4_ZP, quant.pack_nibbles(u), sbits, z).astype(np.float64)
    sf = np.repeat(s, 128, axis=1)
    # where the group range contains 0 the restore error is at most one step s;
    # a one-signed group (row 3) is where the min-max zero point clamps at 0
    wg = w.reshape(5, 2, 128)
    spans0 = np.repeat((wg.min(axis=2) <= 0) & (wg.max(axis=2) >= 0), 128, axis=1)
    ok = (sf > 0) & spans0
    assert (np.abs(w - wq)[ok] <= sf[ok] + 1e-12).all()
    assert not spans0[3, 0]


def test_mxfp4_rule_brute_force():
    r = np.random.default_rng(13)
    w = r.normal(0, 0.02, size=(4, 128)).astype(np.float32)
    w[0, :32] = 0.0
    w[1, 32:64] *= 1e-30                  # tiny block
    codes, e = quant.quant_mxfp4(w)
    assert e[0, 0] == 0 and (codes[0, :32] == 0).all()
    vals = np.concatenate([codecs.E2M1_MAG, -codecs.E2M1_MAG])
    for n in range(4):
        for b in range(4):
            blk = w[n, 32 * b:32 * (b + 1)].astype(np.float64)
            amax = np.abs(blk).max()
            if amax == 0:
                continue
            X = int(e[n, b]) - 127
            # the shared exponent puts amax in [4, 8) times the scale
            assert 4.0 <= amax / 2.0 ** X < 8.0
            for i, wk in enumerate(blk):
                t = min(max(wk / 2.0 ** X, -6.0), 6.0)
                d = np.abs(codecs.E2M1_MAG - abs(t))
                cand = np.nonzero(d == d.min())[0]
                mag = cand[0] if len(cand) == 1 else [c for c in cand if c % 2 == 0][0]
                assert codes[n, 32 * b + i] & 7 == mag
                assert bool(codes[n, 32 * b + i] & 8) == bool(wk < 0)


def test_pack_unpack_all_bytes():
    p = np.arange(256, dtype=np.uint8).reshape(1, 256)
    u = quant.unpack_nibbles(p)
    assert (u[0, 0::2] == np.arange(256) % 16).all() and (u[0, 1::2] == np.arange(256) // 16).all()
    assert np.array_equal(quant.pack_nibbles(u), p)
    r = np.random.default_rng(14)
    for n in (1, 7, 40):
        for k in (128, 256):
            c = r.integers(0, 16, size=(n, k))
            assert np.array_equal(quant.unpack_nibbles(quant.pack_nibbles(c)), c)
    # two's complement packing of signed codes
    q = np.array([[-8, -1, 0, 7]])
    assert list(quant.pack_nibbles(q)[0]) == [0xF8, 0x70]
    assert list(quant.nibble_to_int4(quant.unpack_nibbles(quant.pack_nibbles(q)))[0]) == [-8, -1, 0, 7]


def test_dequant_exact_and_negative_zero():
    r = np.random.default_rng(15)
    for fmt in quant.FORMATS:
        w = r.normal(0, 0.02, size=(8, 256)).astype(np.float32)
        st = quant.quantize(fmt, w)
        d32 = quant.dequant(fmt, st["codes"], st["scales"], st["zeros"])
        # recompute in fp64 from the parts: the fp32 result must equal it exactly
        u = quant.unpack_nibbles(st["codes"]).astype(np.float64)
        if fmt == quant.FMT_MXFP4:
            ref = codecs.e2m1_value(u.astype(np.uint8)) * np.repeat(codecs.e8m0_value(st["scales"]), 32, 1)
        else:
            s = np.repeat(codecs.bf16_value(st["scales"]).astype(np.float64), 128, 1)
            if fmt == quant.FMT_INT4_SYM:
                ref = np.where(u >= 8, u - 16, u) * s
            else:
                ref = (u - np.repeat(st["zeros"].astype(np.float64), 128, 1)) * s
        assert np.array_equal(d32.astype(np.float64), ref)
    p = np.full((1, 16), 0x88, dtype=np.uint8)          # every code 8 = E2M1 -0
    d = quant.dequant(quant.FMT_MXFP4, p, np.full((1, 1), 127, np.uint8))
    assert (d == 0).all() and np.signbit(d).all()


def test_fp8_rows_brute_force_and_torch():
    r = np.random.default_rng(16)
    x32 = r.normal(0, 1, size=(6, 256)).astype(np.float32)
    x32[1] *= 20.0
    x32[2] = 0.0
    x32[3, 5] = -300.0
    from synthetic import to_bf16_bits
    xb = to_bf16_bits(x32)
    codes, s = quant.quant_fp8_rows(xb)
    x = codecs.bf16_value(xb)
    assert s[2] == 0 and (codes[2] == 0).all()
    for m in range(6):
        amax = np.float32(np.abs(x[m]).max())
        assert s[m] == np.float32(amax) / np.float32(448.0)
        if s[m] == 0:
            continue
        qf = (torch.from_numpy(x[m]) / torch.tensor(s[m])).to(torch.float8_e4m3fn)
        assert np.array_equal(codes[m], qf.view(torch.uint8).numpy())
        # the row maximum lands on (or next to) the largest code
        assert codecs.e4m3_value(codes[m]).__abs__().max() == 448.0


def test_bench_weight_bytes_match_storage():
    """bench.py counts algorithmic weight bytes on its own (the product side
    does not import the oracle); the count equals the oracle's storage size."""
    import importlib.util
    import os
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    spec = importlib.util.spec_from_file_location("_bench", os.path.join(root, "bench.py"))
    b = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(b)
    for n, k, name, fmt in [(14336, 4096, "uint4_zp", quant.FMT_UINT4_ZP), (7168, 2048, "mxfp4", quant.FMT_MXFP4),
                            (4096, 7168, "int4_sym", quant.FMT_INT4_SYM), (1792, 4096, "uint4_zp", quant.FMT_UINT4_ZP)]:
        assert b.weight_bytes(n, k, name) == quant.storage_bytes(n, k, fmt)


# ------------------------------------------------------------------ MXINT4 (reading: 1.2 fixed-point INT4
# elements under an E8M0 scale per 32, the MX rule X = floor(log2 amax))

MXI4_VALUES = [0.0, 0.25, 0.5, 0.75, 1.0, 1.25, 1.5, 1.75, -2.0, -1.75, -1.5, -1.25, -1.0, -0.75, -0.5, -0.25]


def test_mxint4_dequant_all_codes():
    """Nibble c is the two's complement q, value q/4 times 2^(b-127), written out."""
    for b in (0, 1, 100, 127, 130, 253):
        codes = quant.pack_nibbles(np.arange(32).reshape(1, 32) % 16)
        got = quant.dequant(quant.FMT_MXINT4, codes, np.array([[b]], dtype=np.uint8))
        want = np.array([MXI4_VALUES[c % 16] * 2.0 ** (b - 127) for c in range(32)], dtype=np.float32)
        assert np.array_equal(got[0], want), b


def test_mxint4_exact_round_trip():
    """A block made of 2^X q / 4 with max |q| = 7 comes back exactly, scale byte X + 127."""
    r = np.random.default_rng(3)
    for x in (-20, -7, 0, 5):
        q = r.integers(-7, 8, 32)
        q[5] = 7 if r.integers(2) else -7
        w = (q * 2.0 ** (x - 2)).astype(np.float32).reshape(1, 32)
        c, e = quant.quant_mxint4(w)
        assert int(e[0, 0]) == x + 127
        assert np.array_equal(c[0], (q & 0xF).astype(np.uint8))


def test_mxint4_brute_force():
    """Pure-Python check on small random blocks: scale byte from the binary
    exponent of amax, each code the nearest of the 16 (ties to even q), the
    top end saturating at 7 and zero blocks all zero."""
    import math
    r = np.random.default_rng(4)
    w = (r.standard_normal((6, 96)) * np.array([1e-3, 0.02, 1.0, 3.0, 1e5, 2.0 ** -120])[:, None]).astype(np.float32)
    w[2, 32:64] = 0.0                                   # a zero block
    w[3, 64] = 1.95 * 2.0 ** 3                          # saturating block: 4 w / 2^X rounds to 8 -> 7
    w[3, 65:96] = np.clip(w[3, 65:96], -15.0, 15.0)
    c, e = quant.quant_mxint4(w)
    for n in range(w.shape[0]):
        for blk in range(3):
            vals = [float(v) for v in w[n, 32 * blk:32 * blk + 32]]
            amax = max(abs(v) for v in vals)
            if amax == 0.0:
                assert e[n, blk] == 0 and all(c[n, 32 * blk + i] == 0 for i in range(32))
                continue
            x = math.frexp(amax)[1] - 1
            assert e[n, blk] == x + 127
            for i, v in enumerate(vals):
                t = 4.0 * v / 2.0 ** x
                best = min(range(-8, 8), key=lambda q: (abs(t - q), q % 2))
                assert c[n, 32 * blk + i] == (best & 0xF), (n, blk, i, v, best)
    assert c[3, 64] == 7


def test_mxint4_storage_and_layout_match_mxfp4():
    """Same standard-format sizes and the same device arrangement as MXFP4."""
    from oracle import layout
    assert quant.storage_bytes(7168, 2048, quant.FMT_MXINT4) == quant.storage_bytes(7168, 2048, quant.FMT_MXFP4)
    assert layout.sizes(quant.FMT_MXINT4, 2, 40, 384) == layout.sizes(quant.FMT_MXFP4, 2, 40, 384)
    r = np.random.default_rng(5)
    codes = r.integers(0, 256, (2, 40, 192), dtype=np.uint8)
    scales = r.integers(0, 255, (2, 40, 12), dtype=np.uint8)
    a = layout.transform_ref(quant.FMT_MXINT4, codes, scales)
    b = layout.transform_ref(quant.FMT_MXFP4, codes, scales)
    assert np.array_equal(a, b)


# ------------------------------------------------------------------ pins of the FP8 row restore and the
# zero-point scale rule (per-token FP8: ywsung.com note, section on weight format / activation / backend;
# zero points: aihaber.org article, Architecture, with the min-max reading of the oracle's header)

def test_fp8_rows_dequant_power_of_two_scale():
    """A row whose largest magnitude is 448 * 2^j has the exact scale s = 2^j,
    and every element that is an E4M3 value times 2^j comes back exactly:
    x_hat = E4M3(code) * s.  The expected values are written out (448, 1.75,
    -0.5, the smallest subnormal 2^-9, 0 and -26 times 2^j), so a restore that
    divided by s, dropped it or took the wrong row's scale fails."""
    from synthetic import to_bf16_bits
    base = np.array([448.0, 1.75, -0.5, 2.0 ** -9, 0.0, -26.0, 448.0, -448.0], dtype=np.float64)
    rows = []
    for j in (-20, -3, 0, 5):
        rows.append(base * 2.0 ** j)
    x = np.array(rows, dtype=np.float32)
    xb = to_bf16_bits(x)
    codes, s = quant.quant_fp8_rows(xb)
    for i, j in enumerate((-20, -3, 0, 5)):
        assert s[i] == np.float32(2.0 ** j)
    xh = quant.fp8_rows_dequant(codes, s)
    want = np.array(rows)
    assert np.array_equal(xh, want)
    # and the codes themselves: 448 -> 0x7E, 1.75 -> 0x3E, -0.5 -> 0xB0, 2^-9 -> 0x01, -26 = -1.625 * 2^4 -> 0xDD
    assert list(codes[0][:6]) == [0x7E, 0x3E, 0xB0, 0x01, 0x00, 0xDD]
    # a row of two rows' scales: the restore uses each row's own scale
    both = quant.fp8_rows_dequant(np.array([[0x38], [0x38]], dtype=np.uint8), np.array([0.25, 8.0], np.float32))
    assert both[0, 0] == 0.25 and both[1, 0] == 8.0


def test_uint4_zp_scale_rule_against_torch():
    """The zero-point format's scale is bf16(fp32((max - min) / 15)) per
    128-group: recomputed here with torch's fp32 division and bf16
    conversion, plus a written-out group (max 1.5, min 0: s = bf16(0.1) =
    0x3DCD, z = 0, and w = 0.7 -> u = rne(0.7 / 0.10009765625) = 7).  A scale
    over 14 or 16 steps, or from max alone, fails."""
    r = np.random.default_rng(21)
    w = r.normal(0, 0.02, size=(7, 384)).astype(np.float32)
    w[4, :128] = np.linspace(0.0, 1.5, 128, dtype=np.float32)
    w[4, 5] = 0.7
    u, sbits, z = quant.quant_uint4_zp(w)
    for n in range(7):
        for g in range(3):
            blk = torch.from_numpy(w[n, 128 * g:128 * (g + 1)].copy())
            s32 = (blk.max() - blk.min()) / torch.tensor(15.0, dtype=torch.float32)
            want = s32.to(torch.bfloat16).view(torch.int16).item() & 0xFFFF
            assert sbits[n, g] == want, (n, g)
    assert sbits[4, 0] == 0x3DCD and z[4, 0] == 0 and u[4, 5] == 7
    assert u[4, 127] == 15 and u[4, 0] == 0


# ------------------------------------------------------------------ MXFP4 activation rows (W4A4)

def test_mxfp4_rows_worked_block():
    """A bf16 block whose largest magnitude is 6 * 2^j takes the scale byte
    j + 127 (X = floor(log2 amax) - 2 = j) and each value v / 2^X rounds to
    the written-out E2M1 code: 6 -> 7, -6 -> 15, 0.25 -> 0 (tie to even),
    0.75 -> 2 (tie to even), 1.25 -> 2, 1.75 -> 4, 2.5 -> 4, 3.5 -> 6, 5 -> 6,
    -0.125 -> 8 (-0), 4.875 -> 6, 5.125 -> 7 (6 above the tie at 5), 0 -> 0."""
    from synthetic import to_bf16_bits
    vals = [6.0, -6.0, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, -0.125, 4.875, 5.125, 0.0, 0.5, 1.0, 1.5]
    want = [7, 15, 0, 2, 2, 4, 4, 6, 6, 8, 6, 7, 0, 1, 2, 3]
    for j in (-10, 0, 3):
        blk = np.array(vals + vals, dtype=np.float32) * np.float32(2.0 ** j)
        xb = to_bf16_bits(blk.reshape(1, 32))
        assert np.array_equal(codecs.bf16_value(xb)[0], blk)          # exact in bf16
        packed, e = quant.quant_mxfp4_rows(xb)
        assert e[0, 0] == j + 127
        codes = quant.unpack_nibbles(packed)[0]
        assert list(codes[:16]) == want and list(codes[16:]) == want
        xh = quant.mxfp4_rows_dequant(packed, e)[0]
        mags = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
        assert xh[0] == 6.0 * 2.0 ** j and xh[8] == 4.0 * 2.0 ** j and np.signbit(xh[9]) and xh[9] == 0.0
        assert all(abs(xh[i]) == mags[want[i] & 7] * 2.0 ** j for i in range(16))
    # a zero row: scale byte 0, zero codes
    packed, e = quant.quant_mxfp4_rows(np.zeros((1, 64), dtype=np.uint16))
    assert (e == 0).all() and (packed == 0).all()


# ------------------------------------------------------------------ 3- and 2-bit zero-point formats

@pytest.mark.parametrize("bits", [2, 3])
def test_uint_zp_narrow_brute_force(bits):
    """The zero-point rule at 3 and 2 bits: scale bf16(fp32((max - min) /
    (2^b - 1))) recomputed with torch, zero point and codes by nearest-value
    search with ties to even, the clamp at 0 and 2^b - 1, s = 0 groups; at 4
    bits the generic rule equals quant_uint4_zp."""
    top = (1 << bits) - 1
    r = np.random.default_rng(30 + bits)
    w = r.normal(0, 0.02, size=(5, 256)).astype(np.float32)
    w[2, 128:] = 0.01                                         # constant group -> s = 0
    w[3, :128] = np.abs(w[3, :128]) + 0.05                    # one-signed -> z clamps at 0
    u, sbits, z = quant.quant_uint_zp(w, bits)
    s = codecs.bf16_value(sbits).astype(np.float64)
    assert u.max() <= top and z.max() <= top
    for n in range(5):
        for g in range(2):
            blk = w[n, g * 128:(g + 1) * 128]
            tb = torch.from_numpy(blk.copy())
            s32 = (tb.max() - tb.min()) / torch.tensor(float(top), dtype=torch.float32)
            assert sbits[n, g] == s32.to(torch.bfloat16).view(torch.int16).item() & 0xFFFF
            if s[n, g] == 0:
                assert z[n, g] == 0 and (u[n, g * 128:(g + 1) * 128] == 0).all()
                continue
            zz = min(max(_brute_nearest(-float(blk.min()) / s[n, g], np.arange(-64, 64.0)), 0), top)
            assert z[n, g] == zz
            for i, wk in enumerate(blk.astype(np.float64)):
                v = _brute_nearest(wk / s[n, g], np.arange(-64, 64.0)) + zz
                assert u[n, g * 128 + i] == min(max(v, 0), top)
    u4, s4, z4 = quant.quant_uint_zp(w, 4)
    u4r, s4r, z4r = quant.quant_uint4_zp(w)
    assert np.array_equal(u4, u4r) and np.array_equal(s4, s4r) and np.array_equal(z4, z4r)


def test_pack_bits_layout_and_round_trips():
    """2-bit: value 4j + i at bits 2i of byte j (every byte value decodes and
    re-encodes); 3-bit: codes 0..7 pack to the 24-bit word 0o76543210 =
    0xFAC688, i.e. bytes 0x88 0xC6 0xFA; random round trips at both widths."""
    p = np.arange(256, dtype=np.uint8).reshape(1, 256)
    u = quant.unpack_bits(p, 2)
    for i in range(4):
        assert (u[0, i::4] == (np.arange(256) >> (2 * i)) & 3).all()
    assert np.array_equal(quant.pack_bits(u, 2), p)
    assert list(quant.pack_bits(np.arange(8).reshape(1, 8), 3)[0]) == [0x88, 0xC6, 0xFA]
    r = np.random.default_rng(7)
    for bits in (2, 3):
        c = r.integers(0, 1 << bits, size=(9, 256))
        assert np.array_equal(quant.unpack_bits(quant.pack_bits(c, bits), bits), c)


def test_narrow_storage_and_dequant():
    """Storage by the pages' formula (codes + 16-bit scale + zero point per
    128): 3.1484375 and 2.140625 bits per value; dequant is s * (u - z) per
    element, recomputed from the unpacked parts."""
    assert quant.bits_per_value(quant.FMT_UINT3_ZP) == (128 * 3 + 16 + 3) / 128
    assert quant.bits_per_value(quant.FMT_UINT2_ZP) == (128 * 2 + 16 + 2) / 128
    r = np.random.default_rng(8)
    w = r.normal(0, 0.02, size=(6, 384)).astype(np.float32)
    for fmt, bits in quant.NARROW_ZP.items():
        st = quant.quantize(fmt, w)
        d = quant.dequant(fmt, st["codes"], st["scales"], st["zeros"]).astype(np.float64)
        u = quant.unpack_bits(st["codes"], bits).astype(np.float64)
        s = np.repeat(codecs.bf16_value(st["scales"]).astype(np.float64), 128, 1)
        z = np.repeat(st["zeros"].astype(np.float64), 128, 1)
        assert np.array_equal(d, (u - z) * s)


def test_int8_sym_brute_force_and_storage():
    """Symmetric INT8 (the INT4 rule at 8 bits): s = bf16(fp32(amax / 127))
    recomputed with torch, each code the nearest of -128..127 (ties to even),
    the clamp, |w - w_hat| <= s / 2; 8.125 bits per value by the pages'
    storage formula; dequant s * q from the signed bytes."""
    r = np.random.default_rng(33)
    w = r.normal(0, 0.02, size=(4, 256)).astype(np.float32)
    w[1, :128] = 0.0
    q, sbits = quant.quant_int8_sym(w)
    s = codecs.bf16_value(sbits).astype(np.float64)
    cands = np.arange(-128, 128, dtype=np.float64)
    for n in range(4):
        for g in range(2):
            blk = w[n, 128 * g:128 * (g + 1)]
            s32 = torch.tensor(float(np.abs(blk).max()), dtype=torch.float32) / 127.0
            assert sbits[n, g] == s32.to(torch.bfloat16).view(torch.int16).item() & 0xFFFF
            for i, wk in enumerate(blk.astype(np.float64)):
                want = 0 if s[n, g] == 0 else _brute_nearest(wk / s[n, g], cands)
                assert q[n, 128 * g + i] == want
    assert quant.quant_int8_sym(np.full((1, 128), 1.0, np.float32))[0].max() == 127
    assert quant.bits_per_value(quant.FMT_INT8_SYM) == 8.125
    st = quant.quantize(quant.FMT_INT8_SYM, w)
    d = quant.dequant(quant.FMT_INT8_SYM, st["codes"], st["scales"]).astype(np.float64)
    assert np.array_equal(d, q.astype(np.float64) * np.repeat(s, 128, 1))
    sr = np.repeat(s, 128, 1)
    assert (np.abs(w - d) <= sr / 2 + 1e-12).all()
