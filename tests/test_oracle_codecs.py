"""Pins for the oracle's number formats, against closed forms, brute force and
torch's own conversions (a library routine independent of the oracle)."""
import numpy as np
import pytest
import torch

from oracle import codecs


def test_bf16_rne_matches_torch():
    r = np.random.default_rng(1)
    x = np.concatenate([
        r.normal(0, 1, 20000), r.normal(0, 1e-30, 2000), r.normal(0, 1e30, 2000),
        [0.0, -0.0, 1.0, -1.0, 3.0e38, 1e-45, -1e-45, 1.00390625, 1.01171875],
    ]).astype(np.float32)
    # exact ties: 1 + 2^-8 (tie, keep even -> 1.0) and 1 + 3*2^-8 (tie -> up)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = codecs.bf16_rne_bits(x)
    assert np.array_equal(got, ref)
    assert codecs.bf16_rne_bits(np.float32(1.00390625)) == 0x3F80
    assert codecs.bf16_rne_bits(np.float32(1.01171875)) == 0x3F82


def test_bf16_value_widening_exact():
    bits = np.arange(0, 65536, dtype=np.uint32).astype(np.uint16)
    v = codecs.bf16_value(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).float().numpy()
    same = (v.view(np.uint32) == ref.view(np.uint32)) | (np.isnan(v) & np.isnan(ref))
    assert same.all()


def test_ulp_bf16_closed_form():
    u = codecs.ulp_bf16(np.array([1.0, 1.5, -1.99, 2.0, 0.0, 2.0 ** -126, 2.0 ** -130, 448.0]))
    assert list(u) == [2.0 ** -7, 2.0 ** -7, 2.0 ** -7, 2.0 ** -6, 2.0 ** -133,
                       2.0 ** -133, 2.0 ** -133, 2.0 ** 1]


def test_e4m3_decode_closed_form_and_torch():
    codes = np.arange(256)
    ref_torch = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    for c in codes:
        s = -1.0 if c & 0x80 else 1.0
        e = (c >> 3) & 15
        m = c & 7
        if e == 15 and m == 7:
            assert np.isnan(codecs.E4M3_TABLE[c]) and np.isnan(ref_torch[c])
            continue
        v = s * np.ldexp(m / 8.0, -6) if e == 0 else s * np.ldexp(1.0 + m / 8.0, e - 7)
        assert codecs.E4M3_TABLE[c] == v == ref_torch[c]
        assert np.signbit(codecs.E4M3_TABLE[c]) == bool(c & 0x80)
    assert codecs.E4M3_TABLE[0x7E] == 448.0
    assert codecs.E4M3_TABLE[1] == 2.0 ** -9


def test_e4m3_roundtrip_all_codes():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    back = codecs.e4m3_rne_sat(codecs.e4m3_value(codes))
    assert np.array_equal(back, codes)


def test_e4m3_encode_matches_torch_in_range():
    r = np.random.default_rng(2)
    x = np.concatenate([r.uniform(-448, 448, 50000), r.normal(0, 1, 50000),
                        r.normal(0, 1e-3, 20000)]).astype(np.float32)
    # add all exact midpoints between consecutive finite codes (ties)
    pos = codecs.E4M3_TABLE[:0x7F]
    mids = ((pos[:-1] + pos[1:]) / 2).astype(np.float32)
    x = np.concatenate([x, mids, -mids])
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = codecs.e4m3_rne_sat(x.astype(np.float64))
    assert np.array_equal(got, ref)


def test_e4m3_saturation_and_edges():
    f = codecs.e4m3_rne_sat
    assert f(np.array([500.0]))[0] == 0x7E
    assert f(np.array([-1e9]))[0] == 0xFE
    assert f(np.array([464.0]))[0] == 0x7E
    assert f(np.array([2.0 ** -10]))[0] == 0          # tie between 0 and 2^-9 -> even (0)
    assert f(np.array([3 * 2.0 ** -10]))[0] == 2      # tie between codes 1 and 2 -> 2
    assert f(np.array([-2.0 ** -12]))[0] == 0x80      # negative underflow keeps sign


def test_e2m1_decode_closed_form():
    for c in range(16):
        s = -1.0 if c & 8 else 1.0
        e = (c >> 1) & 3
        m = c & 1
        v = s * (0.5 * m if e == 0 else 2.0 ** (e - 1) * (1 + m / 2.0))
        assert codecs.e2m1_value(np.array([c]))[0] == v
    assert np.signbit(codecs.e2m1_value(np.array([8]))[0])


def test_e2m1_rne_ties_and_saturation():
    x = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.5, 100.0, -0.25, -5.0])
    vals = codecs.e2m1_value(codecs.e2m1_rne_sat(x))
    assert list(vals) == [0.0, 1.0, 1.0, 2.0, 2.0, 4.0, 4.0, 6.0, 6.0, -0.0, -4.0]


def test_e2m1_encode_brute_force():
    r = np.random.default_rng(3)
    x = np.concatenate([r.uniform(-7, 7, 4000), r.normal(0, 1, 4000)])
    mags = codecs.E2M1_MAG
    got = codecs.e2m1_rne_sat(x)
    for xi, gi in zip(x, got):
        a = min(abs(xi), 6.0)
        d = np.abs(mags - a)
        best = np.nonzero(d == d.min())[0]
        code = best[0] if len(best) == 1 else [b for b in best if b % 2 == 0][0]
        assert (gi & 7) == code and bool(gi & 8) == (xi < 0 or (xi == 0 and np.signbit(xi)))


def test_e8m0():
    v = codecs.e8m0_value(np.array([0, 1, 127, 254, 255]))
    assert v[0] == 2.0 ** -127 and v[1] == 2.0 ** -126 and v[2] == 1.0 and v[3] == 2.0 ** 127
    assert np.isnan(v[4])
    # the smallest product used by MX dequant is representable in fp32
    assert np.float32(0.5 * 2.0 ** -127) == 2.0 ** -128
