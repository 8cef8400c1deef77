"""Pins for the oracle's device-layout builder: every (expert, column, k) of
the standard format is found again at the address the layout rule gives, and
the padding holds value-zero codes."""
import numpy as np
import pytest

from oracle import layout, quant


def _std(fmt, E, N, K, seed):
    r = np.random.default_rng(seed)
    codes = r.integers(0, 256, size=(E, N, K // 2), dtype=np.uint8)
    if fmt == quant.FMT_MXFP4:
        scales = r.integers(0, 255, size=(E, N, K // 32), dtype=np.uint8)
    else:
        scales = r.integers(0, 65536, size=(E, N, K // 128)).astype(np.uint16)
    zeros = r.integers(0, 16, size=(E, N, K // 128), dtype=np.uint8) if fmt == quant.FMT_UINT4_ZP else None
    return codes, scales, zeros


@pytest.mark.parametrize("fmt", quant.FORMATS)
@pytest.mark.parametrize("E,N,K", [(1, 16, 128), (2, 37, 256), (1, 5, 640)])
def test_layout_addresses(fmt, E, N, K):
    codes, scales, zeros = _std(fmt, E, N, K, 3)
    out = layout.transform_ref(fmt, codes, scales, zeros)
    ob, oc, total = layout.sizes(fmt, E, N, K)
    assert out.size == total and ob % 256 == 0 and oc % 256 == 0 and total % 256 == 0
    NB, KG = (N + 15) // 16, K // 128
    for e in range(E):
        for n in range(NB * 16):
            for k in range(K):
                nb, c, g, kk = n // 16, n % 16, k // 128, k % 128
                if fmt == quant.FMT_MXFP4:
                    slot = c + 16 * (kk // 32)
                    byte = (kk % 32) // 2
                    shift = 4 * (k % 2)
                else:
                    # word j = kk // 32 of the slot; value i = kk % 8 sits in nibble
                    # position i/2 (even i) or 4 + (i-1)/2 (odd i) of that word
                    slot = c + 16 * ((kk % 32) // 8)
                    i = kk % 8
                    pos = i // 2 if i % 2 == 0 else 4 + (i - 1) // 2
                    byte = 4 * (kk // 32) + pos // 2
                    shift = 4 * (pos % 2)
                addr = ((e * NB + nb) * KG + g) * 1024 + slot * 16 + byte
                nib = (out[addr] >> shift) & 0xF
                if n < N:
                    src = (codes[e, n, k // 2] >> (4 * (k % 2))) & 0xF
                    want = src ^ 8 if fmt == quant.FMT_INT4_SYM else src
                else:
                    want = 8 if fmt == quant.FMT_INT4_SYM else 0
                assert nib == want
    # scales and zero points
    for e in range(E):
        for n in range(NB * 16):
            nb, c = n // 16, n % 16
            if fmt == quant.FMT_MXFP4:
                KG4 = (KG + 3) // 4
                for blk in range(K // 32):
                    g, h = blk // 4, blk % 4
                    L = c + 16 * h
                    a = ob + (((e * NB + nb) * KG4 + g // 4) * 64 + L) * 4 + g % 4
                    assert out[a] == (scales[e, n, blk] if n < N else 0)
            else:
                for g in range(KG):
                    a = ob + 2 * (((e * NB + nb) * KG + g) * 16 + c)
                    v = int(out[a]) | (int(out[a + 1]) << 8)
                    assert v == (scales[e, n, g] if n < N else 0)
                    if fmt == quant.FMT_UINT4_ZP:
                        za = oc + ((e * NB + nb) * KG + g) * 8 + c // 2
                        zn = (out[za] >> (4 * (c % 2))) & 0xF
                        assert zn == (zeros[e, n, g] if n < N else 0)
