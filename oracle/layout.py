"""Independent implementation of the library's device weight layout
("layout 1"), used only to check the repack kernel byte for byte.

The pages say the weights, scales and zero points are first brought into one
common representation and then padded and re-ordered for the device and the
kernel (ywsung.com note "How vLLM Humming computes 4 bits", section on layout;
aihaber.org article, Architecture).  The re-ordered layout itself is this
library's own design; it is specified here in words and built element by
element from that specification:

E experts, N columns (output features), K (multiple of 128), NB = ceil(N/16)
blocks of 16 columns, KG = K/128 steps of 128 along K.

Region A, codes: E*NB*KG tiles of 1024 bytes, tile index (e*NB + nb)*KG + g.
  A tile is 64 slots of 16 bytes.  Slot L covers column n = 16*nb + L%16 and
  quarter h = L//16.
  * int4 formats: 32-bit word j of slot L (j in 0..3, little endian) holds
    the 8 values k = 128*g + 32*j + 8*h + i, i in 0..7, with value i in nibble
    position i/2 for even i and 4 + (i-1)/2 for odd i (so nibbles p and p+4
    are the consecutive pair 2p, 2p+1).
    Stored value: uint4_zp -> u; int4_sym -> q + 8 (offset binary).
  * mxfp4, mxint4: byte b (0..15) of slot L holds k = 128*g + 32*h + 2*b (low
    nibble) and k+1 (high nibble), the E2M1 / two's complement bits as given.
  Columns n >= N hold the value-zero code (int4_sym 8, others 0).
Region B, scales (starts at the next 256-byte boundary):
  * int4 formats: bf16 entry ((e*NB + nb)*KG + g)*16 + c = scale of column
    16*nb + c, group g.
  * mxfp4, mxint4: KG4 = ceil(KG/4); byte (((e*NB + nb)*KG4 + g//4)*64 + L)*4 + g%4 =
    E8M0 of column 16*nb + L%16 and 32-block 4*g + L//16.
  Padding entries are 0.
Region C, zero points (uint4_zp only, next 256-byte boundary): 8 bytes per
  ((e*NB + nb)*KG + g); byte c//2, nibble c%2 (low nibble for even c) = zero
  point of column 16*nb + c, group g.  Padding 0.
Total size: end of the last region rounded up to 256 bytes.  Every byte not
named above (the alignment gaps between regions) is zero.

uint3_zp and uint2_zp (3- and 2-bit codes with zero points) are widened: their
device bytes are exactly those of uint4_zp built from the same code and zero
point values (each below 8 or 4), with the same scales.

int8_sym (one byte per value): Region A holds E*NB*KG tiles of 2048 bytes,
tile index (e*NB + nb)*KG + g; a tile is two halves of 64 slots of 16 bytes;
slot L of half p covers column 16*nb + L%16 and quarter h = L//16, and its
byte 8*jj + i holds the value k = 128*g + 32*(2*p + jj) + 8*h + i (jj in 0..1,
i in 0..7) as its two's complement byte.  Columns >= N hold 0.  Region B is
the int4 one (bf16 scales); there is no Region C.
"""
import numpy as np

from .quant import (FMT_INT4_SYM, FMT_INT8_SYM, FMT_UINT4_ZP, FMT_MXFP4, MX_FORMATS, NARROW_ZP, pack_nibbles,
                    unpack_bits, unpack_nibbles)


def _align(x, a=256):
    return (x + a - 1) // a * a


def sizes(fmt, E, N, K):
    """(offset_B, offset_C, total) in bytes."""
    if fmt in NARROW_ZP:
        fmt = FMT_UINT4_ZP
    NB = (N + 15) // 16
    KG = K // 128
    a = E * NB * KG * (2048 if fmt == FMT_INT8_SYM else 1024)
    if fmt in MX_FORMATS:
        b = E * NB * ((KG + 3) // 4) * 256
    else:
        b = E * NB * KG * 16 * 2
    c = E * NB * KG * 8 if fmt == FMT_UINT4_ZP else 0
    ob = _align(a)
    oc = _align(ob + b)
    return ob, oc, _align(oc + c)


def transform_ref(fmt, codes, scales, zeros=None):
    """Build the device bytes from the standard format.

    codes  uint8 [E,N,K/2]  (packed nibbles, even k low)
    scales int4: uint16 bf16 bits [E,N,K/128]; mxfp4: uint8 [E,N,K/32]
    zeros  uint8 [E,N,K/128] (uint4_zp only)
    Returns a uint8 array of the total size."""
    if fmt in NARROW_ZP:
        bits = NARROW_ZP[fmt]
        c = np.asarray(codes, dtype=np.uint8)
        wide = np.stack([pack_nibbles(unpack_bits(c[e], bits)) for e in range(c.shape[0])])
        return transform_ref(FMT_UINT4_ZP, wide, scales, np.asarray(zeros) & ((1 << bits) - 1))
    codes = np.asarray(codes, dtype=np.uint8)
    if fmt == FMT_INT8_SYM:
        return _transform_int8_ref(codes, scales)
    E, N, K2 = codes.shape
    K = 2 * K2
    NB = (N + 15) // 16
    KG = K // 128
    ob, oc, total = sizes(fmt, E, N, K)
    out = np.zeros(total, dtype=np.uint8)

    # unsigned nibble values [E, NB*16, K], padded columns at the value-zero code
    u = np.zeros((E, NB * 16, K), dtype=np.uint8)
    if fmt == FMT_INT4_SYM:
        u[:] = 8
    for e in range(E):
        v = unpack_nibbles(codes[e])
        if fmt == FMT_INT4_SYM:
            v = v ^ 8
        u[e, :N] = v

    # Region A: element by element from the slot rule
    tiles = np.zeros((E, NB, KG, 64, 16), dtype=np.uint8)
    L = np.arange(64)
    c = L % 16
    h = L // 16
    if fmt in MX_FORMATS:
        for b in range(16):
            k_lo = 32 * h + 2 * b                          # [64]
            for g in range(KG):
                klo = 128 * g + k_lo
                for nb in range(NB):
                    col = 16 * nb + c
                    tiles[:, nb, g, :, b] = u[:, col, klo] | (u[:, col, klo + 1] << 4)
    else:
        words = np.zeros((E, NB, KG, 64, 4), dtype=np.uint32)
        for j in range(4):
            for i in range(8):
                pos = i // 2 if i % 2 == 0 else 4 + (i - 1) // 2
                for g in range(KG):
                    kk = 128 * g + 32 * j + 8 * h + i        # [64]
                    for nb in range(NB):
                        col = 16 * nb + c
                        words[:, nb, g, :, j] |= u[:, col, kk].astype(np.uint32) << (4 * pos)
        tiles = words.view(np.uint8).reshape(E, NB, KG, 64, 16)
    out[:tiles.size] = tiles.ravel()

    # Region B
    if fmt in MX_FORMATS:
        KG4 = (KG + 3) // 4
        sb = np.zeros((E, NB, KG4, 64, 4), dtype=np.uint8)
        sc = np.asarray(scales, dtype=np.uint8)            # [E, N, K/32]
        for g in range(KG):
            for nb in range(NB):
                for l in range(64):
                    n = 16 * nb + l % 16
                    if n < N:
                        sb[:, nb, g // 4, l, g % 4] = sc[:, n, 4 * g + l // 16]
        out[ob:ob + sb.size] = sb.ravel()
    else:
        sb = np.zeros((E, NB, KG, 16), dtype=np.uint16)
        sc = np.asarray(scales, dtype=np.uint16)           # [E, N, KG]
        for nb in range(NB):
            for cc in range(16):
                n = 16 * nb + cc
                if n < N:
                    sb[:, nb, :, cc] = sc[:, n, :]
        out[ob:ob + sb.size * 2] = sb.view(np.uint8).ravel()

    # Region C
    if fmt == FMT_UINT4_ZP:
        zb = np.zeros((E, NB, KG, 8), dtype=np.uint8)
        zz = np.asarray(zeros, dtype=np.uint8) & 0xF       # [E, N, KG]
        for nb in range(NB):
            for cc in range(16):
                n = 16 * nb + cc
                if n < N:
                    zb[:, nb, :, cc // 2] |= (zz[:, n, :] << (4 * (cc % 2))).astype(np.uint8)
        out[oc:oc + zb.size] = zb.ravel()
    return out


def _transform_int8_ref(codes, scales):
    """int8_sym device bytes, element by element from the rule in the header."""
    E, N, K = codes.shape
    NB = (N + 15) // 16
    KG = K // 128
    ob, _, total = sizes(FMT_INT8_SYM, E, N, K)
    out = np.zeros(total, dtype=np.uint8)
    tiles = np.zeros((E, NB, KG, 2, 64, 16), dtype=np.uint8)
    for p in range(2):
        for L in range(64):
            c, h = L % 16, L // 16
            for jj in range(2):
                for i in range(8):
                    for g in range(KG):
                        k = 128 * g + 32 * (2 * p + jj) + 8 * h + i
                        for nb in range(NB):
                            n = 16 * nb + c
                            if n < N:
                                tiles[:, nb, g, p, L, 8 * jj + i] = codes[:, n, k]
    out[:tiles.size] = tiles.ravel()
    sb = np.zeros((E, NB, KG, 16), dtype=np.uint16)
    sc = np.asarray(scales, dtype=np.uint16)
    for nb in range(NB):
        for cc in range(16):
            n = 16 * nb + cc
            if n < N:
                sb[:, nb, :, cc] = sc[:, n, :]
    out[ob:ob + sb.size * 2] = sb.view(np.uint8).ravel()
    return out


def gated_rows(n):
    """Source row of each device row of the gated layout of a gate_up weight
    with n = 2d rows (gate rows 0..d-1, up rows d..2d-1, n a multiple of 32):
    device 16-row block 2i holds gate rows 16i..16i+15 and block 2i+1 the up
    rows d+16i..d+16i+15, so that one wave's pair of column blocks holds both
    halves of 16 outputs.  The buffer of the gated layout equals transform_ref
    of the weight with its rows taken in this order."""
    assert n % 32 == 0
    d = n // 2
    src = []
    for blk in range(n // 16):
        base = (d if blk % 2 else 0) + 16 * (blk // 2)
        src.extend(range(base, base + 16))
    return np.array(src, dtype=np.int64)
