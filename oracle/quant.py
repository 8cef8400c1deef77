"""Weight quantizers, nibble packing, exact dequantization and per-token FP8
activation quantization (oracle side).

Sources (pages cited by site and section):

* Symmetric INT4: a weight w is stored as q = round(w/s), restored as s*q, and
  the signed 4-bit range is -8..7 with out-of-range values limited separately
  (ywsung.com note "How vLLM Humming computes 4 bits", section on scales).
  Reading: round = round-half-to-even, "limited" = clamp.
* Group-wise scales: one 16-bit scale per 128 weights (same section); 128
  nibbles + one bf16 scale = 66 bytes, 4.125 bits per value.
* Zero points are part of the unified weight representation (aihaber.org
  article, Architecture; ywsung.com note, section on layout, figure on the
  quantization description).  The pages give no formula; the reading used is
  min-max asymmetric quantization with an integer zero point:
  s = (max-min)/15, z = clamp(round(-min/s), 0, 15), u = clamp(round(w/s)+z, 0, 15),
  restored as s*(u-z).
* MXFP4 is named (cocoloop.cn news item, format list; aihaber.org, hardware and
  format support) without a bit layout; the OCP MX v1.0 rule is used: per 32
  values, shared exponent X = floor(log2 amax) - 2 (2 = largest E2M1 exponent),
  clamped to [-127, 127], stored as E8M0 byte X+127; elements E2M1(w / 2^X) with
  round-to-nearest-even and saturation.  amax = 0 gives byte 0 and zero codes.
* Per-token FP8 activations (ywsung.com note, section on weight format /
  activation / backend): per row s = amax/448 in fp32, x8 = E4M3(x/s) with the
  division in fp32, round-to-nearest-even, saturating; amax = 0 gives s = 0 and
  zero codes.

Packing of the standard format: element k = 2j goes to the low nibble of byte
j, k = 2j+1 to the high nibble.  Codes are stored as the 4-bit pattern: two's
complement for symmetric INT4, unsigned for the zero-point format, E2M1 bits
for MXFP4.
"""
import numpy as np

from . import codecs

GROUP_INT4 = 128
GROUP_MX = 32

FMT_INT4_SYM = "int4_sym"
FMT_UINT4_ZP = "uint4_zp"
FMT_MXFP4 = "mxfp4"
FMT_MXINT4 = "mxint4"
FMT_UINT3_ZP = "uint3_zp"
FMT_UINT2_ZP = "uint2_zp"
FMT_INT8_SYM = "int8_sym"
FORMATS = (FMT_INT4_SYM, FMT_UINT4_ZP, FMT_MXFP4)
# narrower unsigned formats with a zero point (INT1..INT8 are in the pages'
# format list, cocoloop.cn news item; GPTQ INT3 is their compatibility case)
NARROW_ZP = {FMT_UINT3_ZP: 3, FMT_UINT2_ZP: 2}
# formats with one E8M0 scale per 32 values (the MX family)
MX_FORMATS = (FMT_MXFP4, FMT_MXINT4)


def _groups(w, g):
    n, k = w.shape
    assert k % g == 0, "K must be a multiple of the group size"
    return w.reshape(n, k // g, g)


# ----------------------------------------------------------------------------- symmetric INT4

def quant_int4_sym_fixed_scale(w, s):
    """q = clamp(round_half_even(w/s), -8, 7) for one given scale s (fp64).
    This is the worked-example form: a fixed scale, no bf16 rounding."""
    w = np.asarray(w, dtype=np.float64)
    return np.clip(np.rint(w / s), -8, 7).astype(np.int8)


def quant_int4_sym(w):
    """Symmetric INT4, group 128 along K, bf16 scales.

    Per (row n, group g):  amax = max|w|;  s = bf16(fp32(amax / 7));
    q = clamp(rne(w / s), -8, 7) with the division in fp64 against the stored
    (bf16) scale, so that s*q is the nearest restore;  s = 0 gives q = 0.
    Returns (q int8 [N,K], scale bf16 bits uint16 [N,K/128])."""
    w = np.asarray(w, dtype=np.float32)
    n, k = w.shape
    wg = _groups(w, GROUP_INT4).astype(np.float64)
    amax = np.abs(wg).max(axis=2)
    s32 = (amax / 7.0).astype(np.float32)         # fp32 quotient (exact double rounding)
    sbits = codecs.bf16_rne_bits(s32)
    s = codecs.bf16_value(sbits).astype(np.float64)
    q = np.zeros(wg.shape, dtype=np.int8)
    nz = s > 0
    q[nz] = np.clip(np.rint(wg[nz] / s[nz][:, None]), -8, 7).astype(np.int8)
    return q.reshape(n, k), sbits


# ----------------------------------------------------------------------------- symmetric INT8

def quant_int8_sym(w):
    """Symmetric INT8 (in the pages' INT1..INT8 weight list, cocoloop.cn news
    item, format list), the INT4 rule at 8 bits: per (row, 128-group)
    s = bf16(fp32(amax / 127)), q = clamp(rne(w / s), -128, 127) against the
    stored scale, s = 0 gives q = 0.  Returns (q int8 [N,K], scale bits)."""
    w = np.asarray(w, dtype=np.float32)
    n, k = w.shape
    wg = _groups(w, GROUP_INT4).astype(np.float64)
    amax = np.abs(wg).max(axis=2)
    sbits = codecs.bf16_rne_bits((amax / 127.0).astype(np.float32))
    s = codecs.bf16_value(sbits).astype(np.float64)
    q = np.zeros(wg.shape, dtype=np.int8)
    nz = s > 0
    q[nz] = np.clip(np.rint(wg[nz] / s[nz][:, None]), -128, 127).astype(np.int8)
    return q.reshape(n, k), sbits


# ----------------------------------------------------------------------------- asymmetric uint4 + zero point

def quant_uint4_zp(w):
    """Asymmetric uint4 with an integer zero point, group 128, bf16 scales.

    Per (row n, group g):  s = bf16(fp32((max - min) / 15));
    z = clamp(rne(-min / s), 0, 15);  u = clamp(rne(w / s) + z, 0, 15);
    s = 0 gives u = z = 0.  Divisions in fp64 against the stored scale.
    Returns (u uint8 [N,K], scale bits uint16 [N,K/128], z uint8 [N,K/128])."""
    w = np.asarray(w, dtype=np.float32)
    n, k = w.shape
    wg = _groups(w, GROUP_INT4).astype(np.float64)
    mx = wg.max(axis=2)
    mn = wg.min(axis=2)
    s32 = ((mx - mn) / 15.0).astype(np.float32)
    sbits = codecs.bf16_rne_bits(s32)
    s = codecs.bf16_value(sbits).astype(np.float64)
    u = np.zeros(wg.shape, dtype=np.uint8)
    z = np.zeros(s.shape, dtype=np.uint8)
    nz = s > 0
    z[nz] = np.clip(np.rint(-mn[nz] / s[nz]), 0, 15).astype(np.uint8)
    u[nz] = np.clip(np.rint(wg[nz] / s[nz][:, None]) + z[nz][:, None].astype(np.float64),
                    0, 15).astype(np.uint8)
    return u.reshape(n, k), sbits, z


def quant_uint_zp(w, bits):
    """The zero-point rule of quant_uint4_zp for b-bit codes (b = 2, 3, 4):
    per 128-group s = bf16(fp32((max - min) / (2^b - 1)));
    z = clamp(rne(-min / s), 0, 2^b - 1);  u = clamp(rne(w / s) + z, 0, 2^b - 1);
    s = 0 gives u = z = 0.  Returns (u uint8 [N,K], scale bits, z uint8)."""
    top = (1 << bits) - 1
    w = np.asarray(w, dtype=np.float32)
    n, k = w.shape
    wg = _groups(w, GROUP_INT4).astype(np.float64)
    mx = wg.max(axis=2)
    mn = wg.min(axis=2)
    s32 = ((mx - mn) / float(top)).astype(np.float32)
    sbits = codecs.bf16_rne_bits(s32)
    s = codecs.bf16_value(sbits).astype(np.float64)
    u = np.zeros(wg.shape, dtype=np.uint8)
    z = np.zeros(s.shape, dtype=np.uint8)
    nz = s > 0
    z[nz] = np.clip(np.rint(-mn[nz] / s[nz]), 0, top).astype(np.uint8)
    u[nz] = np.clip(np.rint(wg[nz] / s[nz][:, None]) + z[nz][:, None].astype(np.float64),
                    0, top).astype(np.uint8)
    return u.reshape(n, k), sbits, z


def pack_bits(codes, bits):
    """[N,K] b-bit codes -> the standard packing: b = 2: four per byte, value
    4j + i at bits 2i..2i+1 of byte j; b = 3: eight per three bytes, value
    8j + i at bits 3i..3i+2 of the little-endian 24-bit word of bytes 3j..3j+2."""
    c = np.asarray(codes).astype(np.int64) & ((1 << bits) - 1)
    n, k = c.shape
    per = 4 if bits == 2 else 8
    assert k % per == 0
    g = c.reshape(n, k // per, per)
    word = np.zeros((n, k // per), dtype=np.int64)
    for i in range(per):
        word |= g[:, :, i] << (bits * i)
    nbytes = bits * per // 8
    out = np.zeros((n, k // per, nbytes), dtype=np.uint8)
    for b in range(nbytes):
        out[:, :, b] = (word >> (8 * b)) & 0xFF
    return out.reshape(n, k * bits // 8)


def unpack_bits(packed, bits):
    """Inverse of pack_bits: [N, K*b/8] bytes -> [N, K] codes (uint8)."""
    p = np.asarray(packed, dtype=np.uint8)
    n, kb = p.shape
    per = 4 if bits == 2 else 8
    nbytes = bits * per // 8
    g = p.reshape(n, kb // nbytes, nbytes).astype(np.int64)
    word = np.zeros(g.shape[:2], dtype=np.int64)
    for b in range(nbytes):
        word |= g[:, :, b] << (8 * b)
    out = np.zeros((n, kb // nbytes, per), dtype=np.uint8)
    for i in range(per):
        out[:, :, i] = (word >> (bits * i)) & ((1 << bits) - 1)
    return out.reshape(n, kb // nbytes * per)


# ----------------------------------------------------------------------------- MXFP4

def mx_shared_exponent(amax):
    """X = floor(log2(amax)) - 2, clamped to [-127, 127]; amax = 0 -> -127.
    floor(log2) is taken exactly from the binary exponent (frexp)."""
    amax = np.asarray(amax, dtype=np.float64)
    _, e = np.frexp(amax)                 # amax = m * 2^e, m in [0.5, 1)
    x = (e - 1) - 2
    x = np.where(amax > 0, x, -127)
    return np.clip(x, -127, 127).astype(np.int64)


def quant_mxfp4(w):
    """MXFP4: E2M1 codes with one E8M0 scale per 32 values along K.
    Returns (codes uint8 [N,K] in 0..15, e8m0 bytes uint8 [N,K/32])."""
    w = np.asarray(w, dtype=np.float32)
    n, k = w.shape
    wg = _groups(w, GROUP_MX).astype(np.float64)
    amax = np.abs(wg).max(axis=2)
    x = mx_shared_exponent(amax)
    scaled = wg / np.ldexp(1.0, x)[:, :, None]          # exact: power-of-two
    codes = codecs.e2m1_rne_sat(scaled)
    codes = np.where((amax > 0)[:, :, None], codes, 0).astype(np.uint8)
    return codes.reshape(n, k), (x + 127).astype(np.uint8)


# ----------------------------------------------------------------------------- MXINT4

def quant_mxint4(w):
    """MXINT4 (named in the pages' format lists, cocoloop.cn item and aihaber.org
    article, hardware and format support, without a definition).  Reading
    taken: the MX scheme with 4-bit two's complement elements read as 1.2
    fixed point, value q/4 with q in -8..7 (range [-2, 1.75], the INT4
    analogue of the MX INT8 element), one E8M0 scale per 32 values along K.
    The shared exponent is X = floor(log2 amax) (the largest element
    magnitude is below 2, so its power-of-two exponent is 0), and
    q = clamp(round-half-even(4 w / 2^X), -8, 7), so w_hat = 2^X q / 4.
    An all-zero block takes X = -127 and zero codes.
    Returns (codes uint8 [N,K] in 0..15 = q & 0xF, e8m0 bytes uint8 [N,K/32])."""
    w = np.asarray(w, dtype=np.float32)
    n, k = w.shape
    wg = _groups(w, GROUP_MX).astype(np.float64)
    amax = np.abs(wg).max(axis=2)
    _, e = np.frexp(amax)                       # amax = m * 2^e, m in [0.5, 1)
    x = np.clip(np.where(amax > 0, e - 1, -127), -127, 127).astype(np.int64)
    scaled = wg / np.ldexp(1.0, x - 2)[:, :, None]      # exact: power of two
    q = np.clip(np.rint(scaled), -8, 7)
    q = np.where((amax > 0)[:, :, None], q, 0).astype(np.int64)
    return (q & 0xF).reshape(n, k).astype(np.uint8), (x + 127).astype(np.uint8)


# ----------------------------------------------------------------------------- packing

def pack_nibbles(codes):
    """[N,K] 4-bit codes (any int dtype; only the low 4 bits are kept) ->
    [N,K/2] bytes, even k in the low nibble."""
    c = np.asarray(codes).astype(np.int64) & 0xF
    n, k = c.shape
    assert k % 2 == 0
    return (c[:, 0::2] | (c[:, 1::2] << 4)).astype(np.uint8)


def unpack_nibbles(packed):
    """[N,K/2] bytes -> [N,K] unsigned 4-bit codes (uint8)."""
    p = np.asarray(packed, dtype=np.uint8)
    n, kb = p.shape
    out = np.empty((n, 2 * kb), dtype=np.uint8)
    out[:, 0::2] = p & 0xF
    out[:, 1::2] = p >> 4
    return out


def nibble_to_int4(u):
    """Unsigned 4-bit pattern -> two's complement value in -8..7."""
    u = np.asarray(u, dtype=np.int64) & 0xF
    return np.where(u >= 8, u - 16, u).astype(np.int8)


# ----------------------------------------------------------------------------- dequantization

def dequant(fmt, packed, scales, zeros=None):
    """Exact restore of the standard format into float32 [N,K].

    int4_sym:  s * q           (q two's complement nibble, s bf16)
    uint4_zp:  s * (u - z)     (z one byte per group, low nibble used)
    mxfp4:     E2M1(code) * 2^(b-127)
    mxint4:    (q / 4) * 2^(b-127)   (q two's complement nibble)
    uint3_zp, uint2_zp: s * (u - z) with u, z 3- or 2-bit (packed as in pack_bits)
    int8_sym:  s * q           (q a two's complement byte, one per value)
    Every product is exact in fp32 (at most 12 significant bits, and the MX
    products stay at or above 2^-129) while it stays below 2^128."""
    if fmt == FMT_INT8_SYM:
        q = np.asarray(packed, dtype=np.uint8).view(np.int8).astype(np.float64)
        n, k = q.shape
        s = codecs.bf16_value(scales).astype(np.float64)
        return (q.reshape(n, k // GROUP_INT4, GROUP_INT4) * s[:, :, None]).reshape(n, k).astype(np.float32)
    if fmt in NARROW_ZP:
        u = unpack_bits(packed, NARROW_ZP[fmt])
        n, k = u.shape
        s = codecs.bf16_value(scales).astype(np.float64)
        z = (np.asarray(zeros, dtype=np.int64) & ((1 << NARROW_ZP[fmt]) - 1)).astype(np.float64)
        d = u.astype(np.float64).reshape(n, k // GROUP_INT4, GROUP_INT4) - z[:, :, None]
        return (d * s[:, :, None]).reshape(n, k).astype(np.float32)
    u = unpack_nibbles(packed)
    n, k = u.shape
    if fmt == FMT_INT4_SYM:
        s = codecs.bf16_value(scales).astype(np.float64)
        q = nibble_to_int4(u).astype(np.float64)
        out = q.reshape(n, k // GROUP_INT4, GROUP_INT4) * s[:, :, None]
    elif fmt == FMT_UINT4_ZP:
        s = codecs.bf16_value(scales).astype(np.float64)
        z = (np.asarray(zeros, dtype=np.int64) & 0xF).astype(np.float64)
        d = u.astype(np.float64).reshape(n, k // GROUP_INT4, GROUP_INT4) - z[:, :, None]
        out = d * s[:, :, None]
    elif fmt == FMT_MXFP4:
        v = codecs.e2m1_value(u).reshape(n, k // GROUP_MX, GROUP_MX)
        out = v * codecs.e8m0_value(scales)[:, :, None]
    elif fmt == FMT_MXINT4:
        v = nibble_to_int4(u).astype(np.float64).reshape(n, k // GROUP_MX, GROUP_MX) / 4.0
        out = v * codecs.e8m0_value(scales)[:, :, None]
    else:
        raise ValueError(fmt)
    return out.reshape(n, k).astype(np.float32)


def quantize(fmt, w):
    """Quantize fp32 W [N,K] into the packed standard format.
    Returns dict(codes=[N,K/2] u8, scales=..., zeros=... or None)."""
    if fmt == FMT_INT4_SYM:
        q, s = quant_int4_sym(w)
        return dict(codes=pack_nibbles(q), scales=s, zeros=None)
    if fmt == FMT_UINT4_ZP:
        u, s, z = quant_uint4_zp(w)
        return dict(codes=pack_nibbles(u), scales=s, zeros=z)
    if fmt == FMT_MXFP4:
        c, e = quant_mxfp4(w)
        return dict(codes=pack_nibbles(c), scales=e, zeros=None)
    if fmt == FMT_MXINT4:
        c, e = quant_mxint4(w)
        return dict(codes=pack_nibbles(c), scales=e, zeros=None)
    if fmt in NARROW_ZP:
        u, s, z = quant_uint_zp(w, NARROW_ZP[fmt])
        return dict(codes=pack_bits(u, NARROW_ZP[fmt]), scales=s, zeros=z)
    if fmt == FMT_INT8_SYM:
        q, s = quant_int8_sym(w)
        return dict(codes=q.view(np.uint8), scales=s, zeros=None)
    raise ValueError(fmt)


# ----------------------------------------------------------------------------- FP8 activation rows

def quant_fp8_rows(x_bf16_bits):
    """Per-token FP8: for each row, amax over the bf16 values;
    s = fp32(amax) / fp32(448) (IEEE fp32 division); x8 = E4M3(fp32(x / s))
    with the division in fp32, round-to-nearest-even, saturating.
    amax = 0 -> s = 0 and every code 0.
    Returns (codes uint8 [M,K], scales float32 [M])."""
    x = codecs.bf16_value(x_bf16_bits)                    # float32, exact
    m, k = x.shape
    amax = np.abs(x).max(axis=1).astype(np.float32) if k else np.zeros(m, np.float32)
    s = (amax / np.float32(448.0)).astype(np.float32)     # fp32 division
    codes = np.zeros((m, k), dtype=np.uint8)
    nz = s > 0
    if nz.any():
        with np.errstate(under="ignore"):
            q = (x[nz] / s[nz][:, None]).astype(np.float32)   # fp32 division
        codes[nz] = codecs.e4m3_rne_sat(q.astype(np.float64))
    return codes, s


def quant_mxfp4_rows(x_bf16_bits):
    """MXFP4 activation rows (the W4A4 pair, cocoloop.cn news item, format
    list): each row's bf16 values are quantized with the same OCP MX rule as
    MXFP4 weights, one E8M0 scale per 32 values along K, E2M1 elements by
    round-to-nearest-even with saturation.  The bf16 values are exact in
    fp32, and the scaling by 2^-X is exact.
    Returns (packed codes uint8 [M, K/2], e8m0 bytes uint8 [M, K/32])."""
    x = codecs.bf16_value(np.asarray(x_bf16_bits, dtype=np.uint16)).astype(np.float32)
    codes, e = quant_mxfp4(x)
    return pack_nibbles(codes), e


def mxfp4_rows_dequant(packed, scales):
    """x_hat = E2M1(code) * 2^(b-127), float64 [M, K]."""
    return dequant(FMT_MXFP4, packed, scales).astype(np.float64)


def fp8_rows_dequant(codes, scales):
    """x_hat = E4M3(code) * s, float64 [M,K]."""
    return codecs.e4m3_value(codes) * np.asarray(scales, dtype=np.float64)[:, None]


# ----------------------------------------------------------------------------- storage accounting

def storage_bytes(n, k, fmt, group=None, scale_bits=16, zero_bits=4):
    """Bytes of the standard format excluding padding and alignment:
    n*k 4-bit codes + one scale per group (+ one zero point per group)."""
    code_bits = NARROW_ZP.get(fmt, 8 if fmt == FMT_INT8_SYM else 4)
    if fmt in NARROW_ZP:
        zero_bits = code_bits
    if fmt in MX_FORMATS:
        group = group or GROUP_MX
        scale_bits = 8
        zero_bits = 0
    else:
        group = group or GROUP_INT4
        if fmt in (FMT_INT4_SYM, FMT_INT8_SYM):
            zero_bits = 0
    groups = n * (k // group)
    bits = n * k * code_bits + groups * (scale_bits + zero_bits)
    return bits / 8.0


def bits_per_value(fmt, group=None, **kw):
    g = group or (GROUP_MX if fmt in MX_FORMATS else GROUP_INT4)
    return storage_bytes(1, g, fmt, group=g, **kw) * 8.0 / g
