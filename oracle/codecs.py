"""Bit-level number formats used by the low-bit GEMM path (oracle side).

Every function works on NumPy arrays and is written from the format's
definition, one value at a time where that keeps it plain:

* bf16: IEEE binary32 with the low 16 bits dropped, round-to-nearest-even.
  Scales are stored in bf16 (ywsung.com note "How vLLM Humming computes 4 bits",
  section on scales: one 16-bit scale per 128 weights).
* E4M3 ("fp8", OCP FN variant): 1 sign, 4 exponent (bias 7), 3 mantissa bits,
  no infinities, 0x7F/0xFF are NaN, largest finite 448, subnormal step 2^-9.
  Per-token FP8 activations are named in the same note, section on weight
  format / activation / backend.
* E2M1 ("fp4"): 1 sign, 2 exponent (bias 1), 1 mantissa bit; magnitudes
  {0, .5, 1, 1.5, 2, 3, 4, 6}.  MXFP4 is named in the cocoloop.cn news item
  (format list) and in the aihaber.org article (hardware and format support).
* E8M0: an unsigned biased exponent, value 2^(b-127); 255 is NaN.

The MX formats follow the public OCP Microscaling v1.0 definitions, which is
the plainest reading of the pages' bare format names.
"""
import numpy as np

# ----------------------------------------------------------------------------- bf16

def bf16_rne_bits(x):
    """fp32 values -> bf16 bit patterns (uint16), round to nearest, ties to even.

    Works on the fp32 bit pattern: add 0x7FFF plus the lsb of the kept half,
    then drop the low 16 bits.  NaN stays NaN (quiet bit forced)."""
    x = np.asarray(x, dtype=np.float32)
    b = x.view(np.uint32).astype(np.uint64)
    lsb = (b >> 16) & 1
    r = ((b + 0x7FFF + lsb) >> 16).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        r = np.where(nan, ((b >> 16) | 0x40).astype(np.uint16), r)
    return r


def bf16_value(bits):
    """bf16 bit patterns (uint16) -> exact values as float32 (a widening)."""
    bits = np.asarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32)


def ulp_bf16(y):
    """One bf16 ulp at |y| (float64 array).

    For a normal bf16 magnitude this is 2^(floor(log2|y|) - 7); below the
    smallest normal (2^-126) and at zero it is the subnormal step 2^-133."""
    y = np.abs(np.asarray(y, dtype=np.float64))
    out = np.full(y.shape, 2.0 ** -133)
    nz = y >= 2.0 ** -126
    if nz.any():
        m, e = np.frexp(y[nz])          # y = m * 2^e, m in [0.5, 1)
        out[nz] = np.ldexp(1.0, (e - 1) - 7)
    return out

# ----------------------------------------------------------------------------- E4M3 (fp8)

def _e4m3_decode_one(c):
    c = int(c) & 0xFF
    s = -1.0 if (c >> 7) else 1.0
    e = (c >> 3) & 0xF
    m = c & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return s * m * 2.0 ** -9           # subnormal: m/8 * 2^(1-7)
    return s * (1.0 + m / 8.0) * 2.0 ** (e - 7)


E4M3_TABLE = np.array([_e4m3_decode_one(c) for c in range(256)], dtype=np.float64)
E4M3_MAX = 448.0
# non-negative finite codes in increasing value order: 0x00 .. 0x7E
_E4M3_POS = E4M3_TABLE[:0x7F].copy()


def e4m3_value(codes):
    """E4M3 codes (uint8) -> values (float64)."""
    return E4M3_TABLE[np.asarray(codes, dtype=np.uint8)]


def e4m3_rne_sat(x):
    """Values -> E4M3 codes: round to nearest representable, ties to the even
    code (even mantissa), magnitudes above 448 saturate to 448.  Never emits NaN.
    A negative value that rounds to zero keeps its sign (code 0x80)."""
    x = np.asarray(x, dtype=np.float64)
    a = np.minimum(np.abs(x), E4M3_MAX)
    # index of the largest table value <= a
    lo = np.searchsorted(_E4M3_POS, a, side="right") - 1
    lo = np.clip(lo, 0, 0x7E)
    hi = np.minimum(lo + 1, 0x7E)
    dlo = a - _E4M3_POS[lo]
    dhi = _E4M3_POS[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi != lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    neg = np.signbit(x)
    return np.where(neg, code | 0x80, code).astype(np.uint8)

# ----------------------------------------------------------------------------- E2M1 (fp4)

E2M1_MAG = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)
E2M1_TABLE = np.concatenate([E2M1_MAG, -E2M1_MAG])   # codes 0..15, 8 = -0.0


def e2m1_value(codes):
    """4-bit E2M1 codes (0..15) -> values (float64); code 8 decodes to -0.0."""
    return E2M1_TABLE[np.asarray(codes, dtype=np.uint8) & 0xF]


def e2m1_rne_sat(x):
    """Values -> 4-bit E2M1 codes: nearest magnitude, ties to the even code,
    saturating at 6; bit 3 carries the sign (negative zero is code 8)."""
    x = np.asarray(x, dtype=np.float64)
    a = np.minimum(np.abs(x), 6.0)
    lo = np.clip(np.searchsorted(E2M1_MAG, a, side="right") - 1, 0, 7)
    hi = np.minimum(lo + 1, 7)
    dlo = a - E2M1_MAG[lo]
    dhi = E2M1_MAG[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi != lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    return np.where(np.signbit(x), code | 0x8, code).astype(np.uint8)

# ----------------------------------------------------------------------------- E8M0

def e8m0_value(b):
    """E8M0 bytes -> 2^(b-127) as float64 (byte 255 -> NaN)."""
    b = np.asarray(b, dtype=np.int64)
    v = np.ldexp(1.0, b - 127)
    return np.where(b == 255, np.nan, v)
