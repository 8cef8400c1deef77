// Shared device helpers and the device weight-layout geometry.
//
// Device layout ("layout 1") for E experts, N columns, K (multiple of 128):
//   NB = ceil(N/16) column blocks, KG = K/128 steps along K.
//   Region A (codes): tile (e, nb, g) of 1024 bytes at ((e*NB + nb)*KG + g)*1024;
//     64 slots of 16 bytes, slot L = column 16*nb + L%16, quarter h = L/16.
//     int4:  u32 j of slot L holds k = 128g + 32j + 8h + i (i = 0..7), value i in
//            nibble i/2 (even i) or 4 + i/2 (odd i), so that the pair (2p, 2p+1)
//            sits in nibbles p and p+4, one per 16-bit half; the u32 j of a slot
//            is the 8 K-values one lane feeds to the j-th 16x16x32 bf16 MFMA of
//            the step.  INT4_SYM is stored offset-binary (q+8).
//     mxfp4, mxint4: byte b of slot L holds k = 128g + 32h + 2b (low), k+1
//            (high); the 16 bytes are the 32 E2M1 (or two's complement)
//            values one lane feeds to a 16x16x128 scaled MFMA (MXFP4).
//     Columns >= N hold the value-zero code.
//   Region B (scales, 256-aligned): int4: bf16 [E][NB][KG][16];
//     mxfp4, mxint4: bytes [E][NB][ceil(KG/4)][64 lanes][4], byte g%4 of lane L's u32
//     = E8M0 of (column 16nb + L%16, 32-block 4g + L/16).
//   Region C (zero points, UINT4_ZP only, 256-aligned): [E][NB][KG] u64,
//     nibble c = zero point of column 16nb + c.
//   Total = end of the last region rounded up to 256 bytes; gap bytes are zero.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

namespace hm {

enum WFmt : int { W_INT4_SYM = 0, W_UINT4_ZP = 1, W_MXFP4 = 2, W_MXINT4 = 3, W_UINT3_ZP = 4, W_UINT2_ZP = 5,
                  W_INT8_SYM = 6 };

// 3- and 2-bit zero-point formats share the 4-bit zero-point device layout
__host__ __device__ inline int device_fmt(int wfmt) {
  return (wfmt == W_UINT3_ZP || wfmt == W_UINT2_ZP) ? W_UINT4_ZP : wfmt;
}

// formats with E8M0 scales per 32 values and the MX slot layout
__host__ __device__ inline bool is_mx(int wfmt) { return wfmt == W_MXFP4 || wfmt == W_MXINT4; }

struct Geom {
  int64_t E, N, K, NB, KG, KG4;
  size_t off_scales, off_zeros, total;
};

__host__ __device__ inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

__host__ __device__ inline Geom make_geom(int wfmt, int64_t E, int64_t N, int64_t K) {
  Geom g;
  g.E = E; g.N = N; g.K = K;
  g.NB = (N + 15) / 16;
  g.KG = K / 128;
  g.KG4 = (g.KG + 3) / 4;
  // INT8: 2048-byte tiles (two 1 KiB halves, MFMA operands 0-1 and 2-3)
  size_t a = (size_t)E * g.NB * g.KG * (wfmt == W_INT8_SYM ? 2048 : 1024);
  size_t b = is_mx(wfmt) ? (size_t)E * g.NB * g.KG4 * 256 : (size_t)E * g.NB * g.KG * 32;
  size_t c = (wfmt == W_UINT4_ZP) ? (size_t)E * g.NB * g.KG * 8 : 0;
  g.off_scales = align256(a);
  g.off_zeros = align256(g.off_scales + b);
  g.total = align256(g.off_zeros + c);
  return g;
}

// ------------------------------------------------------------------ vector types
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ u32x4_t ld16(const void* p) { return *reinterpret_cast<const u32x4_t*>(p); }

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __amdgpu_buffer_rsrc_t rsrc_t;

// Raw buffer over `bytes` bytes from `base` (reads at or past the end return
// zero; larger extents are capped at the 32-bit maximum).
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0,
                                           (int)(uint32_t)(bytes < 0xFFFFFFFFull ? bytes : 0xFFFFFFFFull), 0x00020000);
}

// Direct buffer-to-LDS copies: lane L's `n` bytes at base + voff + soff land at
// lds_base + n L (lds_base wave-uniform).  The buffer form (unlike the global
// one) leaves the compiler's wait counts exact for the loads and LDS reads
// that follow.
__device__ __forceinline__ void b2lds16(rsrc_t r, uint32_t voff, uint32_t soff, uint8_t* lds_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)lds_base, 16, voff, soff, 0, 0);
}
__device__ __forceinline__ void b2lds4(rsrc_t r, uint32_t voff, uint32_t soff, uint8_t* lds_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)lds_base, 4, voff, soff, 0, 0);
}
__device__ __forceinline__ void st16(void* p, u32x4_t v) { *reinterpret_cast<u32x4_t*>(p) = v; }

// Two fp32 -> packed bf16 pair (round to nearest even), low half = a.
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  f32x2_t v = {a, b};
  bf16x2_t h = __builtin_convertvector(v, bf16x2_t);
  return __builtin_bit_cast(uint32_t, h);
}

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// Eight 4-bit unsigned codes in device order (value 2j in nibble j, value
// 2j+1 in nibble j+4) -> eight bf16 of s*u + zs, in value order, as four packed
// pairs.  The fp32 value s*u + zs = s*(u-z) is exact (at most 12 significant
// bits), then rounded once to bf16.
__device__ __forceinline__ u32x4_t dq8_u4(uint32_t w, float s, float zs) {
  u32x4_t r;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t t = (w >> (4 * j)) & 0x000F000Fu;   // values 2j (bits 0-3) and 2j+1 (bits 16-19)
    r[j] = pack_bf16(__builtin_fmaf((float)(t & 0xFFu), s, zs), __builtin_fmaf((float)(t >> 16), s, zs));
  }
  return r;
}

// Eight two's complement bytes (value i in byte i of the two words) -> eight
// bf16 of q, exact, in value order: one sign-extending conversion per value.
__device__ __forceinline__ u32x4_t i8x8_bf16(uint32_t lo, uint32_t hi) {
  auto sb = [](uint32_t x, int b) { return (float)(int8_t)(x >> (8 * b)); };
  return (u32x4_t){pack_bf16(sb(lo, 0), sb(lo, 1)), pack_bf16(sb(lo, 2), sb(lo, 3)),
                   pack_bf16(sb(hi, 0), sb(hi, 1)), pack_bf16(sb(hi, 2), sb(hi, 3))};
}
// Bytes 2 sel and 2 sel + 1 of x (two's complement) times s -> one bf16 pair
// (sel = 0, 1 known at compile time after unrolling).
__device__ __forceinline__ uint32_t i8x2_bf16_scaled(uint32_t x, int sel, float s) {
  return pack_bf16((float)(int8_t)(x >> (16 * sel)) * s, (float)(int8_t)(x >> (16 * sel + 8)) * s);
}
// The same times s, each product rounded once to bf16.
__device__ __forceinline__ u32x4_t i8x8_bf16_scaled(uint32_t lo, uint32_t hi, float s) {
  auto sb = [s](uint32_t x, int b) { return (float)(int8_t)(x >> (8 * b)) * s; };
  return (u32x4_t){pack_bf16(sb(lo, 0), sb(lo, 1)), pack_bf16(sb(lo, 2), sb(lo, 3)),
                   pack_bf16(sb(hi, 0), sb(hi, 1)), pack_bf16(sb(hi, 2), sb(hi, 3))};
}

// Eight unsigned codes of one device-layout word (value 2p in nibble p, 2p+1
// in nibble p+4) minus their zero point z -> eight bf16 of u - z, exact (the
// integers -15..15), in value order.  zc = 0x80808080 - z * 0x01010101: a
// byte u + 128 - z lies in 113..143, so the 32-bit add carries across no byte,
// and the xor with 0x80 leaves the two's complement byte u - z, which a
// sign-extending byte conversion turns into fp32 (one instruction per value).
__device__ __forceinline__ u32x4_t dz8_u4(uint32_t w, uint32_t zc) {
  const uint32_t lo = ((w & 0x0F0F0F0Fu) + zc) ^ 0x80808080u;          // bytes: v0 v4 v1 v5
  const uint32_t hi = (((w >> 4) & 0x0F0F0F0Fu) + zc) ^ 0x80808080u;   // bytes: v2 v6 v3 v7
  auto sb = [](uint32_t x, int b) { return (float)(int8_t)(x >> (8 * b)); };
  return (u32x4_t){pack_bf16(sb(lo, 0), sb(lo, 2)), pack_bf16(sb(hi, 0), sb(hi, 2)),
                   pack_bf16(sb(lo, 1), sb(lo, 3)), pack_bf16(sb(hi, 1), sb(hi, 3))};
}

// Low nibble of byte B of x read as a two's complement 4-bit q -> q / 16 in
// fp32, exactly (gfx9 v_cvt_off_f32_i4 with a byte select).
template <int B>
__device__ __forceinline__ float off_i4(uint32_t x) {
  float r;
  if (B == 0) __asm__("v_cvt_off_f32_i4_sdwa %0, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_0" : "=v"(r) : "v"(x));
  if (B == 1) __asm__("v_cvt_off_f32_i4_sdwa %0, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_1" : "=v"(r) : "v"(x));
  if (B == 2) __asm__("v_cvt_off_f32_i4_sdwa %0, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_2" : "=v"(r) : "v"(x));
  if (B == 3) __asm__("v_cvt_off_f32_i4_sdwa %0, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_3" : "=v"(r) : "v"(x));
  return r;
}

// Eight offset-binary codes q + 8 of one device-layout word (symmetric INT4)
// -> eight bf16 of q / 16, exact, in value order: the xor with 0x8 per nibble
// gives the two's complement q, converted nibble by nibble.
__device__ __forceinline__ u32x4_t dq8_sym16(uint32_t w) {
  const uint32_t lo = w ^ 0x88888888u;     // nibble p of byte b: value 2p of byte b's low nibble
  const uint32_t hi = lo >> 4;             // low nibbles: nibbles 1, 3, 5, 7
  return (u32x4_t){pack_bf16(off_i4<0>(lo), off_i4<2>(lo)), pack_bf16(off_i4<0>(hi), off_i4<2>(hi)),
                   pack_bf16(off_i4<1>(lo), off_i4<3>(lo)), pack_bf16(off_i4<1>(hi), off_i4<3>(hi))};
}

// Opaque copies of constants, so the compiler keeps them in registers.
__device__ __forceinline__ uint32_t in_vgpr(uint32_t v) {
  __asm__ volatile("" : "+v"(v));
  return v;
}
__device__ __forceinline__ uint32_t in_sgpr(uint32_t v) {
  __asm__ volatile("" : "+s"(v));
  return v;
}

// Eight consecutive outputs y[n..n+7] of one row (one 16-byte store when aligned).
__device__ __forceinline__ void store_bf16x8(uint16_t* yrow, int64_t N, int64_t n, u32x4_t v) {
  if ((N & 7) == 0 && n + 7 < N) {
    *reinterpret_cast<u32x4_t*>(yrow + n) = v;
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if (n + e < N) yrow[n + e] = (uint16_t)(v[e >> 1] >> (16 * (e & 1)));
  }
}

__device__ __forceinline__ float ubyte_f(uint32_t x, int b) { return (float)((x >> (8 * b)) & 0xFFu); }

// Eight codes of one device-layout word (value 2p in nibble p, 2p+1 in nibble
// p+4) -> eight bf16 of s*u + zs (= s*(u - z), exact before the bf16 rounding)
// in value order.
// Word r of the result below from the masked bytes lo = w & 0x0F0F0F0F and
// hi = (w >> 4) & 0x0F0F0F0F.
__device__ __forceinline__ uint32_t dq8_word(uint32_t lo, uint32_t hi, int r, float s, float zs) {
  const uint32_t x = (r & 1) ? hi : lo;
  const int b0 = r >> 1;                         // bytes b0 and b0 + 2 of x
  return pack_bf16(fmaf(ubyte_f(x, b0), s, zs), fmaf(ubyte_f(x, b0 + 2), s, zs));
}

__device__ __forceinline__ u32x4_t dq8_bytes(uint32_t w, float s, float zs) {
  // opaque masks: otherwise the compiler folds mask and byte select into one
  // bit-field extract per value instead of converting the masked bytes
  const uint32_t lo = in_vgpr(w & 0x0F0F0F0Fu);          // bytes: v0 v4 v1 v5
  const uint32_t hi = in_vgpr((w >> 4) & 0x0F0F0F0Fu);   // bytes: v2 v6 v3 v7
  u32x4_t r;
  r[0] = pack_bf16(fmaf(ubyte_f(lo, 0), s, zs), fmaf(ubyte_f(lo, 2), s, zs));
  r[1] = pack_bf16(fmaf(ubyte_f(hi, 0), s, zs), fmaf(ubyte_f(hi, 2), s, zs));
  r[2] = pack_bf16(fmaf(ubyte_f(lo, 1), s, zs), fmaf(ubyte_f(lo, 3), s, zs));
  r[3] = pack_bf16(fmaf(ubyte_f(hi, 1), s, zs), fmaf(ubyte_f(hi, 3), s, zs));
  return r;
}

// E8M0 scale byte -> 2^(e - 127) as fp32 (e = 0 is the subnormal 2^-127,
// e = 255 the format's NaN).
__device__ __forceinline__ float e8m0_f32(uint32_t e) {
  return __uint_as_float(e == 0u ? 0x00400000u : (e == 255u ? 0x7FC00000u : e << 23));
}

// Eight E2M1 codes of one mxfp4 layout word (value 2b in the low nibble of
// byte b, 2b + 1 in its high nibble) times the power of two s -> eight bf16
// in value order, by gfx950's scaled fp4 -> bf16 conversion (two values per
// instruction).  Every product is a bf16 number while |code * s| < 2^128.
__device__ __forceinline__ u32x4_t fp4x8_bf16(uint32_t w, float s) {
  u32x4_t r;
  r[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 0));
  r[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 1));
  r[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 2));
  r[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 3));
  return r;
}

// Codes 2 sel, 2 sel + 1 of one word (byte sel, sel = 0..3 known at compile
// time after unrolling) times s -> one bf16 pair.
__device__ __forceinline__ uint32_t fp4x2_bf16(uint32_t w, float s, int sel) {
  switch (sel & 3) {
    case 0: return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 0));
    case 1: return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 1));
    case 2: return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 2));
    default: return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 3));
  }
}

// MXINT4: eight two's complement codes of one word (value 2b in the low
// nibble of byte b, 2b + 1 in its high nibble) times s -> eight bf16 in value
// order; s carries the element's fixed-point factor 1/4.  Exact: q * s has at
// most 4 significant bits.
__device__ __forceinline__ uint32_t i4x2_bf16(uint32_t w, float s, int sel) {
  const int lo = (int)(w << (28 - 8 * sel)) >> 28;       // sign-extended nibble 2 sel
  const int hi = (int)(w << (24 - 8 * sel)) >> 28;       // and 2 sel + 1
  return pack_bf16((float)lo * s, (float)hi * s);
}
__device__ __forceinline__ u32x4_t i4x8_bf16(uint32_t w, float s) {
  return (u32x4_t){i4x2_bf16(w, s, 0), i4x2_bf16(w, s, 1), i4x2_bf16(w, s, 2), i4x2_bf16(w, s, 3)};
}

// 32x32x16 bf16 MFMA: lane L supplies A row L%32 and B column L%32 for K
// = 8*(L/32) + 0..7; C: lane L holds column L%32, rows 8*j + 4*(L/32) + r in
// register 4*j + r (j, r = 0..3).
__device__ __forceinline__ f32x16_t mfma32_bf16(u32x4_t a, u32x4_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// 16x16x32 bf16 MFMA: C[i][j] += sum_k A[i][k] B[k][j]; lane L supplies A row
// L%16 and B column L%16 for K-quarter L/16 (8 values each); C: lane L holds
// column L%16, rows 4*(L/16) + 0..3.
__device__ __forceinline__ f32x4_t mfma_bf16(u32x4_t a, u32x4_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// 16x16x128 scaled MFMA, A = E2M1, B = E4M3 (measured operand layout on gfx950):
//   A: lane L supplies row L%16, K = 32*(L/16) + 0..31 (16 bytes, even K in the
//      low nibble);
//   B: lane L supplies column L%16 with two 16-byte halves: b0 = K 16*(L/16) +
//      0..15 and b1 = K 64 + 16*(L/16) + 0..15;
//   scales: lane r + 16*b supplies the E8M0 byte of row/column r, K-block
//      32b..32b+31, for each operand (sa for A, sb for B).
//   C: same layout as the bf16 MFMA above.
__device__ __forceinline__ f32x4_t mfma_fp4_fp8(u32x4_t a, u32x4_t b0, u32x4_t b1, f32x4_t c,
                                                int sa, int sb) {
  i32x8_t av = {(int)a[0], (int)a[1], (int)a[2], (int)a[3], 0, 0, 0, 0};
  i32x8_t bv = {(int)b0[0], (int)b0[1], (int)b0[2], (int)b0[3],
                (int)b1[0], (int)b1[1], (int)b1[2], (int)b1[3]};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, c, 4, 0, 0, sa, 0, sb);
}

// 16x16x128 scaled MFMA with both operands E2M1 (W4A4): A as above; B lane L
// supplies column L%16, K = 32*(L/16) + 0..31 (16 bytes, even K in the low
// nibble), the same arrangement as A; the E8M0 scales as above.
__device__ __forceinline__ f32x4_t mfma_fp4_fp4(u32x4_t a, u32x4_t b, f32x4_t c, int sa, int sb) {
  i32x8_t av = {(int)a[0], (int)a[1], (int)a[2], (int)a[3], 0, 0, 0, 0};
  i32x8_t bv = {(int)b[0], (int)b[1], (int)b[2], (int)b[3], 0, 0, 0, 0};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, c, 4, 4, 0, sa, 0, sb);
}

// x / s correctly rounded, from r = RN(1 / s), for s in [2^-90, 2^100] and
// bf16 x with |x| <= 2^10 s: q0 = x r is within an ulp of the quotient, the
// FMA residual x - q0 s is then exact (no underflow in this range) and one
// correction step q0 + (x - q0 s) r rounds to the quotient (Markstein's
// correction; checked on gfx950 against the IEEE division for every fp32
// divisor mantissa and every bf16 dividend over 22 binades, 2.4e10 pairs, no
// difference).  Quotients under 2^-12 s may miss by an ulp, which no E4M3
// code can show; the sign comes from x so that -0 stays -0.
__device__ __forceinline__ bool recip_div_ok(float s) { return s >= 0x1p-90f && s <= 0x1p100f; }
__device__ __forceinline__ float div_by_recip(float x, float s, float r) {
  const float q0 = x * r;
  return __builtin_copysignf(__builtin_fmaf(__builtin_fmaf(-q0, s, x), r, q0), x);
}

// Four fp32 -> four E4M3 codes (byte i from value i) by gfx950's packed
// conversion on the values clamped to +-448 (round to nearest even).  It
// equals f32_to_e4m3 below on every non-NaN fp32 input (checked
// exhaustively on the GPU: all 2^32 patterns but NaNs); the kernels use it,
// the software rule documents it.
__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d) {
  auto cl = [](float v) { return __builtin_fminf(__builtin_fmaxf(v, -448.0f), 448.0f); };
  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(cl(a), cl(b), 0, false);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(cl(c), cl(d), lo, true);
}

// fp32 -> E4M3 bits, round to nearest even, saturating; sign kept on zero.
__device__ __forceinline__ uint32_t f32_to_e4m3(float x) {
  const uint32_t b = __float_as_uint(x);
  const uint32_t sign = (b >> 24) & 0x80u;
  const uint32_t a = b & 0x7FFFFFFFu;
  if (a >= 0x43E00000u) return sign | 0x7Eu;           // |x| >= 448: saturate
  if (a < 0x3C800000u) {                                // |x| < 2^-6: subnormal range
    const float m = __builtin_rintf(__uint_as_float(a) * 512.0f);  // units of 2^-9, 0..8
    return sign | (uint32_t)m;                          // 8 -> 0x08 = 2^-6 (exact carry)
  }
  // normal: keep 3 mantissa bits with round-to-nearest-even, then rebias 127 -> 7
  const uint32_t r = a + 0x7FFFFu + ((a >> 20) & 1u);
  return sign | ((r >> 20) - (120u << 3));
}

// silu(g) = g / (1 + e^-g) = g s with s = 1 / (1 + e), e = e^-|g|, for
// g >= 0, and g e s for g < 0.  One exponential, taken as ee = e 2^64 =
// e^(64 ln 2 - |g|), which stays normal for |g| up to about 131 (where e
// alone would leave the normal range below |g| = 87); e = ee 2^-64 and the
// negative branch's g ee s 2^-64 are exact rescalings (the latter rounds once
// if it is subnormal).  The fast exponential (relative error about 3e-6 for
// arguments near 44) and the hardware reciprocal (1 ulp) stay far below the
// final bf16 rounding (2^-9).
__device__ __forceinline__ float silu_f(float g) {
  const float ee = __expf(44.3614195558365f - fabsf(g));
  const float s = __builtin_amdgcn_rcpf(1.0f + ee * 5.421010862427522e-20f);
  return g >= 0.0f ? g * s : ((g * ee) * s) * 5.421010862427522e-20f;
}

__device__ __forceinline__ float lo_bf16(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float hi_bf16(uint32_t v) { return __uint_as_float(v & 0xFFFF0000u); }


// The gated activation of two bf16 pairs: bf16(silu(g) * u) for the low and
// high halves (g, u already rounded to bf16, as a bf16 gate_up output is).
__device__ __forceinline__ uint32_t silu_mul_pair(uint32_t g2, uint32_t u2) {
  return pack_bf16(silu_f(lo_bf16(g2)) * lo_bf16(u2), silu_f(hi_bf16(g2)) * hi_bf16(u2));
}

// Gated (gate / up interleaved) weight layout: device 16-column block 2 i
// holds gate columns 16 i .. 16 i + 15, block 2 i + 1 the matching up
// columns (N a multiple of 32).  Source row of device row n:
__host__ __device__ inline int64_t gated_src_row(int64_t n, int64_t N) {
  const int64_t i = n >> 5, c = n & 15;
  return ((n >> 4) & 1) ? N / 2 + 16 * i + c : 16 * i + c;
}
// Staged bf16 rows of a tile that starts on an even block: output chunk oc
// (8 columns of the tile's output row, which starts at column 8 nb0 of the
// [rows][N/2] output) is the gated product of staged chunk gated_gate_chunk(oc)
// (gate) and that chunk + 2 (up).
__device__ __forceinline__ int gated_gate_chunk(int oc) { return ((oc >> 1) << 2) | (oc & 1); }

}  // namespace hm
