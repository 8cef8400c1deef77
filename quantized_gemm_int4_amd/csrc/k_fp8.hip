// Per-token FP8 activation quantization (the BF16 -> per-token FP8 switch the
// ywsung.com note "How vLLM Humming computes 4 bits" describes in its section
// on weight format / activation / backend):
//   s[m] = amax_k |x[m,k]| / 448  (fp32 division),
//   x8[m,k] = E4M3(x[m,k] / s[m]) (fp32 division, round to nearest even,
//   saturating at 448);  a zero row gives s = 0 and zero codes.
// E4M3 is the OCP "FN" layout: bias 7, no infinities, largest finite 448,
// subnormal step 2^-9.
#include "common.h"
#include "launch.h"

namespace hm {

// One 256-thread block per row; rows of any length k (two passes over the row).
__global__ void __launch_bounds__(256)
k_quant_fp8_rows(const uint16_t* __restrict__ x, int64_t m, int64_t k, uint8_t* __restrict__ x8,
                 float* __restrict__ row_scale) {
  __shared__ float red[4];
  for (int64_t row = blockIdx.x; row < m; row += gridDim.x) {
    const uint16_t* xr = x + row * k;
    uint8_t* qr = x8 + row * k;
    const bool vec = ((k & 7) == 0);
    float amax = 0.0f;
    if (vec) {
      for (int64_t i = threadIdx.x * 8; i < k; i += 256 * 8) {
        const u32x4_t v = ld16(xr + i);
        for (int j = 0; j < 4; ++j) {
          amax = fmaxf(amax, fabsf(bf16_to_f32(v[j] & 0xFFFF)));
          amax = fmaxf(amax, fabsf(bf16_to_f32(v[j] >> 16)));
        }
      }
    } else {
      for (int64_t i = threadIdx.x; i < k; i += 256) amax = fmaxf(amax, fabsf(bf16_to_f32(xr[i])));
    }
    for (int off = 32; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 64));
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = amax;
    __syncthreads();
    amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    __syncthreads();
    const float s = __fdiv_rn(amax, 448.0f);
    if (threadIdx.x == 0) row_scale[row] = s;
    if (vec) {
      for (int64_t i = threadIdx.x * 8; i < k; i += 256 * 8) {
        const u32x4_t v = ld16(xr + i);
        float q[8];
        for (int j = 0; j < 4; ++j) {
          q[2 * j] = s != 0.0f ? __fdiv_rn(bf16_to_f32(v[j] & 0xFFFF), s) : 0.0f;
          q[2 * j + 1] = s != 0.0f ? __fdiv_rn(bf16_to_f32(v[j] >> 16), s) : 0.0f;
        }
        *reinterpret_cast<u32x2_t*>(qr + i) = (u32x2_t){e4m3x4(q[0], q[1], q[2], q[3]), e4m3x4(q[4], q[5], q[6], q[7])};
      }
    } else {
      for (int64_t i = threadIdx.x; i < k; i += 256)
        qr[i] = (s != 0.0f) ? (uint8_t)(e4m3x4(__fdiv_rn(bf16_to_f32(xr[i]), s), 0.0f, 0.0f, 0.0f) & 0xFFu) : (uint8_t)0;
    }
  }
}

// Rows with k % 8 == 0 and k <= 512 CH: one wave per row (four rows per
// block), lane L keeping 16-byte chunks c * 64 + L of the row in registers, so
// the row is read once, the amax is a wave reduction (no block barrier) and
// all of a wave's loads are in flight together.
template <int CH>
__global__ void __launch_bounds__(256)
k_quant_fp8_rows_wave(const uint16_t* __restrict__ x, int64_t m, int64_t k, uint8_t* __restrict__ x8,
                      float* __restrict__ row_scale) {
  const int lane = threadIdx.x & 63;
  const int64_t kc = k / 8;
  for (int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); row < m; row += (int64_t)gridDim.x * 4) {
    const uint16_t* xr = x + row * k;
    u32x4_t v[CH];
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int64_t q = (int64_t)c * 64 + lane;
      v[c] = q < kc ? ld16(xr + 8 * q) : (u32x4_t){0u, 0u, 0u, 0u};
    }
    float amax = 0.0f;
#pragma unroll
    for (int c = 0; c < CH; ++c)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        amax = fmaxf(amax, fabsf(lo_bf16(v[c][j])));
        amax = fmaxf(amax, fabsf(hi_bf16(v[c][j])));
      }
    for (int off = 32; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 64));
    const float s = __fdiv_rn(amax, 448.0f);
    if (lane == 0) row_scale[row] = s;
    // codes of the rounded quotients x / s: by the reciprocal and one
    // correction step when s allows it (the row's s is the same on every
    // lane, so the branch is uniform), else by the IEEE division
    auto put = [&](auto div) __attribute__((always_inline)) {
#pragma unroll
      for (int c = 0; c < CH; ++c) {
        const int64_t q = (int64_t)c * 64 + lane;
        float f[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) f[j] = div((j & 1) ? hi_bf16(v[c][j >> 1]) : lo_bf16(v[c][j >> 1]));
        if (q < kc)
          *reinterpret_cast<u32x2_t*>(x8 + row * k + 8 * q) =
              (u32x2_t){e4m3x4(f[0], f[1], f[2], f[3]), e4m3x4(f[4], f[5], f[6], f[7])};
      }
    };
    if (__builtin_amdgcn_readfirstlane(recip_div_ok(s) ? 1 : 0)) {
      const float r = __fdiv_rn(1.0f, s);
      put([&](float h) { return div_by_recip(h, s, r); });
    } else {
      put([&](float h) { return s != 0.0f ? __fdiv_rn(h, s) : 0.0f; });
    }
  }
}

hipError_t launch_quant_fp8_rows(const uint16_t* x, int64_t m, int64_t k, uint8_t* x8, float* s,
                                 hipStream_t st) {
  if ((k & 7) == 0 && k <= 512 * 16) {
    // one row per wave, held in registers
    const int64_t want = (m + 3) / 4;
    const dim3 g((unsigned)(want < 65536 ? want : 65536));
    if (k <= 512) hipLaunchKernelGGL(k_quant_fp8_rows_wave<1>, g, dim3(256), 0, st, x, m, k, x8, s);
    else if (k <= 1024) hipLaunchKernelGGL(k_quant_fp8_rows_wave<2>, g, dim3(256), 0, st, x, m, k, x8, s);
    else if (k <= 2048) hipLaunchKernelGGL(k_quant_fp8_rows_wave<4>, g, dim3(256), 0, st, x, m, k, x8, s);
    else if (k <= 4096) hipLaunchKernelGGL(k_quant_fp8_rows_wave<8>, g, dim3(256), 0, st, x, m, k, x8, s);
    else hipLaunchKernelGGL(k_quant_fp8_rows_wave<16>, g, dim3(256), 0, st, x, m, k, x8, s);
  } else {
    // one row per block, two passes over the row
    const int64_t blocks = m < 65536 ? m : 65536;
    hipLaunchKernelGGL(k_quant_fp8_rows, dim3((unsigned)blocks), dim3(256), 0, st, x, m, k, x8, s);
  }
  return hipGetLastError();
}

}  // namespace hm

namespace hm {

// MXFP4 activation rows (the W4A4 pair): per 32 consecutive values of a row,
// the OCP MX rule -- shared exponent X = floor(log2 amax) - 2 clamped to
// [-127, 127] (E8M0 byte X + 127; a zero block takes byte 0), elements
// E2M1(x / 2^X) rounded to nearest even and saturated at 6.  The bf16 values
// are exact in fp32 and the scaling by 2^-X is exact, so the codes are those
// of the exact quotient.

// |v| -> E2M1 magnitude code 0..7 (0, 0.5, 1, 1.5, 2, 3, 4, 6): count the
// rounding boundaries below |v|; ties (0.25, 0.75, ..., 5) go to the even code
__device__ __forceinline__ uint32_t e2m1_code(float v) {
  const float a = fabsf(v);
  const uint32_t c = (a > 0.25f) + (a >= 0.75f) + (a > 1.25f) + (a >= 1.75f) + (a > 2.5f) + (a >= 3.5f) +
                     (a > 5.0f);
  return c | ((__float_as_uint(v) >> 28) & 8u);          // sign bit 3 (negative zero keeps it)
}

// One thread per 32-value block: four 16-byte loads, one 16-byte code store
// (value 2i in the low nibble of byte i) and one scale byte.
__global__ void __launch_bounds__(256)
k_quant_mxfp4_rows(const uint16_t* __restrict__ x, int64_t m, int64_t k, uint8_t* __restrict__ codes,
                   uint8_t* __restrict__ scales) {
  const int64_t per_row = k / 32;
  const int64_t n = m * per_row;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t row = i / per_row, b = i - row * per_row;
    const uint16_t* xp = x + row * k + b * 32;
    u32x4_t v[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) v[c] = ld16(xp + 8 * c);
    uint32_t amax_bits = 0;
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        amax_bits = max(amax_bits, (v[c][j] << 16) & 0x7FFFFFFFu);
        amax_bits = max(amax_bits, v[c][j] & 0x7FFF0000u);
      }
    // biased fp32 exponent of amax (0 for zero and subnormal); byte = max(e - 2, 0)
    const int e = (int)(amax_bits >> 23);
    const int byte = e > 2 ? e - 2 : 0;
    const float inv = __uint_as_float((uint32_t)(254 - byte) << 23);   // 2^-(byte - 127)
    uint32_t out[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      uint32_t w = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t lo = e2m1_code(bf16_to_f32(v[c][j] & 0xFFFFu) * inv);
        const uint32_t hi = e2m1_code(bf16_to_f32(v[c][j] >> 16) * inv);
        w |= (lo | (hi << 4)) << (8 * j);
      }
      out[c] = w;
    }
    st16(codes + row * (k / 2) + b * 16, (u32x4_t){out[0], out[1], out[2], out[3]});
    scales[row * per_row + b] = (uint8_t)byte;
  }
}

hipError_t launch_quant_mxfp4_rows(const uint16_t* x, int64_t m, int64_t k, uint8_t* codes, uint8_t* scales,
                                   hipStream_t st) {
  const int64_t n = m * (k / 32);
  int64_t blocks = (n + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(k_quant_mxfp4_rows, dim3((unsigned)blocks), dim3(256), 0, st, x, m, k, codes, scales);
  return hipGetLastError();
}

}  // namespace hm
