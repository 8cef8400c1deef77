// Weight preparation kernels: repack of the standard format into the device
// layout (padding and re-ordering done once before inference, as the pages
// describe the transform step: ywsung.com note "How vLLM Humming computes 4
// bits", section on layout; aihaber.org article, Architecture), and exact
// dequantization of a prepared buffer back to fp32.
#include "common.h"
#include "launch.h"

namespace hm {

// Four nibbles held in the low nibbles of the four bytes of x -> 16 bits.
__device__ __forceinline__ uint32_t compact_nibbles(uint32_t x) {
  x = (x | (x >> 4)) & 0x00FF00FFu;
  return (x | (x >> 8)) & 0x0000FFFFu;
}

// One thread per 16-byte code slot (e, nb, g, L).
__global__ void __launch_bounds__(256)
k_transform_codes(int wfmt, Geom G, const uint8_t* __restrict__ codes, uint8_t* __restrict__ out, int gated) {
  const int64_t slots = G.E * G.NB * G.KG * 64;
  const int64_t row_bytes = G.K / 2;
  for (int64_t s = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; s < slots;
       s += (int64_t)gridDim.x * blockDim.x) {
    const int L = (int)(s & 63);
    int64_t t = s >> 6;
    const int64_t g = t % G.KG; t /= G.KG;
    const int64_t nb = t % G.NB;
    const int64_t e = t / G.NB;
    const int64_t n = nb * 16 + (L & 15);
    const int h = L >> 4;
    u32x4_t v;
    if (n < G.N && (wfmt == W_UINT3_ZP || wfmt == W_UINT2_ZP)) {
      // narrow codes widened to nibbles: word j of the slot holds values
      // k = 128 g + 32 j + 8 h + i, i = 0..7, value 2p in nibble p, 2p+1 in p+4
      const int bits = wfmt == W_UINT3_ZP ? 3 : 2;
      const uint8_t* row = codes + (e * G.N + (gated ? gated_src_row(n, G.N) : n)) * (G.K * bits / 8);
      for (int j = 0; j < 4; ++j) {
        const int64_t k0 = 128 * g + 32 * j + 8 * h;       // multiple of 8
        const uint8_t* p = row + k0 * bits / 8;
        const uint32_t word = bits == 3 ? (uint32_t)p[0] | ((uint32_t)p[1] << 8) | ((uint32_t)p[2] << 16)
                                        : (uint32_t)p[0] | ((uint32_t)p[1] << 8);
        uint32_t o = 0;
        for (int i = 0; i < 8; ++i) {
          const uint32_t val = (word >> (bits * i)) & ((1u << bits) - 1u);
          const int pos = (i & 1) ? 4 + (i >> 1) : (i >> 1);
          o |= val << (4 * pos);
        }
        v[j] = o;
      }
    } else if (n < G.N) {
      const uint8_t* row = codes + (e * G.N + (gated ? gated_src_row(n, G.N) : n)) * row_bytes;
      if (is_mx(wfmt)) {
        v = ld16(row + 64 * g + 16 * h);
      } else {
        const uint8_t* p = row + 64 * g + 4 * h;
        for (int j = 0; j < 4; ++j) {
          // standard order (value i in nibble i) -> device order (value 2p in nibble p,
          // value 2p+1 in nibble p+4): even values to the low half-word, odd to the high
          const uint32_t w = *reinterpret_cast<const uint32_t*>(p + 16 * j);
          v[j] = compact_nibbles(w & 0x0F0F0F0Fu) | (compact_nibbles((w >> 4) & 0x0F0F0F0Fu) << 16);
        }
        if (wfmt == W_INT4_SYM) v ^= 0x88888888u;  // two's complement -> offset binary
      }
    } else {
      const uint32_t z = (wfmt == W_INT4_SYM) ? 0x88888888u : 0u;
      v = (u32x4_t){z, z, z, z};
    }
    st16(out + s * 16, v);
  }
}

// INT8 codes: one thread per 16-byte output chunk (e, nb, g, half p, slot L):
// bytes 8 jj + i = value k = 128 g + 32 (2 p + jj) + 8 h + i of column
// 16 nb + L % 16, h = L / 16; columns past N hold 0.
__global__ void __launch_bounds__(256)
k_transform_codes_i8(Geom G, const uint8_t* __restrict__ codes, uint8_t* __restrict__ out, int gated) {
  const int64_t chunks = G.E * G.NB * G.KG * 128;
  for (int64_t s = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; s < chunks;
       s += (int64_t)gridDim.x * blockDim.x) {
    const int L = (int)(s & 63);
    const int p = (int)((s >> 6) & 1);
    int64_t t = s >> 7;
    const int64_t g = t % G.KG; t /= G.KG;
    const int64_t nb = t % G.NB;
    const int64_t e = t / G.NB;
    const int64_t n = nb * 16 + (L & 15);
    const int h = L >> 4;
    u32x4_t v = {0u, 0u, 0u, 0u};
    if (n < G.N) {
      const uint8_t* row = codes + (e * G.N + (gated ? gated_src_row(n, G.N) : n)) * G.K;
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        const uint8_t* q = row + 128 * g + 32 * (2 * p + jj) + 8 * h;   // 8-byte aligned
        const u32x2_t w = *reinterpret_cast<const u32x2_t*>(q);
        v[2 * jj] = w[0];
        v[2 * jj + 1] = w[1];
      }
    }
    st16(out + s * 16, v);
  }
}

// INT4 scales: one thread per (e, nb, g, c) bf16 entry.
__global__ void __launch_bounds__(256)
k_transform_scales_int4(Geom G, const uint16_t* __restrict__ scales, uint16_t* __restrict__ out, int gated) {
  const int64_t cnt = G.E * G.NB * G.KG * 16;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < cnt;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int c = (int)(i & 15);
    int64_t t = i >> 4;
    const int64_t g = t % G.KG; t /= G.KG;
    const int64_t nb = t % G.NB;
    const int64_t e = t / G.NB;
    const int64_t n = nb * 16 + c;
    out[i] = (n < G.N) ? scales[(e * G.N + (gated ? gated_src_row(n, G.N) : n)) * G.KG + g] : (uint16_t)0;
  }
}

// MX scales: one thread per (e, nb, g4, L) u32 holding the E8M0 bytes of steps 4*g4 + 0..3.
__global__ void __launch_bounds__(256)
k_transform_scales_mx(Geom G, const uint8_t* __restrict__ scales, uint32_t* __restrict__ out, int gated) {
  const int64_t cnt = G.E * G.NB * G.KG4 * 64;
  const int64_t blocks = G.K / 32;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < cnt;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int L = (int)(i & 63);
    int64_t t = i >> 6;
    const int64_t g4 = t % G.KG4; t /= G.KG4;
    const int64_t nb = t % G.NB;
    const int64_t e = t / G.NB;
    const int64_t n = nb * 16 + (L & 15);
    uint32_t v = 0;
    if (n < G.N) {
      for (int gi = 0; gi < 4; ++gi) {
        const int64_t g = 4 * g4 + gi;
        if (g < G.KG)
          v |= (uint32_t)scales[(e * G.N + (gated ? gated_src_row(n, G.N) : n)) * blocks + 4 * g + (L >> 4)]
               << (8 * gi);
      }
    }
    out[i] = v;
  }
}

// Zero points (zero-point formats): one thread per (e, nb, g) u64 of 16
// nibbles; `mask` keeps the code width's bits of each zero-point byte.
__global__ void __launch_bounds__(256)
k_transform_zeros(Geom G, const uint8_t* __restrict__ zeros, uint64_t* __restrict__ out, uint32_t mask, int gated) {
  const int64_t cnt = G.E * G.NB * G.KG;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < cnt;
       i += (int64_t)gridDim.x * blockDim.x) {
    int64_t t = i;
    const int64_t g = t % G.KG; t /= G.KG;
    const int64_t nb = t % G.NB;
    const int64_t e = t / G.NB;
    uint64_t v = 0;
    for (int c = 0; c < 16; ++c) {
      const int64_t n = nb * 16 + c;
      if (n < G.N) v |= (uint64_t)(zeros[(e * G.N + (gated ? gated_src_row(n, G.N) : n)) * G.KG + g] & mask) << (4 * c);
    }
    out[i] = v;
  }
}

// Zero the alignment gaps between the regions (each shorter than 256 bytes),
// so that the whole buffer is a deterministic function of the input.
__global__ void __launch_bounds__(256)
k_zero_gaps(uint8_t* __restrict__ out, size_t a0, size_t a1, size_t b0, size_t b1, size_t c0, size_t c1) {
  const size_t i = threadIdx.x;
  if (a0 + i < a1) out[a0 + i] = 0;
  if (b0 + i < b1) out[b0 + i] = 0;
  if (c0 + i < c1) out[c0 + i] = 0;
}

__device__ __forceinline__ float e2m1_value(uint32_t c) {
  const float mag[8] = {0.0f, 0.5f, 1.0f, 1.5f, 2.0f, 3.0f, 4.0f, 6.0f};
  const float m = mag[c & 7];
  return (c & 8) ? -m : m;
}

__device__ __forceinline__ float e8m0_value(uint32_t b) {
  // 2^(b-127); b = 0 is the fp32 subnormal 2^-127; b = 255 is the format's NaN.
  return (b == 0) ? __uint_as_float(0x00400000u) : (b == 255u ? __uint_as_float(0x7FC00000u) : __uint_as_float(b << 23));
}

// Exact dequantization of expert `e`: one thread per 8 consecutive K-values.
__global__ void __launch_bounds__(256)
k_dequant(int wfmt, Geom G, const uint8_t* __restrict__ w, int64_t e, float* __restrict__ out) {
  const int64_t cnt = G.N * (G.K / 8);
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < cnt;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t n = i / (G.K / 8);
    const int64_t k = (i % (G.K / 8)) * 8;
    const int64_t nb = n / 16, c = n % 16, g = k / 128, kk = k % 128;
    const int64_t tile = (e * G.NB + nb) * G.KG + g;
    float r[8];
    if (wfmt == W_INT8_SYM) {
      const int j = (int)(kk / 32), h = (int)((kk % 32) / 8);
      const int L = (int)c + 16 * h;
      const u32x2_t wv = *reinterpret_cast<const u32x2_t*>(w + tile * 2048 + (j >> 1) * 1024 + L * 16 + 8 * (j & 1));
      const uint16_t* sc = reinterpret_cast<const uint16_t*>(w + G.off_scales);
      const float s = bf16_to_f32(sc[tile * 16 + c]);
      for (int q = 0; q < 8; ++q) r[q] = (float)(int8_t)(wv[q >> 2] >> (8 * (q & 3))) * s;
    } else if (is_mx(wfmt)) {
      const int h = (int)(kk / 32);
      const int L = (int)c + 16 * h;
      const uint32_t word = *reinterpret_cast<const uint32_t*>(w + tile * 1024 + L * 16 + (kk % 32) / 2);
      const uint32_t* sc = reinterpret_cast<const uint32_t*>(w + G.off_scales);
      const uint32_t sb = (sc[((e * G.NB + nb) * G.KG4 + g / 4) * 64 + L] >> (8 * (g % 4))) & 0xFF;
      const float s = e8m0_value(sb);
      if (wfmt == W_MXINT4) {
        // two's complement q, value q / 4 (exact)
        for (int q = 0; q < 8; ++q) r[q] = (float)((int)(word << (28 - 4 * q)) >> 28) * 0.25f * s;
      } else {
        for (int q = 0; q < 8; ++q) r[q] = e2m1_value((word >> (4 * q)) & 0xF) * s;
      }
    } else {
      const int j = (int)(kk / 32), h = (int)((kk % 32) / 8);
      const int L = (int)c + 16 * h;
      const uint32_t word = *reinterpret_cast<const uint32_t*>(w + tile * 1024 + L * 16 + 4 * j);
      const uint16_t* sc = reinterpret_cast<const uint16_t*>(w + G.off_scales);
      const float s = bf16_to_f32(sc[tile * 16 + c]);
      uint32_t z = 8;
      if (wfmt == W_UINT4_ZP) {
        const uint64_t* zz = reinterpret_cast<const uint64_t*>(w + G.off_zeros);
        z = (uint32_t)((zz[tile] >> (4 * c)) & 0xF);
      }
      // (u - z) * s: exact, and the sign of a zero result follows the IEEE product rule
      for (int q = 0; q < 8; ++q) {
        const int pos = (q & 1) ? 4 + (q >> 1) : (q >> 1);   // device nibble order
        r[q] = (float)((int)((word >> (4 * pos)) & 0xF) - (int)z) * s;
      }
    }
    float* o = out + n * G.K + k;
    st16(o, __builtin_bit_cast(u32x4_t, (f32x4_t){r[0], r[1], r[2], r[3]}));
    st16(o + 4, __builtin_bit_cast(u32x4_t, (f32x4_t){r[4], r[5], r[6], r[7]}));
  }
}

static inline unsigned grid_for(int64_t items) {
  int64_t b = (items + 255) / 256;
  if (b > 65536) b = 65536;
  if (b < 1) b = 1;
  return (unsigned)b;
}

hipError_t launch_transform(int wfmt, const Geom& G, const uint8_t* codes, const void* scales,
                            const uint8_t* zeros, uint8_t* out, int gated, hipStream_t st) {
  if (wfmt == W_INT8_SYM)
    hipLaunchKernelGGL(k_transform_codes_i8, dim3(grid_for(G.E * G.NB * G.KG * 128)), dim3(256), 0, st, G, codes,
                       out, gated);
  else
    hipLaunchKernelGGL(k_transform_codes, dim3(grid_for(G.E * G.NB * G.KG * 64)), dim3(256), 0, st,
                       wfmt, G, codes, out, gated);
  if (is_mx(wfmt)) {
    hipLaunchKernelGGL(k_transform_scales_mx, dim3(grid_for(G.E * G.NB * G.KG4 * 64)), dim3(256), 0,
                       st, G, (const uint8_t*)scales, (uint32_t*)(out + G.off_scales), gated);
  } else {
    hipLaunchKernelGGL(k_transform_scales_int4, dim3(grid_for(G.E * G.NB * G.KG * 16)), dim3(256),
                       0, st, G, (const uint16_t*)scales, (uint16_t*)(out + G.off_scales), gated);
  }
  if (device_fmt(wfmt) == W_UINT4_ZP) {
    const uint32_t mask = wfmt == W_UINT3_ZP ? 0x7u : (wfmt == W_UINT2_ZP ? 0x3u : 0xFu);
    hipLaunchKernelGGL(k_transform_zeros, dim3(grid_for(G.E * G.NB * G.KG)), dim3(256), 0, st, G,
                       zeros, (uint64_t*)(out + G.off_zeros), mask, gated);
  }
  // gap ends: codes end .. scales start, scales end .. zeros start, zeros end .. total
  const size_t codes_end = (size_t)G.E * G.NB * G.KG * (wfmt == W_INT8_SYM ? 2048 : 1024);
  const size_t scales_end = G.off_scales + (is_mx(wfmt) ? (size_t)G.E * G.NB * G.KG4 * 256
                                                              : (size_t)G.E * G.NB * G.KG * 32);
  const size_t zeros_end = (device_fmt(wfmt) == W_UINT4_ZP) ? G.off_zeros + (size_t)G.E * G.NB * G.KG * 8 : G.off_zeros;
  hipLaunchKernelGGL(k_zero_gaps, dim3(1), dim3(256), 0, st, out, codes_end, G.off_scales, scales_end,
                     G.off_zeros, zeros_end, G.total);
  return hipGetLastError();
}

hipError_t launch_dequant(int wfmt, const Geom& G, const uint8_t* w, int64_t e, float* out,
                          hipStream_t st) {
  hipLaunchKernelGGL(k_dequant, dim3(grid_for(G.N * (G.K / 8))), dim3(256), 0, st, wfmt, G, w, e,
                     out);
  return hipGetLastError();
}

}  // namespace hm
