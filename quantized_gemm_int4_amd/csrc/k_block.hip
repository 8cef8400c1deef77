// The two elementwise steps of an MoE feed-forward block around its grouped
// GEMMs (tokens split per expert, each token activating only some experts:
// aihaber.org article on Humming, "what problem does it solve"; ywsung.com
// note "How vLLM Humming computes 4 bits", section on one token vs many
// tokens):
//   gated activation  h[r][i]   = silu(gu[r][i]) * gu[r][d + i]
//   weighted combine  out[t][c] = sum_j w[t][j] * y[t*topk + j][c]
// Both only stream bf16 rows through HBM (6 bytes per output of the gated
// activation; 2 * topk + 2 bytes per output of the combine), so each thread
// moves whole 16-byte chunks (eight bf16) and the grid holds one thread per
// chunk: enough waves in flight to cover the memory latency without a loop.
#include "common.h"
#include "launch.h"

namespace hm {


// d % 8 == 0: thread q handles outputs 8 (q % (d/8)) .. + 7 of row q / (d/8)
__global__ void __launch_bounds__(256)
k_silu_mul_v8(const uint16_t* __restrict__ gu, int64_t chunks, int64_t dc, uint16_t* __restrict__ h) {
  const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (q >= chunks) return;
  const int64_t r = q / dc, c = q - r * dc;
  const uint16_t* g = gu + r * (16 * dc) + 8 * c;      // row stride 2d = 16 dc
  const u32x4_t gv = ld16(g), uv = ld16(g + 8 * dc);
  u32x4_t o;
#pragma unroll
  for (int j = 0; j < 4; ++j)
    o[j] = pack_bf16(silu_f(lo_bf16(gv[j])) * lo_bf16(uv[j]), silu_f(hi_bf16(gv[j])) * hi_bf16(uv[j]));
  st16(h + r * (8 * dc) + 8 * c, o);
}

// Gated activation and per-token FP8 quantization of its rows in one pass
// (the input of an MoE block's down projection with FP8 rows): one wave per
// row; lane l holds outputs 8 (64 c + l) .. + 7 (c < CH) of h rounded to bf16
// exactly as k_silu_mul_v8 writes them, the row's amax is a wave reduction,
// and the codes are those k_quant_fp8_rows_wave gives for the bf16 row:
// s = amax / 448, E4M3 of the correctly rounded fp32 quotient h / s.  The
// bf16 h never reaches memory.  d % 8 == 0, d <= 512 CH.
template <int CH>
__global__ void __launch_bounds__(256)
k_silu_mul_fp8(const uint16_t* __restrict__ gu, int64_t rows, int64_t d, uint8_t* __restrict__ h8,
               float* __restrict__ hs) {
  const int lane = threadIdx.x & 63;
  const int64_t dc = d / 8;
  for (int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); r < rows; r += (int64_t)gridDim.x * 4) {
    const uint16_t* g = gu + r * 2 * d;
    u32x4_t gv[CH], uv[CH];
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int64_t q = (int64_t)c * 64 + lane;
      gv[c] = (u32x4_t){0u, 0u, 0u, 0u};
      uv[c] = (u32x4_t){0u, 0u, 0u, 0u};
      if (q < dc) {
        gv[c] = ld16(g + 8 * q);
        uv[c] = ld16(g + d + 8 * q);
      }
    }
    float amax = 0.0f;
#pragma unroll
    for (int c = 0; c < CH; ++c) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        gv[c][j] = pack_bf16(silu_f(lo_bf16(gv[c][j])) * lo_bf16(uv[c][j]),
                             silu_f(hi_bf16(gv[c][j])) * hi_bf16(uv[c][j]));
        amax = fmaxf(amax, fabsf(lo_bf16(gv[c][j])));
        amax = fmaxf(amax, fabsf(hi_bf16(gv[c][j])));
      }
    }
    for (int off = 32; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 64));
    const float s = __fdiv_rn(amax, 448.0f);
    if (lane == 0) hs[r] = s;
    // quotients h / s by the reciprocal and one correction step when s
    // allows it (uniform over the wave's row), else by the IEEE division
    auto put = [&](auto div) __attribute__((always_inline)) {
#pragma unroll
      for (int c = 0; c < CH; ++c) {
        float q[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) q[j] = div((j & 1) ? hi_bf16(gv[c][j >> 1]) : lo_bf16(gv[c][j >> 1]));
        const int64_t qc = (int64_t)c * 64 + lane;
        if (qc < dc)
          *reinterpret_cast<u32x2_t*>(h8 + r * d + 8 * qc) =
              (u32x2_t){e4m3x4(q[0], q[1], q[2], q[3]), e4m3x4(q[4], q[5], q[6], q[7])};
      }
    };
    if (__builtin_amdgcn_readfirstlane(recip_div_ok(s) ? 1 : 0)) {
      const float rs = __fdiv_rn(1.0f, s);
      put([&](float h) { return div_by_recip(h, s, rs); });
    } else {
      put([&](float h) { return s != 0.0f ? __fdiv_rn(h, s) : 0.0f; });
    }
  }
}

// any d: one output per thread
__global__ void __launch_bounds__(256)
k_silu_mul_s(const uint16_t* __restrict__ gu, int64_t total, int64_t d, uint16_t* __restrict__ h) {
  const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (q >= total) return;
  const int64_t r = q / d, i = q - r * d;
  const float g = bf16_to_f32(gu[r * 2 * d + i]), u = bf16_to_f32(gu[r * 2 * d + d + i]);
  h[q] = (uint16_t)(pack_bf16(silu_f(g) * u, 0.0f) & 0xFFFF);
}

// n % 8 == 0: thread q handles columns 8 (q % (n/8)) .. + 7 of token q / (n/8)
__global__ void __launch_bounds__(256)
k_combine_v8(const uint16_t* __restrict__ y, const float* __restrict__ w, int64_t chunks, int64_t nc,
             int topk, uint16_t* __restrict__ out) {
  const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (q >= chunks) return;
  const int64_t t = q / nc, c = q - t * nc;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  const uint16_t* yr = y + t * topk * (8 * nc) + 8 * c;
  for (int j = 0; j < topk; ++j) {
    const float wj = w[t * topk + j];
    const u32x4_t v = ld16(yr + (int64_t)j * (8 * nc));
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc[2 * e] = fmaf(wj, lo_bf16(v[e]), acc[2 * e]);
      acc[2 * e + 1] = fmaf(wj, hi_bf16(v[e]), acc[2 * e + 1]);
    }
  }
  st16(out + t * (8 * nc) + 8 * c, (u32x4_t){pack_bf16(acc[0], acc[1]), pack_bf16(acc[2], acc[3]),
                                             pack_bf16(acc[4], acc[5]), pack_bf16(acc[6], acc[7])});
}

// any n: one output per thread
__global__ void __launch_bounds__(256)
k_combine_s(const uint16_t* __restrict__ y, const float* __restrict__ w, int64_t total, int64_t n, int topk,
            uint16_t* __restrict__ out) {
  const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (q >= total) return;
  const int64_t t = q / n, c = q - t * n;
  float acc = 0.f;
  for (int j = 0; j < topk; ++j) acc = fmaf(w[t * topk + j], bf16_to_f32(y[(t * topk + j) * n + c]), acc);
  out[q] = (uint16_t)(pack_bf16(acc, 0.0f) & 0xFFFF);
}

hipError_t launch_silu_mul_fp8(const uint16_t* gu, int64_t rows, int64_t d, uint8_t* h8, float* hs,
                               hipStream_t st) {
  const int64_t want = (rows + 3) / 4;
  const unsigned blocks = (unsigned)(want < 65536 ? want : 65536);
  if (d <= 512) hipLaunchKernelGGL(k_silu_mul_fp8<1>, dim3(blocks), dim3(256), 0, st, gu, rows, d, h8, hs);
  else if (d <= 2048) hipLaunchKernelGGL(k_silu_mul_fp8<4>, dim3(blocks), dim3(256), 0, st, gu, rows, d, h8, hs);
  else if (d <= 4096) hipLaunchKernelGGL(k_silu_mul_fp8<8>, dim3(blocks), dim3(256), 0, st, gu, rows, d, h8, hs);
  else hipLaunchKernelGGL(k_silu_mul_fp8<16>, dim3(blocks), dim3(256), 0, st, gu, rows, d, h8, hs);
  return hipGetLastError();
}

hipError_t launch_silu_mul(const uint16_t* gu, int64_t rows, int64_t d, uint16_t* h, hipStream_t st) {
  if ((d & 7) == 0) {
    const int64_t chunks = rows * (d / 8);
    hipLaunchKernelGGL(k_silu_mul_v8, dim3((unsigned)((chunks + 255) / 256)), dim3(256), 0, st, gu, chunks,
                       d / 8, h);
  } else {
    const int64_t total = rows * d;
    hipLaunchKernelGGL(k_silu_mul_s, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, st, gu, total, d, h);
  }
  return hipGetLastError();
}

hipError_t launch_combine(const uint16_t* y, const float* w, int64_t t, int topk, int64_t n, uint16_t* out,
                          hipStream_t st) {
  if ((n & 7) == 0) {
    const int64_t chunks = t * (n / 8);
    hipLaunchKernelGGL(k_combine_v8, dim3((unsigned)((chunks + 255) / 256)), dim3(256), 0, st, y, w, chunks,
                       n / 8, topk, out);
  } else {
    const int64_t total = t * n;
    hipLaunchKernelGGL(k_combine_s, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, st, y, w, total, n,
                       topk, out);
  }
  return hipGetLastError();
}

}  // namespace hm

namespace hm {

// Plain streaming read of `bytes` bytes (a multiple of 16): every lane loads
// 16-byte chunks in a grid-stride loop, UNROLL loads in flight, xor-folds
// them and each block writes one word (so no load can be dropped).  The
// decode GEMM reads its weights with the same 16-byte loads; this is the
// floor it is measured against.
template <int UNROLL>
__global__ void __launch_bounds__(256) k_read_probe(const u32x4_t* __restrict__ p, int64_t n16,
                                                    uint32_t* __restrict__ out) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  u32x4_t acc = {0u, 0u, 0u, 0u};
  for (; i + (UNROLL - 1) * stride < n16; i += UNROLL * stride) {
    u32x4_t v[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) v[u] = __builtin_nontemporal_load(p + i + u * stride);
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) acc ^= v[u];
  }
  for (; i < n16; i += stride) acc ^= p[i];
  uint32_t r = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
  for (int off = 32; off >= 1; off >>= 1) r ^= (uint32_t)__shfl_xor((int)r, off, 64);
  __shared__ uint32_t red[4];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = r;
  __syncthreads();
  if (threadIdx.x == 0) out[blockIdx.x] = red[0] ^ red[1] ^ red[2] ^ red[3];
}

hipError_t launch_read_probe(const void* buf, int64_t bytes, int blocks, int unroll, uint32_t* out,
                             hipStream_t st) {
  const int64_t n16 = bytes / 16;
  const u32x4_t* p = reinterpret_cast<const u32x4_t*>(buf);
  if (unroll == 8) hipLaunchKernelGGL(k_read_probe<8>, dim3(blocks), dim3(256), 0, st, p, n16, out);
  else if (unroll == 2) hipLaunchKernelGGL(k_read_probe<2>, dim3(blocks), dim3(256), 0, st, p, n16, out);
  else if (unroll == 1) hipLaunchKernelGGL(k_read_probe<1>, dim3(blocks), dim3(256), 0, st, p, n16, out);
  else hipLaunchKernelGGL(k_read_probe<4>, dim3(blocks), dim3(256), 0, st, p, n16, out);
  return hipGetLastError();
}

}  // namespace hm
