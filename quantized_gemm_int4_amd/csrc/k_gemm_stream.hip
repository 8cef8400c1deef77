// Streaming GEMM for few rows (decode-sized M, and small experts of a grouped
// GEMM).  With few rows, reading and unpacking the weights dominates (ywsung.com
// note "How vLLM Humming computes 4 bits", section on one token vs many
// tokens), so every weight byte is read from HBM exactly once, straight into
// registers: one 16-byte load per lane fetches one 1 KiB tile (16 columns x
// 128 K) of the device layout, which is exactly the operand of four
// 16x16x32 bf16 MFMAs (or of one 16x16x128 scaled fp4 x fp8 MFMA for MXFP4).
// The few activation rows are staged in LDS per chunk of 256 K and shared by
// the block's four waves.  The weights are the MFMA "A" operand (rows = output
// columns n) and the activations the "B" operand, so each lane ends with four
// consecutive n of one row and stores them as one 8-byte write.
// Dense calls split K over blocks and reduce fp32 partials in a second kernel.
#include "common.h"
#include "launch.h"

namespace hm {

constexpr int kChunkG = 2;  // 128-K groups per staged activation chunk

template <bool MX, int MB, int NBW, bool GROUPED>
__global__ void __launch_bounds__(256)
k_gemm_stream(GemmArgs a, int n_tiles) {
  constexpr int ROWS = MB * 16;
  constexpr int XB = MX ? (kChunkG * 128 + 16) : (kChunkG * 256 + 16);  // LDS row stride (bytes)
  constexpr int PIECES_PER_ROW = MX ? kChunkG * 8 : kChunkG * 16;       // 16-byte pieces per row
  constexpr int XLD = (ROWS * PIECES_PER_ROW + 255) / 256;               // pieces per thread
  __shared__ __attribute__((aligned(16))) uint8_t xs_lds[2][ROWS * XB];
  __shared__ int64_t arow_s[ROWS];
  __shared__ int64_t orow_s[ROWS];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const Geom G = a.G;
  const int64_t K = G.K;
  const int n_l = lane & 15, q_l = lane >> 4;
  const uint8_t* xbase = reinterpret_cast<const uint8_t*>(a.x);
  const int64_t xrow_bytes = MX ? K : 2 * K;

  const int64_t n_items = GROUPED ? (int64_t)a.hdr[0] * n_tiles : 1;
  for (int64_t item = GROUPED ? blockIdx.x : 0; item < n_items;
       item += GROUPED ? gridDim.x : 1) {
    int64_t e = 0;
    int nt, rcount, split = 0;
    int64_t g_begin, g_end, m0 = 0;
    if (GROUPED) {
      const int64_t unit = item / n_tiles;
      nt = (int)(item % n_tiles);
      const int32_t* u = a.units + 4 * unit;
      e = u[0];
      rcount = u[2];
      g_begin = 0;
      g_end = G.KG;
      if (tid < ROWS) {
        int64_t ar = -1, orr = -1;
        if (tid < rcount) {
          const int64_t pair = a.sorted_pairs[u[1] + tid];
          if (pair >= 0 && pair < a.P) {
            orr = pair;
            ar = a.rows_are_pairs ? pair : pair / a.topk;
          }
        }
        arow_s[tid] = ar;
        orow_s[tid] = orr;
      }
    } else {
      nt = blockIdx.x;
      split = blockIdx.y;
      m0 = (int64_t)blockIdx.z * ROWS;
      rcount = (int)((a.M - m0) < ROWS ? (a.M - m0) : ROWS);
      g_begin = (int64_t)split * a.ksg;
      g_end = (g_begin + a.ksg < G.KG) ? g_begin + a.ksg : G.KG;
      if (tid < ROWS) {
        arow_s[tid] = (tid < rcount) ? m0 + tid : -1;
        orow_s[tid] = arow_s[tid];
      }
    }
    __syncthreads();

    const int64_t nb0 = ((int64_t)nt * 4 + wave) * NBW;
    const int64_t n_chunks = (g_end - g_begin + kChunkG - 1) / kChunkG;

    // ---- activation chunk: global -> registers -> LDS
    u32x4_t xr[XLD];
    auto load_x = [&](int64_t c) {
      const int64_t gc0 = g_begin + c * kChunkG;
      const int cg = (int)((g_end - gc0) < kChunkG ? (g_end - gc0) : kChunkG);
#pragma unroll
      for (int i = 0; i < XLD; ++i) {
        const int q = tid + 256 * i;
        const int row = q / PIECES_PER_ROW, pc = q % PIECES_PER_ROW;
        u32x4_t v = {0u, 0u, 0u, 0u};
        if (row < ROWS && row < rcount && pc < cg * (PIECES_PER_ROW / kChunkG)) {
          const int64_t ar = arow_s[row];
          if (ar >= 0) v = ld16(xbase + ar * xrow_bytes + gc0 * (MX ? 128 : 256) + pc * 16);
        }
        xr[i] = v;
      }
    };
    auto store_x = [&](int buf) {
#pragma unroll
      for (int i = 0; i < XLD; ++i) {
        const int q = tid + 256 * i;
        const int row = q / PIECES_PER_ROW, pc = q % PIECES_PER_ROW;
        if (row < ROWS) st16(&xs_lds[buf][row * XB + pc * 16], xr[i]);
      }
    };

    // ---- weight registers for one chunk
    u32x4_t bq[NBW][kChunkG];
    float bs[NBW][kChunkG], bz[NBW][kChunkG];
    int bsc[NBW][kChunkG];
    auto load_w = [&](int64_t c, u32x4_t (&q)[NBW][kChunkG], float (&s)[NBW][kChunkG],
                      float (&zs)[NBW][kChunkG], int (&sc)[NBW][kChunkG]) {
      const int64_t gc0 = g_begin + c * kChunkG;
#pragma unroll
      for (int j = 0; j < NBW; ++j) {
        const int64_t nb = nb0 + j;
#pragma unroll
        for (int gl = 0; gl < kChunkG; ++gl) {
          const int64_t g = gc0 + gl;
          q[j][gl] = (u32x4_t){0u, 0u, 0u, 0u};
          s[j][gl] = 0.0f;
          zs[j][gl] = 0.0f;
          sc[j][gl] = 0;
          if (nb < G.NB && g < g_end) {
            const int64_t tile = (e * G.NB + nb) * G.KG + g;
            q[j][gl] = ld16(a.w + tile * 1024 + lane * 16);
            if (MX) {
              const uint32_t* scm = reinterpret_cast<const uint32_t*>(a.w + G.off_scales);
              sc[j][gl] = (int)((scm[((e * G.NB + nb) * G.KG4 + g / 4) * 64 + lane] >> (8 * (g % 4))) & 0xFF);
            } else {
              const uint16_t* s16 = reinterpret_cast<const uint16_t*>(a.w + G.off_scales);
              const float sv = bf16_to_f32(s16[tile * 16 + n_l]);
              float z = 8.0f;
              if (a.wfmt == W_UINT4_ZP) {
                const uint64_t* zz = reinterpret_cast<const uint64_t*>(a.w + G.off_zeros);
                z = (float)((zz[tile] >> (4 * n_l)) & 0xF);
              }
              s[j][gl] = sv;
              zs[j][gl] = -z * sv;
            }
          }
        }
      }
    };

    f32x4_t acc[NBW][MB];
#pragma unroll
    for (int j = 0; j < NBW; ++j)
#pragma unroll
      for (int rb = 0; rb < MB; ++rb) acc[j][rb] = (f32x4_t){0.f, 0.f, 0.f, 0.f};

    u32x4_t nq[NBW][kChunkG];
    float ns[NBW][kChunkG], nz[NBW][kChunkG];
    int nsc[NBW][kChunkG];
    if (n_chunks > 0) {
      load_x(0);
      load_w(0, nq, ns, nz, nsc);
      store_x(0);
    }
    __syncthreads();

    for (int64_t c = 0; c < n_chunks; ++c) {
#pragma unroll
      for (int j = 0; j < NBW; ++j)
#pragma unroll
        for (int gl = 0; gl < kChunkG; ++gl) {
          bq[j][gl] = nq[j][gl]; bs[j][gl] = ns[j][gl]; bz[j][gl] = nz[j][gl]; bsc[j][gl] = nsc[j][gl];
        }
      const bool more = (c + 1 < n_chunks);
      if (more) {
        load_w(c + 1, nq, ns, nz, nsc);
        load_x(c + 1);
      }
      const uint8_t* xl = xs_lds[c & 1];
      const int64_t gc0 = g_begin + c * kChunkG;
#pragma unroll
      for (int gl = 0; gl < kChunkG; ++gl) {
        if (gc0 + gl >= g_end) break;
        if (MX) {
          u32x4_t a0[MB], a1[MB];
#pragma unroll
          for (int rb = 0; rb < MB; ++rb) {
            const uint8_t* p = xl + (rb * 16 + n_l) * XB + gl * 128 + 16 * q_l;
            a0[rb] = ld16(p);
            a1[rb] = ld16(p + 64);
          }
#pragma unroll
          for (int j = 0; j < NBW; ++j) {
            if (nb0 + j >= G.NB) continue;
#pragma unroll
            for (int rb = 0; rb < MB; ++rb)
              acc[j][rb] = mfma_fp4_fp8(bq[j][gl], a0[rb], a1[rb], acc[j][rb], bsc[j][gl], 127);
          }
        } else {
#pragma unroll
          for (int kk = 0; kk < 4; ++kk) {
            u32x4_t af[MB];
#pragma unroll
            for (int rb = 0; rb < MB; ++rb)
              af[rb] = ld16(xl + (rb * 16 + n_l) * XB + (gl * 128 + 32 * kk + 8 * q_l) * 2);
#pragma unroll
            for (int j = 0; j < NBW; ++j) {
              if (nb0 + j >= G.NB) continue;
              const u32x4_t bw = dq8_u4(bq[j][gl][kk], bs[j][gl], bz[j][gl]);
#pragma unroll
              for (int rb = 0; rb < MB; ++rb) acc[j][rb] = mfma_bf16(bw, af[rb], acc[j][rb]);
            }
          }
        }
      }
      if (more) store_x((int)((c + 1) & 1));
      __syncthreads();
    }

    // ---- epilogue: lane holds C[n = 16nb + 4*q_l + r][row = 16rb + n_l]
    const bool partial = (!GROUPED) && (a.part != nullptr);
    const int64_t Np = G.NB * 16;
#pragma unroll
    for (int j = 0; j < NBW; ++j) {
      const int64_t nb = nb0 + j;
      if (nb >= G.NB) continue;
      const int64_t n = nb * 16 + 4 * q_l;
#pragma unroll
      for (int rb = 0; rb < MB; ++rb) {
        const int rl = rb * 16 + n_l;
        if (rl >= rcount || orow_s[rl] < 0) continue;
        f32x4_t v = acc[j][rb];
        if (partial) {
          float* dst = a.part + ((int64_t)split * a.M + m0 + rl) * Np + n;
          st16(dst, __builtin_bit_cast(u32x4_t, v));
          continue;
        }
        if (MX) {
          const float rs = a.xs[arow_s[rl]];
          v = v * rs;
        }
        uint16_t* dst = a.y + orow_s[rl] * G.N + n;
        if ((G.N & 3) == 0 && n + 3 < G.N) {
          *reinterpret_cast<u32x2_t*>(dst) = (u32x2_t){pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3])};
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (n + r < G.N) dst[r] = (uint16_t)(pack_bf16(v[r], 0.0f) & 0xFFFF);
        }
      }
    }
    __syncthreads();  // LDS row tables and buffers are reused by the next item
  }
}

// y[m][n] = bf16( scale(m) * sum_s part[s][m][n] ), four n per thread.
__global__ void __launch_bounds__(256)
k_splitk_reduce(GemmArgs a, int splits) {
  const Geom G = a.G;
  const int64_t Np = G.NB * 16;
  const int64_t cnt = a.M * (Np / 4);
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < cnt;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t m = i / (Np / 4);
    const int64_t n = (i % (Np / 4)) * 4;
    if (n >= G.N) continue;
    f32x4_t v = __builtin_bit_cast(f32x4_t, ld16(a.part + m * Np + n));
    for (int s = 1; s < splits; ++s)
      v += __builtin_bit_cast(f32x4_t, ld16(a.part + ((int64_t)s * a.M + m) * Np + n));
    if (a.xs) v = v * a.xs[m];
    uint16_t* dst = a.y + m * G.N + n;
    if ((G.N & 3) == 0 && n + 3 < G.N) {
      *reinterpret_cast<u32x2_t*>(dst) = (u32x2_t){pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3])};
    } else {
      for (int r = 0; r < 4; ++r)
        if (n + r < G.N) dst[r] = (uint16_t)(pack_bf16(v[r], 0.0f) & 0xFFFF);
    }
  }
}

template <bool MX, int MB, int NBW, bool GROUPED>
static hipError_t go_stream(const GemmArgs& a, const StreamCfg& c, int grid_items, hipStream_t st) {
  const int n_tiles = (int)((a.G.NB + 4 * NBW - 1) / (4 * NBW));
  dim3 grid;
  if (GROUPED) {
    grid = dim3((unsigned)(grid_items > 0 ? grid_items : 1));
  } else {
    const int64_t m_chunks = (a.M + MB * 16 - 1) / (MB * 16);
    grid = dim3((unsigned)n_tiles, (unsigned)c.splits, (unsigned)m_chunks);
  }
  hipLaunchKernelGGL((k_gemm_stream<MX, MB, NBW, GROUPED>), grid, dim3(256), 0, st, a, n_tiles);
  return hipGetLastError();
}

template <bool MX, int MB, bool GROUPED>
static hipError_t go_stream_nbw(const GemmArgs& a, const StreamCfg& c, int gi, hipStream_t st) {
  switch (c.nbw) {
    case 1: return go_stream<MX, MB, 1, GROUPED>(a, c, gi, st);
    case 2: return go_stream<MX, MB, 2, GROUPED>(a, c, gi, st);
    default: return go_stream<MX, MB, 4, GROUPED>(a, c, gi, st);
  }
}

template <bool MX, bool GROUPED>
static hipError_t go_stream_mb(const GemmArgs& a, const StreamCfg& c, int gi, hipStream_t st) {
  return (c.mb == 1) ? go_stream_nbw<MX, 1, GROUPED>(a, c, gi, st)
                     : go_stream_nbw<MX, 2, GROUPED>(a, c, gi, st);
}

hipError_t launch_gemm_stream(const GemmArgs& a, const StreamCfg& c, bool grouped, int grid_items,
                              hipStream_t st) {
  const bool mx = (a.wfmt == W_MXFP4);
  if (mx) return grouped ? go_stream_mb<true, true>(a, c, grid_items, st)
                         : go_stream_mb<true, false>(a, c, grid_items, st);
  return grouped ? go_stream_mb<false, true>(a, c, grid_items, st)
                 : go_stream_mb<false, false>(a, c, grid_items, st);
}

hipError_t launch_splitk_reduce(const GemmArgs& a, int splits, hipStream_t st) {
  const int64_t cnt = a.M * (a.G.NB * 16 / 4);
  int64_t blocks = (cnt + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(k_splitk_reduce, dim3((unsigned)blocks), dim3(256), 0, st, a, splits);
  return hipGetLastError();
}

}  // namespace hm
