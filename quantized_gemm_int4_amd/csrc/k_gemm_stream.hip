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

// activation bytes staged per block: 159 KiB of dynamic LDS, leaving room for the
// row tables within the 160 KiB of a gfx950 compute unit
constexpr int64_t kStreamLdsBudget = 159 * 1024;

// LDS-only barrier: waits for this wave's LDS operations, then meets the other
// waves.  Unlike __syncthreads() it does not wait for outstanding global loads
// (on CDNA one counter covers loads and stores), so the weight prefetch ring
// stays in flight across it.
__device__ __forceinline__ void lds_barrier() {
  __asm__ volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Template parameters: MX (W4A8-MXFP4 vs W4A16), ZP (zero points), MB (16-row
// blocks per unit), NBW (16-column blocks per wave), DW (weight prefetch ring:
// K groups of 128 held in registers ahead of use), GROUPED.
// Runtime: pg = K groups per activation piece staged in LDS (a multiple of DW);
// dynamic LDS = staged rows x (pg * bytes per group + 16).
template <bool MX, bool ZP, int MB, int NBW, int DW, bool GROUPED>
__global__ void __launch_bounds__(256)
k_gemm_stream(GemmArgs a, int n_tiles, int pg) {
  constexpr int ROWS = MB * 16;
  constexpr int GB = MX ? 128 : 256;                    // activation bytes per row per K group
  extern __shared__ __attribute__((aligned(16))) uint8_t xs_lds[];
  __shared__ int64_t arow_s[ROWS];
  __shared__ int64_t orow_s[ROWS];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (scalar)
  const Geom G = a.G;
  const int64_t K = G.K;
  const int n_l = lane & 15, q_l = lane >> 4;
  const uint8_t* xbase = reinterpret_cast<const uint8_t*>(a.x);
  const int64_t xrow_bytes = MX ? K : 2 * K;
  const uint16_t* s16 = reinterpret_cast<const uint16_t*>(a.w + G.off_scales);
  const uint32_t* s32 = reinterpret_cast<const uint32_t*>(a.w + G.off_scales);
  const uint32_t* z32 = reinterpret_cast<const uint32_t*>(a.w + G.off_zeros);
  const int XB = pg * GB + 16;                          // LDS row stride (bytes), padded

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
      rcount = u[2] < ROWS ? u[2] : ROWS;
      g_begin = 0;
      g_end = G.KG;
      if (tid < ROWS) {
        int64_t ar = 0, orr = -1;   // invalid rows read row 0 (always present) and are not stored
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
        const bool ok = tid < rcount;
        arow_s[tid] = ok ? m0 + tid : m0;
        orow_s[tid] = ok ? m0 + tid : -1;
      }
    }
    __syncthreads();

    const int64_t nb0 = ((int64_t)nt * 4 + wave) * NBW;
    const int ng = (int)(g_end - g_begin);
    int64_t nbc[NBW];  // clamped column blocks: loads stay in bounds, results of
                       // blocks >= NB are never stored
#pragma unroll
    for (int j = 0; j < NBW; ++j) nbc[j] = (nb0 + j < G.NB) ? nb0 + j : G.NB - 1;
    // LDS row of each MFMA row block: rows past the staged ones reuse the last
    // staged row (their outputs are never stored)
    int lrow[MB];
#pragma unroll
    for (int rb = 0; rb < MB; ++rb) lrow[rb] = (rb * 16 + n_l < rcount) ? rb * 16 + n_l : rcount - 1;

    // stage activation rows [0, rcount) x groups [gp, gp + plen) into LDS
    auto stage_x = [&](int gp, int plen) {
      const int per_row = plen * (GB / 16);
      const int total = rcount * per_row;
      const int64_t off0 = (g_begin + gp) * GB;
#pragma nounroll
      for (int base = 0; base < total; base += 256 * 4) {
        u32x4_t v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int i = base + u * 256 + tid;
          if (i < total)
            v[u] = ld16(xbase + arow_s[i / per_row] * xrow_bytes + off0 + (i % per_row) * 16);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int i = base + u * 256 + tid;
          if (i < total) st16(xs_lds + (i / per_row) * XB + (i % per_row) * 16, v[u]);
        }
      }
    };

    // ---- weight ring: DW groups ahead, raw scale / zero words kept until use
    u32x4_t wq[DW][NBW];
    // INT4: wsr / wsh hold the bf16 scales of the four output rows 4*q_l + 0..3
    // that this lane accumulates (the MFMA result is scaled, not the operand).
    uint32_t wsr[DW][NBW], wsh[MX ? 1 : DW][MX ? 1 : NBW], wzr[DW][NBW];
    auto load_w = [&](int d, int gl) {                  // gl: group index within [0, ng)
      const int64_t g = g_begin + gl;
#pragma unroll
      for (int j = 0; j < NBW; ++j) {
        const int64_t tile = (e * G.NB + nbc[j]) * G.KG + g;
        wq[d][j] = ld16(a.w + tile * 1024 + lane * 16);
        if (MX) {
          wsr[d][j] = s32[((e * G.NB + nbc[j]) * G.KG4 + g / 4) * 64 + lane];
        } else {
          const u32x2_t sp = *reinterpret_cast<const u32x2_t*>(s16 + tile * 16 + 4 * q_l);
          wsr[d][j] = sp[0];
          wsh[d][j] = sp[1];
          if (ZP) wzr[d][j] = z32[tile * 2 + (n_l >> 3)];
        }
      }
    };

    f32x4_t acc[NBW][MB];
#pragma unroll
    for (int j = 0; j < NBW; ++j)
#pragma unroll
      for (int rb = 0; rb < MB; ++rb) acc[j][rb] = (f32x4_t){0.f, 0.f, 0.f, 0.f};

    // K is walked in pieces of pg groups whose activations fit in LDS.  Each
    // piece restarts its weight ring (one memory latency per piece; a single
    // piece covers the whole K range whenever the rows fit), which keeps the
    // ring's load order identical on every entry to the round loop so that
    // each slot waits only for its own loads.
    const int n_pieces = (ng + pg - 1) / pg;
#pragma nounroll
    for (int p = 0; p < n_pieces; ++p) {
      const int gp = p * pg;
      const int plen = (ng - gp) < pg ? (ng - gp) : pg;
      if (p > 0) lds_barrier();               // everyone is done with the previous piece
      stage_x(gp, plen);
#pragma unroll
      for (int d = 0; d < DW; ++d) load_w(d, gp + (d < plen ? d : plen - 1));
      lds_barrier();
      const int rounds = (plen + DW - 1) / DW;
#pragma nounroll
      for (int r = 0; r < rounds; ++r) {
#pragma unroll
        for (int d = 0; d < DW; ++d) {
          const int lg = r * DW + d;          // group within the piece
          if (lg < plen) {
            const int64_t g = g_begin + gp + lg;
            if (MX) {
              u32x4_t a0[MB], a1[MB];
#pragma unroll
              for (int rb = 0; rb < MB; ++rb) {
                const uint8_t* xp = xs_lds + lrow[rb] * XB + lg * 128 + 16 * q_l;
                a0[rb] = ld16(xp);
                a1[rb] = ld16(xp + 64);
              }
#pragma unroll
              for (int j = 0; j < NBW; ++j) {
                const int sc = (int)((wsr[d][j] >> (8 * (g & 3))) & 0xFF);
#pragma unroll
                for (int rb = 0; rb < MB; ++rb)
                  acc[j][rb] = mfma_fp4_fp8(wq[d][j], a0[rb], a1[rb], acc[j][rb], sc, 127);
              }
            } else {
              // Raw codes: the MFMA sees bf16(1 + u/16) (exact), a second MFMA sees
              // bf16(1 + z/16); their difference is sum_k x_k (u_k - z)/16 for this
              // group, exactly 0 where every code equals the zero point, and 16
              // times the group scale is applied once to the difference.
              f32x4_t raw[NBW][MB], zc[ZP ? NBW : 1][MB];
              u32x4_t bz[ZP ? NBW : 1];
#pragma unroll
              for (int j = 0; j < (ZP ? NBW : 1); ++j) {
                const uint32_t z = ZP ? ((wzr[d][j] >> (4 * (n_l & 7))) & 0xF) : 8u;
                const uint32_t pz = raw_u4_bits(z) * 0x00010001u;
                bz[j] = (u32x4_t){pz, pz, pz, pz};
#pragma unroll
                for (int rb = 0; rb < MB; ++rb) zc[j][rb] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
              }
#pragma unroll
              for (int j = 0; j < NBW; ++j)
#pragma unroll
                for (int rb = 0; rb < MB; ++rb) raw[j][rb] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
#pragma unroll
              for (int kk = 0; kk < 4; ++kk) {
                u32x4_t af[MB];
#pragma unroll
                for (int rb = 0; rb < MB; ++rb)
                  af[rb] = ld16(xs_lds + lrow[rb] * XB + (lg * 128 + 32 * kk + 8 * q_l) * 2);
#pragma unroll
                for (int j = 0; j < NBW; ++j) {
                  const u32x4_t bw = raw8_u4(wq[d][j][kk]);
#pragma unroll
                  for (int rb = 0; rb < MB; ++rb) raw[j][rb] = mfma_bf16(bw, af[rb], raw[j][rb]);
                }
#pragma unroll
                for (int j = 0; j < (ZP ? NBW : 1); ++j)
#pragma unroll
                  for (int rb = 0; rb < MB; ++rb) zc[j][rb] = mfma_bf16(bz[j], af[rb], zc[j][rb]);
              }
#pragma unroll
              for (int j = 0; j < NBW; ++j) {
                const float s0 = bf16_to_f32(wsr[d][j] & 0xFFFFu), s1 = __uint_as_float(wsr[d][j] & 0xFFFF0000u);
                const float s2 = bf16_to_f32(wsh[d][j] & 0xFFFFu), s3 = __uint_as_float(wsh[d][j] & 0xFFFF0000u);
#pragma unroll
                for (int rb = 0; rb < MB; ++rb) {
                  const f32x4_t dl = (raw[j][rb] - zc[ZP ? j : 0][rb]) * 16.f;   // exact scaling
                  acc[j][rb][0] = fmaf(s0, dl[0], acc[j][rb][0]);
                  acc[j][rb][1] = fmaf(s1, dl[1], acc[j][rb][1]);
                  acc[j][rb][2] = fmaf(s2, dl[2], acc[j][rb][2]);
                  acc[j][rb][3] = fmaf(s3, dl[3], acc[j][rb][3]);
                }
              }
            }
          }
          load_w(d, gp + (lg + DW < plen ? lg + DW : plen - 1));
        }
      }
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

template <bool MX, bool ZP, int MB, int NBW, bool GROUPED>
static hipError_t go_stream(const GemmArgs& a, const StreamCfg& c, int grid_items, hipStream_t st) {
  // ring depth: up to 16 groups per 16-column block, within the 63 outstanding
  // vector-memory operations one wave can track (three loads per group)
  constexpr int DW = (NBW == 1) ? (MB == 1 ? 16 : 8) : (NBW == 2 ? 8 : 4);
  const int n_tiles = (int)((a.G.NB + 4 * NBW - 1) / (4 * NBW));
  const int gb = (a.wfmt == W_MXFP4) ? 128 : 256;
  // activation piece: as many K groups as fit the LDS budget, a multiple of DW
  const int64_t rows = GROUPED ? 16 * MB : (a.M < 16 * MB ? a.M : 16 * MB);
  const int64_t ksl = GROUPED ? a.G.KG : a.ksg;
  int64_t pg = (kStreamLdsBudget / rows - 16) / gb;
  pg = pg / DW * DW;
  if (pg < DW) pg = DW;
  const int64_t need = (ksl + DW - 1) / DW * DW;
  if (pg > need) pg = need;
  const size_t lds = (size_t)rows * (pg * gb + 16);
  // allow more than the default dynamic LDS (set once per instance; thread-safe static init)
  static const hipError_t attr_err = hipFuncSetAttribute(
      reinterpret_cast<const void*>(&k_gemm_stream<MX, ZP, MB, NBW, DW, GROUPED>),
      hipFuncAttributeMaxDynamicSharedMemorySize, (int)kStreamLdsBudget);
  if (attr_err != hipSuccess) return attr_err;
  dim3 grid;
  if (GROUPED) {
    grid = dim3((unsigned)(grid_items > 0 ? grid_items : 1));
  } else {
    const int64_t m_chunks = (a.M + MB * 16 - 1) / (MB * 16);
    grid = dim3((unsigned)n_tiles, (unsigned)c.splits, (unsigned)m_chunks);
  }
  hipLaunchKernelGGL((k_gemm_stream<MX, ZP, MB, NBW, DW, GROUPED>), grid, dim3(256), lds, st, a,
                     n_tiles, (int)pg);
  return hipGetLastError();
}

template <bool MX, bool ZP, int MB, bool GROUPED>
static hipError_t go_stream_nbw(const GemmArgs& a, const StreamCfg& c, int gi, hipStream_t st) {
  switch (c.nbw) {
    case 1: return go_stream<MX, ZP, MB, 1, GROUPED>(a, c, gi, st);
    case 2: return go_stream<MX, ZP, MB, 2, GROUPED>(a, c, gi, st);
    default: return go_stream<MX, ZP, MB, 4, GROUPED>(a, c, gi, st);
  }
}

template <bool MX, bool ZP, bool GROUPED>
static hipError_t go_stream_mb(const GemmArgs& a, const StreamCfg& c, int gi, hipStream_t st) {
  return (c.mb == 1) ? go_stream_nbw<MX, ZP, 1, GROUPED>(a, c, gi, st)
                     : go_stream_nbw<MX, ZP, 2, GROUPED>(a, c, gi, st);
}

hipError_t launch_gemm_stream(const GemmArgs& a, const StreamCfg& c, bool grouped, int grid_items,
                              hipStream_t st) {
  if (a.wfmt == W_MXFP4)
    return grouped ? go_stream_mb<true, false, true>(a, c, grid_items, st)
                   : go_stream_mb<true, false, false>(a, c, grid_items, st);
  if (a.wfmt == W_UINT4_ZP)
    return grouped ? go_stream_mb<false, true, true>(a, c, grid_items, st)
                   : go_stream_mb<false, true, false>(a, c, grid_items, st);
  return grouped ? go_stream_mb<false, false, true>(a, c, grid_items, st)
                 : go_stream_mb<false, false, false>(a, c, grid_items, st);
}

hipError_t launch_splitk_reduce(const GemmArgs& a, int splits, hipStream_t st) {
  const int64_t cnt = a.M * (a.G.NB * 16 / 4);
  int64_t blocks = (cnt + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(k_splitk_reduce, dim3((unsigned)blocks), dim3(256), 0, st, a, splits);
  return hipGetLastError();
}

}  // namespace hm
