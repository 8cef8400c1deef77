// MFMA tile GEMM for many rows (prefill-sized M, and large experts of a
// grouped GEMM), where the ~2*M*N*K matrix multiply dominates (ywsung.com note
// "How vLLM Humming computes 4 bits", section on one token vs many tokens).
//
// One 256-thread block computes a 128 x 128 output tile; its four waves each
// own 64 x 64 (4 x 4 MFMA blocks of 16 x 16).  Per 128-K step:
//   * the activation tile (128 rows) is staged in LDS with a padded row stride
//     (conflict-free 16-byte fragment reads);
//   * W4A16: the eight 1 KiB weight tiles are read once per block, unpacked and
//     scaled to bf16 by the block's threads (once per block, not per wave) and
//     written to LDS already in MFMA fragment order;
//   * MXFP4 / MXINT4 with bf16 rows: the same, each lane's eight codes of a
//     fragment scaled to bf16 with their E8M0 scale (the fragment's K run is
//     32 (L/16) + 8 ks + 0..7 instead of 32 ks + 8 (L/16) + 0..7, and the
//     activation fragments follow it);
//   * W4A8-MXFP4: each wave loads its E2M1 fragments straight into registers
//     and feeds them with their E8M0 scales to the 16x16x128 scaled MFMA; the
//     per-token FP8 scale is applied in the epilogue.
// Global loads for step g+1 are issued before the MFMAs of step g.
#include "common.h"
#include "launch.h"

namespace hm {

template <int MODE, bool GROUPED>
__global__ void __launch_bounds__(256)
k_gemm_tile(GemmArgs a, int n_tiles) {
  constexpr bool A4 = MODE == KM_MX_A4;                // MXFP4 rows, scaled fp4 x fp4 MFMA
  constexpr bool MX = MODE == KM_MX_A8 || A4;          // E2M1 weight fragments fed as stored
  constexpr bool F4 = MODE == KM_MX_A16 || MODE == KM_MXI4_A16;  // MX codes scaled to bf16
  constexpr bool I4 = MODE == KM_MXI4_A16;             // MXINT4: two's complement codes / 4
  constexpr bool Q8 = MODE == KM_INT8_A16;             // INT8 weights: 2 KiB tiles in two halves
  constexpr int WLD = Q8 ? 4 : 2;                      // 16-byte weight loads per thread per step
  constexpr int GBX = A4 ? 64 : (MX ? 128 : 256);      // activation bytes per row per K step
  constexpr int XB = GBX + 16;                         // LDS activation row stride (bytes)
  constexpr int XPR = GBX / 16;                        // 16-byte pieces per activation row
  constexpr int XLD = kTileM * XPR / 256;              // pieces per thread
  constexpr int WLDS = MX ? 16 : 8 * 4 * 1024;         // dequantized weight fragments
  __shared__ __attribute__((aligned(16))) uint8_t xs_lds[kTileM * XB];
  __shared__ uint32_t xsc_lds[A4 ? kTileM : 1];        // MXFP4 rows: E8M0 word of each row's step
  __shared__ __attribute__((aligned(16))) uint8_t ws_lds[WLDS];
  __shared__ int64_t arow_s[kTileM];
  __shared__ int64_t orow_s[kTileM];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (scalar)
  const int wm = wave >> 1, wn = wave & 1;
  const int n_l = lane & 15, q_l = lane >> 4;
  const Geom G = a.G;
  const int64_t K = G.K;
  const uint8_t* xbase = reinterpret_cast<const uint8_t*>(a.x);
  const int64_t xrow_bytes = A4 ? K / 2 : (MX ? K : 2 * K);

  const int64_t n_items = GROUPED ? (int64_t)a.hdr[1] * n_tiles : 1;
  for (int64_t item = GROUPED ? blockIdx.x : 0; item < n_items;
       item += GROUPED ? gridDim.x : 1) {
    int64_t e = 0;
    int nt, rcount;
    if (GROUPED) {
      const int64_t unit = item / n_tiles;
      nt = (int)(item % n_tiles);
      const int32_t* u = a.units + 4 * unit;
      e = u[0];
      rcount = u[2];
      if (tid < kTileM) {
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
      const int64_t m0 = (int64_t)blockIdx.y * kTileM;
      rcount = (int)((a.M - m0) < kTileM ? (a.M - m0) : kTileM);
      if (tid < kTileM) {
        const bool ok = tid < rcount;
        arow_s[tid] = ok ? m0 + tid : m0;
        orow_s[tid] = ok ? m0 + tid : -1;
      }
    }
    __syncthreads();

    const int64_t nbt = (int64_t)nt * 8;  // first 16-column block of this tile

    // ---- register staging of one K step.  Loads are unconditional (column
    // blocks clamped into range, invalid rows read a valid row) so that the
    // compiler issues them back to back; scale and zero words stay raw until use.
    const uint16_t* s16 = reinterpret_cast<const uint16_t*>(a.w + G.off_scales);
    const uint32_t* s32 = reinterpret_cast<const uint32_t*>(a.w + G.off_scales);
    const uint32_t* z32 = reinterpret_cast<const uint32_t*>(a.w + G.off_zeros);
    const bool zp = (a.wfmt == W_UINT4_ZP);
    u32x4_t xr[XLD];
    u32x4_t wq[WLD];             // W4A16: two code slots per thread (INT8: four half slots)
    uint32_t wsr[WLD], wzr[WLD];
    u32x4_t mq[4];               // W4A8 / W4A4: this wave's four fragments
    uint32_t msr[4];
    uint32_t xsr = 0;            // W4A4: this thread's row scale word (threads < 128)

    auto load_step = [&](int64_t g) {
#pragma unroll
      for (int i = 0; i < XLD; ++i) {
        const int q = tid + 256 * i;
        const int row = q / XPR, pc = q % XPR;
        xr[i] = ld16(xbase + arow_s[row] * xrow_bytes + g * GBX + pc * 16);
      }
      if (A4 && tid < kTileM)
        xsr = *reinterpret_cast<const uint32_t*>(a.xsb + arow_s[tid] * (G.KG * 4) + g * 4);
      if (MX) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          int64_t nb = nbt + wn * 4 + j;
          if (nb >= G.NB) nb = G.NB - 1;
          const int64_t tile = (e * G.NB + nb) * G.KG + g;
          mq[j] = ld16(a.w + tile * 1024 + lane * 16);
          msr[j] = s32[((e * G.NB + nb) * G.KG4 + g / 4) * 64 + lane];
        }
      } else if (Q8) {
        // load i: column block (q >> 6) & 7, half q >> 9, slot q & 63
#pragma unroll
        for (int i = 0; i < WLD; ++i) {
          const int q = tid + 256 * i;
          int64_t nb = nbt + ((q >> 6) & 7);
          if (nb >= G.NB) nb = G.NB - 1;
          const int L = q & 63;
          const int64_t tile = (e * G.NB + nb) * G.KG + g;
          wq[i] = ld16(a.w + tile * 2048 + (q >> 9) * 1024 + L * 16);
          wsr[i] = s16[tile * 16 + (L & 15)];
          wzr[i] = 0u;
        }
      } else {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const int q = tid + 256 * i;
          int64_t nb = nbt + (q >> 6);
          if (nb >= G.NB) nb = G.NB - 1;
          const int L = q & 63;
          const int64_t tile = (e * G.NB + nb) * G.KG + g;
          wq[i] = ld16(a.w + tile * 1024 + L * 16);
          if (F4) {
            wsr[i] = (s32[((e * G.NB + nb) * G.KG4 + g / 4) * 64 + L] >> (8 * (g & 3))) & 0xFFu;
            wzr[i] = 0u;
          } else {
            wsr[i] = s16[tile * 16 + (L & 15)];
            wzr[i] = zp ? z32[tile * 2 + ((L & 15) >> 3)] : 0u;
          }
        }
      }
    };
    auto store_step = [&]() {
#pragma unroll
      for (int i = 0; i < XLD; ++i) {
        const int q = tid + 256 * i;
        const int row = q / XPR, pc = q % XPR;
        st16(&xs_lds[row * XB + pc * 16], xr[i]);
      }
      if (A4 && tid < kTileM) xsc_lds[tid] = xsr;
      if (Q8) {
        // half p holds the operands of MFMAs 2 p and 2 p + 1, each s * q rounded to bf16
#pragma unroll
        for (int i = 0; i < WLD; ++i) {
          const int q = tid + 256 * i;
          const int nbl = (q >> 6) & 7, p = q >> 9, L = q & 63;
          const float sv = bf16_to_f32(wsr[i] & 0xFFFF);
#pragma unroll
          for (int jj = 0; jj < 2; ++jj)
            st16(&ws_lds[((nbl * 4 + 2 * p + jj) * 64 + L) * 16], i8x8_bf16_scaled(wq[i][2 * jj], wq[i][2 * jj + 1], sv));
        }
      } else if (!MX) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const int q = tid + 256 * i;
          const int nbl = q >> 6, L = q & 63;
          if (F4) {
            const float sf = e8m0_f32(wsr[i]) * (I4 ? 0.25f : 1.0f);
#pragma unroll
            for (int j = 0; j < 4; ++j)
              st16(&ws_lds[((nbl * 4 + j) * 64 + L) * 16], I4 ? i4x8_bf16(wq[i][j], sf) : fp4x8_bf16(wq[i][j], sf));
            continue;
          }
          const float sv = bf16_to_f32(wsr[i] & 0xFFFF);
          const float z = zp ? (float)((wzr[i] >> (4 * (L & 7))) & 0xF) : 8.0f;
          const float zs = -z * sv;
#pragma unroll
          for (int j = 0; j < 4; ++j)
            st16(&ws_lds[((nbl * 4 + j) * 64 + L) * 16], dq8_u4(wq[i][j], sv, zs));
        }
      }
    };

    f32x4_t acc[4][4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[j][i] = (f32x4_t){0.f, 0.f, 0.f, 0.f};

    load_step(0);
    store_step();
    __syncthreads();
    u32x4_t cq[4];
    int csc[4];
    for (int64_t g = 0; g < G.KG; ++g) {
      if (MX) {
#pragma unroll
        for (int j = 0; j < 4; ++j) { cq[j] = mq[j]; csc[j] = (int)((msr[j] >> (8 * (g & 3))) & 0xFF); }
      }
      const bool more = (g + 1 < G.KG);
      if (more) load_step(g + 1);
      if (A4) {
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
          const int r = wm * 64 + mb * 16 + n_l;
          const u32x4_t b = ld16(xs_lds + r * XB + 16 * q_l);
          const int bs = (int)((xsc_lds[r] >> (8 * q_l)) & 0xFFu);
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[j][mb] = mfma_fp4_fp4(cq[j], b, acc[j][mb], csc[j], bs);
        }
      } else if (MX) {
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
          const uint8_t* p = xs_lds + (wm * 64 + mb * 16 + n_l) * XB + 16 * q_l;
          const u32x4_t a0 = ld16(p), a1 = ld16(p + 64);
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[j][mb] = mfma_fp4_fp8(cq[j], a0, a1, acc[j][mb], csc[j], 127);
        }
      } else {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          u32x4_t xf[4], wf[4];
#pragma unroll
          for (int mb = 0; mb < 4; ++mb)
            xf[mb] = ld16(xs_lds + (wm * 64 + mb * 16 + n_l) * XB + (F4 ? 32 * q_l + 8 * ks : 32 * ks + 8 * q_l) * 2);
#pragma unroll
          for (int j = 0; j < 4; ++j) wf[j] = ld16(ws_lds + (((wn * 4 + j) * 4 + ks) * 64 + lane) * 16);
#pragma unroll
          for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int mb = 0; mb < 4; ++mb) acc[j][mb] = mfma_bf16(wf[j], xf[mb], acc[j][mb]);
        }
      }
      __syncthreads();
      if (more) {
        store_step();
        __syncthreads();
      }
    }

    // ---- epilogue: lane holds C[n = 16nb + 4*q_l + r][row = 16mb + n_l]
    if (GROUPED && a.gated) {
      // gated layout: blocks nb (even) and nb + 1 of the lane's j = 2 p and
      // 2 p + 1 are the gate and up halves of output columns 8 nb + 4 q_l + r
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        const int64_t nb = nbt + wn * 4 + 2 * p;
        if (nb >= G.NB) continue;
        const int64_t n = nb * 8 + 4 * q_l;
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
          const int rl = wm * 64 + mb * 16 + n_l;
          if (rl >= rcount || orow_s[rl] < 0) continue;
          f32x4_t vg = acc[2 * p][mb], vu = acc[2 * p + 1][mb];
          if (MX && !A4) {
            const float rs = a.xs[arow_s[rl]];
            vg = vg * rs;
            vu = vu * rs;
          }
          uint16_t* dst = a.y + orow_s[rl] * (G.N / 2) + n;
          *reinterpret_cast<u32x2_t*>(dst) =
              (u32x2_t){silu_mul_pair(pack_bf16(vg[0], vg[1]), pack_bf16(vu[0], vu[1])),
                        silu_mul_pair(pack_bf16(vg[2], vg[3]), pack_bf16(vu[2], vu[3]))};
        }
      }
      __syncthreads();
      continue;
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t nb = nbt + wn * 4 + j;
      if (nb >= G.NB) continue;
      const int64_t n = nb * 16 + 4 * q_l;
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
        const int rl = wm * 64 + mb * 16 + n_l;
        if (rl >= rcount || orow_s[rl] < 0) continue;
        f32x4_t v = acc[j][mb];
        if (MX && !A4) v = v * a.xs[arow_s[rl]];
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
    __syncthreads();
  }
}

template <int MODE, bool GROUPED>
static hipError_t go_tile(const GemmArgs& a, int grid_items, hipStream_t st) {
  const int n_tiles = (int)((a.G.NB + 7) / 8);
  dim3 grid;
  if (GROUPED) grid = dim3((unsigned)(grid_items > 0 ? grid_items : 1));
  else grid = dim3((unsigned)n_tiles, (unsigned)((a.M + kTileM - 1) / kTileM));
  hipLaunchKernelGGL((k_gemm_tile<MODE, GROUPED>), grid, dim3(256), 0, st, a, n_tiles);
  return hipGetLastError();
}

hipError_t launch_gemm_tile(const GemmArgs& a, bool grouped, int grid_items, hipStream_t st) {
  const int mode = kmode_of(a);
  if (mode == KM_MX_A8)
    return grouped ? go_tile<KM_MX_A8, true>(a, grid_items, st) : go_tile<KM_MX_A8, false>(a, grid_items, st);
  if (mode == KM_MX_A4)
    return grouped ? go_tile<KM_MX_A4, true>(a, grid_items, st) : go_tile<KM_MX_A4, false>(a, grid_items, st);
  if (mode == KM_INT8_A16)
    return grouped ? go_tile<KM_INT8_A16, true>(a, grid_items, st) : go_tile<KM_INT8_A16, false>(a, grid_items, st);
  if (mode == KM_MX_A16)
    return grouped ? go_tile<KM_MX_A16, true>(a, grid_items, st) : go_tile<KM_MX_A16, false>(a, grid_items, st);
  if (mode == KM_MXI4_A16)
    return grouped ? go_tile<KM_MXI4_A16, true>(a, grid_items, st) : go_tile<KM_MXI4_A16, false>(a, grid_items, st);
  return grouped ? go_tile<KM_INT4_A16, true>(a, grid_items, st) : go_tile<KM_INT4_A16, false>(a, grid_items, st);
}

}  // namespace hm
