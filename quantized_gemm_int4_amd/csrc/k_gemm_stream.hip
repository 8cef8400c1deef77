// Streaming GEMM for few rows (decode-sized M, and small experts of a grouped
// GEMM).  With few rows, reading and unpacking the weights dominates (ywsung.com
// note "How vLLM Humming computes 4 bits", section on one token vs many
// tokens), so every weight byte is read from HBM exactly once, straight into
// registers: one 16-byte load per lane fetches one 1 KiB tile (16 columns x
// 128 K) of the device layout, which is exactly the operand of four
// 16x16x32 bf16 MFMAs (or of one 16x16x128 scaled fp4 x fp8 MFMA for MXFP4
// with FP8 rows; with bf16 rows the E2M1 (or MXINT4) codes are scaled to bf16 first and fed
// to four bf16 MFMAs, the lane's 32 K values split into four runs of eight and
// the activation fragments read in the same order).
// The few activation rows are copied into LDS with direct global-to-LDS loads
// (issued before the weight loads, so both latencies overlap) and shared by
// the block's four waves.  The weights are the MFMA "A" operand (rows =
// output columns n) and the activations the "B" operand, so each lane ends
// with four consecutive n of one row and stores them as one 8-byte write.
//
// Work split: a block has NW waves (4, or 8 for dense calls, so that a
// block's staged rows feed twice the waves); KS of them share one set of NBW
// 16-column blocks and split its K range, adding their sums through LDS at
// the end; NW/KS such sets make one block.  Dense calls may also split K over
// blocks and reduce fp32 partials in a second kernel.
#include "common.h"
#include "launch.h"

namespace hm {

// dynamic LDS per block: 159 KiB, leaving room for the row tables within the
// 160 KiB of a gfx950 compute unit
constexpr int64_t kStreamLdsBudget = 159 * 1024;

// LDS-only barrier: waits for this wave's LDS operations, then meets the other
// waves.  Unlike __syncthreads() it does not wait for outstanding global loads
// (on CDNA one counter covers loads and stores), so the weight prefetch ring
// stays in flight across it.
__device__ __forceinline__ void lds_barrier() {
  __asm__ volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}


template <int NW, int KS, int NBW, int MB>
struct StreamShape {
  static constexpr int kRedBytes = KS > 1 ? NW * NBW * MB * 1024 : 0;  // K-split sums
};

// Template parameters: MODE (KMode: INT4 / MXFP4 weights, bf16 / FP8 rows), ZP (zero points), MB (16-row
// blocks per unit), NBW (16-column blocks per wave), KS (waves splitting one
// column set's K range), DW (weight prefetch ring: K groups of 128 held in
// registers ahead of use), GROUPED, NW (waves per block).
// Runtime: pg = K groups per activation piece staged in LDS, xb = LDS row
// stride in bytes (a multiple of 1 KiB plus 16).
template <int MODE, bool ZP, int MB, int NBW, int KS, int DW, bool GROUPED, int NW>
__global__ void __launch_bounds__(64 * NW)
k_gemm_stream(GemmArgs a, int n_tiles, int pg, int xb) {
  constexpr bool MX = MODE == KM_MX_A8;                 // FP8 rows, scaled fp4 x fp8 MFMA
  constexpr bool F4 = MODE == KM_MX_A16 || MODE == KM_MXI4_A16;   // MX codes scaled to bf16
  constexpr bool I4 = MODE == KM_MXI4_A16;              // MXINT4: two's complement codes / 4
  constexpr bool A4 = MODE == KM_MX_A4;                 // MXFP4 rows, scaled fp4 x fp4 MFMA
  constexpr bool Q8 = MODE == KM_INT8_A16;              // INT8 weights: 2 KiB tiles, two halves
  constexpr bool MXW = MX || F4 || A4;                  // E8M0 scale words
  constexpr int ROWS = MB * 16;
  constexpr int GB = MX ? 128 : (A4 ? 64 : 256);        // activation bytes per row per K group
  constexpr int CS = NW / KS;                           // column sets per block
  constexpr int RED = StreamShape<NW, KS, NBW, MB>::kRedBytes;
  // vector-memory loads per ring slot: per column block the 1 KiB tile and
  // its scale word(s), plus the zero-point word
  constexpr int kRingLoads = NBW * (MXW ? 2 : (ZP || Q8 ? 3 : 2));
  extern __shared__ __attribute__((aligned(1024))) uint8_t lds[];
  uint8_t* const xs_lds = lds + RED;                    // activations: [rows][xb]
  __shared__ int64_t arow_s[ROWS];
  __shared__ int64_t orow_s[ROWS];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (scalar)
  const int cset = wave / KS, kq = wave % KS;
  const Geom G = a.G;
  const int64_t K = G.K;
  const int n_l = lane & 15, q_l = lane >> 4;
  const uint8_t* xbase = reinterpret_cast<const uint8_t*>(a.x);
  const int64_t xrow_bytes = MX ? K : (A4 ? K / 2 : 2 * K);
  const uint8_t* sbase = a.w + G.off_scales;
  // MXFP4 rows: the E8M0 words of each row's groups (4 blocks of 32 per group)
  // are staged after the rows' codes, `sb` bytes per row
  const int sb = A4 ? ((pg + 63) / 64) * 256 : 0;
  const uint8_t* xsbase = A4 ? a.xsb : nullptr;
  const uint8_t* zbase = a.w + G.off_zeros;
  const uint32_t zshift = 4u * (uint32_t)(n_l & 7);

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

    const int64_t nb0 = ((int64_t)nt * CS + cset) * NBW;
    const int ng = (int)(g_end - g_begin);
    // clamped column blocks (scalar): loads stay in bounds, results of blocks
    // >= NB are never stored
    int64_t wtile0[NBW], stile0[NBW];
#pragma unroll
    for (int j = 0; j < NBW; ++j) {
      const int64_t nbc = (nb0 + j < G.NB) ? nb0 + j : G.NB - 1;
      wtile0[j] = (e * G.NB + nbc) * G.KG;            // tile index of group 0
      stile0[j] = (e * G.NB + nbc) * G.KG4;           // MXFP4 scale word row
    }
    // LDS row of each MFMA row block: rows past the staged ones reuse the last
    // staged row (their outputs are never stored)
    int lrow[MB];
#pragma unroll
    for (int rb = 0; rb < MB; ++rb) lrow[rb] = (rb * 16 + n_l < rcount) ? rb * 16 + n_l : rcount - 1;

    // Byte offset of activation row r (r < ROWS) held by lane r: the copy loop
    // below takes it with readlane, because an LDS read there would have to
    // wait for the copies already in flight (they write LDS too).
    const int64_t xrow_off = arow_s[lane & (ROWS - 1)] * xrow_bytes;
    const uint32_t xro_lo = (uint32_t)xrow_off, xro_hi = (uint32_t)((uint64_t)xrow_off >> 32);
    const int64_t srow_off = A4 ? arow_s[lane & (ROWS - 1)] * G.KG * 4 : 0;    // scale bytes of the row
    const uint32_t sro_lo = (uint32_t)srow_off, sro_hi = (uint32_t)((uint64_t)srow_off >> 32);
    uint8_t* const xsc_lds = xs_lds + rcount * xb;      // MXFP4 rows: staged scale words

    // Copy activation rows [0, rcount) x groups [gp, gp + plen) into LDS: one
    // wave instruction moves 1 KiB of one row (buffer over the row's piece,
    // lane L at byte 16 L of the instruction's 1 KiB); lanes past the row's
    // end fall outside the buffer, read zeros and land in the row's padding.
    // The per-lane offset never changes, so no copy waits for an earlier one.
    const uint32_t lane16 = (uint32_t)lane * 16;
    auto stage_x = [&](int gp, int plen) {
      const int per_row = plen * (GB / 16);             // 16-byte chunks per row
      const int cpr = (per_row + 63) / 64;              // 1 KiB pieces per row
      const int total = rcount * cpr;
      const int64_t off0 = (g_begin + gp) * GB;
#pragma nounroll
      for (int i = wave; i < total; i += NW) {
        const int r = i / cpr, blk = i - (i / cpr) * cpr;
        const uint64_t ro = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)xro_hi, r) << 32) |
                            (uint32_t)__builtin_amdgcn_readlane((int)xro_lo, r);
        b2lds16(make_rsrc(xbase + ro + off0, (uint64_t)per_row * 16), lane16, (uint32_t)blk * 1024,
                xs_lds + r * xb + blk * 1024);
      }
      if (A4) {
        // the rows' scale words of groups [gp, gp + plen): 4-byte copies,
        // 64 words per instruction, lanes past the piece read zeros
        const int cps = (plen + 63) / 64;
        const int tot = rcount * cps;
#pragma nounroll
        for (int i = wave; i < tot; i += NW) {
          const int r = i / cps, blk = i - (i / cps) * cps;
          const uint64_t ro = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)sro_hi, r) << 32) |
                              (uint32_t)__builtin_amdgcn_readlane((int)sro_lo, r);
          b2lds4(make_rsrc(xsbase + ro + (g_begin + gp) * 4, (uint64_t)plen * 4), (uint32_t)lane * 4,
                 (uint32_t)blk * 256, xsc_lds + r * sb + blk * 256);
        }
      }
    };

    // ---- weight ring: DW groups ahead, raw scale / zero words kept until use
    u32x4_t wq[DW][NBW];
    u32x4_t wq2[Q8 ? DW : 1][Q8 ? NBW : 1];            // INT8: the tile's second half
    uint32_t wsr[DW][NBW], wsh[MXW ? 1 : DW][MXW ? 1 : NBW], wzr[ZP ? DW : 1][ZP ? NBW : 1];
    auto load_w = [&](int d, int64_t g) {               // g: group index in [0, KG)
#pragma unroll
      for (int j = 0; j < NBW; ++j) {
        const int64_t tile = wtile0[j] + g;
        if (Q8) {
          wq[d][j] = ld16(a.w + tile * 2048 + lane * 16);
          wq2[Q8 ? d : 0][Q8 ? j : 0] = ld16(a.w + tile * 2048 + 1024 + lane * 16);
        } else {
          wq[d][j] = ld16(a.w + tile * 1024 + lane * 16);
        }
        if (MXW) {
          // four groups' E8M0 scales per lane word: [e][nb][g/4][64 lanes]
          wsr[d][j] = *reinterpret_cast<const uint32_t*>(sbase + ((stile0[j] + g / 4) * 64 + lane) * 4);
        } else {
          // bf16 scales of the four output rows 4*q_l + 0..3 this lane accumulates
          const u32x2_t sp = *reinterpret_cast<const u32x2_t*>(sbase + tile * 32 + q_l * 8);
          wsr[d][j] = sp[0];
          wsh[MXW ? 0 : d][MXW ? 0 : j] = sp[1];
          if (ZP)
            wzr[ZP ? d : 0][ZP ? j : 0] =
                *reinterpret_cast<const uint32_t*>(zbase + tile * 8 + (n_l >> 3) * 4);
        }
      }
    };

    f32x4_t acc[NBW][MB];
#pragma unroll
    for (int j = 0; j < NBW; ++j)
#pragma unroll
      for (int rb = 0; rb < MB; ++rb) acc[j][rb] = (f32x4_t){0.f, 0.f, 0.f, 0.f};

    // K is walked in pieces of pg groups whose activations fit in LDS (a single
    // piece whenever the rows fit).  Inside a piece, wave kq takes the kq-th of
    // KS equal slices.  Each piece restarts the weight ring, which keeps the
    // ring's load order identical on every entry to the round loop so that
    // each slot waits only for its own loads.
    const int n_pieces = (ng + pg - 1) / pg;
#pragma nounroll
    for (int p = 0; p < n_pieces; ++p) {
      const int gp = p * pg;
      const int plen = (ng - gp) < pg ? (ng - gp) : pg;
      const int sub = (plen + KS - 1) / KS;
      const int lo = kq * sub;                              // this wave's slice [lo, lo + sl)
      const int sl = (plen - lo) < sub ? (plen - lo) : sub; // may be <= 0
      const int64_t gw = g_begin + gp + lo;                 // first group of the slice
      const int last = sl > 0 ? sl - 1 : 0;
      const int64_t gsafe = sl > 0 ? gw : g_begin + gp;     // loads of empty slices stay in range
      if (p > 0) lds_barrier();               // everyone is done with the previous piece
      stage_x(gp, plen);
      // the ring's first loads go out after the activation copies (the
      // memory clobber keeps the compiler from hoisting them), so waiting
      // until only those loads are outstanding means the copies landed; the
      // ring slots themselves are waited for one by one where they are used
      __asm__ volatile("" ::: "memory");
#pragma unroll
      for (int d = 0; d < DW; ++d) load_w(d, gsafe + (d < last ? d : last));
      __asm__ volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(DW * kRingLoads) : "memory");
      const int rounds = sl > 0 ? (sl + DW - 1) / DW : 0;
      // group lg of the slice from ring slot d
      auto process = [&](int d, int lg) {
        const int64_t g = gw + lg;
        const uint8_t* xg = xs_lds + (lo + lg) * GB;
        if (A4) {
          // lane L: row n_l of the row block, K block q_l of the group (16
          // bytes of codes) and that block's scale byte
          u32x4_t bq[MB];
          int bs[MB];
#pragma unroll
          for (int rb = 0; rb < MB; ++rb) {
            bq[rb] = ld16(xg + lrow[rb] * xb + 16 * q_l);
            bs[rb] = xsc_lds[lrow[rb] * sb + (lo + lg) * 4 + q_l];
          }
#pragma unroll
          for (int j = 0; j < NBW; ++j) {
            const int sc = (int)((wsr[d][j] >> (8 * (g & 3))) & 0xFF);
#pragma unroll
            for (int rb = 0; rb < MB; ++rb) acc[j][rb] = mfma_fp4_fp4(wq[d][j], bq[rb], acc[j][rb], sc, bs[rb]);
          }
        } else if (MX) {
          u32x4_t a0[MB], a1[MB];
#pragma unroll
          for (int rb = 0; rb < MB; ++rb) {
            const uint8_t* xp = xg + lrow[rb] * xb + 16 * q_l;
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
        } else if (F4) {
          // word kk of the lane's slot holds K = 32 q_l + 8 kk + 0..7 of its
          // column; the activation fragment of MFMA kk covers the same K
          float sf[NBW];
#pragma unroll
          for (int j = 0; j < NBW; ++j) sf[j] = e8m0_f32((wsr[d][j] >> (8 * (g & 3))) & 0xFFu) * (I4 ? 0.25f : 1.0f);
#pragma unroll
          for (int kk = 0; kk < 4; ++kk) {
            u32x4_t af[MB];
#pragma unroll
            for (int rb = 0; rb < MB; ++rb) af[rb] = ld16(xg + lrow[rb] * xb + (32 * q_l + 8 * kk) * 2);
#pragma unroll
            for (int j = 0; j < NBW; ++j) {
              const u32x4_t bw = I4 ? i4x8_bf16(wq[d][j][kk], sf[j]) : fp4x8_bf16(wq[d][j][kk], sf[j]);
#pragma unroll
              for (int rb = 0; rb < MB; ++rb) acc[j][rb] = mfma_bf16(bw, af[rb], acc[j][rb]);
            }
          }
        } else if (Q8) {
          // INT8 codes enter the MFMA exactly (bf16 holds every byte value);
          // operand kk is bytes 8 (kk % 2) .. + 7 of half kk / 2
          f32x4_t t[NBW][MB];
#pragma unroll
          for (int kk = 0; kk < 4; ++kk) {
            u32x4_t af[MB];
#pragma unroll
            for (int rb = 0; rb < MB; ++rb) af[rb] = ld16(xg + lrow[rb] * xb + (32 * kk + 8 * q_l) * 2);
#pragma unroll
            for (int j = 0; j < NBW; ++j) {
              const u32x4_t hv = kk < 2 ? wq[d][j] : wq2[Q8 ? d : 0][Q8 ? j : 0];
              const u32x4_t bw = i8x8_bf16(hv[2 * (kk & 1)], hv[2 * (kk & 1) + 1]);
#pragma unroll
              for (int rb = 0; rb < MB; ++rb)
                t[j][rb] = mfma_bf16(bw, af[rb], kk == 0 ? (f32x4_t){0.f, 0.f, 0.f, 0.f} : t[j][rb]);
            }
          }
#pragma unroll
          for (int j = 0; j < NBW; ++j) {
            const uint32_t lo2 = wsr[d][j], hi2 = wsh[MXW ? 0 : d][MXW ? 0 : j];
            const float s0 = bf16_to_f32(lo2 & 0xFFFFu), s1 = __uint_as_float(lo2 & 0xFFFF0000u);
            const float s2 = bf16_to_f32(hi2 & 0xFFFFu), s3 = __uint_as_float(hi2 & 0xFFFF0000u);
#pragma unroll
            for (int rb = 0; rb < MB; ++rb) {
              acc[j][rb][0] = fmaf(s0, t[j][rb][0], acc[j][rb][0]);
              acc[j][rb][1] = fmaf(s1, t[j][rb][1], acc[j][rb][1]);
              acc[j][rb][2] = fmaf(s2, t[j][rb][2], acc[j][rb][2]);
              acc[j][rb][3] = fmaf(s3, t[j][rb][3], acc[j][rb][3]);
            }
          }
        } else {
          // INT4 codes enter the MFMA exactly: u - z (zero-point format) or
          // q / 16 (symmetric), so the per-group chain holds sum x (u - z)
          // (or sum x q / 16) with fp32 rounding relative to sum |x w|; the
          // group scale of each of the lane's four output rows multiplies
          // the chain's result once, and the symmetric factor 16 is applied
          // in the epilogue (exact).
          uint32_t zc[ZP ? NBW : 1];
#pragma unroll
          for (int j = 0; j < (ZP ? NBW : 1); ++j) {
            const uint32_t z = ZP ? ((wzr[ZP ? d : 0][ZP ? j : 0] >> zshift) & 0xFu) : 8u;
            zc[j] = 0x80808080u - z * 0x01010101u;
          }
          f32x4_t t[NBW][MB];
#pragma unroll
          for (int kk = 0; kk < 4; ++kk) {
            u32x4_t af[MB];
#pragma unroll
            for (int rb = 0; rb < MB; ++rb) af[rb] = ld16(xg + lrow[rb] * xb + (32 * kk + 8 * q_l) * 2);
#pragma unroll
            for (int j = 0; j < NBW; ++j) {
              const u32x4_t bw = ZP ? dz8_u4(wq[d][j][kk], zc[ZP ? j : 0]) : dq8_sym16(wq[d][j][kk]);
#pragma unroll
              for (int rb = 0; rb < MB; ++rb)
                t[j][rb] = mfma_bf16(bw, af[rb], kk == 0 ? (f32x4_t){0.f, 0.f, 0.f, 0.f} : t[j][rb]);
            }
          }
#pragma unroll
          for (int j = 0; j < NBW; ++j) {
            const uint32_t lo2 = wsr[d][j], hi2 = wsh[MXW ? 0 : d][MXW ? 0 : j];
            const float s0 = bf16_to_f32(lo2 & 0xFFFFu), s1 = __uint_as_float(lo2 & 0xFFFF0000u);
            const float s2 = bf16_to_f32(hi2 & 0xFFFFu), s3 = __uint_as_float(hi2 & 0xFFFF0000u);
#pragma unroll
            for (int rb = 0; rb < MB; ++rb) {
              acc[j][rb][0] = fmaf(s0, t[j][rb][0], acc[j][rb][0]);
              acc[j][rb][1] = fmaf(s1, t[j][rb][1], acc[j][rb][1]);
              acc[j][rb][2] = fmaf(s2, t[j][rb][2], acc[j][rb][2]);
              acc[j][rb][3] = fmaf(s3, t[j][rb][3], acc[j][rb][3]);
            }
          }
        }
      };
      // Every round but the last refills each slot right after its use (with
      // a repeat of the last group when the slice runs out), so each round
      // issues the same loads and the waits for the slots stay exact; the
      // last round refills nothing.
      int r = 0;
#pragma nounroll
      for (; r + 1 < rounds; ++r) {
#pragma unroll
        for (int d = 0; d < DW; ++d) {
          const int lg = r * DW + d;
          process(d, lg);
          load_w(d, gsafe + (lg + DW < last ? lg + DW : last));
        }
      }
      if (rounds > 0) {
#pragma unroll
        for (int d = 0; d < DW; ++d) {
          const int lg = r * DW + d;
          if (lg < sl) process(d, lg);
        }
      }
      // slots past a short slice were loaded but never used: let them land
      // here (a wait the compiler sees), so that the next piece's ring loads
      // do not wait behind its activation copies for them
      __builtin_amdgcn_s_waitcnt(0x0F70);             // vmcnt(0)
    }

    // ---- K-split sum: waves kq > 0 park their sums in LDS, wave kq == 0 adds them
    if (KS > 1) {
      f32x4_t* red = reinterpret_cast<f32x4_t*>(lds);
      if (kq > 0) {
#pragma unroll
        for (int j = 0; j < NBW; ++j)
#pragma unroll
          for (int rb = 0; rb < MB; ++rb) red[((wave * NBW + j) * MB + rb) * 64 + lane] = acc[j][rb];
      }
      lds_barrier();
      if (kq == 0) {
#pragma unroll
        for (int k2 = 1; k2 < KS; ++k2)
#pragma unroll
          for (int j = 0; j < NBW; ++j)
#pragma unroll
            for (int rb = 0; rb < MB; ++rb) acc[j][rb] += red[(((wave + k2) * NBW + j) * MB + rb) * 64 + lane];
      }
    }

    // ---- epilogue: lane holds C[n = 16nb + 4*q_l + r][row = 16rb + n_l]
    if (NBW == 2 && GROUPED && a.gated && kq == 0) {
      // gated layout: the wave's blocks nb0 (even) and nb0 + 1 are the gate
      // and up halves of output columns 8 nb0 + 4 q_l + r of [rows][N/2]
      if (nb0 < G.NB) {
        const int64_t n = nb0 * 8 + 4 * q_l;
#pragma unroll
        for (int rb = 0; rb < MB; ++rb) {
          const int rl = rb * 16 + n_l;
          if (rl >= rcount || orow_s[rl] < 0) continue;
          f32x4_t vg = acc[0][rb], vu = acc[NBW - 1][rb];
          if (MODE == KM_INT4_A16 && !ZP) {
            vg = vg * 16.f;
            vu = vu * 16.f;
          }
          if (MX) {
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
    } else if (kq == 0) {
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
          if (MODE == KM_INT4_A16 && !ZP) v = v * 16.f;   // symmetric sums carry a factor 1/16 (exact)
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


// LDS plan of one launch: K groups per activation piece and the row stride.
static void stream_lds_plan(const GemmArgs& a, const StreamCfg& c, bool grouped, int red_bytes,
                            int* pg_out, int* xb_out, size_t* bytes_out) {
  const bool a4 = kmode_of(a) == KM_MX_A4;
  const int64_t gb = (kmode_of(a) == KM_MX_A8) ? 128 : (a4 ? 64 : 256);
  const int64_t rows = grouped ? 16 * c.mb : (a.M < 16 * c.mb ? a.M : 16 * c.mb);
  const int64_t ksl = grouped ? a.G.KG : a.ksg;         // groups one block walks
  const int64_t gq = 1024 / gb;                         // groups per 1 KiB of a row
  // largest piece (a multiple of gq groups) whose rows fit the budget
  const int64_t budget = (c.lds_kb > 0 && c.lds_kb * 1024 < kStreamLdsBudget) ? c.lds_kb * 1024 : kStreamLdsBudget;
  const int64_t avail = budget - red_bytes;
  // MXFP4 rows add 4 scale bytes per group (staged in 256-byte pieces)
  int64_t pg = a4 ? ((avail / rows - 16 - 256) / (1024 + 4 * gq)) * gq : ((avail / rows - 16) / 1024) * gq;
  if (pg < gq) pg = gq;
  const int64_t need = (ksl + gq - 1) / gq * gq;
  if (pg > need) pg = need;
  const int64_t xb = (pg * gb + 1023) / 1024 * 1024 + 16;
  const int64_t sb = a4 ? (pg + 63) / 64 * 256 : 0;
  *pg_out = (int)pg;
  *xb_out = (int)xb;
  *bytes_out = (size_t)(red_bytes + rows * (xb + sb));
}

template <int MODE, bool ZP, int MB, int NBW, int KS, bool GROUPED, int NW>
static hipError_t go_stream(const GemmArgs& a, const StreamCfg& c, int grid_items, hipStream_t st) {
  // ring depth in K groups, within the 63 outstanding vector-memory operations
  // one wave can track (up to three loads per group and column block) and a
  // register budget that leaves room for four waves per SIMD at small M
  constexpr int DW = (NBW == 1 && MB == 1 && KS < 4 && MODE != KM_INT8_A16) ? 16 : 8;
  constexpr int RED = StreamShape<NW, KS, NBW, MB>::kRedBytes;
  auto kern = &k_gemm_stream<MODE, ZP, MB, NBW, KS, DW, GROUPED, NW>;
  int pg, xb;
  size_t lds;
  stream_lds_plan(a, c, GROUPED, RED, &pg, &xb, &lds);
  // allow more than the default dynamic LDS (set once per instance; thread-safe static init)
  static const hipError_t attr_err = hipFuncSetAttribute(
      reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
      (int)kStreamLdsBudget);
  if (attr_err != hipSuccess) return attr_err;
  const int64_t n_tiles = stream_n_tiles(a.G, c);
  dim3 grid;
  if (GROUPED) {
    grid = dim3((unsigned)(grid_items > 0 ? grid_items : 1));
  } else {
    const int64_t m_chunks = (a.M + MB * 16 - 1) / (MB * 16);
    grid = dim3((unsigned)n_tiles, (unsigned)c.splits, (unsigned)m_chunks);
  }
  hipLaunchKernelGGL(kern, grid, dim3(64 * NW), lds, st, a, (int)n_tiles, pg, xb);
  return hipGetLastError();
}

template <int MODE, bool ZP, int MB, int NBW, bool GROUPED>
static hipError_t go_stream_ks(const GemmArgs& a, const StreamCfg& c, int gi, hipStream_t st) {
  if (!GROUPED && c.nw == 8) {
    // eight waves per block (dense only): K split over 2, 4 or 8 of them
    switch (c.ks) {
      case 8: return go_stream<MODE, ZP, MB, NBW, 8, GROUPED, 8>(a, c, gi, st);
      case 4: return go_stream<MODE, ZP, MB, NBW, 4, GROUPED, 8>(a, c, gi, st);
      default: return go_stream<MODE, ZP, MB, NBW, 2, GROUPED, 8>(a, c, gi, st);
    }
  }
  switch (c.ks) {
    case 4: return go_stream<MODE, ZP, MB, NBW, 4, GROUPED, 4>(a, c, gi, st);
    case 2: return go_stream<MODE, ZP, MB, NBW, 2, GROUPED, 4>(a, c, gi, st);
    default: return go_stream<MODE, ZP, MB, NBW, 1, GROUPED, 4>(a, c, gi, st);
  }
}

template <int MODE, bool ZP, int MB, bool GROUPED>
static hipError_t go_stream_nbw(const GemmArgs& a, const StreamCfg& c, int gi, hipStream_t st) {
  return (c.nbw == 2) ? go_stream_ks<MODE, ZP, MB, 2, GROUPED>(a, c, gi, st)
                      : go_stream_ks<MODE, ZP, MB, 1, GROUPED>(a, c, gi, st);
}

template <int MODE, bool ZP, bool GROUPED>
static hipError_t go_stream_mb(const GemmArgs& a, const StreamCfg& c, int gi, hipStream_t st) {
  return (c.mb == 1) ? go_stream_nbw<MODE, ZP, 1, GROUPED>(a, c, gi, st)
                     : go_stream_nbw<MODE, ZP, 2, GROUPED>(a, c, gi, st);
}

hipError_t launch_gemm_stream(const GemmArgs& a, const StreamCfg& c, bool grouped, int grid_items,
                              hipStream_t st) {
  const int mode = kmode_of(a);
  if (mode == KM_MX_A8)
    return grouped ? go_stream_mb<KM_MX_A8, false, true>(a, c, grid_items, st)
                   : go_stream_mb<KM_MX_A8, false, false>(a, c, grid_items, st);
  if (mode == KM_MX_A4)
    return grouped ? go_stream_mb<KM_MX_A4, false, true>(a, c, grid_items, st)
                   : go_stream_mb<KM_MX_A4, false, false>(a, c, grid_items, st);
  if (mode == KM_INT8_A16)
    return grouped ? go_stream_mb<KM_INT8_A16, false, true>(a, c, grid_items, st)
                   : go_stream_mb<KM_INT8_A16, false, false>(a, c, grid_items, st);
  if (mode == KM_MX_A16)
    return grouped ? go_stream_mb<KM_MX_A16, false, true>(a, c, grid_items, st)
                   : go_stream_mb<KM_MX_A16, false, false>(a, c, grid_items, st);
  if (mode == KM_MXI4_A16)
    return grouped ? go_stream_mb<KM_MXI4_A16, false, true>(a, c, grid_items, st)
                   : go_stream_mb<KM_MXI4_A16, false, false>(a, c, grid_items, st);
  if (a.wfmt == W_UINT4_ZP)
    return grouped ? go_stream_mb<KM_INT4_A16, true, true>(a, c, grid_items, st)
                   : go_stream_mb<KM_INT4_A16, true, false>(a, c, grid_items, st);
  return grouped ? go_stream_mb<KM_INT4_A16, false, true>(a, c, grid_items, st)
                 : go_stream_mb<KM_INT4_A16, false, false>(a, c, grid_items, st);
}

hipError_t launch_splitk_reduce(const GemmArgs& a, int splits, hipStream_t st) {
  const int64_t cnt = a.M * (a.G.NB * 16 / 4);
  int64_t blocks = (cnt + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(k_splitk_reduce, dim3((unsigned)blocks), dim3(256), 0, st, a, splits);
  return hipGetLastError();
}

}  // namespace hm
