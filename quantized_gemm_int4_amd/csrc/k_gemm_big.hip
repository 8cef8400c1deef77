// MFMA GEMM for many rows (prefill-sized M, and 256-row units of a grouped
// GEMM), where the ~2*M*N*K matrix multiply dominates (ywsung.com note "How
// vLLM Humming computes 4 bits", section on one token vs many tokens).
//
// One block computes a 256 x 256 output tile.  Activations reach LDS through
// 16-byte direct global-to-LDS loads laid out in MFMA fragment order (lane L
// of a 1 KiB fragment at byte 16 L), so every operand read is one
// conflict-free 1 KiB sweep.  Three LDS stages: copies run two K steps ahead.
//   * W4A16 (K step 64, eight waves, two per SIMD): each wave owns 128 rows x
//     64 columns as 32x32x16 bf16 MFMA blocks (128 accumulators per lane) and
//     unpacks its columns' weights, copied into LDS one step ahead of the
//     activations, to bf16 s * (u - z) after its MFMAs of the step, while the
//     other wave of the SIMD multiplies.
//   * W4A8-MXFP4 (K step 128, eight waves of 64 x 128): E2M1 weight tiles and
//     their E8M0 scale words are copied to LDS too and fed as stored to the
//     16x16x128 scaled MFMA; the per-token FP8 scale is applied in the
//     epilogue.
// Dense tiles are assigned XCD by XCD: blocks are dispatched round-robin over
// the eight XCDs, so block b runs on XCD b % 8; each XCD gets a contiguous
// range of tiles, visited in groups of four tile rows, so the blocks that
// share an XCD's L2 also share activation and weight slices.
#include <algorithm>
#include <type_traits>

#include "common.h"
#include "launch.h"

namespace hm {

namespace {

typedef __attribute__((address_space(3))) void lds_void_t;

__device__ __forceinline__ void g2lds(const void* src, uint8_t* lds_base) {
  __builtin_amdgcn_global_load_lds(src, (lds_void_t*)lds_base, 16, 0, 0);
}

// Four consecutive outputs y[n..n+3] of one row as bf16 (one 8-byte store when aligned).
__device__ __forceinline__ void store_bf16x4(uint16_t* yrow, int64_t N, int64_t n, f32x4_t v) {
  if ((N & 3) == 0 && n + 3 < N) {
    *reinterpret_cast<u32x2_t*>(yrow + n) = (u32x2_t){pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3])};
  } else {
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (n + r < N) yrow[n + r] = (uint16_t)(pack_bf16(v[r], 0.0f) & 0xFFFF);
  }
}

__device__ __forceinline__ float ubyte_f(uint32_t x, int b) { return (float)((x >> (8 * b)) & 0xFFu); }

// Eight codes of one device-layout word (value 2p in nibble p, 2p+1 in nibble
// p+4) -> eight bf16 of s*u + zs (= s*(u - z), exact before the bf16 rounding)
// in value order.
__device__ __forceinline__ u32x4_t dq8_bytes(uint32_t w, float s, float zs) {
  const uint32_t lo = w & 0x0F0F0F0Fu;          // bytes: v0 v4 v1 v5
  const uint32_t hi = (w >> 4) & 0x0F0F0F0Fu;   // bytes: v2 v6 v3 v7
  u32x4_t r;
  r[0] = pack_bf16(fmaf(ubyte_f(lo, 0), s, zs), fmaf(ubyte_f(lo, 2), s, zs));
  r[1] = pack_bf16(fmaf(ubyte_f(hi, 0), s, zs), fmaf(ubyte_f(hi, 2), s, zs));
  r[2] = pack_bf16(fmaf(ubyte_f(lo, 1), s, zs), fmaf(ubyte_f(lo, 3), s, zs));
  r[3] = pack_bf16(fmaf(ubyte_f(hi, 1), s, zs), fmaf(ubyte_f(hi, 3), s, zs));
  return r;
}

}  // namespace

constexpr int kBigM = 256;        // rows per block
constexpr int kBigCB = 16;        // 16-column blocks per block (256 columns)
constexpr int kBigStages = 3;     // LDS stages: loads run two K steps ahead

// LDS bytes of one stage: activation fragments (32 x 1 KiB) and the block's
// 16 weight tiles (16 KiB), plus MXFP4: their E8M0 scale words (16 x 256 B);
// INT4: per wave 256 B of bf16 scales and 256 B of zero-point words.
__host__ __device__ constexpr int big_stage_bytes(bool mx) { return mx ? (32 + 16 + 4) * 1024 : (32 + 16 + 2) * 1024; }
__host__ __device__ constexpr int big_lds_bytes(bool mx) { return kBigStages * big_stage_bytes(mx); }

// Dense: one block per 256 x 256 tile.  Grouped (MoE): a persistent grid
// walks (unit, 256-column tile) items; a unit is up to 256 rows of one
// expert, whose activation rows are gathered through the sorted pair list
// and whose outputs are written in pair order.
template <bool MX, bool ZP, bool GROUPED>
__global__ void __launch_bounds__(512, 1)
k_gemm_big(GemmArgs a, int tiles_n, int tiles_m) {
  constexpr int SB = big_stage_bytes(MX);
  extern __shared__ __attribute__((aligned(1024))) uint8_t lds[];
  __shared__ int64_t arow_s[GROUPED ? kBigM : 1];
  __shared__ int64_t orow_s[GROUPED ? kBigM : 1];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n_l = lane & 15, q_l = lane >> 4;
  const Geom G = a.G;
  const int64_t K = G.K;
  const int64_t row_bytes = MX ? K : 2 * K;

  const int64_t n_items = GROUPED ? (int64_t)a.hdr[2] * tiles_n : 1;
  for (int64_t item = GROUPED ? blockIdx.x : 0; item < n_items; item += GROUPED ? gridDim.x : 1) {
    int64_t e = 0, m0 = 0, nb0;
    int64_t rows_left;                               // valid rows of this tile (>= 1)
    if (GROUPED) {
      const int32_t* u = a.units + 4 * (item / tiles_n);
      e = u[0];
      rows_left = u[2] < kBigM ? u[2] : kBigM;
      nb0 = (item % tiles_n) * kBigCB;
      if (tid < kBigM) {
        int64_t ar = 0, orr = -1;   // invalid rows read row 0 (always present) and are not stored
        if (tid < rows_left) {
          const int64_t pair = a.sorted_pairs[u[1] + tid];
          if (pair >= 0 && pair < a.P) {
            orr = pair;
            ar = a.rows_are_pairs ? pair : pair / a.topk;
          }
        }
        arow_s[tid] = ar;
        orow_s[tid] = orr;
      }
      __syncthreads();
    } else {
      // tile of this block (XCD-aware order, see the file comment)
      const int total = tiles_n * tiles_m;
      const int xcd = blockIdx.x % 8, idx = blockIdx.x / 8;
      const int base = total / 8, extra = total % 8;
      const int t = xcd * base + (xcd < extra ? xcd : extra) + idx;
      constexpr int GM = 4;
      const int grp = t / (GM * tiles_n);
      const int first_m = grp * GM;
      const int gm = (tiles_m - first_m) < GM ? (tiles_m - first_m) : GM;
      const int tin = t - grp * GM * tiles_n;
      const int tm = first_m + tin % gm, tn = tin / gm;
      m0 = (int64_t)tm * kBigM;
      nb0 = (int64_t)tn * kBigCB;
      rows_left = a.M - m0;
    }
    // activation bytes: dense offsets are relative to the tile's first row,
    // grouped offsets to the start of A (the launcher checks they fit 32 bits)
    const uint8_t* xblk = reinterpret_cast<const uint8_t*>(a.x) + m0 * row_bytes;
    auto xrow = [&](int64_t r) -> uint32_t {         // local row -> byte offset from xblk
      if (r >= rows_left) r = rows_left - 1;         // rows past the tile's end load a valid row, never stored
      return (uint32_t)((GROUPED ? arow_s[r] : r) * row_bytes);
    };
    auto out_row = [&](int64_t r) -> int64_t {       // local row -> output row, or -1
      if (r >= rows_left) return -1;
      return GROUPED ? orow_s[r] : m0 + r;
    };
    auto in_row = [&](int64_t r) -> int64_t {        // local row -> activation row (for the A8 scale)
      return GROUPED ? arow_s[r] : m0 + r;
    };
    const int64_t wbase = e * G.NB;                  // first column block of this expert
    auto barrier_after = [&](bool exact, auto n_c) {
      // wait for this wave's copies into the next stage (all but the n most
      // recent vector-memory operations) and its LDS operations, then meet the
      // other waves; the memory clobber keeps the compiler from moving LDS
      // accesses across
      constexpr int n = decltype(n_c)::value;
      if (exact) __asm__ volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(n) : "memory");
      else __asm__ volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    };

    if constexpr (MX) {
      // ================================ W4A8-MXFP4: K step 128 = one K group;
      // eight waves, two per SIMD: wave w owns rows 64 (w & 3) + 0..63 and
      // columns 128 (w >> 2) + 0..127 (4 x 8 blocks of 16 x 16, 128
      // accumulators per lane)
      const int wm = wave & 3, wn = wave >> 2;
      f32x4_t acc[8][4];
#pragma unroll
      for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[j][i] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
      // activation fragments this thread copies: fragment f = w + 8 i (i = 0..3)
      // covers row block f >> 1 and the 16-byte halves at 16 q_l (f even) or
      // 64 + 16 q_l (f odd) of a 128-K step
      uint32_t xoff[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int f = wave + 8 * i;
        xoff[i] = xrow((f >> 1) * 16 + n_l) + 16 * q_l + 64 * (f & 1);
      }
      auto copy_x = [&](int64_t step, uint8_t* stage) {
        const uint8_t* src = xblk + step * 128;   // 128 fp8 per K step
#pragma unroll
        for (int i = 0; i < 4; ++i) g2lds(src + xoff[i], stage + (wave + 8 * i) * 1024);
      };
      // weight tiles and scale words this wave copies per stage: column blocks w and w + 8
      const uint8_t* wsrc[2];
      const uint8_t* ssrc[2];
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        int64_t nb = nb0 + wave + 8 * c;
        if (nb >= G.NB) nb = G.NB - 1;
        wsrc[c] = a.w + (wbase + nb) * G.KG * 1024 + lane * 16;
        ssrc[c] = a.w + G.off_scales + (wbase + nb) * G.KG4 * 256 + lane * 4;
      }
      auto copy_stage = [&](int64_t s, uint8_t* st) {
        copy_x(s, st);
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          const int cb = wave + 8 * c;
          g2lds(wsrc[c] + s * 1024, st + 32 * 1024 + cb * 1024);
          __builtin_amdgcn_global_load_lds(ssrc[c] + (s / 4) * 256, (lds_void_t*)(st + 48 * 1024 + cb * 256), 4, 0, 0);
        }
      };
      constexpr int kPer = 8;                         // copies per wave per stage
      const int64_t S = G.KG;
      copy_stage(0, lds);
      if (S > 1) copy_stage(1, lds + SB);
      barrier_after(S > 1, std::integral_constant<int, kPer>());
#pragma nounroll
      for (int64_t s = 0; s < S; ++s) {
        const uint8_t* st = lds + (s % kBigStages) * SB;
        const bool issue = s + 2 < S;
        if (issue) copy_stage(s + 2, lds + ((s + 2) % kBigStages) * SB);
        const int sh = 8 * (int)(s & 3);
        u32x4_t wq[8];
        int wsc[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int cb = wn * 8 + j;
          wq[j] = ld16(st + 32 * 1024 + cb * 1024 + lane * 16);
          wsc[j] = (int)((*reinterpret_cast<const uint32_t*>(st + 48 * 1024 + cb * 256 + lane * 4) >> sh) & 0xFF);
        }
        u32x4_t b0[4], b1[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int rb = wm * 4 + i;
          b0[i] = ld16(st + (rb * 2 + 0) * 1024 + lane * 16);
          b1[i] = ld16(st + (rb * 2 + 1) * 1024 + lane * 16);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 8; ++j) acc[j][i] = mfma_fp4_fp8(wq[j], b0[i], b1[i], acc[j][i], wsc[j], 127);
        // the next stage was issued one step ago, this step's copies after it
        barrier_after(issue, std::integral_constant<int, kPer>());
      }

      // ---- epilogue: lane holds C[n = 16 nb + 4 q_l + r][row = 16 rb + n_l]
      __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");   // no copy may land after the stages are reused
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t lr = (wm * 4 + i) * 16 + n_l;
        const int64_t row = out_row(lr);
        if (row < 0) continue;
        const float rs = a.xs[in_row(lr)];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int64_t nb = nb0 + wn * 8 + j;
          if (nb >= G.NB) continue;
          store_bf16x4(a.y + row * G.N, G.N, nb * 16 + 4 * q_l, acc[j][i] * rs);
        }
      }
    } else {
      // ================================ W4A16: K step 64 = half a K group;
      // eight waves, two per SIMD: wave w owns rows 128 (w & 1) + 0..127 and
      // columns 64 (w >> 1) + 0..63 as 2 x 4 blocks of 32 x 32
      // (v_mfma_f32_32x32x16_bf16; unlike the 16x16x32 form it keeps the
      // matrix core busy).  Each wave unpacks the weights of its 64 columns
      // into MFMA operands after its MFMAs of the step; the other wave on the
      // SIMD multiplies meanwhile.  32x32x16 operands: A row / B column =
      // lane % 32, K = 8 (lane / 32) + 0..7; result: column lane % 32, rows
      // 8 j + 4 (lane / 32) + r in register 4 j + r.
      const int wm = wave & 1, wn = wave >> 1;
      f32x16_t acc[2][4];
#pragma unroll
      for (int nb2 = 0; nb2 < 2; ++nb2)
#pragma unroll
        for (int mb = 0; mb < 4; ++mb)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[nb2][mb][r] = 0.f;
      const int l32 = lane & 31, hi = lane >> 5;
      // activation fragments: fragment f = 4 mb + kq (row block of 32, K part
      // of 16); wave w copies K part w & 3 of row blocks 4 (w >> 2) + 0..3
      uint32_t xoff[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int mb = 4 * (wave >> 2) + i;
        xoff[i] = xrow(mb * 32 + l32) + 2 * (16 * (wave & 3) + 8 * hi);
      }
      auto copy_x = [&](int64_t step, uint8_t* stg) {
        const uint8_t* src = xblk + step * 128;     // 64 bf16 per K step
#pragma unroll
        for (int i = 0; i < 4; ++i)
          g2lds(src + xoff[i], stg + ((4 * (wave >> 2) + i) * 4 + (wave & 3)) * 1024);
      };
      // Weight tiles of the block's 16 column blocks: wave w copies tiles
      // 4 wn + 2 wm + {0, 1}; wave wm = 0 also copies its column quarter's
      // bf16 scales (lane L: tile L / 8 of the quarter, bytes 4 (L % 8)), wave
      // wm = 1 the zero-point words (lane L: tile (L / 2) % 4, word L % 2).
      // Lanes past the useful ones repeat in-range addresses into unused bytes.
      const uint8_t* wsrc[2];
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        int64_t nb = nb0 + 4 * wn + 2 * wm + c;
        if (nb >= G.NB) nb = G.NB - 1;
        wsrc[c] = a.w + (wbase + nb) * G.KG * 1024 + lane * 16;
      }
      const int sz_c = wm == 0 ? ((lane >> 3) & 3) : ((lane >> 1) & 3);
      int64_t nbq = nb0 + 4 * wn + sz_c;
      if (nbq >= G.NB) nbq = G.NB - 1;
      const uint8_t* szsrc = wm == 0 ? a.w + G.off_scales + (wbase + nbq) * G.KG * 32 + (lane & 7) * 4
                                     : a.w + G.off_zeros + (wbase + nbq) * G.KG * 8 + (lane & 1) * 4;
      const int64_t szstride = wm == 0 ? 32 : 8;
      constexpr int kWOff = 32 * 1024, kSOff = 48 * 1024, kZOff = 49 * 1024;
      // weights of K step s (group s / 2) into the weight part of stage s % 3
      auto copy_w = [&](int64_t s, uint8_t* stg) {
        const int64_t g = s >> 1;
#pragma unroll
        for (int c = 0; c < 2; ++c) g2lds(wsrc[c] + g * 1024, stg + kWOff + (4 * wn + 2 * wm + c) * 1024);
        if (wm == 0 || ZP)
          __builtin_amdgcn_global_load_lds(szsrc + g * szstride,
                                           (lds_void_t*)(stg + (wm == 0 ? kSOff : kZOff) + wn * 256), 4, 0, 0);
      };
      // copies per wave per step: 4 + 2 + 1, except the zero-point copy is
      // missing for symmetric weights on waves wm = 1; the wait below uses the
      // smaller count (waiting for one more copy than needed is harmless)
      constexpr int kPer = 4 + 2 + (ZP ? 1 : 0);
      // A operands of one step: 32-column block nb2, K part kq.  Lane row n =
      // 32 nb2 + l32 of the quarter lies in tile 4 wn + 2 nb2 + l32 / 16 at
      // column l32 % 16; K = 64 h + 16 kq + 8 hi is word 2 h + kq / 2 of slot
      // (l32 % 16) + 16 ((2 kq + hi) % 4) of that tile.
      u32x4_t af[2][4];
      auto unpack_from = [&](const uint8_t* stg, int h) {
#pragma unroll
        for (int nb2 = 0; nb2 < 2; ++nb2) {
          const int c = 2 * nb2 + (l32 >> 4), c16 = l32 & 15;
          const uint8_t* tile = stg + kWOff + (4 * wn + c) * 1024;
          const float sv = bf16_to_f32(*reinterpret_cast<const uint16_t*>(stg + kSOff + wn * 256 + c * 32 + c16 * 2));
          const uint32_t zw = ZP ? *reinterpret_cast<const uint32_t*>(stg + kZOff + wn * 256 + c * 8 + (c16 >> 3) * 4) : 0u;
          const float z = ZP ? (float)((zw >> (4 * (c16 & 7))) & 0xFu) : 8.0f;
          const float zs = -z * sv;
#pragma unroll
          for (int kq = 0; kq < 4; ++kq) {
            const int slot = c16 + 16 * ((2 * kq + hi) & 3);
            const uint32_t w = *reinterpret_cast<const uint32_t*>(tile + slot * 16 + 4 * (2 * h + (kq >> 1)));
            af[nb2][kq] = dq8_bytes(w, sv, zs);
          }
        }
      };
      const int64_t S = 2 * G.KG;
      auto stage = [&](int64_t s) { return lds + (s % kBigStages) * SB; };
      // prologue: weights of steps 0, 1, 2 and activations of steps 0, 1 (their
      // stages), operands of step 0
      copy_w(0, stage(0));
      copy_w(std::min<int64_t>(1, S - 1), stage(1));
      copy_w(std::min<int64_t>(2, S - 1), stage(2));
      copy_x(0, stage(0));
      copy_x(std::min<int64_t>(1, S - 1), stage(1));
      __syncthreads();
      unpack_from(stage(0), 0);
      // Step s multiplies stage s % 3 with operands af, then unpacks the
      // operands of step s + 1 from stage s + 1.  It first issues the
      // activations of step s + 2 and the weights of step s + 3.  No branches:
      // near the end the copies repeat the last step into parts no longer read,
      // so every step issues the same copies and the wait count is exact.
#pragma nounroll
      for (int64_t s = 0; s < S; ++s) {
        copy_x(std::min<int64_t>(s + 2, S - 1), stage(s + 2));
        copy_w(std::min<int64_t>(s + 3, S - 1), stage(s + 3));
        const uint8_t* stg = stage(s);
        // each accumulator takes its four K parts back to back (clustered
        // updates keep the register allocation in place)
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
          const uint8_t* fr = stg + ((4 * wm + mb) * 4) * 1024 + lane * 16;
          u32x4_t b[4];
#pragma unroll
          for (int kq = 0; kq < 4; ++kq) b[kq] = ld16(fr + kq * 1024);
#pragma unroll
          for (int kq = 0; kq < 4; ++kq)
#pragma unroll
            for (int nb2 = 0; nb2 < 2; ++nb2) acc[nb2][mb] = mfma32_bf16(af[nb2][kq], b[kq], acc[nb2][mb]);
        }
        unpack_from(stage(s + 1), (int)((s + 1) & 1));
        // stage s + 1 (activations) came one step earlier, weights two; after
        // them only this step's copies
        __asm__ volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(kPer) : "memory");
      }

      // ---- epilogue: lane holds C[n = 64 wn + 32 nb2 + 8 j + 4 hi + r][row = 128 wm + 32 mb + l32]
      __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");   // no copy may land after the stages are reused
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
        const int64_t row = out_row(128 * wm + mb * 32 + l32);
        if (row < 0) continue;
#pragma unroll
        for (int nb2 = 0; nb2 < 2; ++nb2)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const f32x4_t v = {acc[nb2][mb][4 * j], acc[nb2][mb][4 * j + 1], acc[nb2][mb][4 * j + 2], acc[nb2][mb][4 * j + 3]};
            store_bf16x4(a.y + row * G.N, G.N, nb0 * 16 + wn * 64 + nb2 * 32 + 8 * j + 4 * hi, v);
          }
      }
    }
    __syncthreads();  // row tables and LDS stages are reused by the next item
  }
}

template <bool MX, bool ZP, bool GROUPED>
static hipError_t go_big(const GemmArgs& a, int grid_items, hipStream_t st) {
  auto kern = &k_gemm_big<MX, ZP, GROUPED>;
  static const hipError_t attr_err = hipFuncSetAttribute(
      reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize, big_lds_bytes(MX));
  if (attr_err != hipSuccess) return attr_err;
  const int tiles_n = (int)((a.G.NB + kBigCB - 1) / kBigCB);
  const int tiles_m = GROUPED ? 0 : (int)((a.M + kBigM - 1) / kBigM);
  const unsigned grid = GROUPED ? (unsigned)(grid_items > 0 ? grid_items : 1) : (unsigned)(tiles_n * tiles_m);
  hipLaunchKernelGGL(kern, dim3(grid), dim3(512), big_lds_bytes(MX), st, a, tiles_n, tiles_m);
  return hipGetLastError();
}

int64_t big_n_tiles(const Geom& G) { return (G.NB + kBigCB - 1) / kBigCB; }

hipError_t launch_gemm_big(const GemmArgs& a, bool grouped, int grid_items, hipStream_t st) {
  if (a.wfmt == W_MXFP4)
    return grouped ? go_big<true, false, true>(a, grid_items, st) : go_big<true, false, false>(a, 0, st);
  if (a.wfmt == W_UINT4_ZP)
    return grouped ? go_big<false, true, true>(a, grid_items, st) : go_big<false, true, false>(a, 0, st);
  return grouped ? go_big<false, false, true>(a, grid_items, st) : go_big<false, false, false>(a, 0, st);
}

}  // namespace hm
