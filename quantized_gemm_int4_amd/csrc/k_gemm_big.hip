// MFMA GEMM for many rows (prefill-sized M), where the ~2*M*N*K matrix
// multiply dominates (ywsung.com note "How vLLM Humming computes 4 bits",
// section on one token vs many tokens).
//
// One 256-thread block computes a 256 x 256 output tile; each of its four
// waves owns 128 x 128 (8 x 8 MFMA blocks of 16 x 16, 256 fp32 accumulators
// per lane), which halves the LDS operand traffic per MFMA compared with
// 64 x 64 wave tiles.  Activations reach LDS through 16-byte direct
// global-to-LDS loads laid out in MFMA fragment order (lane L of a 1 KiB
// fragment at byte 16 L), so every operand read is one conflict-free 1 KiB
// sweep.  Two LDS stages: the loads of step s+1 fly while step s multiplies.
//   * W4A16 (K step 64): the block's threads unpack the next step's weights
//     to bf16 s * (u - z) between the MFMAs of the current step and write them
//     to LDS in fragment order.  Codes, scales and zero points of a K group are
//     fetched one step before their first use.
//   * W4A8-MXFP4 (K step 128): each wave loads its E2M1 weight tiles straight
//     into registers (they are already the A operand of the 16x16x128 scaled
//     MFMA) and passes their E8M0 scales; the per-token FP8 scale is applied
//     in the epilogue.
// Tiles are assigned XCD by XCD: blocks are dispatched round-robin over the
// eight XCDs, so block b runs on XCD b % 8; each XCD gets a contiguous range
// of tiles, visited in groups of four tile rows, so the blocks that share an
// XCD's L2 also share activation and weight slices.
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
__global__ void __launch_bounds__(256, 1)
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
      {
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
      // waves 2 x 2, each 128 rows x 128 columns (8 x 8 MFMA blocks)
      f32x4_t acc[8][8];
  #pragma unroll
      for (int j = 0; j < 8; ++j)
  #pragma unroll
        for (int i = 0; i < 8; ++i) acc[j][i] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
      // activation fragments this thread copies: fragment f = w + 4 i (i = 0..7)
      // covers row block f >> 1 and the 16-byte halves at 16 q_l (f even) or
      // 64 + 16 q_l (f odd) of a 128-K step.  Offsets are 32-bit from the block's
      // first row (256 rows of at most K bytes each).
      uint32_t xoff[8];
  #pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int f = wave + 4 * i;
        xoff[i] = xrow((f >> 1) * 16 + n_l) + 16 * q_l + 64 * (f & 1);
      }
      auto copy_x = [&](int64_t step, uint8_t* stage) {
        const uint8_t* src = xblk + step * 128;   // 128 fp8 per K step
  #pragma unroll
        for (int i = 0; i < 8; ++i) g2lds(src + xoff[i], stage + (wave + 4 * i) * 1024);
      };
      const int wm = wave >> 1, wn = wave & 1;
      // weight tiles and scale words this wave copies per stage: column blocks wave + 4 c
      const uint8_t* wsrc[4];
      const uint8_t* ssrc[4];
  #pragma unroll
      for (int c = 0; c < 4; ++c) {
        int64_t nb = nb0 + wave + 4 * c;
        if (nb >= G.NB) nb = G.NB - 1;
        wsrc[c] = a.w + (wbase + nb) * G.KG * 1024 + lane * 16;
        ssrc[c] = a.w + G.off_scales + (wbase + nb) * G.KG4 * 256 + lane * 4;
      }
      auto copy_stage = [&](int64_t s, uint8_t* st) {
        copy_x(s, st);
  #pragma unroll
        for (int c = 0; c < 4; ++c) {
          const int cb = wave + 4 * c;
          g2lds(wsrc[c] + s * 1024, st + 32 * 1024 + cb * 1024);
          __builtin_amdgcn_global_load_lds(ssrc[c] + (s / 4) * 256, (lds_void_t*)(st + 48 * 1024 + cb * 256), 4, 0, 0);
        }
      };
      constexpr int kPer = 16;                        // copies per wave per stage
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
        // B fragments of row block i, read one row block ahead
        u32x4_t b0 = ld16(st + (wm * 8 * 2 + 0) * 1024 + lane * 16);
        u32x4_t b1 = ld16(st + (wm * 8 * 2 + 1) * 1024 + lane * 16);
  #pragma unroll
        for (int i = 0; i < 8; ++i) {
          u32x4_t n0 = b0, n1 = b1;
          if (i + 1 < 8) {
            const int rb = wm * 8 + i + 1;
            n0 = ld16(st + (rb * 2 + 0) * 1024 + lane * 16);
            n1 = ld16(st + (rb * 2 + 1) * 1024 + lane * 16);
          }
  #pragma unroll
          for (int j = 0; j < 8; ++j) acc[j][i] = mfma_fp4_fp8(wq[j], b0, b1, acc[j][i], wsc[j], 127);
          b0 = n0;
          b1 = n1;
        }
        // the next stage was issued one step ago, this step's copies after it
        barrier_after(issue, std::integral_constant<int, kPer>());
      }

      // ---- epilogue: lane holds C[n = 16 nb + 4 q_l + r][row = 16 rb + n_l]
      __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");   // no copy may land after the stages are reused
  #pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int64_t lr = (wm * 8 + i) * 16 + n_l;
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
      // wave w owns columns 64w..64w+63 for all 256 rows as 2 x 8 blocks of
      // 32 x 32 (v_mfma_f32_32x32x16_bf16: unlike the 16x16x32 form, one wave
      // per SIMD keeps the matrix core busy), and unpacks its own weights into
      // MFMA operands.  32x32x16 operands: A row / B column = lane % 32, K =
      // 8 (lane / 32) + 0..7; result: column lane % 32, rows 8 j + 4 (lane / 32) + r
      // in register 4 j + r.
      f32x16_t acc[2][8];
  #pragma unroll
      for (int nb2 = 0; nb2 < 2; ++nb2)
  #pragma unroll
        for (int mb = 0; mb < 8; ++mb)
  #pragma unroll
          for (int r = 0; r < 16; ++r) acc[nb2][mb][r] = 0.f;
      const int l32 = lane & 31, hi = lane >> 5;
      // activation fragments: fragment f = 4 mb + kq (row block of 32, K part of
      // 16); wave w copies kq = w for mb = 0..7
      uint32_t xoff[8];
  #pragma unroll
      for (int mb = 0; mb < 8; ++mb) {
        xoff[mb] = xrow(mb * 32 + l32) + 2 * (16 * wave + 8 * hi);
      }
      auto copy_x = [&](int64_t step, uint8_t* stg) {
        const uint8_t* src = xblk + step * 128;     // 64 bf16 per K step
  #pragma unroll
        for (int mb = 0; mb < 8; ++mb) g2lds(src + xoff[mb], stg + (mb * 4 + wave) * 1024);
      };
      // This wave's four weight tiles per K group, copied to LDS with their
      // scales and zero points: one 1 KiB tile per copy; one 4-byte-per-lane
      // copy for the 4 x 32 B of bf16 scales (lane L: tile L / 8, bytes 4 (L % 8));
      // one for the 4 x 8 B of zero-point words (lane L: tile (L / 2) % 4, word L % 2).
      // Lanes past the useful ones repeat in-range addresses into unused bytes.
      const uint8_t* wsrc[4];
  #pragma unroll
      for (int c = 0; c < 4; ++c) {
        int64_t nb = nb0 + wave * 4 + c;
        if (nb >= G.NB) nb = G.NB - 1;
        wsrc[c] = a.w + (wbase + nb) * G.KG * 1024 + lane * 16;
      }
      const int sc_c = (lane >> 3) & 3, zc_c = (lane >> 1) & 3;
      int64_t nbs = nb0 + wave * 4 + sc_c, nbz = nb0 + wave * 4 + zc_c;
      if (nbs >= G.NB) nbs = G.NB - 1;
      if (nbz >= G.NB) nbz = G.NB - 1;
      const uint8_t* ssrc = a.w + G.off_scales + (wbase + nbs) * G.KG * 32 + (lane & 7) * 4;
      const uint8_t* zsrc = a.w + G.off_zeros + (wbase + nbz) * G.KG * 8 + (lane & 1) * 4;
      constexpr int kWOff = 32 * 1024, kSOff = 48 * 1024, kZOff = 49 * 1024;
      // weights of K step s (group s / 2) into the weight part of stage s % 3
      auto copy_w = [&](int64_t s, uint8_t* stg) {
        const int64_t g = s >> 1;
  #pragma unroll
        for (int c = 0; c < 4; ++c) g2lds(wsrc[c] + g * 1024, stg + kWOff + (wave * 4 + c) * 1024);
        __builtin_amdgcn_global_load_lds(ssrc + g * 32, (lds_void_t*)(stg + kSOff + wave * 256), 4, 0, 0);
        if (ZP) __builtin_amdgcn_global_load_lds(zsrc + g * 8, (lds_void_t*)(stg + kZOff + wave * 256), 4, 0, 0);
      };
      constexpr int kPer = 8 + 4 + 1 + (ZP ? 1 : 0);    // copies per wave per step
      // A operands of the current step (af) and the next (an): 32-column block
      // nb2, K part kq.  Lane row n = 32 nb2 + l32 lies in tile 2 nb2 + l32 / 16
      // at column l32 % 16; K = 64 h + 16 kq + 8 hi is word 2 h + kq / 2 of slot
      // (l32 % 16) + 16 ((2 kq + hi) % 4) of that tile.
      u32x4_t af[2][4], an[2][4];
      auto unpack_from = [&](const uint8_t* stg, int h, auto out_c, int part) {
        constexpr int o = decltype(out_c)::value;
        // part = -1: all operands; part = 0..3: column block part >> 1, K parts
        // 2 (part & 1) and 2 (part & 1) + 1
  #pragma unroll
        for (int nb2 = 0; nb2 < 2; ++nb2) {
          if (part >= 0 && nb2 != (part >> 1)) continue;
          const int c = 2 * nb2 + (l32 >> 4), c16 = l32 & 15;
          const uint8_t* tile = stg + kWOff + (wave * 4 + c) * 1024;
          const float sv = bf16_to_f32(*reinterpret_cast<const uint16_t*>(stg + kSOff + wave * 256 + c * 32 + c16 * 2));
          const uint32_t zw = ZP ? *reinterpret_cast<const uint32_t*>(stg + kZOff + wave * 256 + c * 8 + (c16 >> 3) * 4) : 0u;
          const float z = ZP ? (float)((zw >> (4 * (c16 & 7))) & 0xFu) : 8.0f;
          const float zs = -z * sv;
  #pragma unroll
          for (int kq = 0; kq < 4; ++kq) {
            if (part >= 0 && (kq >> 1) != (part & 1)) continue;
            const int slot = c16 + 16 * ((2 * kq + hi) & 3);
            const uint32_t w = *reinterpret_cast<const uint32_t*>(tile + slot * 16 + 4 * (2 * h + (kq >> 1)));
            if (o == 0) af[nb2][kq] = dq8_bytes(w, sv, zs);
            else an[nb2][kq] = dq8_bytes(w, sv, zs);
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
      unpack_from(stage(0), 0, std::integral_constant<int, 0>(), -1);
      // Step s multiplies stage s % 3 with operands af.  It first issues the
      // activations of step s + 2 and the weights of step s + 3 (weights run one
      // step further ahead: the operands of step s + 1 are unpacked from stage
      // s + 1 during step s, between the MFMAs).  No branches: near the end the
      // copies repeat the last step into parts no longer read, so every step
      // issues the same copies and the wait count is exact.
  #pragma nounroll
      for (int64_t s = 0; s < S; ++s) {
        const uint8_t* stg = stage(s);
        const uint8_t* nxt = stage(s + 1);
        const int hn = (int)((s + 1) & 1);
        // row blocks in pairs; the four K parts of a pair's accumulators run back
        // to back (clustered updates keep them in place), B fragments one K part ahead
  #pragma unroll
        for (int mp = 0; mp < 4; ++mp) {
          u32x4_t b0 = ld16(stg + ((2 * mp) * 4 + 0) * 1024 + lane * 16);
          u32x4_t b1 = ld16(stg + ((2 * mp + 1) * 4 + 0) * 1024 + lane * 16);
  #pragma unroll
          for (int kq = 0; kq < 4; ++kq) {
            u32x4_t n0 = b0, n1 = b1;
            if (kq + 1 < 4) {
              n0 = ld16(stg + ((2 * mp) * 4 + kq + 1) * 1024 + lane * 16);
              n1 = ld16(stg + ((2 * mp + 1) * 4 + kq + 1) * 1024 + lane * 16);
            }
  #pragma unroll
            for (int nb2 = 0; nb2 < 2; ++nb2) {
              acc[nb2][2 * mp] = mfma32_bf16(af[nb2][kq], b0, acc[nb2][2 * mp]);
              acc[nb2][2 * mp + 1] = mfma32_bf16(af[nb2][kq], b1, acc[nb2][2 * mp + 1]);
            }
            b0 = n0;
            b1 = n1;
          }
          if (mp == 0) copy_x(std::min<int64_t>(s + 2, S - 1), stage(s + 2));
          if (mp == 2) copy_w(std::min<int64_t>(s + 3, S - 1), stage(s + 3));
          unpack_from(nxt, hn, std::integral_constant<int, 1>(), mp);
        }
  #pragma unroll
        for (int nb2 = 0; nb2 < 2; ++nb2)
  #pragma unroll
          for (int kq = 0; kq < 4; ++kq) af[nb2][kq] = an[nb2][kq];
        // stage s + 1 (activations) came one step earlier, weights two; after
        // them only this step's copies
        __asm__ volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(kPer) : "memory");
      }

      // ---- epilogue: lane holds C[n = 64 w + 32 nb2 + 8 j + 4 hi + r][row = 32 mb + l32]
      __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");   // no copy may land after the stages are reused
  #pragma unroll
      for (int mb = 0; mb < 8; ++mb) {
        const int64_t row = out_row(mb * 32 + l32);
        if (row < 0) continue;
  #pragma unroll
        for (int nb2 = 0; nb2 < 2; ++nb2)
  #pragma unroll
          for (int j = 0; j < 4; ++j) {
            const f32x4_t v = {acc[nb2][mb][4 * j], acc[nb2][mb][4 * j + 1], acc[nb2][mb][4 * j + 2], acc[nb2][mb][4 * j + 3]};
            store_bf16x4(a.y + row * G.N, G.N, nb0 * 16 + wave * 64 + nb2 * 32 + 8 * j + 4 * hi, v);
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
  hipLaunchKernelGGL(kern, dim3(grid), dim3(256), big_lds_bytes(MX), st, a, tiles_n, tiles_m);
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
