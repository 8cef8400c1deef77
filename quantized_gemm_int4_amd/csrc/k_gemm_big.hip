// MFMA GEMM for many rows (prefill-sized M, and 256-row units of a grouped
// GEMM), where the ~2*M*N*K matrix multiply dominates (ywsung.com note "How
// vLLM Humming computes 4 bits", section on one token vs many tokens).
//
// One block computes a 256 x 256 output tile.  Activations and weights reach
// LDS through 16-byte direct buffer-to-LDS loads; each activation copy reads
// whole 128-byte lines (eight rows of one K step), which the L1 path moves
// about three times faster than copies that gather 32 bytes from each of 32
// rows.  The row-major activation stage is XOR-swizzled so that the MFMA
// operand reads stay free of bank conflicts.  Three LDS stages: copies run
// two K steps ahead.
//   * W4A16 (K step 64, four waves, one per SIMD): each wave owns all 256
//     rows x 64 columns as 2 x 8 blocks of 32x32x16 bf16 MFMA (256
//     accumulators per lane) and unpacks its columns' weights, copied into
//     LDS per K group through a ring of group slots, to bf16 s * (u - z) in
//     between its MFMAs of the previous step.  A tile of at most 128 rows
//     (the last round's half tiles of a dense grid, a short unit) runs only
//     four of the eight row blocks.
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

}  // namespace

// first column block of expert e
__device__ __forceinline__ int64_t wbase_of(int64_t e, const Geom& G) { return e * G.NB; }

constexpr int kBigStages = 3;     // LDS stages: loads run two K steps ahead

// LDS bytes of one stage: activation fragments (32 x 1 KiB; MXFP4 rows 16 x
// 1 KiB) and the block's 16 weight tiles (16 KiB), plus MXFP4: their E8M0
// scale words (16 x 256 B) and, with MXFP4 rows, the rows' E8M0 words (8 x
// 256 B); INT4: per wave 256 B of bf16 scales and 256 B of zero-point words.
__host__ __device__ constexpr int big_stage_bytes(bool mx, bool a4 = false) {
  return a4 ? (16 + 16 + 4 + 2) * 1024 : (mx ? (32 + 16 + 4) * 1024 : (32 + 16 + 2) * 1024);
}
__host__ __device__ constexpr int big_lds_bytes(bool mx, bool a4 = false) { return kBigStages * big_stage_bytes(mx, a4); }
// MXFP4: eight waves (two per SIMD); W4A16: four (one per SIMD, 256 accumulators each)
__host__ __device__ constexpr int big_threads(bool mx) { return mx ? 512 : 256; }

// Unit swizzles of the epilogue slabs (8-byte units, 64 per 512-byte row),
// chosen so that the accumulator writes of 32 lanes hit distinct banks:
// W4A16 lanes write 32 rows of one unit, MXFP4 lanes 16 rows x 2 units.
struct Swz16 {
  __device__ static int swz(int r) { return r & 31; }
};
struct SwzMx {
  __device__ static int swz(int r) { return 2 * (r & 15); }
};

// One 256 x 256 output tile: expert, first row (dense), first 16-column
// block, valid rows (1..256) and, grouped, its first index into the sorted
// pair list.
struct BigTile {
  int64_t e, m0, nb0, rows, first;
};

// What one thread's copies of a tile need: buffers over the tile's
// activation rows and its 16 weight column blocks, and per-lane byte offsets.
template <int NX, int NWT>
struct BigCopy {
  rsrc_t rx, rw;
  uint32_t xoff[NX];  // activation copies (row offset + swizzled chunk)
  uint32_t wvo[NWT];  // weight tile copies
  uint32_t svo[2];    // MXFP4: scale words of the two tiles; INT4: scale / zero gather
  rsrc_t rxs;         // MXFP4 rows: buffer over the rows' E8M0 bytes
  uint32_t xso;       // MXFP4 rows: this lane's row of E8M0 bytes
};

// A persistent grid: block b takes tiles b, b + grid, b + 2 grid, ...  Dense
// tiles are visited XCD by XCD: blocks are dispatched round-robin over the
// eight XCDs, so item i runs on XCD i % 8 (the grid is a multiple of 8 or a
// single round); each XCD walks a contiguous range of tiles in groups of four
// tile rows, so the blocks sharing an XCD's L2 also share activation and
// weight slices.  Grouped (MoE) items are (unit, 256-column tile) pairs; a
// unit is up to 256 rows of one expert, whose activation rows are gathered
// through the sorted pair list and whose outputs are written in pair order.
//
// With three or more K steps per tile the copies run on across tiles: the
// last steps of a tile copy the first steps of the block's next tile, whose
// MFMAs then start right after this tile's epilogue, and the output stores
// drain while the next tile computes.
// W4A16 K-step loop of one tile (the body of k_gemm_big below, written once
// and expanded there for MB_ = 8 or 4 32-row blocks; it uses the kernel's
// locals).  A function or lambda here would make the compiler keep the two
// copy-descriptor sets in scratch memory.
#define HM_BIG_W4A16_STEPS(MB_)                                                                                     \
  do {                                                                                                              \
        constexpr int MB = MB_;                                                                                     \
        constexpr int NI = 4 * MB;                                                                                  \
        constexpr int WPI = 32 / NI;                                                                                \
_Pragma("nounroll")                                                                                                 \
        for (int s = 0; s < S; ++s) {                                                                               \
          if (GROUPED && chained && s == 1) {                                                                       \
            write_table(tp);                                                                                        \
            if (has_next) nc = make_copy(nxt, prn);                                                                 \
          }                                                                                                         \
          const int KGt = S >> 1;                                                                                   \
          const int t2 = s + 2, tg = (s >> 1) + 2, wh = s & 1;                                                      \
          const bool xnext = chained && has_next && t2 >= S, wnext = chained && has_next && tg >= KGt;              \
          const int xls = t2 < S ? t2 : (xnext ? t2 - S : S - 1);                                                   \
          const int wg = tg < KGt ? tg : (wnext ? tg - KGt : KGt - 1);                                              \
          uint8_t* d2 = lds + so[2];                                                                                \
          uint8_t* dw = lds + wso[2];                                                                               \
          /* INT8 weights travel per step, three steps ahead, through the ring of weight slots */                  \
          const int t3 = s + 3;                                                                                     \
          const bool w8next = chained && has_next && t3 >= S;                                                       \
          const int w8s = t3 < S ? t3 : (w8next ? t3 - S : S - 1);                                                  \
          uint8_t* dw8 = lds + wso[0];                                                                              \
          auto dma = [&](int q) __attribute__((always_inline)) {                                                    \
            if (q < NX) {                                                                                           \
              const rsrc_t r = xnext ? nc.rx : cc.rx;                                                               \
              b2lds16(r, xnext ? nc.xoff[q] : cc.xoff[q], (uint32_t)(xls * 128), d2 + (NX * wave + q) * 1024);      \
            } else if (Q8 && q < NX + 4) {                                                                          \
              /* INT8: step s + 3's half (1 KiB) of each 2 KiB tile into the free weight slot */                    \
              const int k0 = q - NX;                                                                                \
              b2lds16(w8next ? nc.rw : cc.rw, w8next ? nc.wvo[k0] : cc.wvo[k0],                                     \
                      (uint32_t)((w8s >> 1) * 2048 + (w8s & 1) * 1024), dw8 + kWOff + (NWT * wave + k0) * 1024);    \
            } else if (Q8) {                                                                                        \
              b2lds4(rsz, (w8next ? nc.svo[0] : cc.svo[0]) + (uint32_t)(w8s >> 1) * szstride, 0u,                   \
                     dw8 + kSOff + wave * 256);                                                                     \
            } else if (q < NX + 2) {                                                                                \
              /* tile k0 + 2 wh of the wave: selected operands, no branch (a branch here splits */                  \
              /* the step into blocks and the compiler then bunches the unpacking of later K parts) */             \
              const rsrc_t r = wnext ? nc.rw : cc.rw;                                                               \
              const int k0 = q - NX;                                                                                \
              const uint32_t vlo = wnext ? nc.wvo[k0] : cc.wvo[k0], vhi = wnext ? nc.wvo[2 + k0] : cc.wvo[2 + k0];  \
              b2lds16(r, wh ? vhi : vlo, (uint32_t)(wg * 1024), dw + kWOff + (NWT * wave + k0 + 2 * wh) * 1024);    \
            } else if (F4) {                                                                                        \
              b2lds16(rsz, (wnext ? nc.svo[0] : cc.svo[0]) + (uint32_t)(wg >> 2) * 256, 0u,                         \
                      dw + kSOff + wave * 1024);                                                                    \
            } else {                                                                                                \
              b2lds4(rsz, (wnext ? nc.svo[0] : cc.svo[0]) + (uint32_t)wg * szstride, 0u, dw + kSOff + wave * 256);  \
            }                                                                                                       \
          };                                                                                                        \
          const uint8_t* xs = lds + so[0];                                                                          \
          uint32_t wv[2][4];                                                                                        \
          float svn[2], zsn[2], sfn[2][2];                                                                          \
          u32x2_t wv8[2][4];                                                                                        \
          if (Q8)                                                                                                   \
            fetch8(lds + wso[1], wv8, svn);                                                                         \
          else if (F4)                                                                                              \
            fetch_f4(lds + ((s & 1) ? wso[1] : wso[0]), (s + 1) & 1, (s + 1 < S ? (s + 1) >> 1 : 0) & 3, wv, sfn); \
          else                                                                                                      \
            fetch(lds + ((s & 1) ? wso[1] : wso[0]), (s + 1) & 1, wv, svn, zsn);                                    \
          u32x4_t b[NI];                                                                                            \
_Pragma("unroll")                                                                                                   \
          for (int i = 0; i < kD; ++i) b[i] = ld16(xs + (i % MB) * 4096 + xo[i / MB]);                              \
          uint32_t lo = 0, hi4 = 0;                                                                                 \
_Pragma("unroll")                                                                                                   \
          for (int i = 0; i < NI; ++i) {                                                                            \
            const int kq = i / MB, mb = i % MB;                                                                     \
_Pragma("unroll")                                                                                                   \
            for (int nb2 = 0; nb2 < 2; ++nb2) acc[nb2][mb] = mfma32_bf16(af[nb2][kq], b[i], acc[nb2][mb]);          \
            if (i + kD < NI) {                                                                                      \
              const int j = i + kD;                                                                                 \
              b[j] = ld16(xs + (j % MB) * 4096 + xo[j / MB]);                                                       \
            }                                                                                                       \
_Pragma("unroll")                                                                                                   \
            for (int e = 0; e < WPI; ++e) {                                                                         \
              const int wi = WPI * i + e, nb2 = (wi >> 2) & 1, u = wi & 3;                                          \
              const uint32_t w = kq == 0 ? w3c[nb2] : wv[nb2][kq - 1];                                              \
              if (Q8) {                                                                                             \
                const u32x2_t w8 = kq == 0 ? w3c8[nb2] : wv8[nb2][kq - 1];                                          \
                const float sv = kq == 0 ? sv3c[nb2] : svn[nb2];                                                    \
                af[nb2][(kq + 3) & 3][u] = i8x2_bf16_scaled(w8[u >> 1], u & 1, sv);                                \
              } else if (F4) {                                                                                      \
                const float sf = kq == 0 ? sv3c[nb2] : sfn[nb2][(kq - 1) >> 1];                                     \
                af[nb2][(kq + 3) & 3][u] = I4 ? i4x2_bf16(w, sf, u) : fp4x2_bf16(w, sf, u);                          \
              } else {                                                                                              \
                const float sv = kq == 0 ? sv3c[nb2] : svn[nb2], zs = kq == 0 ? zs3c[nb2] : zsn[nb2];               \
                if (u == 0) {                                                                                       \
                  lo = in_vgpr(w & 0x0F0F0F0Fu);                                                                    \
                  hi4 = in_vgpr((w >> 4) & 0x0F0F0F0Fu);                                                            \
                }                                                                                                   \
                af[nb2][(kq + 3) & 3][u] = dq8_word(lo, hi4, u, sv, zs);                                            \
              }                                                                                                     \
            }                                                                                                       \
            if (MB == 8) {                                                                                          \
              if ((i & 1) && (i >> 1) < kPer) dma(i >> 1);                                                          \
            } else {                                                                                                \
              if (i >= 1 && i - 1 < kPer) dma(i - 1);                                                               \
            }                                                                                                       \
            __builtin_amdgcn_sched_barrier(0);                                                                      \
          }                                                                                                         \
_Pragma("unroll")                                                                                                   \
          for (int nb2 = 0; nb2 < 2; ++nb2) {                                                                       \
            w3c[nb2] = wv[nb2][3];                                                                                  \
            if (Q8) w3c8[nb2] = wv8[nb2][3];                                                                        \
            sv3c[nb2] = F4 ? sfn[nb2][1] : svn[nb2];                                                                \
            zs3c[nb2] = F4 ? 0.f : zsn[nb2];                                                                        \
          }                                                                                                         \
          wait_barrier(std::integral_constant<int, kPer>());                                                        \
          rotate();                                                                                                 \
          if (Q8 || (s & 1)) rotate_w();                                                                            \
        }                                                                                                           \
  } while (0)

template <bool MX, bool ZP, bool GROUPED, bool A4 = false, bool F4 = false, bool I4 = false, bool Q8 = false>
__global__ void __launch_bounds__(big_threads(MX), 1)
k_gemm_big(GemmArgs a, int tiles_n, int tiles_m, int n_full) {
  static_assert(!A4 || MX, "MXFP4 rows go with MXFP4 weights");
  static_assert(!F4 || (!MX && !ZP), "MX weights with bf16 rows take the bf16 path");
  static_assert(!I4 || F4, "MXINT4 codes take the MX bf16-row path");
  static_assert(!Q8 || (!MX && !ZP && !F4), "INT8 weights take the bf16 path");
  constexpr int SB = big_stage_bytes(MX || F4, A4);
  constexpr int NW = big_threads(MX) / 64;         // waves
  constexpr int NX = A4 ? 2 : 32 / NW;             // activation copies per lane per step
  constexpr int NPR = A4 ? NX + 1 : NX;            // grouped: pair rows a thread's copies read
  constexpr int NWT = 16 / NW;                     // weight tiles copied per wave per step
  constexpr int XSTEP = A4 ? 64 : 128;             // activation bytes per row per K step
  typedef BigCopy<NX, NWT> Copy;
  extern __shared__ __attribute__((aligned(1024))) uint8_t lds[];
  __shared__ int32_t arow_s[GROUPED ? kBigM : 1];   // activation row of each local row
  __shared__ int32_t orow_s[GROUPED ? kBigM : 1];   // output row, or -1 (not stored)

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n_l = lane & 15, q_l = lane >> 4, l32 = lane & 31, hi = lane >> 5;
  const Geom G = a.G;
  const int64_t row_bytes = A4 ? G.K / 2 : (MX ? G.K : 2 * G.K);
  const int S = (int)(MX ? G.KG : 2 * G.KG);      // K steps per tile
  const bool chained = S >= 3;
  // dense: tiles n_full.. of the visiting order run as two 128-row halves
  const int64_t n_items = GROUPED ? (int64_t)a.hdr[2] * tiles_n
                                  : (int64_t)n_full + 2 * ((int64_t)tiles_n * tiles_m - n_full);
  int64_t item = blockIdx.x;
  if (item >= n_items) return;

  auto decode = [&](int64_t it) __attribute__((always_inline)) -> BigTile {
    BigTile t;
    if (GROUPED) {
      const int32_t* u = a.units + 4 * (it / tiles_n);
      t.e = u[0];
      t.first = u[1];
      t.rows = u[2] < kBigM ? u[2] : kBigM;
      t.m0 = 0;
      t.nb0 = (it % tiles_n) * kBigCB;
    } else {
      const int total = tiles_n * tiles_m;
      // item j of a range of cnt items -> its position in the range: the
      // items of one XCD (j % 8) take a contiguous part
      auto spread = [](int j, int cnt) __attribute__((always_inline)) {
        const int xcd = j % 8, idx = j / 8, base = cnt / 8, extra = cnt % 8;
        return xcd * base + (xcd < extra ? xcd : extra) + idx;
      };
      int tt, half = -1;
      if (it < n_full) {
        tt = spread((int)it, n_full);
      } else {
        const int h = spread((int)(it - n_full), 2 * (total - n_full));
        tt = n_full + (h >> 1);
        half = h & 1;
      }
      constexpr int GM = 4;
      const int grp = tt / (GM * tiles_n);
      const int first_m = grp * GM;
      const int gm = (tiles_m - first_m) < GM ? (tiles_m - first_m) : GM;
      const int tin = tt - grp * GM * tiles_n;
      const int tm = first_m + tin % gm, tn = tin / gm;
      t.e = 0;
      t.first = 0;
      t.m0 = (int64_t)tm * kBigM + (half > 0 ? kBigM / 2 : 0);
      t.nb0 = (int64_t)tn * kBigCB;
      const int64_t cap = half >= 0 ? kBigM / 2 : kBigM;
      t.rows = (a.M - t.m0) < cap ? (a.M - t.m0) : cap;
    }
    return t;
  };
  // grouped: activation row of a sorted pair (invalid pairs read row 0 and are not stored)
  auto act_row = [&](int32_t pair) __attribute__((always_inline)) -> int64_t {
    if (pair < 0 || pair >= a.P) return 0;
    return a.rows_are_pairs ? pair : pair / a.topk;
  };
  // grouped: sorted pair of local row r, clamped to the tile
  auto pair_of = [&](const BigTile& t, int r) __attribute__((always_inline)) -> int32_t {
    return a.sorted_pairs[t.first + (r < t.rows ? r : t.rows - 1)];
  };

  // Activations of one K step (128 bytes per row: 64 bf16 or 128 fp8) are
  // staged row-major, 256 rows x 128 bytes, with 16-byte chunk c of row r in
  // slot c ^ ((r >> 1) & 7), so that the 16 lanes of an operand read (16
  // rows, one chunk each) hit all 64 banks once.  Copy j = NX w + i (i <
  // NX) of wave w covers rows 8 j .. 8 j + 7: lane L row 8 j + L / 8, slot
  // L % 8, so every copy reads eight whole 128-byte lines.
  const rsrc_t rsz = make_rsrc(a.w + G.off_scales, G.total - G.off_scales);
  // INT4: lanes 0..31 gather the bf16 scales of the wave's four column blocks
  // (tile (L / 8) % 4, bytes 4 (L % 8)), lanes 32..39 their zero-point words
  // (tile (L / 2) % 4, word L % 2)
  const bool zlane = !MX && ZP && lane >= 32 && lane < 40;
  const uint32_t szstride = zlane ? 8 : 32;
  auto make_copy = [&](const BigTile& t, const int32_t (&pr)[NPR]) __attribute__((always_inline)) -> Copy {
    Copy c;
    c.rx = make_rsrc(reinterpret_cast<const uint8_t*>(a.x) + t.m0 * row_bytes,
                     GROUPED ? 0xFFFFFFFFull : (uint64_t)t.rows * row_bytes);
    const int64_t wb = wbase_of(t.e, G);
    constexpr int TB = Q8 ? 2048 : 1024;             // bytes of one (column block, group) tile
    c.rw = make_rsrc(a.w + (wb + t.nb0) * G.KG * TB, (uint64_t)kBigCB * G.KG * TB);
#pragma unroll
    for (int i = 0; i < NX; ++i) {
      // MXFP4 rows (64 bytes a step): 16 rows a copy, lane L row 16 j + L / 4,
      // chunk slot L % 4; else 8 rows a copy, lane L row 8 j + L / 8, slot L % 8
      const int r = A4 ? 16 * (NX * wave + i) + (lane >> 2) : 8 * (NX * wave + i) + (lane >> 3);
      // dense rows past the tile's end lie outside the buffer: zeros, no memory traffic
      const int64_t src = GROUPED ? act_row(pr[i]) : (r < t.rows ? r : t.rows);
      c.xoff[i] = (uint32_t)(src * row_bytes) +
                  (A4 ? 16 * ((lane & 3) ^ ((r >> 2) & 3)) : 16 * ((lane & 7) ^ ((r >> 1) & 7)));
    }
    if (A4) {
      // the rows' E8M0 bytes (K / 32 per row, one 4-byte word per K step):
      // lanes L and L + 32 of wave w copy the word of row 32 w + L % 32
      const int64_t kb = G.K / 32;
      c.rxs = make_rsrc(a.xsb + (GROUPED ? 0 : t.m0 * kb), GROUPED ? 0xFFFFFFFFull : (uint64_t)t.rows * kb);
      const int r = 32 * wave + (lane & 31);
      const int64_t src = GROUPED ? act_row(pr[NX]) : (r < t.rows ? r : t.rows);
      c.xso = (uint32_t)(src * kb);
    }
#pragma unroll
    for (int k = 0; k < NWT; ++k) {
      int64_t nb = MX ? t.nb0 + wave + 8 * k : t.nb0 + NWT * wave + k;
      if (nb >= G.NB) nb = G.NB - 1;
      c.wvo[k] = (uint32_t)((nb - t.nb0) * G.KG * TB + lane * 16);
      if (MX) c.svo[k & 1] = (uint32_t)((wb + nb) * G.KG4 * 256 + lane * 4);
    }
    if (F4) {
      // MXFP4 with bf16 rows: lane L copies 16 bytes (four lanes' E8M0
      // words) of the word array of column block 4 w + L / 16
      c.svo[1] = 0u;
      int64_t nbq = t.nb0 + NWT * wave + (lane >> 4);
      if (nbq >= G.NB) nbq = G.NB - 1;
      c.svo[0] = (uint32_t)((wb + nbq) * G.KG4 * 256 + (lane & 15) * 16);
    } else if (!MX) {
      c.svo[1] = 0u;
      int64_t nbq = t.nb0 + NWT * wave + (zlane ? ((lane >> 1) & 3) : ((lane >> 3) & 3));
      if (nbq >= G.NB) nbq = G.NB - 1;
      c.svo[0] = (uint32_t)(zlane ? (G.off_zeros - G.off_scales) + (wb + nbq) * G.KG * 8 + (lane & 1) * 4
                                  : (wb + nbq) * G.KG * 32 + (lane & 7) * 4);
    }
    return c;
  };
  // grouped: this thread's copy rows of tile t, and its row of the tables
  auto load_rows = [&](const BigTile& t, int32_t (&pr)[NPR], int32_t& tp) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < NX; ++i)
      pr[i] = pair_of(t, A4 ? 16 * (NX * wave + i) + (lane >> 2) : 8 * (NX * wave + i) + (lane >> 3));
    if (A4) pr[NPR - 1] = pair_of(t, 32 * wave + (lane & 31));
    tp = (tid < t.rows) ? a.sorted_pairs[t.first + tid] : -1;
  };
  auto write_table = [&](int32_t tp) __attribute__((always_inline)) {
    if (GROUPED && tid < kBigM) {
      const bool ok = tp >= 0 && tp < a.P;
      arow_s[tid] = (int32_t)act_row(tp);
      orow_s[tid] = ok ? tp : -1;
    }
  };
  // LDS offsets of the stages of the current step and the next two (the one
  // after those is the current one again), rotated after every step
  uint32_t so[3] = {0u, (uint32_t)SB, 2u * SB};
  auto rotate = [&]() __attribute__((always_inline)) {
    const uint32_t t = so[0];
    so[0] = so[1];
    so[1] = so[2];
    so[2] = t;
  };
  auto copy_x = [&](const Copy& c, int ls, uint8_t* stg) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < NX; ++i) b2lds16(c.rx, c.xoff[i], (uint32_t)(ls * XSTEP), stg + (NX * wave + i) * 1024);
  };
  auto wait_barrier = [&](auto n_c) __attribute__((always_inline)) {
    // wait for this wave's copies except the n most recent vector-memory
    // operations and for its LDS operations, then meet the other waves; the
    // memory clobber keeps the compiler from moving LDS accesses across
    __asm__ volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(decltype(n_c)::value) : "memory");
  };
  // LDS-only barrier for the epilogue's staging: the output stores drain on
  // their own (the next step's wait covers them, vector memory completes in order)
  auto lds_barrier = [&]() __attribute__((always_inline)) { __asm__ volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); };
  auto local_row = [&](const BigTile& t, int64_t r, int64_t& out, int64_t& in) __attribute__((always_inline)) {
    if (r >= t.rows) { out = -1; in = 0; return; }
    out = GROUPED ? (int64_t)orow_s[r] : t.m0 + r;
    in = GROUPED ? (int64_t)arow_s[r] : t.m0 + r;
  };

  // Epilogue through LDS: the tile leaves in four slabs of 64 rows, staged
  // as bf16 in the activation part of the last step's stage (free until the
  // next tile's first step), 512 bytes per row with 8-byte unit u of row r
  // at unit u ^ g(r); each thread then stores 16-byte chunks, 32 lanes per
  // row, so every store writes whole 128-byte lines.
  auto store_slab = [&](const BigTile& t, const uint8_t* ost, int p, auto gfun) __attribute__((always_inline)) {
    constexpr int RS = 2 * NW;                     // rows per sweep of the block
#pragma unroll
    for (int k = 0; k < 64 / RS; ++k) {
      const int r = RS * k + (tid >> 5), c = tid & 31;
      const int g = decltype(gfun)::swz(r);
      const u32x2_t v0 = *reinterpret_cast<const u32x2_t*>(ost + r * 512 + ((2 * c) ^ g) * 8);
      const u32x2_t v1 = *reinterpret_cast<const u32x2_t*>(ost + r * 512 + ((2 * c + 1) ^ g) * 8);
      int64_t row, arow;
      local_row(t, 64 * p + r, row, arow);
      if (GROUPED && a.gated) {
        // gated layout: lane c takes half c & 1 (4 values) of output chunk
        // c >> 1, from the same half of its gate and up chunks
        const int oc = c >> 1, hf = c & 1, gc = gated_gate_chunk(oc);
        const u32x2_t gv = *reinterpret_cast<const u32x2_t*>(ost + r * 512 + ((2 * gc + hf) ^ g) * 8);
        const u32x2_t uv = *reinterpret_cast<const u32x2_t*>(ost + r * 512 + ((2 * gc + 4 + hf) ^ g) * 8);
        if (row >= 0)
          *reinterpret_cast<u32x2_t*>(a.y + row * (G.N / 2) + t.nb0 * 8 + 8 * oc + 4 * hf) =
              (u32x2_t){silu_mul_pair(gv[0], uv[0]), silu_mul_pair(gv[1], uv[1])};
      } else if (row >= 0) {
        store_bf16x8(a.y + row * G.N, G.N, t.nb0 * 16 + 8 * c, (u32x4_t){v0[0], v0[1], v1[0], v1[1]});
      }
    }
  };

  BigTile cur = decode(item);
  int32_t pr[NPR] = {}, tp = -1;
  if (GROUPED) load_rows(cur, pr, tp);
  Copy cc = make_copy(cur, pr);
  bool first = true;

  if constexpr (MX) {
    // ================================ W4A8-MXFP4: K step 128 = one K group;
    // eight waves, two per SIMD: wave w owns rows 64 (w & 3) + 0..63 and
    // columns 128 (w >> 2) + 0..127 (4 x 8 blocks of 16 x 16, 128
    // accumulators per lane)
    const int wm = wave & 3, wn = wave >> 2;
    // stage layout: activations (kXB bytes), weight tiles at kWO, their
    // scale words at kSO, MXFP4 rows: the rows' E8M0 words at kAO (256 B per
    // wave, rows 32 w + 0..31 twice)
    constexpr int kXB = A4 ? 16 * 1024 : 32 * 1024, kWO = kXB, kSO = kXB + 16 * 1024, kAO = kSO + 4 * 1024;
    // operand rows 16 rb + n_l: K chunks q_l and 4 + q_l (16 fp8 each); MXFP4
    // rows: chunk q_l (32 E2M1 values), slot q_l ^ ((n_l >> 2) & 3)
    const int xsw = (n_l >> 1) & 7;
    const uint32_t xo0 = A4 ? n_l * 64 + 16 * (q_l ^ ((n_l >> 2) & 3)) : n_l * 128 + 16 * (q_l ^ xsw);
    const uint32_t xo1 = n_l * 128 + 16 * ((4 + q_l) ^ xsw);
    // copies of one stage: activations, weight tiles (column blocks w and
    // w + 8) and their scale words, [the rows' scale words]
    auto copy_stage = [&](const Copy& c, int ls, uint8_t* st) __attribute__((always_inline)) {
      copy_x(c, ls, st);
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const int cb = wave + 8 * k;
        b2lds16(c.rw, c.wvo[k], (uint32_t)(ls * 1024), st + kWO + cb * 1024);
        b2lds4(rsz, c.svo[k], (uint32_t)((ls / 4) * 256), st + kSO + cb * 256);
      }
      if (A4) b2lds4(c.rxs, c.xso, (uint32_t)(ls * 4), st + kAO + wave * 256);
    };
    constexpr int kPer = A4 ? 7 : 8;                // copies per wave per stage
    while (true) {
      const int64_t nitem = item + gridDim.x;
      const bool has_next = nitem < n_items;
      const BigTile nxt = has_next ? decode(nitem) : cur;
      int32_t prn[NPR] = {}, tpn = -1;
      if (!chained || first) {
        // stand-alone start: earlier copies and stores done, all waves past
        // the previous epilogue
        if (!first) {
          __asm__ volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
          if (GROUPED) load_rows(cur, pr, tp);
          cc = make_copy(cur, pr);
        }
        write_table(tp);
        copy_stage(cc, 0, lds + so[0]);
        if (S > 1) {
          copy_stage(cc, 1, lds + so[1]);
          wait_barrier(std::integral_constant<int, kPer>());
        } else {
          wait_barrier(std::integral_constant<int, 0>());
        }
      }
      // the next tile's rows load before this tile's copies (done by the end of step 0)
      if (GROUPED && chained && has_next) load_rows(nxt, prn, tpn);
      Copy nc = cc;
      if (!GROUPED && chained && has_next) nc = make_copy(nxt, prn);

      f32x4_t acc[8][4];
#pragma unroll
      for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[j][i] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
#pragma nounroll
      for (int s = 0; s < S; ++s) {
        if (GROUPED && chained && s == 1) {
          write_table(tp);
          if (has_next) nc = make_copy(nxt, prn);
        }
        const uint8_t* st = lds + so[0];
        // copies for step s + 2: this tile's, the next tile's, or (none left)
        // a repeat of the last one into a stage no longer read
        // copies for step s + 2 (this tile's, the next tile's, or, none
        // left, repeats of this tile's last step into a stage no longer
        // read), one after every four MFMAs: activations q < 4, then per
        // weight tile its 1 KiB and its scale words
        const int t2 = s + 2;
        const bool xnext = chained && has_next && t2 >= S;
        const int ls = t2 < S ? t2 : (xnext ? t2 - S : S - 1);
        uint8_t* d2 = lds + so[2];
        auto dma = [&](int q) __attribute__((always_inline)) {
          const Copy& c = xnext ? nc : cc;
          if (q < NX) {
            b2lds16(c.rx, c.xoff[q], (uint32_t)(ls * XSTEP), d2 + (NX * wave + q) * 1024);
          } else if (q < NX + 4) {
            const int k = (q - NX) >> 1, cb = wave + 8 * k;
            if (((q - NX) & 1) == 0) b2lds16(c.rw, c.wvo[k], (uint32_t)(ls * 1024), d2 + kWO + cb * 1024);
            else b2lds4(rsz, c.svo[k], (uint32_t)((ls / 4) * 256), d2 + kSO + cb * 256);
          } else if (A4) {
            b2lds4(c.rxs, c.xso, (uint32_t)(ls * 4), d2 + kAO + wave * 256);
          }
        };
        // operands: the wave's eight weight tiles and their scales (kept for
        // the step), activation halves of one row block at a time, read one
        // row block ahead
        const int sh = 8 * (s & 3);
        const uint8_t* wbase = st + kWO + wn * 8 * 1024 + lane * 16;
        const uint8_t* sbase = st + kSO + wn * 8 * 256 + lane * 4;
        constexpr int XRB = A4 ? 1024 : 2048;         // bytes of one 16-row block of the stage
        const uint8_t* xbase = st + wm * 4 * XRB;
        u32x4_t wq[8];
        int wsc[8];
        uint32_t swd[8], xsw4[4];
        u32x4_t b0[2], b1[2];
        // every read of the step's first MFMAs goes out before any of them is
        // used, in the order they are needed (LDS returns in order): the
        // scale words, row block 0's activations, then the tiles one by one,
        // so the first MFMA waits for a fifth of the step's reads and each
        // later one for its own tile
#pragma unroll
        for (int j = 0; j < 8; ++j) swd[j] = *reinterpret_cast<const uint32_t*>(sbase + j * 256);
        // MXFP4 rows: the E8M0 byte of row 64 wm + 16 i + n_l and K block q_l
        // (word of row r at kAO + (r / 32) 256 + (r % 32) 4)
        if (A4) {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            xsw4[i] = *reinterpret_cast<const uint32_t*>(st + kAO + (2 * wm + (i >> 1)) * 256 + (16 * (i & 1) + n_l) * 4);
        }
        b0[0] = ld16(xbase + xo0);
        if (!A4) b1[0] = ld16(xbase + xo1);
#pragma unroll
        for (int j = 0; j < 8; ++j) wq[j] = ld16(wbase + j * 1024);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < 8; ++j) wsc[j] = (int)((swd[j] >> sh) & 0xFF);
        int xsc[4] = {127, 127, 127, 127};
        if (A4) {
#pragma unroll
          for (int i = 0; i < 4; ++i) xsc[i] = (int)((xsw4[i] >> (8 * q_l)) & 0xFF);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (i + 1 < 4) {
            b0[(i + 1) & 1] = ld16(xbase + (i + 1) * XRB + xo0);
            if (!A4) b1[(i + 1) & 1] = ld16(xbase + (i + 1) * XRB + xo1);
          }
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            if (A4) acc[j][i] = mfma_fp4_fp4(wq[j], b0[i & 1], acc[j][i], wsc[j], xsc[i]);
            else acc[j][i] = mfma_fp4_fp8(wq[j], b0[i & 1], b1[i & 1], acc[j][i], wsc[j], 127);
            if ((j & 3) == 3) {
              if (2 * i + (j >> 2) < kPer) dma(2 * i + (j >> 2));
              __builtin_amdgcn_sched_barrier(0);
            }
          }
        }
        // the next stage was issued one step ago, this step's copies after it
        wait_barrier(std::integral_constant<int, kPer>());
        rotate();
      }

      // ---- epilogue: lane holds C[n = 16 nb + 4 q_l + r][row = 16 rb + n_l];
      // slab p holds the rows of the two waves with wm = p; the copies still
      // in flight finish first (the stores then never overtake a copy)
      float rs[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        int64_t row, arow;
        local_row(cur, (wm * 4 + i) * 16 + n_l, row, arow);
        rs[i] = A4 ? 1.0f : a.xs[arow];              // MXFP4 rows: scaled inside the MFMA
      }
      __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
      uint8_t* ost = lds + so[2];                    // the last step's stage
      for (int p = 0; p < 4; ++p) {
        if (wm == p) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int r = 16 * i + n_l;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
              const f32x4_t v = acc[j][i] * rs[i];
              const int u = 32 * wn + 4 * j + q_l;
              *reinterpret_cast<u32x2_t*>(ost + r * 512 + (u ^ SwzMx::swz(r)) * 8) =
                  (u32x2_t){pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3])};
            }
          }
        }
        lds_barrier();
        store_slab(cur, ost, p, SwzMx());
        lds_barrier();
      }
      if (!has_next) break;
      cur = nxt;
      cc = nc;
      tp = tpn;
      item = nitem;
      first = false;
    }
  } else {
    // ================================ W4A16: K step 64 = half a K group;
    // four waves, one per SIMD: wave w owns columns 64 w + 0..63 and all 256
    // rows as 2 x 8 blocks of 32 x 32 (v_mfma_f32_32x32x16_bf16, 256
    // accumulators per lane), so every weight is unpacked by one wave and
    // every activation fragment read from LDS feeds two MFMAs.  32x32x16
    // operands: A row / B column = lane % 32, K = 8 (lane / 32) + 0..7;
    // result: column lane % 32, rows 8 j + 4 (lane / 32) + r in register
    // 4 j + r.  The unpacking of the next step's operands is interleaved with
    // this step's MFMAs, so it runs on the vector ALU while the matrix core
    // works.
    // operand rows 32 mb + l32, K part kq: chunk 2 kq + hi (8 bf16)
    const int xsw = (l32 >> 1) & 7;
    uint32_t xo[4];
#pragma unroll
    for (int kq = 0; kq < 4; ++kq) xo[kq] = l32 * 128 + 16 * ((2 * kq + hi) ^ xsw);
    // Weights travel per K group (two steps): the weight parts of the three
    // stages form a ring of group slots (group slot offsets wso, rotated
    // every second step), and group g + 2 is copied during the two steps of
    // group g, half of the wave's four tiles per step.  Wave w copies its own
    // tiles (column blocks 4 w .. 4 w + 3) and one 4-byte-per-lane gather of
    // their scales and zero points into its 256-byte slot at kSOff + 256 w
    // (scales at 0, zero-point words at 128), repeated in both steps.
    constexpr int kWOff = 32 * 1024, kSOff = 48 * 1024;
    uint32_t wso[3] = {0u, (uint32_t)SB, 2u * SB};
    auto rotate_w = [&]() __attribute__((always_inline)) {
      const uint32_t t = wso[0];
      wso[0] = wso[1];
      wso[1] = wso[2];
      wso[2] = t;
    };
    // all four tiles of group g and the gather (MXFP4 weights: the E8M0 word
    // arrays of the four column blocks for groups 4 (g / 4) .. + 3, 1 KiB per
    // wave at kSOff + 1024 w)
    auto copy_w = [&](const Copy& c, int g, uint8_t* slot) __attribute__((always_inline)) {
#pragma unroll
      for (int k = 0; k < NWT; ++k)
        b2lds16(c.rw, c.wvo[k], (uint32_t)(g * 1024), slot + kWOff + (NWT * wave + k) * 1024);
      if (F4) b2lds16(rsz, c.svo[0] + (uint32_t)(g >> 2) * 256, 0u, slot + kSOff + wave * 1024);
      else b2lds4(rsz, c.svo[0] + (uint32_t)g * szstride, 0u, slot + kSOff + wave * 256);
    };
    // copies per wave per step: activations, half of the wave's code tiles
    // (INT8: the step's half of all four) and the scale / zero-point gather
    constexpr int kPer = Q8 ? NX + 4 + 1 : NX + 2 + 1;
    // A operands of one step: column half nb2, K part kq.  Lane row n =
    // 64 w + 32 nb2 + l32 lies in tile 4 w + 2 nb2 + l32 / 16 at column
    // l32 % 16; K = 64 h + 16 kq + 8 hi is word 2 h + kq / 2 of slot
    // (l32 % 16) + 16 ((2 kq + hi) % 4).
    const int c_l = l32 >> 4, c16 = l32 & 15;
    auto fetch = [&](const uint8_t* stg, int h, uint32_t (&wv)[2][4], float (&sv)[2], float (&zs)[2]) __attribute__((always_inline)) {
      const uint8_t* sz = stg + kSOff + wave * 256;
#pragma unroll
      for (int nb2 = 0; nb2 < 2; ++nb2) {
        const uint8_t* tile = stg + kWOff + (NWT * wave + 2 * nb2 + c_l) * 1024;
        // K parts kq and kq + 2 are words 2 h and 2 h + 1 of one slot: one 8-byte read
#pragma unroll
        for (int kq = 0; kq < 2; ++kq) {
          const u32x2_t v = *reinterpret_cast<const u32x2_t*>(tile + (c16 + 16 * (2 * kq + hi)) * 16 + 8 * h);
          wv[nb2][kq] = v[0];
          wv[nb2][kq + 2] = v[1];
        }
        const int t4 = 2 * nb2 + c_l;
        sv[nb2] = bf16_to_f32(*reinterpret_cast<const uint16_t*>(sz + t4 * 32 + c16 * 2));
        const uint32_t zw = ZP ? *reinterpret_cast<const uint32_t*>(sz + 128 + t4 * 8 + (c16 >> 3) * 4) : 0u;
        const float z = ZP ? (float)((zw >> (4 * (c16 & 7))) & 0xFu) : 8.0f;
        zs[nb2] = -z * sv[nb2];
      }
    };
    // MXFP4 weights with bf16 rows: K = 64 h + 16 kq + 8 hi (the same K run
    // of the lane as for INT4, so the activation side is unchanged) is word
    // 2 (kq % 2) + hi of slot (l32 % 16) + 16 (2 h + kq / 2), scaled by the
    // E8M0 byte gsel of that slot's word (groups 4 (g / 4) + gsel)
    auto fetch_f4 = [&](const uint8_t* stg, int h, int gsel, uint32_t (&wv)[2][4], float (&sf)[2][2])
        __attribute__((always_inline)) {
      const uint8_t* sz = stg + kSOff + wave * 1024;
#pragma unroll
      for (int nb2 = 0; nb2 < 2; ++nb2) {
        const int t4 = 2 * nb2 + c_l;
        const uint8_t* tile = stg + kWOff + (NWT * wave + t4) * 1024;
#pragma unroll
        for (int kh = 0; kh < 2; ++kh) {
          const int slot = c16 + 16 * (2 * h + kh);
          wv[nb2][2 * kh] = *reinterpret_cast<const uint32_t*>(tile + slot * 16 + 4 * hi);
          wv[nb2][2 * kh + 1] = *reinterpret_cast<const uint32_t*>(tile + slot * 16 + 8 + 4 * hi);
          sf[nb2][kh] = e8m0_f32((*reinterpret_cast<const uint32_t*>(sz + t4 * 256 + slot * 4) >> (8 * gsel)) & 0xFFu) *
                        (I4 ? 0.25f : 1.0f);                   // MXINT4: q / 4
        }
      }
    };
    // INT8 weights (the step's half of a 2 KiB tile; per step, through the
    // ring of weight slots: at step s slot wso[1] holds step s + 1, wso[2]
    // step s + 2, and step s + 3 is copied into wso[0], free since step s's
    // operands were read during step s - 1):
    // K = 16 kq + 8 hi of the step is bytes 8 (kq / 2) .. + 7 of slot
    // (l32 % 16) + 16 (2 (kq % 2) + hi); one bf16 scale per column and group
    auto fetch8 = [&](const uint8_t* stg, u32x2_t (&wv8)[2][4], float (&sv)[2]) __attribute__((always_inline)) {
      const uint8_t* sz = stg + kSOff + wave * 256;
#pragma unroll
      for (int nb2 = 0; nb2 < 2; ++nb2) {
        const int t4 = 2 * nb2 + c_l;
        const uint8_t* tile = stg + kWOff + (NWT * wave + t4) * 1024;
        const u32x4_t va = ld16(tile + (c16 + 16 * hi) * 16), vb = ld16(tile + (c16 + 16 * (2 + hi)) * 16);
        wv8[nb2][0] = (u32x2_t){va[0], va[1]};
        wv8[nb2][1] = (u32x2_t){vb[0], vb[1]};
        wv8[nb2][2] = (u32x2_t){va[2], va[3]};
        wv8[nb2][3] = (u32x2_t){vb[2], vb[3]};
        sv[nb2] = bf16_to_f32(*reinterpret_cast<const uint16_t*>(sz + t4 * 32 + c16 * 2));
      }
    };
    // INT8: all four tiles' halves of step st and the scale gather of its group
    auto copy_w8 = [&](const Copy& c, int st, uint8_t* stage) __attribute__((always_inline)) {
#pragma unroll
      for (int k = 0; k < NWT; ++k)
        b2lds16(c.rw, c.wvo[k], (uint32_t)((st >> 1) * 2048 + (st & 1) * 1024), stage + kWOff + (NWT * wave + k) * 1024);
      b2lds4(rsz, c.svo[0] + (uint32_t)(st >> 1) * szstride, 0u, stage + kSOff + wave * 256);
    };
    u32x4_t af[2][4];
    u32x2_t w3c8[2] = {};                           // INT8: code bytes of operands (nb2, 3)
    uint32_t w3c[2] = {0u, 0u};                     // code words of operands (nb2, 3), their scales and offsets
    float sv3c[2] = {0.f, 0.f}, zs3c[2] = {0.f, 0.f};
    while (true) {
      const int64_t nitem = item + gridDim.x;
      const bool has_next = nitem < n_items;
      const BigTile nxt = has_next ? decode(nitem) : cur;
      int32_t prn[NPR] = {}, tpn = -1;
      if (!chained || first) {
        // stand-alone start: weights of steps 0, 1, 2 and activations of
        // steps 0, 1, then operands 0..2 of step 0
        if (!first) {
          __asm__ volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
          if (GROUPED) load_rows(cur, pr, tp);
          cc = make_copy(cur, pr);
        }
        write_table(tp);
        const int KGt = S >> 1;
        if (Q8) {
          copy_w8(cc, 0, lds + wso[0]);
          copy_w8(cc, std::min(1, S - 1), lds + wso[1]);
          copy_w8(cc, std::min(2, S - 1), lds + wso[2]);
        } else {
          copy_w(cc, 0, lds + wso[0]);
          copy_w(cc, std::min(1, KGt - 1), lds + wso[1]);
        }
        copy_x(cc, 0, lds + so[0]);
        copy_x(cc, std::min(1, S - 1), lds + so[1]);
        wait_barrier(std::integral_constant<int, 0>());
        uint32_t wv[2][4];
        if (Q8) {
          u32x2_t w8[2][4];
          fetch8(lds + wso[0], w8, sv3c);
#pragma unroll
          for (int nb2 = 0; nb2 < 2; ++nb2) {
#pragma unroll
            for (int kq = 0; kq < 3; ++kq) af[nb2][kq] = i8x8_bf16_scaled(w8[nb2][kq][0], w8[nb2][kq][1], sv3c[nb2]);
            af[nb2][3] = (u32x4_t){0u, 0u, 0u, 0u};
            w3c8[nb2] = w8[nb2][3];
          }
        } else if (F4) {
          float sf[2][2];
          fetch_f4(lds + wso[0], 0, 0, wv, sf);
#pragma unroll
          for (int nb2 = 0; nb2 < 2; ++nb2) {
#pragma unroll
            for (int kq = 0; kq < 3; ++kq)
              af[nb2][kq] = I4 ? i4x8_bf16(wv[nb2][kq], sf[nb2][kq >> 1]) : fp4x8_bf16(wv[nb2][kq], sf[nb2][kq >> 1]);
            af[nb2][3] = (u32x4_t){0u, 0u, 0u, 0u};
            w3c[nb2] = wv[nb2][3];
            sv3c[nb2] = sf[nb2][1];
          }
        } else {
          fetch(lds + wso[0], 0, wv, sv3c, zs3c);
#pragma unroll
          for (int nb2 = 0; nb2 < 2; ++nb2) {
#pragma unroll
            for (int kq = 0; kq < 3; ++kq) af[nb2][kq] = dq8_bytes(wv[nb2][kq], sv3c[nb2], zs3c[nb2]);
            af[nb2][3] = (u32x4_t){0u, 0u, 0u, 0u};
            w3c[nb2] = wv[nb2][3];
          }
        }
      }
      if (GROUPED && chained && has_next) load_rows(nxt, prn, tpn);
      Copy nc = cc;
      if (!GROUPED && chained && has_next) nc = make_copy(nxt, prn);

      f32x16_t acc[2][8];
#pragma unroll
      for (int nb2 = 0; nb2 < 2; ++nb2)
#pragma unroll
        for (int mb = 0; mb < 8; ++mb)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[nb2][mb][r] = 0.f;
      // Step s runs its MFMAs K part by K part (kq = 0..3; row blocks 0..MB-1,
      // each activation fragment feeding both column halves, so no
      // accumulator is updated twice in a row) with the fragments read kD
      // fragments ahead.  Operands (nb2, kq) are free once their MFMAs are
      // issued, so the unpacking follows behind: during K part 0 operands
      // (nb2, 3) of this step (from the words carried over), during K part
      // kq = 1..3 operands (nb2, kq - 1) of the next step (this tile's or, at
      // the last step, the next tile's first), 32 result words spread evenly
      // over the step's MFMA pairs.  The scheduling barriers keep this
      // interleaving as written.  Each step first issues the activations of
      // step s + 2 and the weights of step s + 3 (of this tile or the next,
      // else repeats of this tile's last step into parts no longer read), so
      // the wait count is exact.  A tile of at most 128 rows (a half tile, or
      // the last rows of M) runs only row blocks 0..3.
      constexpr int kD = 4;
      if (cur.rows > kBigM / 2) HM_BIG_W4A16_STEPS(8);
      else HM_BIG_W4A16_STEPS(4);

      // ---- epilogue: lane holds C[n = 64 w + 32 nb2 + 8 j + 4 hi + r][row = 32 mb + l32];
      // slab p holds row blocks 2 p and 2 p + 1 of every wave; the copies still
      // in flight finish first (the stores then never overtake a copy)
      __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
      uint8_t* ost = lds + so[2];                    // the last step's stage
      const int n_slabs = cur.rows > kBigM / 2 ? 4 : 2;
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        if (p < n_slabs) {
  #pragma unroll
          for (int mm = 0; mm < 2; ++mm) {
            const int mb = 2 * p + mm, r = 32 * mm + l32;
  #pragma unroll
            for (int nb2 = 0; nb2 < 2; ++nb2)
  #pragma unroll
              for (int j = 0; j < 4; ++j) {
                const int u = 16 * wave + 8 * nb2 + 2 * j + hi;
                *reinterpret_cast<u32x2_t*>(ost + r * 512 + (u ^ Swz16::swz(r)) * 8) =
                    (u32x2_t){pack_bf16(acc[nb2][mb][4 * j], acc[nb2][mb][4 * j + 1]),
                              pack_bf16(acc[nb2][mb][4 * j + 2], acc[nb2][mb][4 * j + 3])};
              }
          }
          lds_barrier();
          store_slab(cur, ost, p, Swz16());
          lds_barrier();
        }
      }
      if (!has_next) break;
      cur = nxt;
      cc = nc;
      tp = tpn;
      item = nitem;
      first = false;
    }
  }
  __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");   // no copy may land after the block ends
}

// Dense tiles that run whole; the rest of the visiting order runs as two
// 128-row halves.  When the tiles fill the persistent grid a whole number of
// rounds plus at most half a round (896 tiles of M = 4096, N = 14336 on 256
// CUs: 3.5), the last round's tiles are split so that every CU takes part in
// it; W4A16 only (the half tiles compute four of the eight row blocks), and
// not where the second half of a last tile row would be empty.

template <bool MX, bool ZP, bool GROUPED, bool A4 = false, bool F4 = false, bool I4 = false, bool Q8 = false>
static hipError_t go_big(const GemmArgs& a, int grid_items, hipStream_t st) {
  auto kern = &k_gemm_big<MX, ZP, GROUPED, A4, F4, I4, Q8>;
  static const hipError_t attr_err = hipFuncSetAttribute(
      reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize, big_lds_bytes(MX || F4, A4));
  if (attr_err != hipSuccess) return attr_err;
  const int tiles_n = (int)((a.G.NB + kBigCB - 1) / kBigCB);
  const int tiles_m = GROUPED ? 0 : (int)((a.M + kBigM - 1) / kBigM);
  // dense: one round of tiles, or a persistent grid of one block per CU
  // (a multiple of 8, so a block's items stay on its XCD)
  const int64_t tiles = (int64_t)tiles_n * tiles_m;
  const int n_full = GROUPED ? 0 : (int)big_full_tiles(a.G, a.M, MX);
  const int64_t items = GROUPED ? 0 : 2 * tiles - n_full;
  const unsigned grid = GROUPED ? (unsigned)(grid_items > 0 ? grid_items : 1)
                                : (unsigned)(items <= kBigGrid ? items : kBigGrid);
  hipLaunchKernelGGL(kern, dim3(grid), dim3(big_threads(MX)), big_lds_bytes(MX || F4, A4), st, a, tiles_n, tiles_m,
                     n_full);
  return hipGetLastError();
}


hipError_t launch_gemm_big(const GemmArgs& a, bool grouped, int grid_items, hipStream_t st) {
  if (kmode_of(a) == KM_INT8_A16)
    return grouped ? go_big<false, false, true, false, false, false, true>(a, grid_items, st)
                   : go_big<false, false, false, false, false, false, true>(a, 0, st);
  // scale and zero-point copies use 32-bit offsets from the scale region
  if (a.G.total - a.G.off_scales > 0xFFFFFFFFull) return hipErrorInvalidValue;
  if (kmode_of(a) == KM_MX_A4)
    return grouped ? go_big<true, false, true, true>(a, grid_items, st) : go_big<true, false, false, true>(a, 0, st);
  if (kmode_of(a) == KM_MX_A16)
    return grouped ? go_big<false, false, true, false, true>(a, grid_items, st)
                   : go_big<false, false, false, false, true>(a, 0, st);
  if (kmode_of(a) == KM_MXI4_A16)
    return grouped ? go_big<false, false, true, false, true, true>(a, grid_items, st)
                   : go_big<false, false, false, false, true, true>(a, 0, st);
  if (a.wfmt == W_MXFP4)
    return grouped ? go_big<true, false, true>(a, grid_items, st) : go_big<true, false, false>(a, 0, st);
  if (a.wfmt == W_UINT4_ZP)
    return grouped ? go_big<false, true, true>(a, grid_items, st) : go_big<false, true, false>(a, 0, st);
  return grouped ? go_big<false, false, true>(a, grid_items, st) : go_big<false, false, false>(a, 0, st);
}

}  // namespace hm
