// C ABI entry points: argument checks, tile-configuration choice and launches.
// Every check runs before any launch; the library allocates nothing.
#include <hip/hip_runtime.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <mutex>

#include "../../include/hm.h"
#include "common.h"
#include "launch.h"

#define HM_API extern "C" __attribute__((visibility("default")))

namespace {

using namespace hm;

constexpr int kStreamMaxRows = 32;   // dense rows of one streaming block (two 16-row blocks)
constexpr int64_t kStreamWideRows = 256;      // narrow-N dense calls stream up to this many rows ...
constexpr int64_t kStreamChunkCols = 16384;   // ... while 32-row chunks x N stays within this
constexpr int64_t kA8StreamChunkCols = 28672;  // W4A8 (FP8 rows, half the bytes): the same rule's limit
constexpr int64_t kStreamLdsBytes = 159 * 1024;  // dynamic LDS one streaming block may use
constexpr int kMoeStreamRows = 16;   // rows per grouped streaming unit
// Experts with at most this many rows use the streaming kernel (as units of
// kMoeStreamRows rows that share the expert's weights through the L2), with
// this many 16-column blocks per wave.  Measured on the 256-expert top-8
// workloads: W4A16 64 rows and two blocks per wave (T = 64 / 1024 / 8192:
// -19% / -5% / -5% against 16 rows and one block); MXFP4 rows keep 16 and one.
constexpr int kMoeStreamMaxA16 = 64, kMoeStreamNbwA16 = 2;
constexpr int kMoeStreamMaxMx = 16, kMoeStreamNbwMx = 1;
// FP8 rows (W4A8): 32-row units, experts of up to 128 rows streaming, two
// blocks per wave (T = 1024 gate_up / down 583 / 334 -> 504 / 313 us; T =
// 16384 0.3 / 1.2% faster), as dense W4A8 streams up to 128 rows
constexpr int kMoeStreamRowsA8 = 32, kMoeStreamMaxA8 = 128, kMoeStreamNbwA8 = 2;
// MXINT4 (bf16 rows): its streaming kernel is bound by the code conversion,
// so 32-row units (each conversion serving twice the rows) with experts of
// up to 128 rows streaming: T = 64 / 1024 / 8192 0.448 / 1.756 / 8.954 ms
// against 0.463 / 1.826 / 9.018 with 16-row units up to 64 rows
constexpr int kMoeStreamRowsMxi4 = 32, kMoeStreamMaxMxi4 = 128;
// LDS per grouped streaming block: 48 KiB (three blocks per CU; rows longer
// than that are staged in K pieces).  Measured against 79 KiB (two blocks),
// 256 experts top-8: INT4 T = 64 / 1024 / 8192 gate_up 250 / 905 / 4087 ->
// 205 / 835 / 4026 us, down 127 / 558 / 2347 -> 112 / 506 / 2318; MXFP4 bf16
// rows and FP8 rows 1-8% faster; 20-32 KiB (four or more blocks) no better
// than 79.  MXINT4 (32-row units) keeps 79 KiB: 48 was within +-3%.
constexpr int kMoeStreamLdsKb = 48, kMoeStreamLdsKbMxi4 = 79;
constexpr int64_t kBigMinRows = 512;  // dense rows from which 256 x 256 tiles may be used
// An expert remainder of at least this many rows gets a 256-row unit (a unit
// of at most 128 rows runs four of the eight 32-row MFMA blocks) instead of
// 128 x 64 tile units, which copy the unit's activation rows once per 64
// columns.  Measured against 192: W4A16 T = 1024 -12%, T = 8192 -2%; W4A8
// T = 16384 -3..4% (65 and 129 rows).  With K <= 2048 (a down projection:
// short K loops, so a 128 x 64 tile's staging weighs more) from 49 rows:
// N = 7168 K = 2048, T = 1024 -5..7% for bf16 rows (INT4, MXFP4), -2% for
// FP8 rows, T = 8192 within +-1%; with K = 7168 49 rows was 3-7% slower.
constexpr int kMoeBigMinRows = 97;
constexpr int kMoeBigMinRowsShortK = 49;
constexpr int64_t kMoeShortK = 2048;
constexpr int kGroupedGridStream = 2048;
constexpr int kGroupedGridTile = 1024;
constexpr int kGroupedGridMid = 256;     // one 128 x 64 tile block per compute unit (LDS-bound)
constexpr int kGroupedGridBig = 256;     // one 256-tile block per compute unit (LDS-bound)
constexpr uint64_t kAddr32 = 1ull << 32; // extent of one 32-bit buffer offset

enum Path : int { P_AUTO = 0, P_STREAM = 1, P_MID = 2, P_BIG = 3, P_TILE = 4 };

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

hm_status check_desc(const hm_wdesc* d) {
  if (!d) return HM_ERR_NULL;
  if (d->abi != HM_ABI_VERSION) return HM_ERR_ABI;
  if (d->wfmt < HM_W_INT4_SYM || d->wfmt > HM_W_INT8_SYM) return HM_ERR_UNSUPPORTED;
  const int want_group = is_mx(d->wfmt) ? 32 : 128;
  if (d->group != want_group) return HM_ERR_SHAPE;
  if (d->num_experts < 1 || d->num_experts > 512 || d->n < 1 || d->k < 128 || (d->k % 128) != 0)
    return HM_ERR_SHAPE;
  if (d->n > (1ll << 24) || d->k > (1ll << 20)) return HM_ERR_SHAPE;
  return HM_OK;
}

hm_status check_pair(const hm_wdesc* d, int32_t afmt) {
  if (afmt != HM_A_BF16 && afmt != HM_A_FP8_ROWSCALE && afmt != HM_A_MXFP4) return HM_ERR_UNSUPPORTED;
  // FP8 and MXFP4 rows pair with MXFP4 weights only; bf16 rows with every format
  if (afmt != HM_A_BF16 && d->wfmt != HM_W_MXFP4) return HM_ERR_UNSUPPORTED;
  return HM_OK;
}

// MX weights (MXFP4, MXINT4) with bf16 rows (codes scaled to bf16 inside the kernels)
bool mx_a16(const hm_wdesc* d, int32_t afmt) { return is_mx(d->wfmt) && afmt == HM_A_BF16; }

const char* pair_name(const hm_wdesc* d, int32_t afmt) {
  if (d->wfmt == HM_W_MXFP4) return afmt == HM_A_BF16 ? "w4a16-mxfp4" : (afmt == HM_A_MXFP4 ? "w4a4-mxfp4" : "w4a8-mxfp4");
  if (d->wfmt == HM_W_MXINT4) return "w4a16-mxint4";
  if (d->wfmt == HM_W_UINT3_ZP) return "w3a16-uint3zp";
  if (d->wfmt == HM_W_UINT2_ZP) return "w2a16-uint2zp";
  if (d->wfmt == HM_W_INT8_SYM) return "w8a16-int8sym";
  return d->wfmt == HM_W_UINT4_ZP ? "w4a16-uint4zp" : "w4a16-int4sym";
}

// the device layout's geometry (3- and 2-bit zero-point formats use the 4-bit one)
Geom geom_of(const hm_wdesc* d) { return make_geom(device_fmt(d->wfmt), d->num_experts, d->n, d->k); }

// The 128-row and 256-row tile kernels address the scale / zero-point region
// with 32-bit offsets from its start.
bool scales_addr32(const Geom& G) { return G.total - G.off_scales < kAddr32; }

// ---------------------------------------------------------------- tuning
struct Tune {
  int path, sks, snbw, ssplits, swaves, mrows, mmax, mnbw, mks, mlds, mbig, mtile;
};

bool in_set(int v, std::initializer_list<int> ok) {
  for (int x : ok)
    if (v == x) return true;
  return false;
}

hm_status read_tuning(const hm_tuning* t, Tune* out) {
  *out = Tune{};
  if (!t) return HM_OK;
  if (t->abi != HM_ABI_VERSION) return HM_ERR_ABI;
  const bool ok = in_set(t->path, {0, 1, 2, 3, 4}) && in_set(t->stream_ks, {0, 1, 2, 4, 8}) &&
                  in_set(t->stream_nbw, {0, 1, 2}) && t->stream_splits >= 0 &&
                  in_set(t->stream_waves, {0, 4, 8}) && !(t->stream_ks == 8 && t->stream_waves != 8) &&
                  !(t->stream_ks == 1 && t->stream_waves == 8) &&
                  in_set(t->moe_stream_rows, {0, 16, 32}) && t->moe_stream_max >= 0 &&
                  t->moe_stream_max <= 4096 && in_set(t->moe_stream_nbw, {0, 1, 2}) &&
                  in_set(t->moe_stream_ks, {0, 1, 2, 4}) &&
                  (t->moe_stream_lds_kb == 0 || (t->moe_stream_lds_kb >= 20 && t->moe_stream_lds_kb <= 159)) &&
                  t->moe_big_min >= -1 && t->moe_big_min <= kBigRows && in_set(t->moe_tile, {0, 1, 2});
  if (!ok) return HM_ERR_TUNING;
  *out = Tune{t->path, t->stream_ks, t->stream_nbw, t->stream_splits, t->stream_waves, t->moe_stream_rows, t->moe_stream_max,
              t->moe_stream_nbw, t->moe_stream_ks, t->moe_stream_lds_kb, t->moe_big_min, t->moe_tile};
  return HM_OK;
}

// ---------------------------------------------------------------- dense plan
struct DensePlan {
  int path;          // P_STREAM, P_MID (128-row tiles), P_BIG (256 x 256), P_TILE (128 x 128)
  StreamCfg sc;
  int ksg;
  size_t ws_bytes;
};

// one block per tile of the dense 128-row tile kernels (a 32-bit grid)
bool mid_grid_fits(const Geom& G, bool a8, int64_t m) {
  const int64_t tiles_m = a8 ? (m + 63) / 64 : (m + kTileM - 1) / kTileM;
  const int64_t tiles_n = a8 ? (G.NB + 7) / 8 : mid_n_tiles(G, false);
  return tiles_n * tiles_m <= 0x7FFFFFFFll;
}

// Dense rows: the 128 x 128 kernel's grid has one block row per 128 rows.
constexpr int64_t kMaxDenseRows = 65535ll * kTileM;

hm_status plan_dense(const hm_wdesc* d, int32_t afmt, int64_t m, const Tune& tu, DensePlan* out) {
  DensePlan p{};
  if (m < 1 || m > kMaxDenseRows) return HM_ERR_SHAPE;
  const Geom G = geom_of(d);
  const bool f4 = mx_a16(d, afmt);
  const bool a8 = afmt == HM_A_FP8_ROWSCALE;
  const bool a4 = afmt == HM_A_MXFP4;
  const bool tiles32 = scales_addr32(G);        // 128-row and 256-row kernels can address the scales
  if (tu.path == P_STREAM && m > kStreamWideRows) return HM_ERR_TUNING;
  // W4A4 and INT8 weights have no 128-row tile kernel
  const bool int8 = d->wfmt == HM_W_INT8_SYM;
  const bool no_mid = a4 || int8;
  if (no_mid && tu.path == P_MID) return HM_ERR_TUNING;
  if ((tu.path == P_MID || tu.path == P_BIG) && (!tiles32 || !mid_grid_fits(G, a8, m))) return HM_ERR_TUNING;
  // W4A16 up to 256 rows also streams (in 32-row chunks, each re-reading the
  // weights from the L2) when N is narrow: measured at K = 4096, a streaming
  // launch costs ~8 us + 0.8 ns per (chunk x column) and a round of 128 x 64
  // tiles 23-25 us, so chunks x N <= 16384 streams (N = 1792, M = 128: 14.9
  // against 23.4 us; N = 7168, M = 128 stays on tiles: 25.3 against 28.8 us)
  const bool narrow = !is_mx(d->wfmt) && m <= kStreamWideRows &&
                      ((m + kStreamMaxRows - 1) / kStreamMaxRows) * d->n <= kStreamChunkCols;
  // W4A8 chunks: eight-wave blocks of four column sets (K split over two
  // waves), one column block per wave for two chunks and two for more; taken
  // where that grid has at least 128 blocks without a K split (measured up to
  // four chunks)
  const int64_t a8_nchunks = (m + kStreamMaxRows - 1) / kStreamMaxRows;
  const int a8_nbw = a8_nchunks <= 2 ? 1 : 2;
  const bool a8_chunks = a8 && m > kStreamMaxRows && m <= 4 * kStreamMaxRows &&
                         a8_nchunks * d->n <= kA8StreamChunkCols &&
                         (G.NB + 4 * a8_nbw - 1) / (4 * a8_nbw) * a8_nchunks >= 128;
  if (tu.path != P_AUTO) {
    p.path = tu.path;
  } else if (m <= kStreamMaxRows || narrow || (a4 && m <= kStreamWideRows) || a8_chunks) {
    // (W4A4 rows are 1/4 of bf16 bytes: streaming 32-row chunks beats the
    // 128 x 128 tiles up to 256 rows, N = 7168 K = 2048: M = 64 7.0 against
    // 15.5 us, M = 256 12.4 against 18.1.  W4A8 likewise while chunks x N
    // <= 28672, N = 7168 K = 2048: M = 64 6.1 against 9.3 us on 64 x 128
    // tiles, M = 128 7.6 against 9.6; M = 256 stays on tiles, 10.1 against
    // 10.8)
    p.path = P_STREAM;
  } else if (int8) {
    // INT8: 128 x 128 or 256 x 256 tiles by the round costs of the MX
    // bf16-row choice below (the same two kernels' step loops)
    const int64_t mt = (m + kTileM - 1) / kTileM, bt = (m + kBigRows - 1) / kBigRows;
    const int64_t c_tile = 170 * ((((G.NB + 7) / 8) * mt + 255) / 256) + 120;
    const int64_t c_big = 580 * std::max<int64_t>(big_n_tiles(G) * bt, 256) / 256;
    p.path = c_big < c_tile ? P_BIG : P_TILE;
  } else if (a4) {
    // W4A4: 128 x 128 or 256 x 256 tiles by the round costs of the MX bf16-row
    // choice below (M = 512, N = 7168: 16.9 against 23.5 us; M = 4096 on
    // 256 x 256 tiles)
    const int64_t mt = (m + kTileM - 1) / kTileM, bt = (m + kBigRows - 1) / kBigRows;
    const int64_t c_tile = 170 * ((((G.NB + 7) / 8) * mt + 255) / 256) + 120;
    const int64_t c_big = 580 * std::max<int64_t>(big_n_tiles(G) * bt, 256) / 256;
    p.path = c_big < c_tile ? P_BIG : P_TILE;
  } else if (f4) {
    // MX weights with bf16 rows: the kernel with the least estimated time
    // (0.1 us per 2048 of K), fitted to MXFP4 and MXINT4 at N = 7168 K = 2048
    // and N = 14336 K = 4096, M = 256 .. 4096: 128 x 64 tiles 13.4 a round of
    // the chip, 128 x 128 tiles 17 a round plus 12, 256 x 256 tiles 58 a round
    // (fractional: the last round's half tiles) and at least one round.
    // Picks: N = 7168, M = 512 128 x 64 (28.0 us against 34.4 / 55.4), M =
    // 1024 128 x 128 (45.8 against 53.5 / 57.3), M = 4096 256 x 256 (116.8
    // against 272.6 / 142.8); N = 14336, M = 512 128 x 128 (83.3 against
    // 96.8 / 106.4), M = 1024 and 4096 256 x 256 (114.0, 409.8)
    const int64_t mt = (m + kTileM - 1) / kTileM, bt = (m + kBigRows - 1) / kBigRows;
    const int64_t c_mid = 134 * ((mid_n_tiles(G, false) * mt + 255) / 256) + 10;
    const int64_t c_tile = 170 * ((((G.NB + 7) / 8) * mt + 255) / 256) + 120;
    const int64_t c_big = 580 * std::max<int64_t>(big_n_tiles(G) * bt, 256) / 256;
    p.path = (c_big < c_mid && c_big < c_tile) ? P_BIG : (c_tile < c_mid ? P_TILE : P_MID);
  } else {
    // 256 x 256 tiles unless 128 x 64 tiles take fewer rounds of the chip by
    // the measured cost of a round (one of 256 x 256 tiles ~ 3.8 of 128 x 64
    // tiles, N = 1792 / 7168 / 14336, K = 4096): a narrow N (one rank's
    // column shard, N = 1792, M = 1024: 28 large tiles) runs 3.5x faster on
    // the smaller tiles
    const int64_t big_rounds = (big_n_tiles(G) * ((m + kBigRows - 1) / kBigRows) + 255) / 256;
    const int64_t mid_rounds = (mid_n_tiles(G, false) * ((m + kTileM - 1) / kTileM) + 255) / 256;
    const bool mid_fewer = (!is_mx(d->wfmt) || f4) && mid_rounds * 10 < big_rounds * 38;
    p.path = (m >= kBigMinRows && !mid_fewer) ? P_BIG : P_MID;
  }
  // kernels with 32-bit offsets fall back to the 128 x 128 kernel (64-bit addressing)
  if (tu.path == P_AUTO && (p.path == P_MID || p.path == P_BIG) && (!tiles32 || !mid_grid_fits(G, a8, m)))
    p.path = P_TILE;
  if (p.path != P_STREAM) {
    *out = p;
    return HM_OK;
  }
  p.sc.mb = (m <= 16) ? 1 : 2;
  const int64_t rows = (m < 16 * p.sc.mb) ? m : 16 * p.sc.mb;
  const int64_t m_chunks = (m + 16 * p.sc.mb - 1) / (16 * p.sc.mb);
  const int64_t gb = a8 ? 128 : (a4 ? 68 : 256);   // activation bytes per row per group (A4: + scales)
  // Launch shape: (ks, nbw) from the narrowest block (most waves, least work
  // per wave) to the widest, take the first whose blocks all fit on the chip
  // at once.  A block keeps its activation rows in LDS, so the LDS footprint
  // decides how many blocks share a compute unit (at most 5: the register
  // budget allows 5 waves per SIMD).
  // (ks, nbw) per block width, narrowest block first
  static const int kShapes4[6][2] = {{4, 1}, {2, 1}, {4, 2}, {2, 2}, {1, 1}, {1, 2}};
  static const int kShapes8[6][2] = {{8, 1}, {4, 1}, {8, 2}, {2, 1}, {4, 2}, {2, 2}};
  const int64_t row_bytes = std::min<int64_t>(G.KG * gb + 16, kStreamLdsBytes / rows);
  // the first shape (matching the forced fields) whose blocks all fit on the
  // chip at once; per_cu returns the blocks one compute unit holds
  auto search = [&](int nw, int ks, int nbw, int* pick, int64_t* per_cu) {
    const int (*shapes)[2] = nw == 8 ? kShapes8 : kShapes4;
    *pick = -1;
    for (int i = 0; i < 6; ++i) {
      const int cks = shapes[i][0], cnbw = shapes[i][1];
      if ((ks && cks != ks) || (nbw && cnbw != nbw)) continue;
      if (G.KG < 2 * cks && cks > 1 && !ks) continue;         // >= 2 groups per wave
      StreamCfg t = p.sc;
      t.ks = cks;
      t.nbw = cnbw;
      t.nw = nw;
      const int64_t lds = rows * row_bytes + (cks > 1 ? nw * cnbw * p.sc.mb * 1024 : 0);
      // blocks per compute unit: LDS, and at most 20 waves (the register budget)
      *per_cu = std::max<int64_t>(1, std::min<int64_t>(20 / nw, kStreamLdsBytes / lds));
      *pick = i;
      if (stream_n_tiles(G, t) * m_chunks <= 256 * *per_cu) break;
    }
    return shapes;
  };
  int ks = tu.sks, nbw = tu.snbw, nw = tu.swaves ? tu.swaves : (ks == 8 ? 8 : 4);
  // W4A4 in several 32-row chunks: two column blocks per wave, so each
  // block stages its rows for twice the columns (N = 7168 K = 2048, M = 256:
  // 12.4 against 16.6 us with one)
  if (a4 && m_chunks > 1 && !nbw) nbw = 2;
  // W4A8 in several 32-row chunks (N = 7168 K = 2048: M = 64 6.1 us against
  // 7.2 for the first shape that fits, M = 128 7.6 against 8.3; a K split
  // over two blocks doubled the time)
  const bool a8_shape = a8_chunks && tu.path == P_AUTO && !ks && !nbw && !tu.swaves;
  if (a8_shape) {
    nw = 8;
    ks = 2;
    nbw = a8_nbw;
  }
  if (!ks || !nbw) {
    int pick;
    int64_t per_cu;
    const int (*shapes)[2] = search(nw, ks, nbw, &pick, &per_cu);
    // A block whose staged rows fill a compute unit's LDS runs alone on it:
    // eight waves then share the rows (measured at N = 14336, K = 4096: M =
    // 16 15.9 -> 15.4 us, M = 32 21.5 -> 18.4 us; M = 1, five blocks per
    // compute unit, gains nothing)
    if (!tu.swaves && ks != 1 && pick >= 0 && per_cu == 1) {
      int pick8;
      int64_t per_cu8;
      const int (*shapes8)[2] = search(8, ks, nbw, &pick8, &per_cu8);
      if (pick8 >= 0) {
        shapes = shapes8;
        pick = pick8;
        nw = 8;
      }
    }
    if (pick < 0) return HM_ERR_TUNING;                        // no shape matches the forced fields
    ks = shapes[pick][0];
    nbw = shapes[pick][1];
  }
  p.sc.ks = ks;
  p.sc.nbw = nbw;
  p.sc.nw = nw;
  const int64_t n_tiles = stream_n_tiles(G, p.sc);
  int64_t splits = tu.ssplits;
  if (splits > G.KG) return HM_ERR_TUNING;
  if (splits <= 0 && a8_shape) splits = 1;
  if (splits <= 0) {
    // enough waves to keep every SIMD streaming (1024 SIMDs); split K over
    // blocks only below that
    const int64_t target_waves = 800;
    const int64_t waves = n_tiles * 4 * m_chunks;
    splits = (target_waves + waves - 1) / waves;
  }
  if (splits > G.KG) splits = G.KG;
  if (splits < 1) splits = 1;
  if (splits > 65535 || n_tiles > 0x7FFFFFFFll) return HM_ERR_SHAPE;
  p.ksg = (int)((G.KG + splits - 1) / splits);
  p.sc.splits = (int)((G.KG + p.ksg - 1) / p.ksg);
  p.ws_bytes = (p.sc.splits > 1) ? (size_t)p.sc.splits * m * G.NB * 16 * sizeof(float) : 0;
  *out = p;
  return HM_OK;
}

// ---------------------------------------------------------------- MoE plan
struct MoePlan {
  int64_t P, max_s, max_t, max_b;
  size_t off_su, off_tu, off_bu, ws_bytes;
  int nbw, ks, lds_kb, s_rows, s_max;
  int big_min;       // 0: no 256-row units
  int tile;          // kernel of the up-to-128-row units: P_MID or P_TILE
  bool a64;          // activations of 4 GiB or more (64-bit row addressing only)
};

// Work-list sizes and workspace layout (independent of the activation size);
// kernel choices need rows_are_pairs (< 0: sizes only).
hm_status plan_moe(const hm_wdesc* d, int32_t afmt, int64_t t, int32_t topk, int rows_are_pairs,
                   const Tune& tu, MoePlan* out, bool gated = false) {
  MoePlan p{};
  p.P = t * topk;
  const int64_t act = (p.P < d->num_experts) ? p.P : d->num_experts;
  const bool mxi4 = d->wfmt == HM_W_MXINT4;
  const bool a8 = afmt != HM_A_BF16;          // FP8 or MXFP4 rows
  const bool a4 = afmt == HM_A_MXFP4;
  const bool f4 = mx_a16(d, afmt);
  const bool fp8 = afmt == HM_A_FP8_ROWSCALE;
  p.s_rows = tu.mrows ? tu.mrows : (fp8 ? kMoeStreamRowsA8 : (mxi4 ? kMoeStreamRowsMxi4 : kMoeStreamRows));
  p.s_max = tu.mmax ? tu.mmax
                    : (fp8 ? kMoeStreamMaxA8 : (a8 ? kMoeStreamMaxMx : (mxi4 ? kMoeStreamMaxMxi4 : kMoeStreamMaxA16)));
  p.nbw = tu.mnbw ? tu.mnbw : (fp8 ? kMoeStreamNbwA8 : (a8 ? kMoeStreamNbwMx : kMoeStreamNbwA16));
  if (gated) {
    // the gated epilogue pairs a wave's two column blocks (gate, up)
    if (d->n % 32 != 0) return HM_ERR_SHAPE;
    if (tu.mnbw == 1) return HM_ERR_TUNING;
    p.nbw = 2;
  }
  p.ks = tu.mks ? tu.mks : 1;
  p.lds_kb = tu.mlds ? tu.mlds : (mxi4 ? kMoeStreamLdsKbMxi4 : kMoeStreamLdsKb);
  // an expert remainder of at least big_min rows takes a 256-row unit
  const int big_min = tu.mbig > 0 ? tu.mbig : (d->k <= kMoeShortK ? kMoeBigMinRowsShortK : kMoeBigMinRows);
  p.max_s = p.P / p.s_rows + act;
  p.max_t = (p.P + kTileM - 1) / kTileM + act;
  p.max_b = p.P / big_min + 1;              // every 256-row unit holds >= big_min rows
  p.off_su = 256;
  p.off_tu = align256(p.off_su + (size_t)p.max_s * 16);
  p.off_bu = align256(p.off_tu + (size_t)p.max_t * 16);
  p.ws_bytes = align256(p.off_bu + (size_t)p.max_b * 16);
  if (rows_are_pairs >= 0) {
    const Geom G = geom_of(d);
    const int64_t a_rows = rows_are_pairs ? p.P : t;
    p.a64 = (uint64_t)a_rows * (uint64_t)d->k * (a4 ? 1u : (a8 ? 2u : 4u)) >= 2 * kAddr32;
    const bool tiles32 = scales_addr32(G);
    // 256-row units address activation rows and scales with 32-bit offsets
    const bool int8 = d->wfmt == HM_W_INT8_SYM;
    const bool tile_only = a4 || int8;                       // no 128-row tile kernel
    const bool big_ok = !p.a64 && tiles32;
    if (tu.mbig > 0 && !big_ok) return HM_ERR_TUNING;
    p.big_min = (tu.mbig == -1 || !big_ok) ? 0 : big_min;
    // up-to-128-row units: the 128-row tile kernel (32-bit offsets), or the
    // 128 x 128 kernel for MX weights with bf16 rows when all pairs in
    // 128-row units would take many rounds of 128 x 64 tiles (T = 8192:
    // 7.92 against 8.30 ms)
    const bool mid_ok = !tile_only && !p.a64 && tiles32;
    if (tu.mtile == 1 && !mid_ok) return HM_ERR_TUNING;
    if (tu.mtile == 1) p.tile = P_MID;
    else if (tu.mtile == 2) p.tile = P_TILE;
    else p.tile = mid_ok ? P_MID : P_TILE;
  }
  *out = p;
  return HM_OK;
}


// The launches of one grouped GEMM: the schedule, then the grouped streaming,
// 128-row and 256-row unit kernels (each a persistent grid over its units).
hm_status launch_moe(const hm_wdesc* d, int32_t afmt, const void* w_dev, const void* a_in, const void* a_scales,
                     int32_t a_rows_are_pairs, int64_t t, int32_t topk, const int32_t* offsets,
                     const int32_t* sorted_pairs, uint16_t* y, uint8_t* w8, const MoePlan& p, hipStream_t stream,
                     bool gated = false) {
  int32_t* hdr = (int32_t*)w8;
  int32_t* su = (int32_t*)(w8 + p.off_su);
  int32_t* tu = (int32_t*)(w8 + p.off_tu);
  int32_t* bu = (int32_t*)(w8 + p.off_bu);
  GemmArgs a{};
  a.w = (const uint8_t*)w_dev;
  a.G = geom_of(d);
  a.wfmt = device_fmt(d->wfmt);
  a.a8 = afmt == HM_A_FP8_ROWSCALE;
  a.a4 = afmt == HM_A_MXFP4;
  a.x = a_in;
  a.xs = a.a8 ? (const float*)a_scales : nullptr;
  a.xsb = a.a4 ? (const uint8_t*)a_scales : nullptr;
  a.M = 0;
  a.y = y;
  a.hdr = hdr;
  a.sorted_pairs = sorted_pairs;
  a.topk = topk;
  a.rows_are_pairs = a_rows_are_pairs;
  a.P = p.P;
  a.gated = gated ? 1 : 0;
  (void)t;
  hipError_t e = launch_moe_schedule(offsets, d->num_experts, p.P, p.s_rows, p.s_max, kTileM, p.big_min,
                                     p.max_s, p.max_t, p.max_b, hdr, su, tu, bu, stream);
  if (e == hipSuccess) {
    StreamCfg sc{p.s_rows / 16, p.nbw, 1, p.ks, p.lds_kb, 4};
    const int64_t nts = stream_n_tiles(a.G, sc);
    int64_t gi = p.max_s * nts;
    if (gi > kGroupedGridStream) gi = kGroupedGridStream;
    a.units = su;
    if (gi > 0) e = launch_gemm_stream(a, sc, true, (int)gi, stream);
  }
  if (e == hipSuccess) {
    const bool mid = p.tile == P_MID;
    const int64_t ntt = mid ? mid_n_tiles(a.G, a.a8) : (a.G.NB + 7) / 8;
    int64_t gi = p.max_t * ntt;
    const int64_t cap = mid ? kGroupedGridMid : kGroupedGridTile;
    if (gi > cap) gi = cap;
    a.units = tu;
    if (gi > 0) e = mid ? launch_gemm_mid(a, true, (int)gi, stream) : launch_gemm_tile(a, true, (int)gi, stream);
  }
  if (e == hipSuccess && p.big_min > 0) {
    int64_t gi = p.max_b * big_n_tiles(a.G);
    if (gi > kGroupedGridBig) gi = kGroupedGridBig;
    a.units = bu;
    if (gi > 0) e = launch_gemm_big(a, true, (int)gi, stream);
  }
  return (e == hipSuccess) ? HM_OK : HM_ERR_HIP;
}

}  // namespace

// =====================================================================================

HM_API const char* hm_status_string(int32_t s) {
  switch (s) {
    case HM_OK: return "ok";
    case HM_ERR_NULL: return "null pointer";
    case HM_ERR_SHAPE: return "bad shape, group or count";
    case HM_ERR_ALIGN: return "misaligned pointer";
    case HM_ERR_UNSUPPORTED: return "unsupported format or format/activation pair";
    case HM_ERR_WORKSPACE: return "workspace too small";
    case HM_ERR_HIP: return "HIP launch failed";
    case HM_ERR_ABI: return "descriptor ABI version mismatch";
    case HM_ERR_TUNING: return "tuning field out of range, or the forced kernel cannot run this call";
  }
  return "unknown status";
}

HM_API hm_status hm_transform_size(const hm_wdesc* d, size_t* bytes) {
  hm_status s = check_desc(d);
  if (s) return s;
  if (!bytes) return HM_ERR_NULL;
  *bytes = geom_of(d).total;
  return HM_OK;
}

static hm_status transform_impl(const hm_wdesc* d, const uint8_t* codes, const void* scales,
                                const uint8_t* zeros, void* w_dev, size_t w_bytes, bool gated,
                                hipStream_t stream) {
  hm_status s = check_desc(d);
  if (s) return s;
  if (gated && d->n % 32 != 0) return HM_ERR_SHAPE;
  if (!codes || !scales || !w_dev) return HM_ERR_NULL;
  if (device_fmt(d->wfmt) == HM_W_UINT4_ZP && !zeros) return HM_ERR_NULL;
  if (!aligned(codes, 16) || !aligned(w_dev, 256)) return HM_ERR_ALIGN;
  if (!aligned(scales, is_mx(d->wfmt) ? 1 : 2)) return HM_ERR_ALIGN;
  const Geom G = geom_of(d);
  if (w_bytes < G.total) return HM_ERR_WORKSPACE;
  if (launch_transform(d->wfmt, G, codes, scales, zeros, (uint8_t*)w_dev, gated ? 1 : 0, stream) != hipSuccess)
    return HM_ERR_HIP;
  return HM_OK;
}

HM_API hm_status hm_transform(const hm_wdesc* d, const uint8_t* codes, const void* scales,
                              const uint8_t* zeros, void* w_dev, size_t w_bytes,
                              hipStream_t stream) {
  return transform_impl(d, codes, scales, zeros, w_dev, w_bytes, false, stream);
}

HM_API hm_status hm_transform_gated(const hm_wdesc* d, const uint8_t* codes, const void* scales,
                                    const uint8_t* zeros, void* w_dev, size_t w_bytes,
                                    hipStream_t stream) {
  return transform_impl(d, codes, scales, zeros, w_dev, w_bytes, true, stream);
}

HM_API hm_status hm_dequant(const hm_wdesc* d, const void* w_dev, size_t w_bytes, int32_t expert,
                            float* out, hipStream_t stream) {
  hm_status s = check_desc(d);
  if (s) return s;
  if (!w_dev || !out) return HM_ERR_NULL;
  if (!aligned(w_dev, 256) || !aligned(out, 16)) return HM_ERR_ALIGN;
  if (expert < 0 || expert >= d->num_experts) return HM_ERR_SHAPE;
  const Geom G = geom_of(d);
  if (w_bytes < G.total) return HM_ERR_WORKSPACE;
  if (launch_dequant(device_fmt(d->wfmt), G, (const uint8_t*)w_dev, expert, out, stream) != hipSuccess)
    return HM_ERR_HIP;
  return HM_OK;
}

HM_API hm_status hm_quant_fp8_rows(const uint16_t* x, int64_t m, int64_t k, uint8_t* x8,
                                   float* row_scale, hipStream_t stream) {
  if (m < 0 || k < 1) return HM_ERR_SHAPE;
  if (m == 0) return HM_OK;
  if (!x || !x8 || !row_scale) return HM_ERR_NULL;
  if (!aligned(x, 16) || !aligned(x8, 16) || !aligned(row_scale, 16)) return HM_ERR_ALIGN;
  if (launch_quant_fp8_rows(x, m, k, x8, row_scale, stream) != hipSuccess) return HM_ERR_HIP;
  return HM_OK;
}

HM_API hm_status hm_quant_mxfp4_rows(const uint16_t* x, int64_t m, int64_t k, uint8_t* codes, uint8_t* scales,
                                     hipStream_t stream) {
  if (m < 0 || k < 32 || (k % 32) != 0) return HM_ERR_SHAPE;
  if (m == 0) return HM_OK;
  if (!x || !codes || !scales) return HM_ERR_NULL;
  if (!aligned(x, 16) || !aligned(codes, 16)) return HM_ERR_ALIGN;
  if (launch_quant_mxfp4_rows(x, m, k, codes, scales, stream) != hipSuccess) return HM_ERR_HIP;
  return HM_OK;
}

HM_API hm_status hm_silu_mul(const uint16_t* gu, int64_t rows, int64_t d, uint16_t* h, hipStream_t stream) {
  if (rows < 0 || d <= 0) return HM_ERR_SHAPE;
  if (rows == 0) return HM_OK;
  if (!gu || !h) return HM_ERR_NULL;
  if (!aligned(gu, 16) || !aligned(h, 16)) return HM_ERR_ALIGN;
  // one thread per 16-byte chunk (or per element): the grid's x extent is 32-bit
  if ((rows * d + 255) / 256 > 0x7FFFFFFFll) return HM_ERR_SHAPE;
  if (launch_silu_mul(gu, rows, d, h, stream) != hipSuccess) return HM_ERR_HIP;
  return HM_OK;
}

HM_API hm_status hm_silu_mul_fp8(const uint16_t* gu, int64_t rows, int64_t d, uint8_t* h8, float* h_scales,
                                 hipStream_t stream) {
  if (rows < 0 || d <= 0 || (d % 8) != 0 || d > 8192) return HM_ERR_SHAPE;
  if (rows == 0) return HM_OK;
  if (!gu || !h8 || !h_scales) return HM_ERR_NULL;
  if (!aligned(gu, 16) || !aligned(h8, 16) || !aligned(h_scales, 4)) return HM_ERR_ALIGN;
  if (launch_silu_mul_fp8(gu, rows, d, h8, h_scales, stream) != hipSuccess) return HM_ERR_HIP;
  return HM_OK;
}

HM_API hm_status hm_moe_combine(const uint16_t* y, const float* w, int64_t t, int32_t topk, int64_t n,
                                uint16_t* out, hipStream_t stream) {
  if (t < 0 || n <= 0 || topk < 1) return HM_ERR_SHAPE;
  if (t == 0) return HM_OK;
  if (!y || !w || !out) return HM_ERR_NULL;
  if (!aligned(y, 16) || !aligned(out, 16) || !aligned(w, 4)) return HM_ERR_ALIGN;
  if ((t * n + 255) / 256 > 0x7FFFFFFFll) return HM_ERR_SHAPE;
  if (launch_combine(y, w, t, topk, n, out, stream) != hipSuccess) return HM_ERR_HIP;
  return HM_OK;
}

HM_API hm_status hm_read_probe(const void* buf, int64_t bytes, int32_t blocks, int32_t unroll, uint32_t* out,
                               hipStream_t stream) {
  if (bytes <= 0 || (bytes % 16) != 0 || blocks < 1 || blocks > 65535) return HM_ERR_SHAPE;
  if (unroll != 1 && unroll != 2 && unroll != 4 && unroll != 8) return HM_ERR_SHAPE;
  if (!buf || !out) return HM_ERR_NULL;
  if (!aligned(buf, 16) || !aligned(out, 4)) return HM_ERR_ALIGN;
  return launch_read_probe(buf, bytes, blocks, unroll, out, stream) == hipSuccess ? HM_OK : HM_ERR_HIP;
}

HM_API hm_status hm_gemm_workspace_size(const hm_wdesc* d, int32_t afmt, int64_t m, const hm_tuning* tune,
                                        size_t* bytes) {
  hm_status s = check_desc(d);
  if (s) return s;
  if ((s = check_pair(d, afmt))) return s;
  if (!bytes) return HM_ERR_NULL;
  if (m < 0) return HM_ERR_SHAPE;
  Tune tu;
  if ((s = read_tuning(tune, &tu))) return s;
  if (m == 0) {
    *bytes = 0;
    return HM_OK;
  }
  DensePlan p;
  if ((s = plan_dense(d, afmt, m, tu, &p))) return s;
  *bytes = p.ws_bytes;
  return HM_OK;
}

HM_API hm_status hm_gemm_plan(const hm_wdesc* d, int32_t afmt, int64_t m, const hm_tuning* tune, char* buf,
                              size_t buf_len) {
  hm_status s = check_desc(d);
  if (s) return s;
  if ((s = check_pair(d, afmt))) return s;
  if (!buf || buf_len == 0) return HM_ERR_NULL;
  if (m < 0) return HM_ERR_SHAPE;
  Tune tu;
  if ((s = read_tuning(tune, &tu))) return s;
  DensePlan p;
  if ((s = plan_dense(d, afmt, m > 0 ? m : 1, tu, &p))) return s;
  const char* w = pair_name(d, afmt);
  const bool a8 = afmt != HM_A_BF16;        // scaled f8f6f4 MFMA (FP8 or MXFP4 rows)
  if (p.path == P_STREAM)
    snprintf(buf, buf_len, "%s stream mb=%d nbw=%d ks=%d waves=%d splits=%d ksg=%d mfma=%s", w, p.sc.mb,
             p.sc.nbw, p.sc.ks, p.sc.nw, p.sc.splits, p.ksg,
             afmt == HM_A_MXFP4 ? "scale_16x16x128_f8f6f4_fp4xfp4" : (a8 ? "scale_16x16x128_f8f6f4" : "16x16x32_bf16"));
  else if (p.path == P_BIG) {
    const Geom G = make_geom(device_fmt(d->wfmt), 1, d->n, d->k);
    const int64_t tiles = big_n_tiles(G) * ((m + kBigRows - 1) / kBigRows);
    const bool mxk = afmt != HM_A_BF16;       // the scaled-MFMA path of the kernel
    const int64_t halves = 2 * (tiles - big_full_tiles(G, m, mxk));
    snprintf(buf, buf_len, "%s tile 256x256 waves=%s mfma=%s half_tiles=%lld", w, mxk ? "4x2" : "1x4",
             afmt == HM_A_MXFP4 ? "scale_16x16x128_f8f6f4_fp4xfp4"
                                : (mxk ? "scale_16x16x128_f8f6f4" : "32x32x16_bf16"),
             (long long)halves);
  }
  else if (p.path == P_MID && a8)
    snprintf(buf, buf_len, "%s tile 64x128 waves=2x2 mfma=scale_16x16x128_f8f6f4", w);
  else if (p.path == P_MID)
    snprintf(buf, buf_len, "%s tile 128x64 waves=4 (K split) mfma=32x32x16_bf16", w);
  else
    snprintf(buf, buf_len, "%s tile %dx%d waves=2x2 mfma=%s", w, kTileM, kTileN,
             afmt == HM_A_MXFP4 ? "scale_16x16x128_f8f6f4_fp4xfp4" : (a8 ? "scale_16x16x128_f8f6f4" : "16x16x32_bf16"));
  return HM_OK;
}

HM_API hm_status hm_gemm(const hm_wdesc* d, const void* w_dev, int32_t afmt, const void* x,
                         const void* x_scales, int64_t m, uint16_t* y, void* ws, size_t ws_bytes,
                         const hm_tuning* tune, hipStream_t stream) {
  hm_status s = check_desc(d);
  if (s) return s;
  if ((s = check_pair(d, afmt))) return s;
  if (d->num_experts != 1) return HM_ERR_SHAPE;
  if (m < 0 || m > kMaxDenseRows) return HM_ERR_SHAPE;
  Tune tu;
  if ((s = read_tuning(tune, &tu))) return s;
  if (m == 0) return HM_OK;
  if (!w_dev || !x || !y) return HM_ERR_NULL;
  if (afmt != HM_A_BF16 && !x_scales) return HM_ERR_NULL;
  if (!aligned(w_dev, 256) || !aligned(x, 16) || !aligned(y, 16)) return HM_ERR_ALIGN;
  if (x_scales && !aligned(x_scales, 4)) return HM_ERR_ALIGN;
  DensePlan p;
  if ((s = plan_dense(d, afmt, m, tu, &p))) return s;
  if (p.ws_bytes) {
    if (!ws) return HM_ERR_NULL;
    if (ws_bytes < p.ws_bytes) return HM_ERR_WORKSPACE;
    if (!aligned(ws, 256)) return HM_ERR_ALIGN;
  }
  GemmArgs a{};
  a.w = (const uint8_t*)w_dev;
  a.G = geom_of(d);
  a.wfmt = device_fmt(d->wfmt);
  a.a8 = afmt == HM_A_FP8_ROWSCALE;
  a.a4 = afmt == HM_A_MXFP4;
  a.x = x;
  a.xs = (afmt == HM_A_FP8_ROWSCALE) ? (const float*)x_scales : nullptr;
  a.xsb = a.a4 ? (const uint8_t*)x_scales : nullptr;
  a.M = m;
  a.y = y;
  hipError_t e;
  if (p.path == P_STREAM) {
    a.part = (p.sc.splits > 1) ? (float*)ws : nullptr;
    a.ksg = p.ksg;
    e = launch_gemm_stream(a, p.sc, false, 0, stream);
    if (e == hipSuccess && p.sc.splits > 1) e = launch_splitk_reduce(a, p.sc.splits, stream);
  } else {
    e = p.path == P_BIG ? launch_gemm_big(a, false, 0, stream)
        : (p.path == P_MID ? launch_gemm_mid(a, false, 0, stream) : launch_gemm_tile(a, false, 0, stream));
  }
  return (e == hipSuccess) ? HM_OK : HM_ERR_HIP;
}

// Per-chunk expert counts of the GPU-wide sort (none for one block).
static size_t sort_ws_bytes(int64_t P, int E) {
  const int nb = moe_sort_blocks(P, nullptr);
  return nb > 1 ? (size_t)nb * (size_t)E * sizeof(int32_t) : 0;
}

HM_API hm_status hm_moe_sort_workspace_size(int64_t t, int32_t topk, int32_t num_experts,
                                            size_t* bytes) {
  if (!bytes) return HM_ERR_NULL;
  if (t < 0 || topk < 1 || num_experts < 1 || num_experts > 512 || topk > num_experts)
    return HM_ERR_SHAPE;
  if (t * (int64_t)topk >= (1ll << 31)) return HM_ERR_SHAPE;
  *bytes = sort_ws_bytes(t * topk, num_experts);
  return HM_OK;
}

HM_API hm_status hm_moe_sort(const int32_t* topk_ids, int64_t t, int32_t topk, int32_t num_experts,
                             int32_t* counts, int32_t* offsets, int32_t* sorted_pairs, void* ws,
                             size_t ws_bytes, hipStream_t stream) {
  if (t < 0 || topk < 1 || num_experts < 1 || num_experts > 512 || topk > num_experts)
    return HM_ERR_SHAPE;
  if (t * (int64_t)topk >= (1ll << 31)) return HM_ERR_SHAPE;
  if (t == 0) return HM_OK;
  if (!topk_ids || !counts || !offsets || !sorted_pairs) return HM_ERR_NULL;
  if (!aligned(topk_ids, 4) || !aligned(counts, 4) || !aligned(offsets, 4) || !aligned(sorted_pairs, 4))
    return HM_ERR_ALIGN;
  const size_t need = sort_ws_bytes(t * topk, num_experts);
  if (need) {
    if (!ws) return HM_ERR_NULL;
    if (ws_bytes < need) return HM_ERR_WORKSPACE;
    if (!aligned(ws, 4)) return HM_ERR_ALIGN;
  }
  if (launch_moe_sort(topk_ids, t * topk, num_experts, counts, offsets, sorted_pairs,
                      static_cast<int32_t*>(ws), stream) != hipSuccess)
    return HM_ERR_HIP;
  return HM_OK;
}

// Common checks of the grouped GEMM's size query, plan and call.
static hm_status moe_common(const hm_wdesc* d, int32_t afmt, int64_t t, int32_t topk, const hm_tuning* tune,
                            Tune* tu) {
  hm_status s = check_desc(d);
  if (s) return s;
  if ((s = check_pair(d, afmt))) return s;
  if (t < 0 || topk < 1 || topk > d->num_experts) return HM_ERR_SHAPE;
  if (t * (int64_t)topk >= (1ll << 31)) return HM_ERR_SHAPE;
  return read_tuning(tune, tu);
}

HM_API hm_status hm_moe_gemm_workspace_size(const hm_wdesc* d, int32_t afmt, int64_t t, int32_t topk,
                                            const hm_tuning* tune, size_t* bytes) {
  Tune tu;
  hm_status s = moe_common(d, afmt, t, topk, tune, &tu);
  if (s) return s;
  if (!bytes) return HM_ERR_NULL;
  MoePlan p;
  if ((s = plan_moe(d, afmt, t, topk, -1, tu, &p))) return s;
  *bytes = p.ws_bytes;
  return HM_OK;
}

static hm_status moe_plan_text(const hm_wdesc* d, int32_t afmt, int64_t t, int32_t topk, int32_t a_rows_are_pairs,
                               const hm_tuning* tune, char* buf, size_t buf_len, bool gated) {
  Tune tu;
  hm_status s = moe_common(d, afmt, t, topk, tune, &tu);
  if (s) return s;
  if (a_rows_are_pairs != 0 && a_rows_are_pairs != 1) return HM_ERR_SHAPE;
  if (!buf || buf_len == 0) return HM_ERR_NULL;
  MoePlan p;
  if ((s = plan_moe(d, afmt, t, topk, a_rows_are_pairs, tu, &p, gated))) return s;
  const bool a8 = afmt == HM_A_FP8_ROWSCALE;
  const char* tile = p.tile == P_TILE ? "k_gemm_tile 128x128"
                     : (a8 ? "k_gemm_mid_mx 64x128" : "k_gemm_mid 128x64");
  char big[64];
  if (p.big_min > 0) snprintf(big, sizeof big, "k_gemm_big from %d rows", p.big_min);
  else snprintf(big, sizeof big, "none");
  snprintf(buf, buf_len,
           "%s moe%s stream(rows=%d max=%d nbw=%d ks=%d lds=%dKiB)=k_gemm_stream tile(<=128 rows)=%s "
           "big(256 rows)=%s%s ws=%zu",
           pair_name(d, afmt), gated ? " gated(silu epilogue)" : "", p.s_rows, p.s_max, p.nbw, p.ks, p.lds_kb, tile,
           big, p.a64 ? " activations>=4GiB" : "", p.ws_bytes);
  return HM_OK;
}

HM_API hm_status hm_moe_gemm_plan(const hm_wdesc* d, int32_t afmt, int64_t t, int32_t topk,
                                  int32_t a_rows_are_pairs, const hm_tuning* tune, char* buf, size_t buf_len) {
  return moe_plan_text(d, afmt, t, topk, a_rows_are_pairs, tune, buf, buf_len, false);
}

HM_API hm_status hm_moe_gemm_gated_plan(const hm_wdesc* d, int32_t afmt, int64_t t, int32_t topk,
                                        int32_t a_rows_are_pairs, const hm_tuning* tune, char* buf,
                                        size_t buf_len) {
  return moe_plan_text(d, afmt, t, topk, a_rows_are_pairs, tune, buf, buf_len, true);
}

static hm_status moe_gemm_impl(const hm_wdesc* d, const void* w_dev, int32_t afmt, const void* a_in,
                               const void* a_scales, int32_t a_rows_are_pairs, int64_t t, int32_t topk,
                               const int32_t* offsets, const int32_t* sorted_pairs, uint16_t* y, void* ws,
                               size_t ws_bytes, const hm_tuning* tune, bool gated, hipStream_t stream) {
  Tune tu;
  hm_status s = moe_common(d, afmt, t, topk, tune, &tu);
  if (s) return s;
  if (a_rows_are_pairs != 0 && a_rows_are_pairs != 1) return HM_ERR_SHAPE;
  if (t == 0) return HM_OK;
  if (!w_dev || !a_in || !offsets || !sorted_pairs || !y || !ws) return HM_ERR_NULL;
  if (afmt != HM_A_BF16 && !a_scales) return HM_ERR_NULL;
  if (!aligned(w_dev, 256) || !aligned(a_in, 16) || !aligned(y, 16) || !aligned(ws, 256) ||
      !aligned(offsets, 4) || !aligned(sorted_pairs, 4))
    return HM_ERR_ALIGN;
  if (a_scales && !aligned(a_scales, 4)) return HM_ERR_ALIGN;
  MoePlan p;
  if ((s = plan_moe(d, afmt, t, topk, a_rows_are_pairs, tu, &p, gated))) return s;
  if (ws_bytes < p.ws_bytes) return HM_ERR_WORKSPACE;
  return launch_moe(d, afmt, w_dev, a_in, a_scales, a_rows_are_pairs, t, topk, offsets, sorted_pairs, y,
                    (uint8_t*)ws, p, stream, gated);
}

HM_API hm_status hm_moe_gemm(const hm_wdesc* d, const void* w_dev, int32_t afmt, const void* a_in,
                             const void* a_scales, int32_t a_rows_are_pairs, int64_t t,
                             int32_t topk, const int32_t* offsets, const int32_t* sorted_pairs,
                             uint16_t* y, void* ws, size_t ws_bytes, const hm_tuning* tune,
                             hipStream_t stream) {
  return moe_gemm_impl(d, w_dev, afmt, a_in, a_scales, a_rows_are_pairs, t, topk, offsets, sorted_pairs, y, ws,
                       ws_bytes, tune, false, stream);
}

HM_API hm_status hm_moe_gemm_gated(const hm_wdesc* d, const void* w_dev, int32_t afmt, const void* a_in,
                                   const void* a_scales, int32_t a_rows_are_pairs, int64_t t,
                                   int32_t topk, const int32_t* offsets, const int32_t* sorted_pairs,
                                   uint16_t* h, void* ws, size_t ws_bytes, const hm_tuning* tune,
                                   hipStream_t stream) {
  return moe_gemm_impl(d, w_dev, afmt, a_in, a_scales, a_rows_are_pairs, t, topk, offsets, sorted_pairs, h, ws,
                       ws_bytes, tune, true, stream);
}

// ------------------------------------------------ allocation-free grouped GEMM
//
// The work lists of hm_moe_gemm_static live in this file-scope device array
// (each GPU the library runs on holds its own copy until the process ends).
// In host code its name is only a stand-in: the device address comes from
// hipGetSymbolAddress, resolved once per device with that device current.
namespace {
constexpr size_t kStaticScratchBytes = 4u << 20;
constexpr int kMaxDevices = 64;
__device__ __align__(256) uint8_t scratch[kStaticScratchBytes];
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

hm_status scratch_of_current_device(uint8_t** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return HM_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return HM_ERR_HIP;
    g_scratch_ptr[dev] = ptr;
  }
  *out = (uint8_t*)g_scratch_ptr[dev];
  return HM_OK;
}
}  // namespace

HM_API size_t hm_moe_gemm_static_max_workspace(void) { return kStaticScratchBytes; }

HM_API hm_status hm_moe_gemm_static(const hm_wdesc* d, const void* w_dev, int32_t afmt, const void* a_in,
                                    const void* a_scales, int32_t a_rows_are_pairs, int64_t t, int32_t topk,
                                    const int32_t* offsets, const int32_t* sorted_pairs, uint16_t* y,
                                    const hm_tuning* tune, hipStream_t stream) {
  Tune tu;
  hm_status s = moe_common(d, afmt, t, topk, tune, &tu);
  if (s) return s;
  if (a_rows_are_pairs != 0 && a_rows_are_pairs != 1) return HM_ERR_SHAPE;
  if (t == 0) return HM_OK;
  if (!w_dev || !a_in || !offsets || !sorted_pairs || !y) return HM_ERR_NULL;
  if (afmt != HM_A_BF16 && !a_scales) return HM_ERR_NULL;
  if (!aligned(w_dev, 256) || !aligned(a_in, 16) || !aligned(y, 16) || !aligned(offsets, 4) ||
      !aligned(sorted_pairs, 4))
    return HM_ERR_ALIGN;
  if (a_scales && !aligned(a_scales, 4)) return HM_ERR_ALIGN;
  MoePlan p;
  if ((s = plan_moe(d, afmt, t, topk, a_rows_are_pairs, tu, &p))) return s;
  if (p.ws_bytes > kStaticScratchBytes) return HM_ERR_WORKSPACE;
  uint8_t* ws = nullptr;
  if ((s = scratch_of_current_device(&ws))) return s;
  // the schedule writes the header and every unit it counts, so nothing of
  // the previous call's contents is read
  return launch_moe(d, afmt, w_dev, a_in, a_scales, a_rows_are_pairs, t, topk, offsets, sorted_pairs, y, ws, p,
                    stream);
}
