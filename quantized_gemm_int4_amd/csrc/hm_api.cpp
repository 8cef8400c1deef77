// C ABI entry points: argument checks, tile-configuration choice and launches.
// Every check runs before any launch; the library allocates nothing.
#include <hip/hip_runtime.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>

#include "../../include/hm.h"
#include "common.h"
#include "launch.h"

#define HM_API extern "C" __attribute__((visibility("default")))

namespace {

using namespace hm;

constexpr int kStreamMaxRows = 32;   // dense rows of one streaming block (two 16-row blocks)
constexpr int64_t kStreamWideRows = 256;      // narrow-N dense calls stream up to this many rows ...
constexpr int64_t kStreamChunkCols = 16384;   // ... while 32-row chunks x N stays within this
constexpr int64_t kStreamLdsBytes = 159 * 1024;  // dynamic LDS one streaming block may use
constexpr int kMoeStreamRows = 16;   // rows per grouped streaming unit
// Experts with at most this many rows use the streaming kernel (as units of
// kMoeStreamRows rows that share the expert's weights through the L2), with
// this many 16-column blocks per wave.  Measured on the 256-expert top-8
// workloads: W4A16 64 rows and two blocks per wave (T = 64 / 1024 / 8192:
// -19% / -5% / -5% against 16 rows and one block); MXFP4 keeps 16 and one.
constexpr int kMoeStreamMaxA16 = 64, kMoeStreamNbwA16 = 2;
constexpr int kMoeStreamMaxMx = 16, kMoeStreamNbwMx = 1;
// MXINT4 (bf16 rows): its streaming kernel is bound by the code conversion,
// so 32-row units (each conversion serving twice the rows) with experts of
// up to 128 rows streaming: T = 64 / 1024 / 8192 0.448 / 1.756 / 8.954 ms
// against 0.463 / 1.826 / 9.018 with 16-row units up to 64 rows
constexpr int kMoeStreamRowsMxi4 = 32, kMoeStreamMaxMxi4 = 128;
constexpr int64_t kBigMinRows = 512;  // dense rows from which 256 x 256 tiles may be used
// An expert remainder of at least this many rows gets a 256-row unit (a unit
// of at most 128 rows runs four of the eight 32-row MFMA blocks) instead of
// 128 x 64 tile units, which copy the unit's activation rows once per 64
// columns.  Measured against 192: W4A16 T = 1024 -12%, T = 8192 -2%; W4A8
// T = 16384 -3..4% (65 and 129 rows).
constexpr int kMoeBigMinRows = 97;
constexpr int kGroupedGridStream = 2048;
constexpr int kGroupedGridTile = 1024;
constexpr int kGroupedGridMid = 256;     // one 128 x 64 tile block per compute unit (LDS-bound)
constexpr int kGroupedGridBig = 256;     // one 256-tile block per compute unit (LDS-bound)

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

hm_status check_desc(const hm_wdesc* d) {
  if (!d) return HM_ERR_NULL;
  if (d->abi != HM_ABI_VERSION) return HM_ERR_ABI;
  if (d->wfmt != HM_W_INT4_SYM && d->wfmt != HM_W_UINT4_ZP && d->wfmt != HM_W_MXFP4 && d->wfmt != HM_W_MXINT4)
    return HM_ERR_UNSUPPORTED;
  const int want_group = is_mx(d->wfmt) ? 32 : 128;
  if (d->group != want_group) return HM_ERR_SHAPE;
  if (d->num_experts < 1 || d->n < 1 || d->k < 128 || (d->k % 128) != 0) return HM_ERR_SHAPE;
  if (d->n > (1ll << 24) || d->k > (1ll << 24)) return HM_ERR_SHAPE;
  return HM_OK;
}

hm_status check_pair(const hm_wdesc* d, int32_t afmt) {
  if (afmt != HM_A_BF16 && afmt != HM_A_FP8_ROWSCALE) return HM_ERR_UNSUPPORTED;
  // FP8 rows pair with MXFP4 weights only; bf16 rows with every format
  if (afmt == HM_A_FP8_ROWSCALE && d->wfmt != HM_W_MXFP4) return HM_ERR_UNSUPPORTED;
  return HM_OK;
}

// MX weights (MXFP4, MXINT4) with bf16 rows (codes scaled to bf16 inside the kernels)
bool mx_a16(const hm_wdesc* d, int32_t afmt) { return is_mx(d->wfmt) && afmt == HM_A_BF16; }

const char* pair_name(const hm_wdesc* d, int32_t afmt) {
  if (d->wfmt == HM_W_MXFP4) return afmt == HM_A_BF16 ? "w4a16-mxfp4" : "w4a8-mxfp4";
  if (d->wfmt == HM_W_MXINT4) return "w4a16-mxint4";
  return d->wfmt == HM_W_UINT4_ZP ? "w4a16-uint4zp" : "w4a16-int4sym";
}

Geom geom_of(const hm_wdesc* d) { return make_geom(d->wfmt, d->num_experts, d->n, d->k); }

int env_int(const char* name, int dflt) {
  const char* s = getenv(name);
  return (s && *s) ? atoi(s) : dflt;
}

// ---------------------------------------------------------------- dense plan
struct DensePlan {
  bool stream;
  bool big;          // 256 x 256 tiles (large M)
  bool mid;          // W4A16 128 x 64 tiles with the K groups split over the waves
  StreamCfg sc;
  int ksg;
  size_t ws_bytes;
};

// MX weights with bf16 rows: rows that take the 128 x 128 kernel instead of the
// 128 x 64 one (at least 8 rounds of 128 x 64 tiles on the 256 compute units)
bool f4_wide_tiles(const Geom& G, int64_t rows) {
  const int64_t mt = (rows + kTileM - 1) / kTileM;
  const int64_t mid_rounds = (mid_n_tiles(G, false) * mt + 255) / 256;
  const int64_t tile_rounds = (((G.NB + 7) / 8) * mt + 255) / 256;
  return mid_rounds >= 8 && tile_rounds < mid_rounds;
}

DensePlan plan_dense(const hm_wdesc* d, int32_t afmt, int64_t m) {
  DensePlan p{};
  const Geom G = geom_of(d);
  const bool f4 = mx_a16(d, afmt);
  // 1 = streaming, 2 = 128-row tiles, 3 = 256-row tiles, 4 = W4A16 128 x 128 tiles
  const int force = env_int("HM_FORCE_PATH", 0);
  // W4A16 up to 256 rows also streams (in 32-row chunks, each re-reading the
  // weights from the L2) when N is narrow: measured at K = 4096, a streaming
  // launch costs ~8 us + 0.8 ns per (chunk x column) and a round of 128 x 64
  // tiles 23-25 us, so chunks x N <= 16384 streams (N = 1792, M = 128: 14.9
  // against 23.4 us; N = 7168, M = 128 stays on tiles: 25.3 against 28.8 us)
  const bool narrow = !is_mx(d->wfmt) && m <= kStreamWideRows &&
                      ((m + kStreamMaxRows - 1) / kStreamMaxRows) * d->n <= kStreamChunkCols;
  p.stream = (force == 1) || (force == 0 && (m <= kStreamMaxRows || narrow));
  if (force == 1 && m > kStreamWideRows) p.stream = false;  // forced streaming: up to 256 rows
  if (!p.stream) {
    // W4A16: 256 x 256 tiles unless 128 x 64 tiles take fewer rounds of the
    // chip by the measured cost of a round (one of 256 x 256 tiles ~ 3.8 of
    // 128 x 64 tiles, N = 1792 / 7168 / 14336, K = 4096): a narrow N (one
    // rank's column shard, N = 1792, M = 1024: 28 large tiles) runs 3.5x
    // faster on the smaller tiles
    const int64_t big_rounds = (big_n_tiles(G) * ((m + kBigRows - 1) / kBigRows) + 255) / 256;
    const int64_t mid_rounds = (mid_n_tiles(G, false) * ((m + kTileM - 1) / kTileM) + 255) / 256;
    const bool mid_fewer = !is_mx(d->wfmt) && mid_rounds * 10 < big_rounds * 38;
    p.big = (force == 3) || (force == 0 && m >= kBigMinRows && !mid_fewer);
    p.mid = !p.big && force != 4;
    // MX weights with bf16 rows (no 256 x 256 kernel): 128 x 64 tiles, or 128 x
    // 128 tiles once the 128 x 64 ones take many rounds of the chip.
    // Measured at N = 7168 K = 2048 / N = 14336 K = 4096: M = 256 / 128 on
    // 128 x 64 tiles 14.9 / 23.9 us against 30.1 / 63.2 (one round each),
    // M = 1024 even (4 / 7 rounds against 2 / 4), M = 4096 147 / 520 us on
    // 128 x 128 tiles against 273 / 1039 (14 / 28 rounds against 7 / 14)
    if (f4) {
      p.big = false;
      p.mid = (force == 2 || force == 3) || (force == 0 && !f4_wide_tiles(G, m));
    }
    return p;
  }
  p.sc.mb = (m <= 16) ? 1 : 2;
  const int64_t rows = (m < 16 * p.sc.mb) ? m : 16 * p.sc.mb;
  const int64_t m_chunks = (m + 16 * p.sc.mb - 1) / (16 * p.sc.mb);
  const int64_t gb = (afmt == HM_A_FP8_ROWSCALE) ? 128 : 256;   // activation bytes per row per group
  // Launch shape: (ks, nbw) from the narrowest block (most waves, least work
  // per wave) to the widest, take the first whose blocks all fit on the chip
  // at once.  A block keeps its activation rows in LDS, so the LDS footprint
  // decides how many blocks share a compute unit (at most 5: the register
  // budget allows 5 waves per SIMD).
  int ks = env_int("HM_STREAM_KS", 0), nbw = env_int("HM_STREAM_NBW", 0);
  static const int kShapes[6][2] = {{4, 1}, {2, 1}, {4, 2}, {2, 2}, {1, 1}, {1, 2}};
  if (ks != 1 && ks != 2 && ks != 4) ks = 0;
  if (nbw != 1 && nbw != 2) nbw = 0;
  if (!ks || !nbw) {
    const int64_t row_bytes = std::min<int64_t>(G.KG * gb + 16, kStreamLdsBytes / rows);
    int pick = 5;
    for (int i = 0; i < 6; ++i) {
      const int cks = kShapes[i][0], cnbw = kShapes[i][1];
      if ((ks && cks != ks) || (nbw && cnbw != nbw)) continue;
      if (G.KG < 2 * cks && cks > 1) continue;                  // >= 2 groups per wave
      StreamCfg t = p.sc;
      t.ks = cks;
      t.nbw = cnbw;
      const int64_t lds = rows * row_bytes + (cks > 1 ? 4 * cnbw * p.sc.mb * 1024 : 0);
      const int64_t per_cu = std::max<int64_t>(1, std::min<int64_t>(5, kStreamLdsBytes / lds));
      const int64_t blocks = stream_n_tiles(G, t) * m_chunks;
      pick = i;
      if (blocks <= 256 * per_cu) break;
    }
    ks = kShapes[pick][0];
    nbw = kShapes[pick][1];
  }
  p.sc.ks = ks;
  p.sc.nbw = nbw;
  const int64_t n_tiles = stream_n_tiles(G, p.sc);
  int64_t splits = env_int("HM_STREAM_SPLITS", 0);
  if (splits <= 0) {
    // enough waves to keep every SIMD streaming (1024 SIMDs); split K over
    // blocks only below that
    const int64_t target_waves = 800;
    const int64_t waves = n_tiles * 4 * m_chunks;
    splits = (target_waves + waves - 1) / waves;
  }
  if (splits > G.KG) splits = G.KG;
  if (splits < 1) splits = 1;
  p.ksg = (int)((G.KG + splits - 1) / splits);
  p.sc.splits = (int)((G.KG + p.ksg - 1) / p.ksg);
  p.ws_bytes = (p.sc.splits > 1) ? (size_t)p.sc.splits * m * G.NB * 16 * sizeof(float) : 0;
  return p;
}

// ---------------------------------------------------------------- MoE plan
struct MoePlan {
  int64_t P, max_s, max_t, max_b;
  size_t off_su, off_tu, off_bu, ws_bytes;
  int nbw, ks, lds_kb, s_rows, s_max, big_min;
};

MoePlan plan_moe(const hm_wdesc* d, int32_t afmt, int64_t t, int32_t topk) {
  MoePlan p{};
  p.P = t * topk;
  const int64_t act = (p.P < d->num_experts) ? p.P : d->num_experts;
  const bool mxi4 = d->wfmt == HM_W_MXINT4;
  const int rows_dflt = mxi4 ? kMoeStreamRowsMxi4 : kMoeStreamRows;
  p.s_rows = env_int("HM_MOE_STREAM_ROWS", rows_dflt);
  if (p.s_rows != 16 && p.s_rows != 32) p.s_rows = rows_dflt;
  // experts with up to s_max rows stream, as ceil(rows / s_rows) units
  const bool mx = afmt == HM_A_FP8_ROWSCALE;
  p.s_max = env_int("HM_MOE_STREAM_MAX", mx ? kMoeStreamMaxMx : (mxi4 ? kMoeStreamMaxMxi4 : kMoeStreamMaxA16));
  if (p.s_max < p.s_rows) p.s_max = p.s_rows;
  p.max_s = p.P / p.s_rows + act;
  p.max_t = (p.P + kTileM - 1) / kTileM + act;
  // an expert remainder of at least big_min rows takes a 256-row unit
  p.big_min = env_int("HM_MOE_BIG_MIN", kMoeBigMinRows);
  if (p.big_min < 1 || p.big_min > kBigRows) p.big_min = kMoeBigMinRows;
  p.max_b = p.P / p.big_min + 1;              // every 256-row unit holds >= big_min rows
  p.off_su = 256;
  p.off_tu = align256(p.off_su + (size_t)p.max_s * 16);
  p.off_bu = align256(p.off_tu + (size_t)p.max_t * 16);
  p.ws_bytes = align256(p.off_bu + (size_t)p.max_b * 16);
  p.nbw = env_int("HM_MOE_STREAM_NBW", mx ? kMoeStreamNbwMx : kMoeStreamNbwA16);
  if (p.nbw != 1 && p.nbw != 2) p.nbw = mx ? kMoeStreamNbwMx : kMoeStreamNbwA16;
  p.ks = env_int("HM_MOE_STREAM_KS", 1);
  if (p.ks != 1 && p.ks != 2 && p.ks != 4) p.ks = 1;
  // LDS per streaming block: a unit stages up to s_rows rows, so K is walked in
  // pieces that fit this budget; a smaller budget lets more blocks share a
  // compute unit
  p.lds_kb = env_int("HM_MOE_STREAM_LDS_KB", 79);
  if (p.lds_kb < 20 || p.lds_kb > 159) p.lds_kb = 79;
  return p;
}

}  // namespace

// =====================================================================================

HM_API const char* hm_status_string(hm_status s) {
  switch (s) {
    case HM_OK: return "ok";
    case HM_ERR_NULL: return "null pointer";
    case HM_ERR_SHAPE: return "bad shape, group or count";
    case HM_ERR_ALIGN: return "misaligned pointer";
    case HM_ERR_UNSUPPORTED: return "unsupported format or format/activation pair";
    case HM_ERR_WORKSPACE: return "workspace too small";
    case HM_ERR_HIP: return "HIP launch failed";
    case HM_ERR_ABI: return "descriptor ABI version mismatch";
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

HM_API hm_status hm_transform(const hm_wdesc* d, const uint8_t* codes, const void* scales,
                              const uint8_t* zeros, void* w_dev, size_t w_bytes,
                              hipStream_t stream) {
  hm_status s = check_desc(d);
  if (s) return s;
  if (!codes || !scales || !w_dev) return HM_ERR_NULL;
  if (d->wfmt == HM_W_UINT4_ZP && !zeros) return HM_ERR_NULL;
  if (!aligned(codes, 16) || !aligned(w_dev, 256)) return HM_ERR_ALIGN;
  if (!aligned(scales, is_mx(d->wfmt) ? 1 : 2)) return HM_ERR_ALIGN;
  const Geom G = geom_of(d);
  if (w_bytes < G.total) return HM_ERR_WORKSPACE;
  if (launch_transform(d->wfmt, G, codes, scales, zeros, (uint8_t*)w_dev, stream) != hipSuccess)
    return HM_ERR_HIP;
  return HM_OK;
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
  if (launch_dequant(d->wfmt, G, (const uint8_t*)w_dev, expert, out, stream) != hipSuccess)
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

HM_API hm_status hm_gemm_workspace_size(const hm_wdesc* d, int32_t afmt, int64_t m, size_t* bytes) {
  hm_status s = check_desc(d);
  if (s) return s;
  if ((s = check_pair(d, afmt))) return s;
  if (!bytes) return HM_ERR_NULL;
  if (m < 0) return HM_ERR_SHAPE;
  *bytes = (m == 0) ? 0 : plan_dense(d, afmt, m).ws_bytes;
  return HM_OK;
}

HM_API hm_status hm_gemm_plan(const hm_wdesc* d, int32_t afmt, int64_t m, char* buf,
                              size_t buf_len) {
  hm_status s = check_desc(d);
  if (s) return s;
  if ((s = check_pair(d, afmt))) return s;
  if (!buf || buf_len == 0) return HM_ERR_NULL;
  if (m < 0) return HM_ERR_SHAPE;
  const DensePlan p = plan_dense(d, afmt, m);
  const char* w = pair_name(d, afmt);
  const bool a8 = afmt == HM_A_FP8_ROWSCALE;
  if (p.stream)
    snprintf(buf, buf_len, "%s stream mb=%d nbw=%d ks=%d splits=%d ksg=%d mfma=%s", w, p.sc.mb,
             p.sc.nbw, p.sc.ks, p.sc.splits, p.ksg, a8 ? "scale_16x16x128_f8f6f4" : "16x16x32_bf16");
  else if (p.big) {
    const Geom G = make_geom(d->wfmt, 1, d->n, d->k);
    const int64_t tiles = big_n_tiles(G) * ((m + kBigRows - 1) / kBigRows);
    const int64_t halves = 2 * (tiles - big_full_tiles(G, m, d->wfmt == HM_W_MXFP4));
    snprintf(buf, buf_len, "%s tile 256x256 waves=%s mfma=%s half_tiles=%lld", w,
             d->wfmt == HM_W_MXFP4 ? "4x2" : "1x4", d->wfmt == HM_W_MXFP4 ? "scale_16x16x128_f8f6f4" : "32x32x16_bf16",
             (long long)halves);
  }
  else if (p.mid && a8)
    snprintf(buf, buf_len, "%s tile 64x128 waves=2x2 mfma=scale_16x16x128_f8f6f4", w);
  else if (p.mid)
    snprintf(buf, buf_len, "%s tile 128x64 waves=4 (K split) mfma=32x32x16_bf16", w);
  else
    snprintf(buf, buf_len, "%s tile %dx%d waves=2x2 mfma=%s", w, kTileM, kTileN,
             a8 ? "scale_16x16x128_f8f6f4" : "16x16x32_bf16");
  return HM_OK;
}

HM_API hm_status hm_gemm(const hm_wdesc* d, const void* w_dev, int32_t afmt, const void* x,
                         const float* x_row_scale, int64_t m, uint16_t* y, void* ws,
                         size_t ws_bytes, hipStream_t stream) {
  hm_status s = check_desc(d);
  if (s) return s;
  if ((s = check_pair(d, afmt))) return s;
  if (d->num_experts != 1) return HM_ERR_SHAPE;
  if (m < 0 || m > 65535ll * kTileM) return HM_ERR_SHAPE;
  if (m == 0) return HM_OK;
  if (!w_dev || !x || !y) return HM_ERR_NULL;
  if (afmt == HM_A_FP8_ROWSCALE && !x_row_scale) return HM_ERR_NULL;
  if (!aligned(w_dev, 256) || !aligned(x, 16) || !aligned(y, 16)) return HM_ERR_ALIGN;
  if (x_row_scale && !aligned(x_row_scale, 4)) return HM_ERR_ALIGN;
  const DensePlan p = plan_dense(d, afmt, m);
  if (p.ws_bytes) {
    if (!ws) return HM_ERR_NULL;
    if (ws_bytes < p.ws_bytes) return HM_ERR_WORKSPACE;
    if (!aligned(ws, 256)) return HM_ERR_ALIGN;
  }
  GemmArgs a{};
  a.w = (const uint8_t*)w_dev;
  a.G = geom_of(d);
  a.wfmt = d->wfmt;
  a.a8 = afmt == HM_A_FP8_ROWSCALE;
  a.x = x;
  a.xs = (afmt == HM_A_FP8_ROWSCALE) ? x_row_scale : nullptr;
  a.M = m;
  a.y = y;
  hipError_t e;
  if (p.stream) {
    a.part = (p.sc.splits > 1) ? (float*)ws : nullptr;
    a.ksg = p.ksg;
    e = launch_gemm_stream(a, p.sc, false, 0, stream);
    if (e == hipSuccess && p.sc.splits > 1) e = launch_splitk_reduce(a, p.sc.splits, stream);
  } else {
    e = p.big ? launch_gemm_big(a, false, 0, stream)
              : (p.mid ? launch_gemm_mid(a, false, 0, stream) : launch_gemm_tile(a, false, 0, stream));
  }
  return (e == hipSuccess) ? HM_OK : HM_ERR_HIP;
}

HM_API hm_status hm_moe_sort_workspace_size(int64_t t, int32_t topk, int32_t num_experts,
                                            size_t* bytes) {
  if (!bytes) return HM_ERR_NULL;
  if (t < 0 || topk < 1 || num_experts < 1 || num_experts > 512 || topk > num_experts)
    return HM_ERR_SHAPE;
  *bytes = 0;
  return HM_OK;
}

HM_API hm_status hm_moe_sort(const int32_t* topk_ids, int64_t t, int32_t topk, int32_t num_experts,
                             int32_t* counts, int32_t* offsets, int32_t* sorted_pairs, void* ws,
                             size_t ws_bytes, hipStream_t stream) {
  (void)ws;
  (void)ws_bytes;
  if (t < 0 || topk < 1 || num_experts < 1 || num_experts > 512 || topk > num_experts)
    return HM_ERR_SHAPE;
  if (t * (int64_t)topk >= (1ll << 31)) return HM_ERR_SHAPE;
  if (t == 0) return HM_OK;
  if (!topk_ids || !counts || !offsets || !sorted_pairs) return HM_ERR_NULL;
  if (!aligned(topk_ids, 4) || !aligned(counts, 4) || !aligned(offsets, 4) || !aligned(sorted_pairs, 4))
    return HM_ERR_ALIGN;
  if (launch_moe_sort(topk_ids, t * topk, num_experts, counts, offsets, sorted_pairs, stream) !=
      hipSuccess)
    return HM_ERR_HIP;
  return HM_OK;
}

HM_API hm_status hm_moe_gemm_workspace_size(const hm_wdesc* d, int32_t afmt, int64_t t, int32_t topk,
                                            size_t* bytes) {
  hm_status s = check_desc(d);
  if (s) return s;
  if ((s = check_pair(d, afmt))) return s;
  if (!bytes) return HM_ERR_NULL;
  if (t < 0 || topk < 1 || topk > d->num_experts || d->num_experts > 512) return HM_ERR_SHAPE;
  *bytes = plan_moe(d, afmt, t, topk).ws_bytes;
  return HM_OK;
}

HM_API hm_status hm_moe_gemm(const hm_wdesc* d, const void* w_dev, int32_t afmt, const void* a_in,
                             const float* a_row_scale, int32_t a_rows_are_pairs, int64_t t,
                             int32_t topk, const int32_t* offsets, const int32_t* sorted_pairs,
                             uint16_t* y, void* ws, size_t ws_bytes, hipStream_t stream) {
  hm_status s = check_desc(d);
  if (s) return s;
  if ((s = check_pair(d, afmt))) return s;
  if (t < 0 || topk < 1 || topk > d->num_experts || d->num_experts > 512) return HM_ERR_SHAPE;
  if (t * (int64_t)topk >= (1ll << 31)) return HM_ERR_SHAPE;
  if (a_rows_are_pairs != 0 && a_rows_are_pairs != 1) return HM_ERR_SHAPE;
  if (t == 0) return HM_OK;
  if (!w_dev || !a_in || !offsets || !sorted_pairs || !y || !ws) return HM_ERR_NULL;
  if (afmt == HM_A_FP8_ROWSCALE && !a_row_scale) return HM_ERR_NULL;
  if (!aligned(w_dev, 256) || !aligned(a_in, 16) || !aligned(y, 16) || !aligned(ws, 256) ||
      !aligned(offsets, 4) || !aligned(sorted_pairs, 4))
    return HM_ERR_ALIGN;
  if (a_row_scale && !aligned(a_row_scale, 4)) return HM_ERR_ALIGN;
  const MoePlan p = plan_moe(d, afmt, t, topk);
  if (ws_bytes < p.ws_bytes) return HM_ERR_WORKSPACE;

  uint8_t* w8 = (uint8_t*)ws;
  int32_t* hdr = (int32_t*)w8;
  int32_t* su = (int32_t*)(w8 + p.off_su);
  int32_t* tu = (int32_t*)(w8 + p.off_tu);
  int32_t* bu = (int32_t*)(w8 + p.off_bu);
  GemmArgs a{};
  a.w = (const uint8_t*)w_dev;
  a.G = geom_of(d);
  a.wfmt = d->wfmt;
  a.a8 = afmt == HM_A_FP8_ROWSCALE;
  a.x = a_in;
  a.xs = (afmt == HM_A_FP8_ROWSCALE) ? a_row_scale : nullptr;
  a.M = 0;
  a.y = y;
  a.hdr = hdr;
  a.sorted_pairs = sorted_pairs;
  a.topk = topk;
  a.rows_are_pairs = a_rows_are_pairs;

  a.P = p.P;
  // 256-row units address activation rows with 32-bit byte offsets
  const int64_t a_bytes = (a_rows_are_pairs ? p.P : t) * d->k * (afmt == HM_A_FP8_ROWSCALE ? 1 : 2);
  const bool f4 = mx_a16(d, afmt);   // MX weights with bf16 rows: streaming and 128-row units only
  const int big_min = (!f4 && a_bytes < (1ll << 32) && env_int("HM_MOE_BIG", 1)) ? p.big_min : 0;
  hipError_t e = launch_moe_schedule(offsets, d->num_experts, p.P, p.s_rows, p.s_max, kTileM, big_min,
                                     p.max_s, p.max_t, p.max_b, hdr, su, tu, bu, stream);
  if (e == hipSuccess) {
    StreamCfg sc{p.s_rows / 16, p.nbw, 1, p.ks, p.lds_kb};
    const int64_t nts = stream_n_tiles(a.G, sc);
    int64_t gi = p.max_s * nts;
    if (gi > kGroupedGridStream) gi = kGroupedGridStream;
    a.units = su;
    if (gi > 0) e = launch_gemm_stream(a, sc, true, (int)gi, stream);
  }
  if (e == hipSuccess) {
    // units of up to 128 rows: W4A16 on 128 x 64 tiles, W4A8 on 64 x 128
    // tiles (one block per compute unit, LDS-bound); HM_MOE_MID=0 keeps
    // them on the 128 x 128 kernel
    // MX weights with bf16 rows: the 128 x 128 kernel when all pairs in 128-row
    // units would take many rounds of 128 x 64 tiles (T = 8192: 7.92 against
    // 8.30 ms)
    const bool mid = env_int("HM_MOE_MID", 1) != 0 && !(f4 && f4_wide_tiles(a.G, p.P));
    const int64_t ntt = mid ? mid_n_tiles(a.G, afmt == HM_A_FP8_ROWSCALE) : (a.G.NB + 7) / 8;
    int64_t gi = p.max_t * ntt;
    const int64_t cap = mid ? kGroupedGridMid : kGroupedGridTile;
    if (gi > cap) gi = cap;
    a.units = tu;
    if (gi > 0) e = mid ? launch_gemm_mid(a, true, (int)gi, stream) : launch_gemm_tile(a, true, (int)gi, stream);
  }
  if (e == hipSuccess && big_min > 0) {
    int64_t gi = p.max_b * big_n_tiles(a.G);
    if (gi > kGroupedGridBig) gi = kGroupedGridBig;
    a.units = bu;
    if (gi > 0) e = launch_gemm_big(a, true, (int)gi, stream);
  }
  return (e == hipSuccess) ? HM_OK : HM_ERR_HIP;
}
