// Internal launchers (host side) for the kernels of the library.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>
#include "common.h"

namespace hm {

constexpr int kBigRows = 256;   // rows of a 256 x 256 tile (and of a grouped 256-row unit)

// Launch geometry the planner shares with the kernels.
constexpr int kBigM = kBigRows;  // rows per 256 x 256 block
constexpr int kBigCB = 16;       // 16-column blocks per 256 x 256 block (256 columns)
constexpr int kBigGrid = 256;    // persistent dense 256 x 256 grid: one block per CU
constexpr int kMidCB = 4;        // 16-column blocks per W4A16 128 x 64 tile (64 columns)
constexpr int kMxCB = 8;         // 16-column blocks per W4A8 64 x 128 tile (128 columns)

// Kernel variants by (weight format, activation format): INT4 codes with
// bf16 rows, MXFP4 with FP8 rows (scaled fp4 x fp8 MFMA), MXFP4 / MXINT4 with bf16 rows
// (E2M1 converted to bf16 with its E8M0 scale, bf16 MFMA).
// (MXINT4 weights with bf16 rows take the MXFP4 path with integer codes.)
enum KMode : int { KM_INT4_A16 = 0, KM_MX_A8 = 1, KM_MX_A16 = 2, KM_MXI4_A16 = 3, KM_MX_A4 = 4, KM_INT8_A16 = 5 };

// Arguments shared by the GEMM kernels.
struct GemmArgs {
  const uint8_t* w;        // device weight layout (all experts)
  Geom G;
  int wfmt;                // W_INT4_SYM / W_UINT4_ZP / W_MXFP4 / W_MXINT4
  int a8;                  // 1: x is E4M3 bytes with fp32 row scales (MXFP4 only); 0: bf16
  int a4;                  // 1: x is E2M1 codes [rows][K/2] with E8M0 bytes xsb [rows][K/32] (MXFP4 only)
  const uint8_t* xsb;      // E8M0 activation scales (a4) or null
  const void* x;           // activations: bf16 [rows][K] or E4M3 bytes [rows][K]
  const float* xs;         // fp32 row scales (A8) or null
  int64_t M;               // dense: rows of x and y
  uint16_t* y;             // bf16 output [rows][N]
  float* part;             // split-K partials [splits][M][NB*16] (dense streaming only)
  int ksg;                 // K groups per split (dense streaming)
  // grouped (MoE) mode
  const int32_t* units;    // {expert, first, count, 0} per unit
  const int32_t* hdr;      // hdr[0] streaming units, hdr[1] tile units, hdr[2] 256-row units
  const int32_t* sorted_pairs;
  int topk;
  int rows_are_pairs;
  int64_t P;               // routed pairs (row ids outside [0, P) are skipped)
  // 1: weights in the gated layout (gate / up 16-column blocks interleaved,
  // N % 32 == 0) and y is [rows][N/2] = bf16(silu(bf16 gate) * bf16 up)
  int gated;
};

// gated: device row n takes source row gated_src_row(n, N) (N % 32 == 0)
hipError_t launch_transform(int wfmt, const Geom& G, const uint8_t* codes, const void* scales,
                            const uint8_t* zeros, uint8_t* out, int gated, hipStream_t st);
hipError_t launch_dequant(int wfmt, const Geom& G, const uint8_t* w, int64_t e, float* out,
                          hipStream_t st);
hipError_t launch_quant_fp8_rows(const uint16_t* x, int64_t m, int64_t k, uint8_t* x8, float* s,
                                 hipStream_t st);
hipError_t launch_quant_mxfp4_rows(const uint16_t* x, int64_t m, int64_t k, uint8_t* codes, uint8_t* scales,
                                   hipStream_t st);
// Expert sort: up to kSortOneBlock pairs in one block; more are cut into
// moe_sort_blocks(P) chunks of *chunk pairs (about kSortChunk, at most
// kSortMaxBlocks chunks) whose per-expert counts go to cnt [chunks][E].
constexpr int64_t kSortOneBlock = 4096;
constexpr int64_t kSortChunk = 2048;
constexpr int kSortMaxBlocks = 512;
int moe_sort_blocks(int64_t P, int64_t* chunk);
hipError_t launch_moe_sort(const int32_t* ids, int64_t P, int E, int32_t* counts, int32_t* offsets,
                           int32_t* sorted_pairs, int32_t* cnt, hipStream_t st);
hipError_t launch_moe_schedule(const int32_t* offsets, int E, int64_t P, int s_rows, int s_max, int bm,
                               int big_min, int64_t max_s, int64_t max_t, int64_t max_b, int32_t* hdr,
                               int32_t* su, int32_t* tu, int32_t* bu, hipStream_t st);

// MoE block steps around the grouped GEMMs (bf16 rows, 16-byte chunks when
// d (n) is a multiple of 8).  Grids of one thread per chunk: the caller keeps
// rows * d (t * n) / 8 under 2^31 * 256.
hipError_t launch_silu_mul(const uint16_t* gu, int64_t rows, int64_t d, uint16_t* h, hipStream_t st);
// gated activation + per-token FP8 rows in one pass (d % 8 == 0, d <= 8192)
hipError_t launch_silu_mul_fp8(const uint16_t* gu, int64_t rows, int64_t d, uint8_t* h8, float* hs,
                               hipStream_t st);
hipError_t launch_combine(const uint16_t* y, const float* w, int64_t t, int topk, int64_t n, uint16_t* out,
                          hipStream_t st);
// plain streaming read of a buffer (16-byte loads), one word per block written
hipError_t launch_read_probe(const void* buf, int64_t bytes, int blocks, int unroll, uint32_t* out,
                             hipStream_t st);

// Streaming (small-M) kernel.  Dense: grid (n_tiles, splits, m_chunks).
// Grouped: persistent over (streaming unit x n tile) items.
struct StreamCfg {
  int mb;      // 16-row blocks per unit: 1 or 2
  int nbw;     // 16-column blocks per wave: 1 or 2
  int splits;  // dense split-K factor (over blocks, fp32 partials)
  int ks;      // waves of a block splitting one column set's K range: 1, 2 or 4 (8 with nw = 8)
  int lds_kb;  // dynamic LDS budget per block in KiB (0: the 159 KiB maximum)
  int nw;      // waves per block: 4, or 8 (dense only, ks 2, 4 or 8)
};
// blocks along N (dense) or n tiles per unit (grouped) of a streaming launch
int64_t stream_n_tiles(const Geom& G, const StreamCfg& c);
hipError_t launch_gemm_stream(const GemmArgs& a, const StreamCfg& c, bool grouped, int grid_items,
                              hipStream_t st);
hipError_t launch_splitk_reduce(const GemmArgs& a, int splits, hipStream_t st);

// MFMA tile kernel, 128x128 output tiles.  Dense: grid (n_tiles, m_tiles).
// Grouped: persistent over (tile unit x n tile) items.
constexpr int kTileM = 128;
constexpr int kTileN = 128;
hipError_t launch_gemm_tile(const GemmArgs& a, bool grouped, int grid_items, hipStream_t st);

// Mid-M MFMA kernels: W4A16 128 x 64 output tiles (K groups split over the
// four waves; INT4, and MXFP4 / MXINT4 with bf16 rows), W4A8-MXFP4 64 x 128 tiles.  Dense: one block per tile.
// Grouped: persistent over items of hdr[1] units of up to 128 rows; items
// per unit from mid_n_tiles (MXFP4: two 64-row halves per column tile).
hipError_t launch_gemm_mid(const GemmArgs& a, bool grouped, int grid_items, hipStream_t st);
int64_t mid_n_tiles(const Geom& G, bool mx);

// MFMA kernel with 256 x 256 output tiles.  Dense: one block per tile, or a
// persistent grid of one block per CU when there are more tiles than CUs (the
// last round's tiles split into 128-row halves when they fill half the grid
// or less, W4A16).  Grouped: persistent over (256-row unit x 256-column tile)
// items, hdr[2] units.
hipError_t launch_gemm_big(const GemmArgs& a, bool grouped, int grid_items, hipStream_t st);
int64_t big_n_tiles(const Geom& G);
// dense: tiles of the visiting order that run whole (the rest as 128-row halves)
int64_t big_full_tiles(const Geom& G, int64_t M, bool mx);

inline int kmode_of(const GemmArgs& a) {
  if (a.wfmt == W_MXINT4) return KM_MXI4_A16;
  if (a.wfmt == W_INT8_SYM) return KM_INT8_A16;
  if (a.wfmt == W_MXFP4 && a.a4) return KM_MX_A4;
  return a.wfmt != W_MXFP4 ? KM_INT4_A16 : (a.a8 ? KM_MX_A8 : KM_MX_A16);
}

}  // namespace hm
