// Launch-geometry helpers of the planner (host code only): how many column
// tiles each kernel's launch covers, which dense 256 x 256 tiles run whole,
// and how the expert sort cuts its pairs into chunks.
#include "launch.h"

namespace hm {

int64_t stream_n_tiles(const Geom& G, const StreamCfg& c) {
  const int64_t cols = (int64_t)(c.nw / c.ks) * c.nbw;   // 16-column blocks per block
  return (G.NB + cols - 1) / cols;
}

int64_t mid_n_tiles(const Geom& G, bool mx) {
  return mx ? 2 * ((G.NB + kMxCB - 1) / kMxCB) : (G.NB + kMidCB - 1) / kMidCB;
}

int64_t big_n_tiles(const Geom& G) { return (G.NB + kBigCB - 1) / kBigCB; }

// Dense 256 x 256 launches run more tiles than one block per CU as a
// persistent grid; a last round that fills half the grid or less (and whose
// row tail is more than 128 rows, or none) runs as 128-row halves.
int64_t big_full_tiles(const Geom& G, int64_t M, bool mx) {
  const int64_t tiles_n = (G.NB + kBigCB - 1) / kBigCB, tiles_m = (M + kBigM - 1) / kBigM;
  const int64_t tiles = tiles_n * tiles_m, rest = tiles % kBigGrid;
  const bool tail_ok = (M % kBigM) == 0 || (M % kBigM) > kBigM / 2;
  if (mx || tiles <= kBigGrid || rest == 0 || 2 * rest > kBigGrid || !tail_ok) return tiles;
  return tiles - rest;
}

int moe_sort_blocks(int64_t P, int64_t* chunk) {
  int nb = 1;
  if (P > kSortOneBlock) {
    const int64_t want = (P + kSortChunk - 1) / kSortChunk;
    nb = (int)(want < kSortMaxBlocks ? want : kSortMaxBlocks);
  }
  if (chunk) *chunk = (P + nb - 1) / nb;
  return nb;
}

}  // namespace hm
