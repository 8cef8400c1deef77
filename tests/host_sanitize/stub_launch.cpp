// Host-only stand-ins for the kernel launchers, linked with the library's
// host code (hm_api.cpp, plan_host.cpp) into a sanitizer build that runs on
// a machine without a GPU.  Each launcher checks the arguments the planner
// hands it against what the real kernel assumes, counts the call, and
// returns hipSuccess without touching device memory.  A violated assumption
// aborts the program with a message.
#include <stdio.h>
#include <stdlib.h>

#include "launch.h"

namespace hm {

long g_launches = 0;

static void need(bool ok, const char* what) {
  if (!ok) {
    fprintf(stderr, "launcher check failed: %s\n", what);
    abort();
  }
}

static void check_gemm(const GemmArgs& a, bool grouped, int grid_items) {
  need(a.w != nullptr && a.x != nullptr && a.y != nullptr, "weights, activations and output set");
  need(a.G.N >= 1 && a.G.K >= 128 && a.G.K % 128 == 0 && a.G.NB * 16 >= a.G.N, "geometry");
  need(!a.a8 || a.xs != nullptr, "FP8 rows come with row scales");
  need(!a.a4 || a.xsb != nullptr, "MXFP4 rows come with block scales");
  need(!(a.a8 && a.a4), "one activation format");
  need(!a.gated || (a.G.N % 32 == 0 && grouped), "gated output: grouped, N a multiple of 32");
  if (grouped) {
    need(grid_items >= 1, "grouped launches have items");
    need(a.units != nullptr && a.hdr != nullptr && a.sorted_pairs != nullptr, "grouped work lists");
    need(a.topk >= 1 && a.P >= 1, "routed pairs");
  } else {
    need(a.M >= 1, "dense rows");
  }
  ++g_launches;
}

hipError_t launch_transform(int wfmt, const Geom& G, const uint8_t* codes, const void* scales,
                            const uint8_t* zeros, uint8_t* out, int gated, hipStream_t) {
  need(wfmt >= 0 && wfmt <= 6 && codes && scales && out && G.total > 0, "transform arguments");
  need(!gated || G.N % 32 == 0, "gated layout pairs whole 16-column blocks");
  (void)zeros;
  ++g_launches;
  return hipSuccess;
}

hipError_t launch_dequant(int wfmt, const Geom& G, const uint8_t* w, int64_t e, float* out, hipStream_t) {
  need(wfmt >= 0 && wfmt <= 6 && w && out && e >= 0 && e < G.E, "dequant arguments");
  ++g_launches;
  return hipSuccess;
}

hipError_t launch_quant_fp8_rows(const uint16_t* x, int64_t m, int64_t k, uint8_t* x8, float* s, hipStream_t) {
  need(x && x8 && s && m >= 1 && k >= 1, "fp8 row arguments");
  ++g_launches;
  return hipSuccess;
}

hipError_t launch_quant_mxfp4_rows(const uint16_t* x, int64_t m, int64_t k, uint8_t* codes, uint8_t* scales,
                                   hipStream_t) {
  need(x && codes && scales && m >= 1 && k >= 32 && k % 32 == 0, "mxfp4 row arguments");
  ++g_launches;
  return hipSuccess;
}

hipError_t launch_moe_sort(const int32_t* ids, int64_t P, int E, int32_t* counts, int32_t* offsets,
                           int32_t* sorted_pairs, int32_t* cnt, hipStream_t) {
  need(ids && counts && offsets && sorted_pairs && P >= 1 && E >= 1 && E <= 512, "sort arguments");
  need(moe_sort_blocks(P, nullptr) == 1 || cnt != nullptr, "chunked sort has its count buffer");
  ++g_launches;
  return hipSuccess;
}

hipError_t launch_moe_schedule(const int32_t* offsets, int E, int64_t P, int s_rows, int s_max, int bm,
                               int big_min, int64_t max_s, int64_t max_t, int64_t max_b, int32_t* hdr,
                               int32_t* su, int32_t* tu, int32_t* bu, hipStream_t) {
  need(offsets && hdr && su && tu && bu && E >= 1 && E <= 512 && P >= 1, "schedule arguments");
  need((s_rows == 16 || s_rows == 32) && s_max >= 0 && bm >= 1 && bm <= 128 && big_min >= 0, "unit sizes");
  need(max_s >= 1 && max_t >= 1 && max_b >= 1, "unit list capacities");
  ++g_launches;
  return hipSuccess;
}

hipError_t launch_silu_mul(const uint16_t* gu, int64_t rows, int64_t d, uint16_t* h, hipStream_t) {
  need(gu && h && rows >= 1 && d >= 1, "silu arguments");
  ++g_launches;
  return hipSuccess;
}

hipError_t launch_silu_mul_fp8(const uint16_t* gu, int64_t rows, int64_t d, uint8_t* h8, float* hs, hipStream_t) {
  need(gu && h8 && hs && rows >= 1 && d % 8 == 0 && d >= 8 && d <= 8192, "fused silu arguments");
  ++g_launches;
  return hipSuccess;
}

hipError_t launch_combine(const uint16_t* y, const float* w, int64_t t, int topk, int64_t n, uint16_t* out,
                          hipStream_t) {
  need(y && w && out && t >= 1 && topk >= 1 && n >= 1, "combine arguments");
  ++g_launches;
  return hipSuccess;
}

hipError_t launch_read_probe(const void* buf, int64_t bytes, int blocks, int unroll, uint32_t* out, hipStream_t) {
  need(buf && out && bytes >= 16 && blocks >= 1 && unroll >= 1, "read probe arguments");
  ++g_launches;
  return hipSuccess;
}

hipError_t launch_gemm_stream(const GemmArgs& a, const StreamCfg& c, bool grouped, int grid_items, hipStream_t) {
  check_gemm(a, grouped, grouped ? grid_items : 1);
  need(c.mb == 1 || c.mb == 2, "stream rows per unit");
  need(c.nbw == 1 || c.nbw == 2, "stream column blocks per wave");
  need(c.nw == 4 || (c.nw == 8 && !grouped), "stream waves per block");
  need(c.ks == 1 || c.ks == 2 || c.ks == 4 || (c.ks == 8 && c.nw == 8), "stream K split over waves");
  need(c.nw == 4 || c.ks >= 2, "eight-wave blocks split K");
  need(c.splits >= 1 && (c.splits == 1 || (!grouped && a.part != nullptr)), "split-K partials");
  need(grouped || a.M <= 256, "dense streaming rows");
  return hipSuccess;
}

hipError_t launch_splitk_reduce(const GemmArgs& a, int splits, hipStream_t) {
  need(splits >= 2 && a.part && a.y && a.M >= 1, "split-K reduction arguments");
  ++g_launches;
  return hipSuccess;
}

hipError_t launch_gemm_tile(const GemmArgs& a, bool grouped, int grid_items, hipStream_t) {
  check_gemm(a, grouped, grid_items);
  return hipSuccess;
}

hipError_t launch_gemm_mid(const GemmArgs& a, bool grouped, int grid_items, hipStream_t) {
  check_gemm(a, grouped, grid_items);
  need(kmode_of(a) != KM_MX_A4 && kmode_of(a) != KM_INT8_A16, "128-row tile kernel formats");
  if (grouped) {
    const int64_t xrows = a.rows_are_pairs ? a.P : (a.P + a.topk - 1) / a.topk;
    need(xrows * (a.a8 ? 1 : 2) * a.G.K <= 0xFFFFFFFFll, "grouped 128-row units address rows in 32 bits");
  }
  return hipSuccess;
}

hipError_t launch_gemm_big(const GemmArgs& a, bool grouped, int grid_items, hipStream_t) {
  check_gemm(a, grouped, grid_items);
  const int km = kmode_of(a);
  need(km >= KM_INT4_A16 && km <= KM_INT8_A16, "256 x 256 kernel formats");
  need(a.G.total - a.G.off_scales <= 0xFFFFFFFFull, "scale region addressed in 32 bits");
  return hipSuccess;
}

}  // namespace hm
