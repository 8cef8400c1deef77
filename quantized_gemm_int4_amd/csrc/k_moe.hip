// MoE expert sort and grouped-GEMM scheduling.
//
// Tokens are split per expert, so every expert's GEMM has its own M that
// depends on the routing load (ywsung.com note "How vLLM Humming computes 4
// bits", section on one token vs many tokens).  The sort groups the
// (token, expert) pairs by expert; the scheduler cuts every expert's segment
// into row units for the two GEMM kernels (short segments to the streaming
// kernel, long ones to the MFMA tile kernel).
#include "common.h"
#include "launch.h"

namespace hm {

constexpr int kSortThreads = 1024;
constexpr int kSortWaves = kSortThreads / 64;

// Inclusive scan of one value per thread over the first 512 threads of a
// block (8 waves).  `wsum` is 8 ints of shared scratch.  Must be reached by
// every thread of the block.
__device__ int block_scan512(int v, int* wsum) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int off = 1; off < 64; off <<= 1) {
    const int u = __shfl_up(v, off, 64);
    if (lane >= off) v += u;
  }
  if (lane == 63 && wave < 8) wsum[wave] = v;
  __syncthreads();
  int pre = 0;
  for (int w = 0; w < wave && w < 8; ++w) pre += wsum[w];
  __syncthreads();
  return v + pre;
}

// Places the pairs of [lo, hi) stably: wave w owns the contiguous subrange
// [lo + w*chunk, ...), its per-expert base positions are base[e] plus the
// counts of earlier waves, and inside a wave each batch of 64 pairs is ranked
// in lane order with ballot matching.  hist is the block's [16][512] LDS
// array (zeroed here); base[e] (LDS) is the first position of this range's
// pairs of expert e.  Must be reached by every thread of the block.
__device__ void sort_range(const int32_t* __restrict__ ids, int64_t lo, int64_t hi, int E, const int* base,
                           int (*hist)[512], int32_t* __restrict__ sorted_pairs) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int i = tid; i < kSortWaves * 512; i += kSortThreads) (&hist[0][0])[i] = 0;
  __syncthreads();
  const int64_t chunk = (hi - lo + kSortWaves - 1) / kSortWaves;
  const int64_t beg = lo + wave * chunk;
  const int64_t end = (beg + chunk < hi) ? beg + chunk : hi;
  for (int64_t b = beg; b < end; b += 64) {
    const int64_t p = b + lane;
    if (p < end) {
      const int e = ids[p];
      if (e >= 0 && e < E) atomicAdd(&hist[wave][e], 1);
    }
  }
  __syncthreads();
  if (tid < E) {
    int run = base[tid];
    for (int w = 0; w < kSortWaves; ++w) {
      const int c = hist[w][tid];
      hist[w][tid] = run;
      run += c;
    }
  }
  __syncthreads();
  int nbits = 0;
  while ((1 << nbits) < E) ++nbits;
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int64_t b = beg; b < end; b += 64) {
    const int64_t p = b + lane;
    int e = -1;
    if (p < end) e = ids[p];
    const bool valid = (e >= 0 && e < E);
    uint64_t m = __ballot(valid);
    for (int bit = 0; bit < nbits; ++bit) {
      const uint64_t x = __ballot(valid && ((e >> bit) & 1));
      m &= ((e >> bit) & 1) ? x : ~x;
    }
    if (valid) {
      const int rank = __popcll(m & lt);
      const int pos = hist[wave][e] + rank;
      sorted_pairs[pos] = (int32_t)p;
    }
    __builtin_amdgcn_wave_barrier();
    if (valid && __popcll(m & lt) == 0) hist[wave][e] += __popcll(m);
    __builtin_amdgcn_wave_barrier();
  }
}

// Exclusive scan of the per-expert totals tot[] (LDS) into base[] (LDS,
// adding what base[] holds), and, when `out` is set, the counts and offsets.
__device__ void expert_offsets(const int* tot, int* base, int E, int* wsum, bool out, int32_t* __restrict__ counts,
                               int32_t* __restrict__ offsets) {
  const int tid = threadIdx.x;
  const int total = tid < E ? tot[tid] : 0;
  const int incl = block_scan512(tid < 512 ? total : 0, wsum);
  const int excl = incl - total;
  if (tid < E) {
    base[tid] += excl;
    if (out) {
      counts[tid] = total;
      offsets[tid] = excl;
      if (tid == E - 1) offsets[E] = incl;
    }
  }
  __syncthreads();
}

// Deterministic, stable counting sort of pair ids by expert in one block
// (few pairs).
__global__ void __launch_bounds__(kSortThreads)
k_moe_sort(const int32_t* __restrict__ ids, int64_t P, int E, int32_t* __restrict__ counts,
           int32_t* __restrict__ offsets, int32_t* __restrict__ sorted_pairs) {
  __shared__ int hist[kSortWaves][512];
  __shared__ int tot[512], base[512];
  __shared__ int wsum[8];
  const int tid = threadIdx.x;
  for (int i = tid; i < 512; i += kSortThreads) { tot[i] = 0; base[i] = 0; }
  __syncthreads();
  for (int64_t p = tid; p < P; p += kSortThreads) {
    const int e = ids[p];
    if (e >= 0 && e < E) atomicAdd(&tot[e], 1);
  }
  __syncthreads();
  expert_offsets(tot, base, E, wsum, true, counts, offsets);
  sort_range(ids, 0, P, E, base, hist, sorted_pairs);
}

// GPU-wide sort, pass 1: block b counts the pairs of its chunk
// [b*C, min((b+1)*C, P)) per expert into cnt[b][e] (every e < E written).
__global__ void __launch_bounds__(kSortThreads)
k_moe_sort_count(const int32_t* __restrict__ ids, int64_t P, int E, int64_t C, int32_t* __restrict__ cnt) {
  __shared__ int h[512];
  const int tid = threadIdx.x;
  for (int i = tid; i < 512; i += kSortThreads) h[i] = 0;
  __syncthreads();
  const int64_t lo = (int64_t)blockIdx.x * C;
  const int64_t hi = (lo + C < P) ? lo + C : P;
  for (int64_t p = lo + tid; p < hi; p += kSortThreads) {
    const int e = ids[p];
    if (e >= 0 && e < E) atomicAdd(&h[e], 1);
  }
  __syncthreads();
  for (int e = tid; e < E; e += kSortThreads) cnt[(int64_t)blockIdx.x * E + e] = h[e];
}

// Pass 2: block b sums every chunk's counts per expert (the totals) and those
// of the chunks before its own, scans the totals into the expert offsets
// (block 0 writes counts and offsets), and places its chunk's pairs after
// those of the earlier chunks: the order is stable over the whole input.
__global__ void __launch_bounds__(kSortThreads)
k_moe_sort_place(const int32_t* __restrict__ ids, int64_t P, int E, int64_t C, int nb,
                 const int32_t* __restrict__ cnt, int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                 int32_t* __restrict__ sorted_pairs) {
  __shared__ int hist[kSortWaves][512];
  __shared__ int tot[512], base[512];
  __shared__ int wsum[8];
  const int tid = threadIdx.x;
  const int b = blockIdx.x;
  for (int i = tid; i < 512; i += kSortThreads) { tot[i] = 0; base[i] = 0; }
  __syncthreads();
  const int64_t all = (int64_t)nb * E;
  for (int64_t i = tid; i < all; i += kSortThreads) {
    const int bb = (int)(i / E), e = (int)(i - (int64_t)bb * E);
    const int c = cnt[i];
    if (c) {
      atomicAdd(&tot[e], c);
      if (bb < b) atomicAdd(&base[e], c);
    }
  }
  __syncthreads();
  expert_offsets(tot, base, E, wsum, b == 0, counts, offsets);
  const int64_t lo = (int64_t)b * C;
  const int64_t hi = (lo + C < P) ? lo + C : P;
  sort_range(ids, lo, hi, E, base, hist, sorted_pairs);
}

// Work units of a grouped GEMM from the expert offsets (one thread per
// expert, E <= 512).  An expert with 1..s_max rows becomes ceil(rows/s_rows)
// consecutive streaming units of at most s_rows rows (the streaming kernel
// takes s_rows rows per unit; consecutive units of one expert run side by
// side and share its weights through the L2).  A larger one is cut into
// 256-row units while big_min > 0 (a remainder of at least big_min rows is
// one more 256-row unit) and what is left into units of at most bm rows for
// the 128-row tile kernel.  Units are {expert, first index into
// sorted_pairs, rows, 0}; hdr = {streaming units, tile units, 256-row
// units}, each capped at its array size.
__global__ void __launch_bounds__(512)
k_moe_schedule(const int32_t* __restrict__ offsets, int E, int64_t P, int s_rows, int s_max, int bm, int big_min,
               int64_t max_s, int64_t max_t, int64_t max_b, int32_t* __restrict__ hdr,
               int32_t* __restrict__ su, int32_t* __restrict__ tu, int32_t* __restrict__ bu) {
  __shared__ int wsum[8];
  const int e = threadIdx.x;
  int c = 0, beg = 0;
  if (e < E) {
    // clamp to [0, P] so that malformed offsets can never address outside the pairs
    int64_t b = offsets[e], f = offsets[e + 1];
    b = b < 0 ? 0 : (b > P ? P : b);
    f = f < b ? b : (f > P ? P : f);
    beg = (int)b;
    c = (int)(f - b);
  }
  const int ns = (c > 0 && c <= s_max) ? (c + s_rows - 1) / s_rows : 0;
  int nb = 0, rest = 0;
  if (c > s_max) {
    if (big_min > 0) {
      nb = c / kBigRows;
      rest = c - nb * kBigRows;
      if (rest >= big_min) { ++nb; rest = 0; }
    } else {
      rest = c;
    }
  }
  const int nt = (rest + bm - 1) / bm;
  const int is = block_scan512(ns, wsum);
  const int it = block_scan512(nt, wsum);
  const int ib = block_scan512(nb, wsum);
  for (int i = 0; i < ns; ++i) {
    if (is - ns + i >= max_s) break;
    int32_t* u = su + 4 * (is - ns + i);
    const int r0 = i * s_rows;
    u[0] = e; u[1] = beg + r0; u[2] = (c - r0 < s_rows) ? c - r0 : s_rows; u[3] = 0;
  }
  for (int i = 0; i < nb; ++i) {
    if (ib - nb + i >= max_b) break;
    int32_t* u = bu + 4 * (ib - nb + i);
    const int r0 = i * kBigRows;
    u[0] = e; u[1] = beg + r0; u[2] = (c - r0 < kBigRows) ? c - r0 : kBigRows; u[3] = 0;
  }
  const int t0 = c - rest;                        // first row left for the tile units
  for (int i = 0; i < nt; ++i) {
    if (it - nt + i >= max_t) break;
    int32_t* u = tu + 4 * (it - nt + i);
    const int r0 = t0 + i * bm;
    u[0] = e; u[1] = beg + r0; u[2] = (c - r0 < bm) ? c - r0 : bm; u[3] = 0;
  }
  if (e == 511) {
    hdr[0] = (int32_t)(is < max_s ? is : max_s);
    hdr[1] = (int32_t)(it < max_t ? it : max_t);
    hdr[2] = (int32_t)(ib < max_b ? ib : max_b);
  }
}


hipError_t launch_moe_sort(const int32_t* ids, int64_t P, int E, int32_t* counts, int32_t* offsets,
                           int32_t* sorted_pairs, int32_t* cnt, hipStream_t st) {
  int64_t C = 0;
  const int nb = moe_sort_blocks(P, &C);
  if (nb == 1) {
    hipLaunchKernelGGL(k_moe_sort, dim3(1), dim3(kSortThreads), 0, st, ids, P, E, counts, offsets,
                       sorted_pairs);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(k_moe_sort_count, dim3(nb), dim3(kSortThreads), 0, st, ids, P, E, C, cnt);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_moe_sort_place, dim3(nb), dim3(kSortThreads), 0, st, ids, P, E, C, nb, cnt, counts,
                     offsets, sorted_pairs);
  return hipGetLastError();
}

hipError_t launch_moe_schedule(const int32_t* offsets, int E, int64_t P, int s_rows, int s_max, int bm,
                               int big_min, int64_t max_s, int64_t max_t, int64_t max_b, int32_t* hdr,
                               int32_t* su, int32_t* tu, int32_t* bu, hipStream_t st) {
  hipLaunchKernelGGL(k_moe_schedule, dim3(1), dim3(512), 0, st, offsets, E, P, s_rows, s_max, bm, big_min,
                     max_s, max_t, max_b, hdr, su, tu, bu);
  return hipGetLastError();
}

}  // namespace hm
