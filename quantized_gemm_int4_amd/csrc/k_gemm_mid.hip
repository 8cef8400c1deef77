// W4A16 MFMA GEMM for mid-sized M (tens to a few hundred rows, and the
// up-to-128-row units of a grouped GEMM), where the matrix multiply already
// dominates but a 256 x 256 tile would leave most compute units idle (ywsung.com
// note "How vLLM Humming computes 4 bits", section on one token vs many
// tokens: the dequantized weights feed the matrix cores once the batch is
// large enough).
//
// One 256-thread block computes a 128 x 64 output tile over the whole K range,
// so a 128-row batch already gives N / 64 blocks.  The K range runs in groups
// of 128 (one scale per column and group); the four waves split every group:
// wave w takes its K values 32 w .. 32 w + 31 for all 128 rows and 64 columns
// (2 x 4 blocks of 32x32x16 bf16 MFMAs, 128 accumulators per lane), so each
// weight nibble is unpacked once per block and each activation byte read once
// from LDS.  The four partial tiles are summed through LDS at the end.
//
// Data movement, all by 16-byte (4-byte for scales) direct buffer-to-LDS
// copies, issued between the MFMAs:
//   * activations: 128 rows x 256 bytes per group, row-major with chunk c of
//     row r at slot c ^ (r % 16) (the 16 lanes of an operand read hit all 64
//     banks once); each copy reads four whole rows (eight 128-byte lines);
//     four stages, copied three groups ahead;
//   * weights: the tile's four 1 KiB code tiles of a group plus a gather of
//     their bf16 scales and zero points; six group slots, copied five groups
//     ahead (they come from HBM, the activations mostly from L2).
// Operands of the next group's first K part are unpacked during the second
// K part of the current one, so each group starts with ready operands.
//
// MX weights with bf16 rows (F4: MXFP4, and MXINT4 with I4, whose two's
// complement codes are converted on the vector ALU) run the same kernel: wave w's K values
// 32 w .. 32 w + 31 are exactly the E2M1 codes of quarter w of each 16-byte
// slot, whose words 2 kk' + hi the lanes read, with one E8M0 scale per lane
// and column half; the gather copies the 256 bytes of scale words of the
// wave's column block (four groups each) and the codes are scaled to bf16
// by the hardware conversion instead of the INT4 arithmetic.
//
// W4A8-MXFP4 (k_gemm_mid_mx): one K group (128 values) is a single scaled
// 16x16x128 fp4 x fp8 MFMA, so the waves split the tile instead: 64 rows x
// 128 columns per 256-thread block (224 blocks for M = 256, N = 7168), each
// wave 32 rows x 64 columns (2 x 4 MFMA blocks).  E2M1 code tiles and their
// E8M0 scale words are fed to the MFMA as stored; the per-token FP8 scale is
// applied in the epilogue.  Six LDS stages of one group each (activations,
// the eight code tiles, their scale words), copied five groups ahead; the
// fragments of the next group are read during the current one.
#include <algorithm>

#include "common.h"
#include "launch.h"

namespace hm {

namespace {

constexpr int kMidM = 128;                       // rows per tile
constexpr int kMidDX = 3;                        // activation groups copied ahead
constexpr int kMidDW = 5;                        // weight groups copied ahead
constexpr int kMidXS = kMidDX + 1;               // activation stages
constexpr int kMidWS = kMidDW + 1;               // weight group slots
constexpr int kMidXBytes = kMidM * 256;          // one activation stage (32 KiB)
constexpr int kMidWBytes = kMidCB * 1024 + kMidCB * 256;   // code tiles + scale gathers
constexpr int kMidLds = kMidXS * kMidXBytes + kMidWS * kMidWBytes;   // 158 KiB
constexpr int kMidCopies = 8 + 2;                // copies per wave per group

struct MidTile {
  int64_t e, m0, nb0, rows, first;
};

constexpr int kMxM = 64;                         // rows per W4A8 tile
// six stages: eight (one K group each, copied seven ahead) measured no
// faster at M = 64..256 (N = 7168, K = 2048: 10.1-10.8 us against 10.0)
constexpr int kMxStages = 6;                     // one K group each, copied five ahead
constexpr int kMxSB = 8 * 1024 + kMxCB * 1024 + kMxCB * 256;   // activations, code tiles, scale words
constexpr int kMxLds = kMxStages * kMxSB;        // 108 KiB
constexpr int kMxCopies = 6;                     // copies per wave per group

// One group's operands of a wave: its four code tiles and their scale words,
// and both 16-byte halves of its two row blocks' activation fragments.
struct MxFrag {
  u32x4_t wq[4];
  uint32_t ws[4];
  u32x4_t b0[2], b1[2];
};

}  // namespace

template <bool ZP, bool GROUPED, bool F4, bool I4>
__global__ void __launch_bounds__(256, 1)
k_gemm_mid(GemmArgs a, int tiles_n, int tiles_m) {
  extern __shared__ __attribute__((aligned(1024))) uint8_t lds[];
  __shared__ int32_t orow_s[GROUPED ? kMidM : 1];   // output row of each local row, or -1

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hi = lane >> 5, c_l = l32 >> 4, c16 = l32 & 15;
  const Geom G = a.G;
  const int64_t row_bytes = 2 * G.K;
  const int KG = (int)G.KG;
  const int64_t n_items = GROUPED ? (int64_t)a.hdr[1] * tiles_n : (int64_t)tiles_n * tiles_m;

  auto decode = [&](int64_t it) -> MidTile {
    MidTile t;
    if (GROUPED) {
      const int32_t* u = a.units + 4 * (it / tiles_n);
      t.e = u[0];
      t.first = u[1];
      t.rows = u[2] < kMidM ? u[2] : kMidM;
      t.m0 = 0;
      t.nb0 = (it % tiles_n) * kMidCB;
    } else {
      // block b runs on XCD b % 8: each XCD takes a contiguous range of
      // tiles, row tiles fastest, so its blocks share weight columns
      const int total = tiles_n * tiles_m;
      const int xcd = (int)(it % 8), idx = (int)(it / 8);
      const int base = total / 8, extra = total % 8;
      const int tt = (total >= 8) ? xcd * base + (xcd < extra ? xcd : extra) + idx : (int)it;
      t.e = 0;
      t.first = 0;
      t.m0 = (int64_t)(tt % tiles_m) * kMidM;
      t.nb0 = (int64_t)(tt / tiles_m) * kMidCB;
      t.rows = (a.M - t.m0) < kMidM ? (a.M - t.m0) : kMidM;
    }
    return t;
  };
  auto act_row = [&](int32_t pair) -> int64_t {
    if (pair < 0 || pair >= a.P) return 0;
    return a.rows_are_pairs ? pair : pair / a.topk;
  };

  // scale / zero-point gather of the wave's column block: lanes 0..7 the 16
  // bf16 scales (4 bytes each), lanes 8, 9 the two zero-point words
  const bool zlane = ZP && (lane == 8 || lane == 9);
  const uint32_t szstride = zlane ? 8u : 32u;
  const rsrc_t rsz = make_rsrc(a.w + G.off_scales, G.total - G.off_scales);

  // ---- per-lane operand offsets (constant over the tile)
  // B operand (activations) of row block mb, K part kk (= 2 w + kk' within
  // the group): row 32 mb + l32, 16-byte chunk 2 kk + hi
  uint32_t xo[2];
#pragma unroll
  for (int k2 = 0; k2 < 2; ++k2) xo[k2] = (uint32_t)(l32 * 256 + 16 * ((4 * wave + 2 * k2 + hi) ^ (l32 & 15)));
  // A operand (weights) of column half nb2, K part kk': column 32 nb2 + l32 in
  // code tile 2 nb2 + c_l, word w of slot c16 + 16 (2 kk' + hi) (INT4), word
  // 2 kk' + hi of slot c16 + 16 w (MXFP4)
  uint32_t wo[2][2];
#pragma unroll
  for (int nb2 = 0; nb2 < 2; ++nb2)
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2)
      wo[nb2][k2] = F4 ? (uint32_t)((2 * nb2 + c_l) * 1024 + (c16 + 16 * wave) * 16 + 4 * (2 * k2 + hi))
                       : (uint32_t)((2 * nb2 + c_l) * 1024 + (c16 + 16 * (2 * k2 + hi)) * 16 + 4 * wave);

  int64_t item = blockIdx.x;
  while (item < n_items) {
    const MidTile t = decode(item);
    // ---- copy descriptors of this tile
    const rsrc_t rx = make_rsrc(reinterpret_cast<const uint8_t*>(a.x) + t.m0 * row_bytes,
                                GROUPED ? 0xFFFFFFFFull : (uint64_t)t.rows * row_bytes);
    uint32_t xoff[8];   // activation copy j: rows 32 w + 4 j + L / 16, slot L % 16
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int r = 32 * wave + 4 * j + (lane >> 4);
      const int rc = r < t.rows ? r : (int)t.rows - 1;
      const int64_t src = GROUPED ? act_row(a.sorted_pairs[t.first + rc]) : rc;
      xoff[j] = (uint32_t)(src * row_bytes) + 16u * (uint32_t)((lane & 15) ^ (r & 15));
    }
    const int64_t wb = t.e * G.NB;
    int64_t nbw = t.nb0 + wave;
    if (nbw >= G.NB) nbw = G.NB - 1;
    const rsrc_t rw = make_rsrc(a.w + (wb + nbw) * G.KG * 1024, (uint64_t)G.KG * 1024);
    const uint32_t wvo = (uint32_t)lane * 16u;
    const uint32_t svo = F4 ? (uint32_t)((wb + nbw) * G.KG4 * 256 + lane * 4)
                         : zlane ? (uint32_t)((G.off_zeros - G.off_scales) + (wb + nbw) * G.KG * 8 + (lane - 8) * 4)
                                 : (uint32_t)((wb + nbw) * G.KG * 32 + (lane & 7) * 4);
    if (GROUPED && tid < kMidM) {
      const int32_t p = tid < t.rows ? a.sorted_pairs[t.first + tid] : -1;
      orow_s[tid] = (p >= 0 && p < a.P) ? p : -1;
    }

    // stage / slot offsets of groups g .. g + kMidDX (activations) and
    // g .. g + kMidDW (weights), rotated after every group
    uint32_t xso[kMidXS], wso[kMidWS];
#pragma unroll
    for (int i = 0; i < kMidXS; ++i) xso[i] = (uint32_t)(i * kMidXBytes);
#pragma unroll
    for (int i = 0; i < kMidWS; ++i) wso[i] = (uint32_t)(kMidXS * kMidXBytes + i * kMidWBytes);

    auto copy_x = [&](int q, int g, uint32_t so) {
      b2lds16(rx, xoff[q], (uint32_t)(g * 256), lds + so + (8 * wave + q) * 1024);
    };
    auto copy_w = [&](int g, uint32_t so) {
      b2lds16(rw, wvo, (uint32_t)(g * 1024), lds + so + wave * 1024);
    };
    auto copy_sz = [&](int g, uint32_t so) {
      // MXFP4: the scale words of groups 4 (g / 4) .. + 3, 256 bytes
      b2lds4(rsz, F4 ? svo + (uint32_t)(g >> 2) * 256u : svo + (uint32_t)g * szstride, 0u,
             lds + so + kMidCB * 1024 + wave * 256);
    };

    // ---- prologue: weights of groups 0 .. DW - 1 and activations of 0 .. DX
    // - 1 (those that exist); the first group needs weights 0, 1 and
    // activations 0, 1, issued first, so the wait leaves the rest in flight
    auto pro_w = [&](int g) {
      if (g < KG) {
        copy_w(g, wso[g]);
        copy_sz(g, wso[g]);
      }
    };
    auto pro_x = [&](int g) {
      if (g < KG) {
#pragma unroll
        for (int q = 0; q < 8; ++q) copy_x(q, g, xso[g]);
      }
    };
    pro_w(0);
    pro_w(1);
    pro_x(0);
    pro_x(1);
    pro_w(2);
    pro_x(2);
    pro_w(3);
    pro_w(4);
    if (KG >= 5) __asm__ volatile("s_waitcnt vmcnt(14)\n\ts_barrier" ::: "memory");
    else __asm__ volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");

    // code word, scale and s * (-z) of column half nb2, K part kk' of group g in slot so
    auto fetch = [&](uint32_t so, int g, uint32_t (&wq)[2][2], float (&sv)[2], float (&zs)[2]) {
      const uint8_t* slot = lds + so;
#pragma unroll
      for (int nb2 = 0; nb2 < 2; ++nb2) {
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2) wq[nb2][k2] = *reinterpret_cast<const uint32_t*>(slot + wo[nb2][k2]);
        const uint8_t* sz = slot + kMidCB * 1024 + (2 * nb2 + c_l) * 256;
        if (F4) {
          // E8M0 of (column c16, K block w): byte g % 4 of scale word c16 + 16 w
          const uint32_t sw = *reinterpret_cast<const uint32_t*>(sz + 4 * (c16 + 16 * wave));
          sv[nb2] = e8m0_f32((sw >> (8 * (g & 3))) & 0xFFu) * (I4 ? 0.25f : 1.0f);   // MXINT4: q / 4
          zs[nb2] = 0.f;
          continue;
        }
        sv[nb2] = bf16_to_f32(*reinterpret_cast<const uint16_t*>(sz + 2 * c16));
        const uint32_t zw = ZP ? *reinterpret_cast<const uint32_t*>(sz + 32 + 4 * (c16 >> 3)) : 0u;
        const float z = ZP ? (float)((zw >> (4 * (c16 & 7))) & 0xFu) : 8.0f;
        zs[nb2] = -z * sv[nb2];
      }
    };

    u32x4_t af[2][2];        // operands (nb2, kk') of the current group
    uint32_t c1[2];          // code words of K part 1 of the current group
    float csv[2], czs[2];
    {
      uint32_t wq[2][2];
      fetch(wso[0], 0, wq, csv, czs);
#pragma unroll
      for (int nb2 = 0; nb2 < 2; ++nb2) {
        af[nb2][0] = I4 ? i4x8_bf16(wq[nb2][0], csv[nb2])
                     : F4 ? fp4x8_bf16(wq[nb2][0], csv[nb2]) : dq8_bytes(wq[nb2][0], csv[nb2], czs[nb2]);
        af[nb2][1] = (u32x4_t){0u, 0u, 0u, 0u};
        c1[nb2] = wq[nb2][1];
      }
    }
    f32x16_t acc[2][4];
#pragma unroll
    for (int nb2 = 0; nb2 < 2; ++nb2)
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[nb2][mb][r] = 0.f;

    // activation fragments (row block i % 4, K part i / 4), read kD ahead
    constexpr int kD = 4;
    u32x4_t b[8];
#pragma unroll
    for (int i = 0; i < kD; ++i) b[i] = ld16(lds + xso[0] + (i & 3) * 8192 + xo[i >> 2]);

    // Group g: 16 MFMAs per wave in eight pairs (K part kk' = i / 4, row
    // block i % 4, both column halves).  During K part 0 the operands of K
    // part 1 are unpacked, during K part 1 those of the next group's K part
    // 0 (two result words per pair).  Copy q of the group (activations of
    // group g + DX, then the weight tile and scale gather of group g + DW,
    // while those exist) is issued after pair max(0, q - 2) / (q < 4 ? 2 :
    // 1), spreading the ten copies over the group.
#pragma nounroll
    for (int g = 0; g < KG; ++g) {
      uint32_t nq[2][2];
      float nsv[2], nzs[2];
      fetch(wso[1], g + 1, nq, nsv, nzs);
      // past the end: repeats of the last group into slots no longer read
      const int xg = std::min(g + kMidDX, KG - 1), wg = std::min(g + kMidDW, KG - 1);
      const uint32_t xd = xso[kMidDX], wd = wso[kMidDW];
      auto dma = [&](int q) {
        if (q < 8) copy_x(q, xg, xd);
        else if (q == 8) copy_w(wg, wd);
        else copy_sz(wg, wd);
      };
      const uint8_t* xs = lds + xso[0];
      uint32_t lo = 0, hi4 = 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int k2 = i >> 2, mb = i & 3;
#pragma unroll
        for (int nb2 = 0; nb2 < 2; ++nb2) acc[nb2][mb] = mfma32_bf16(af[nb2][k2], b[i], acc[nb2][mb]);
        if (i + kD < 8) b[i + kD] = ld16(xs + ((i + kD) & 3) * 8192 + xo[(i + kD) >> 2]);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int wi = 2 * (i & 3) + h;          // result word 0..7 of this K part's pair of operands
          const int nb2 = wi >> 2, u = wi & 3;
          const uint32_t w = k2 == 0 ? c1[nb2] : nq[nb2][0];
          const float sv = k2 == 0 ? csv[nb2] : nsv[nb2], zs = k2 == 0 ? czs[nb2] : nzs[nb2];
          if (F4) {
            af[nb2][k2 ^ 1][u] = I4 ? i4x2_bf16(w, sv, u) : fp4x2_bf16(w, sv, u);
            continue;
          }
          if (u == 0) {
            lo = in_vgpr(w & 0x0F0F0F0Fu);
            hi4 = in_vgpr((w >> 4) & 0x0F0F0F0Fu);
          }
          af[nb2][k2 ^ 1][u] = dq8_word(lo, hi4, u, sv, zs);
        }
        if (i == 0) { dma(0); dma(1); }
        else if (i == 1) { dma(2); dma(3); }
        else dma(i + 2);
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int nb2 = 0; nb2 < 2; ++nb2) {
        c1[nb2] = nq[nb2][1];
        csv[nb2] = nsv[nb2];
        czs[nb2] = nzs[nb2];
      }
      // rotate the stages: group g + 1 becomes the current one
      {
        const uint32_t x0 = xso[0];
#pragma unroll
        for (int i = 0; i + 1 < kMidXS; ++i) xso[i] = xso[i + 1];
        xso[kMidXS - 1] = x0;
        const uint32_t w0 = wso[0];
#pragma unroll
        for (int i = 0; i + 1 < kMidWS; ++i) wso[i] = wso[i + 1];
        wso[kMidWS - 1] = w0;
      }
      // the next group's activations landed before the last barrier: read
      // its first fragments, then wait for all but this group's copies (which covers the activations
      // of group g + 2, read during the next group, and the weights of group
      // g + 4) and meet the other waves
#pragma unroll
      for (int i = 0; i < kD; ++i) b[i] = ld16(lds + xso[0] + (i & 3) * 8192 + xo[i >> 2]);
      __asm__ volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(kMidCopies) : "memory");
    }

    // ---- epilogue: sum the four waves' partial tiles.  Lane holds
    // C[n = 32 nb2 + 8 j + 4 hi + r][row = 32 mb + l32] in acc[nb2][mb][4 j + r];
    // every wave stores its partial of row block mb in LDS region (wave,
    // mb), 8 KiB each, and wave w sums the four partials of row block w.
    // The repeats of the last groups land first.
    __asm__ volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      uint8_t* reg = lds + (wave * 4 + mb) * 8192;
#pragma unroll
      for (int nb2 = 0; nb2 < 2; ++nb2)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          *reinterpret_cast<f32x4_t*>(reg + ((nb2 * 4 + j) * 64 + lane) * 16) =
              (f32x4_t){acc[nb2][mb][4 * j], acc[nb2][mb][4 * j + 1], acc[nb2][mb][4 * j + 2], acc[nb2][mb][4 * j + 3]};
    }
    __asm__ volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    f32x16_t sum[2];
#pragma unroll
    for (int nb2 = 0; nb2 < 2; ++nb2)
#pragma unroll
      for (int r = 0; r < 16; ++r) sum[nb2][r] = 0.f;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const uint8_t* reg = lds + (s * 4 + wave) * 8192;
#pragma unroll
      for (int nb2 = 0; nb2 < 2; ++nb2)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const f32x4_t v = *reinterpret_cast<const f32x4_t*>(reg + ((nb2 * 4 + j) * 64 + lane) * 16);
#pragma unroll
          for (int r = 0; r < 4; ++r) sum[nb2][4 * j + r] += v[r];
        }
    }
    // bf16 rows of block w staged in region (w, w), which only this wave
    // reads, 128 bytes per row with 16-byte chunk c of row r at c ^ (r % 8),
    // then stored as whole rows (eight lanes per row)
    uint8_t* ost = lds + (wave * 4 + wave) * 8192;
    __asm__ volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
    for (int nb2 = 0; nb2 < 2; ++nb2)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int cidx = 4 * nb2 + j;              // 16-byte chunk of columns 8 cidx .. 8 cidx + 7
        *reinterpret_cast<u32x2_t*>(ost + l32 * 128 + ((cidx ^ (l32 & 7)) * 16) + 8 * hi) =
            (u32x2_t){pack_bf16(sum[nb2][4 * j], sum[nb2][4 * j + 1]), pack_bf16(sum[nb2][4 * j + 2], sum[nb2][4 * j + 3])};
      }
    __asm__ volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int r = 8 * k + (lane >> 3), cidx = lane & 7;
      const u32x4_t v = *reinterpret_cast<const u32x4_t*>(ost + r * 128 + ((cidx ^ (r & 7)) * 16));
      const int lr = 32 * wave + r;
      if (GROUPED && a.gated) {
        // gated layout: lane cidx takes half cidx & 1 (4 values) of output
        // chunk cidx >> 1, from the same half of its gate and up chunks
        const int oc = cidx >> 1, hf = cidx & 1, gc = gated_gate_chunk(oc);
        const u32x2_t gv = *reinterpret_cast<const u32x2_t*>(ost + r * 128 + ((gc ^ (r & 7)) * 16) + 8 * hf);
        const u32x2_t uv = *reinterpret_cast<const u32x2_t*>(ost + r * 128 + (((gc + 2) ^ (r & 7)) * 16) + 8 * hf);
        if (lr < t.rows) {
          const int64_t row = orow_s[lr];
          if (row >= 0)
            *reinterpret_cast<u32x2_t*>(a.y + row * (G.N / 2) + t.nb0 * 8 + 8 * oc + 4 * hf) =
                (u32x2_t){silu_mul_pair(gv[0], uv[0]), silu_mul_pair(gv[1], uv[1])};
        }
      } else if (lr < t.rows) {
        const int64_t row = GROUPED ? (int64_t)orow_s[lr] : t.m0 + lr;
        if (row >= 0) store_bf16x8(a.y + row * G.N, G.N, t.nb0 * 16 + 8 * cidx, v);
      }
    }
    item += gridDim.x;
    // the next tile's copies overwrite the reduction regions and the row table
    __asm__ volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  }
}

template <bool GROUPED>
__global__ void __launch_bounds__(256, 1)
k_gemm_mid_mx(GemmArgs a, int tiles_n, int tiles_m) {
  extern __shared__ __attribute__((aligned(1024))) uint8_t lds[];
  __shared__ int32_t orow_s[GROUPED ? kMxM : 1];   // output row of each local row, or -1
  __shared__ int32_t arow_s[GROUPED ? kMxM : 1];   // activation row of each local row

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n_l = lane & 15, q_l = lane >> 4;
  const int wm = wave & 1, wn = wave >> 1;         // rows 32 wm .. + 31, column blocks 4 wn .. 4 wn + 3
  const Geom G = a.G;
  const int64_t row_bytes = G.K;                   // fp8 activations
  const int KG = (int)G.KG;
  // grouped items: (128-row unit, 64-row half, 128-column tile)
  const int64_t n_items = GROUPED ? (int64_t)a.hdr[1] * 2 * tiles_n : (int64_t)tiles_n * tiles_m;

  auto act_row = [&](int32_t pair) -> int64_t {
    if (pair < 0 || pair >= a.P) return 0;
    return a.rows_are_pairs ? pair : pair / a.topk;
  };
  const rsrc_t rsz = make_rsrc(a.w + G.off_scales, G.total - G.off_scales);
  // operand rows 16 rb + n_l: 16-byte K chunks q_l and 4 + q_l, at slot
  // c ^ ((r >> 1) & 7) of the row (the copies place them so)
  const int xsw = (n_l >> 1) & 7;
  const uint32_t xo0 = n_l * 128 + 16 * (q_l ^ xsw), xo1 = n_l * 128 + 16 * ((4 + q_l) ^ xsw);

  int64_t item = blockIdx.x;
  for (; item < n_items; item += gridDim.x) {
    MidTile t;
    if (GROUPED) {
      const int64_t unit = item / (2 * tiles_n);
      const int half = (int)((item / tiles_n) & 1);
      const int32_t* u = a.units + 4 * unit;
      t.e = u[0];
      t.first = (int64_t)u[1] + kMxM * half;
      t.rows = std::min<int64_t>((int64_t)u[2] - kMxM * half, kMxM);
      t.m0 = 0;
      t.nb0 = (item % tiles_n) * kMxCB;
      if (t.rows <= 0) continue;                   // block-uniform: a unit of <= 64 rows
    } else {
      const int total = tiles_n * tiles_m;
      const int xcd = (int)(item % 8), idx = (int)(item / 8);
      const int base = total / 8, extra = total % 8;
      const int tt = (total >= 8) ? xcd * base + (xcd < extra ? xcd : extra) + idx : (int)item;
      t.e = 0;
      t.first = 0;
      t.m0 = (int64_t)(tt % tiles_m) * kMxM;
      t.nb0 = (int64_t)(tt / tiles_m) * kMxCB;
      t.rows = (a.M - t.m0) < kMxM ? (a.M - t.m0) : kMxM;
    }
    // ---- copy descriptors: activation copy j = 2 w + q covers rows 8 j ..
    // 8 j + 7 (lane L: row 8 j + L / 8, slot L % 8); weight copies k = 0, 1
    // the code tile and scale words of column block 2 w + k
    const rsrc_t rx = make_rsrc(reinterpret_cast<const uint8_t*>(a.x) + t.m0 * row_bytes,
                                GROUPED ? 0xFFFFFFFFull : (uint64_t)t.rows * row_bytes);
    uint32_t xoff[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int r = 8 * (2 * wave + q) + (lane >> 3);
      const int rc = r < t.rows ? r : (int)t.rows - 1;
      const int64_t src = GROUPED ? act_row(a.sorted_pairs[t.first + rc]) : rc;
      xoff[q] = (uint32_t)(src * row_bytes) + 16u * (uint32_t)((lane & 7) ^ ((r >> 1) & 7));
    }
    const int64_t wb = t.e * G.NB;
    const rsrc_t rw = make_rsrc(a.w + (wb + t.nb0) * G.KG * 1024, (uint64_t)kMxCB * G.KG * 1024);
    uint32_t wvo[2], svo[2];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      int64_t nb = t.nb0 + 2 * wave + k;
      if (nb >= G.NB) nb = G.NB - 1;
      wvo[k] = (uint32_t)((nb - t.nb0) * G.KG * 1024 + lane * 16);
      svo[k] = (uint32_t)((wb + nb) * G.KG4 * 256 + lane * 4);
    }
    if (GROUPED && tid < kMxM) {
      const int32_t p = tid < t.rows ? a.sorted_pairs[t.first + tid] : -1;
      orow_s[tid] = (p >= 0 && p < a.P) ? p : -1;
      arow_s[tid] = (int32_t)act_row(p);
    }
    uint32_t so[kMxStages];
#pragma unroll
    for (int i = 0; i < kMxStages; ++i) so[i] = (uint32_t)(i * kMxSB);
    // the six copies of group g into the stage at offset st (q = 0, 1
    // activations, 2, 3 code tiles, 4, 5 scale words)
    auto dma = [&](int q, int g, uint32_t st) {
      uint8_t* d = lds + st;
      if (q < 2) b2lds16(rx, xoff[q], (uint32_t)(g * 128), d + (2 * wave + q) * 1024);
      else if (q < 4) b2lds16(rw, wvo[q - 2], (uint32_t)(g * 1024), d + 8 * 1024 + (2 * wave + q - 2) * 1024);
      else b2lds4(rsz, svo[q - 4], (uint32_t)((g / 4) * 256), d + 16 * 1024 + (2 * wave + q - 4) * 256);
    };
    // ---- prologue: groups 0 .. kMxStages - 2 (past the end: repeats of the
    // last), then wait for groups 0 and 1
#pragma unroll
    for (int i = 0; i < kMxStages - 1; ++i)
#pragma unroll
      for (int q = 0; q < kMxCopies; ++q) dma(q, std::min(i, KG - 1), so[i]);
    __asm__ volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"((kMxStages - 3) * kMxCopies) : "memory");

    auto load = [&](MxFrag& f, uint32_t st) {
      const uint8_t* wbase = lds + st + 8 * 1024 + 4 * wn * 1024 + lane * 16;
      const uint8_t* sbase = lds + st + 16 * 1024 + 4 * wn * 256 + lane * 4;
      const uint8_t* xbase = lds + st + wm * 2 * 2048;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        f.wq[c] = ld16(wbase + c * 1024);
        f.ws[c] = *reinterpret_cast<const uint32_t*>(sbase + c * 256);
      }
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        f.b0[rb] = ld16(xbase + rb * 2048 + xo0);
        f.b1[rb] = ld16(xbase + rb * 2048 + xo1);
      }
    };
    f32x4_t acc[4][2];
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) acc[c][rb] = (f32x4_t){0.f, 0.f, 0.f, 0.f};

    // Group g: eight MFMAs from fragments read during group g - 1, while the
    // fragments of group g + 1 (landed two groups ago) are read and the
    // copies of group g + kMxStages - 1 go out, one after each MFMA from the
    // second.
    auto group = [&](int g, const MxFrag& cur, MxFrag& nxt) {
      load(nxt, so[1]);
      const int dg = std::min(g + kMxStages - 1, KG - 1);
      const uint32_t dst = so[kMxStages - 1];
      const int sh = 8 * (g & 3);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int c = i & 3, rb = i >> 2;
        acc[c][rb] = mfma_fp4_fp8(cur.wq[c], cur.b0[rb], cur.b1[rb], acc[c][rb], (int)((cur.ws[c] >> sh) & 0xFFu), 127);
        if (i >= 1 && i <= kMxCopies) dma(i - 1, dg, dst);
        __builtin_amdgcn_sched_barrier(0);
      }
      const uint32_t s0 = so[0];
#pragma unroll
      for (int i = 0; i + 1 < kMxStages; ++i) so[i] = so[i + 1];
      so[kMxStages - 1] = s0;
      // all but the copies of groups g + 3 .. g + kMxStages - 1: group g + 2 has landed
      __asm__ volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"((kMxStages - 3) * kMxCopies) : "memory");
    };
    MxFrag f0, f1;
    load(f0, so[0]);
    int g = 0;
#pragma nounroll
    for (; g + 1 < KG; g += 2) {
      group(g, f0, f1);
      group(g + 1, f1, f0);
    }
    if (g < KG) group(g, f0, f1);

    // ---- epilogue: lane holds C[n = 16 (4 wn + c) + 4 q_l + r][row = 32 wm +
    // 16 rb + n_l]; rows scaled by their token scale, staged as bf16 (8-byte
    // unit u of row r at u ^ 2 (r % 16), 256 bytes per row), then stored as
    // 16-byte chunks, 16 lanes per row
    float rs[2];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      const int lr = 32 * wm + 16 * rb + n_l;
      const int lc = lr < t.rows ? lr : 0;
      rs[rb] = a.xs[GROUPED ? (int64_t)arow_s[lc] : t.m0 + lc];
    }
    __asm__ volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      const int r = 32 * wm + 16 * rb + n_l;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const f32x4_t v = acc[c][rb] * rs[rb];
        const int u = 4 * (4 * wn + c) + q_l;
        *reinterpret_cast<u32x2_t*>(lds + r * 256 + (u ^ (2 * (r & 15))) * 8) =
            (u32x2_t){pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3])};
      }
    }
    __asm__ volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int r = 16 * k + (tid >> 4), c16 = tid & 15;
      const u32x4_t v = *reinterpret_cast<const u32x4_t*>(lds + r * 256 + ((2 * c16) ^ (2 * (r & 15))) * 8);
      if (GROUPED && a.gated) {
        // gated layout: lane c16 takes half c16 & 1 (4 values) of output
        // chunk c16 >> 1, from the same half of its gate and up chunks
        const int oc = c16 >> 1, hf = c16 & 1, gc = gated_gate_chunk(oc);
        const u32x2_t gv = *reinterpret_cast<const u32x2_t*>(lds + r * 256 + ((2 * gc + hf) ^ (2 * (r & 15))) * 8);
        const u32x2_t uv =
            *reinterpret_cast<const u32x2_t*>(lds + r * 256 + ((2 * gc + 4 + hf) ^ (2 * (r & 15))) * 8);
        if (r < t.rows) {
          const int64_t row = orow_s[r];
          if (row >= 0)
            *reinterpret_cast<u32x2_t*>(a.y + row * (G.N / 2) + t.nb0 * 8 + 8 * oc + 4 * hf) =
                (u32x2_t){silu_mul_pair(gv[0], uv[0]), silu_mul_pair(gv[1], uv[1])};
        }
      } else if (r < t.rows) {
        const int64_t row = GROUPED ? (int64_t)orow_s[r] : t.m0 + r;
        if (row >= 0) store_bf16x8(a.y + row * G.N, G.N, t.nb0 * 16 + 8 * c16, v);
      }
    }
    // the next tile's copies overwrite the staging and the row tables
    __asm__ volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  }
}

template <bool GROUPED>
static hipError_t go_mid_mx(const GemmArgs& a, int grid_items, hipStream_t st) {
  auto kern = &k_gemm_mid_mx<GROUPED>;
  static const hipError_t attr_err = hipFuncSetAttribute(
      reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize, kMxLds);
  if (attr_err != hipSuccess) return attr_err;
  const int tiles_n = (int)((a.G.NB + kMxCB - 1) / kMxCB);
  const int tiles_m = GROUPED ? 0 : (int)((a.M + kMxM - 1) / kMxM);
  const int64_t tiles = (int64_t)tiles_n * tiles_m;
  if (!GROUPED && tiles > 0x7FFFFFFF) return hipErrorInvalidValue;
  const unsigned grid = GROUPED ? (unsigned)(grid_items > 0 ? grid_items : 1) : (unsigned)tiles;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(256), kMxLds, st, a, tiles_n, tiles_m);
  return hipGetLastError();
}

template <bool ZP, bool GROUPED, bool F4 = false, bool I4 = false>
static hipError_t go_mid(const GemmArgs& a, int grid_items, hipStream_t st) {
  auto kern = &k_gemm_mid<ZP, GROUPED, F4, I4>;
  static const hipError_t attr_err = hipFuncSetAttribute(
      reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize, kMidLds);
  if (attr_err != hipSuccess) return attr_err;
  const int tiles_n = (int)((a.G.NB + kMidCB - 1) / kMidCB);
  const int tiles_m = GROUPED ? 0 : (int)((a.M + kMidM - 1) / kMidM);
  const int64_t tiles = (int64_t)tiles_n * tiles_m;
  if (!GROUPED && tiles > 0x7FFFFFFF) return hipErrorInvalidValue;
  const unsigned grid = GROUPED ? (unsigned)(grid_items > 0 ? grid_items : 1) : (unsigned)tiles;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(256), kMidLds, st, a, tiles_n, tiles_m);
  return hipGetLastError();
}


hipError_t launch_gemm_mid(const GemmArgs& a, bool grouped, int grid_items, hipStream_t st) {
  // W4A4 and INT8 weights have no 128-row tile kernel
  if (kmode_of(a) == KM_MX_A4 || kmode_of(a) == KM_INT8_A16) return hipErrorInvalidValue;
  // scale and zero-point copies use 32-bit offsets from the scale region
  if (a.G.total - a.G.off_scales > 0xFFFFFFFFull) return hipErrorInvalidValue;
  // grouped activation rows are addressed by 32-bit offsets from x
  if (grouped) {
    const int64_t xrows = a.rows_are_pairs ? a.P : (a.P + a.topk - 1) / a.topk;
    if (xrows * (a.a8 ? 1 : 2) * a.G.K > 0xFFFFFFFFll) return hipErrorInvalidValue;
  }
  if (kmode_of(a) == KM_MX_A16)
    return grouped ? go_mid<false, true, true>(a, grid_items, st) : go_mid<false, false, true>(a, 0, st);
  if (kmode_of(a) == KM_MXI4_A16)
    return grouped ? go_mid<false, true, true, true>(a, grid_items, st) : go_mid<false, false, true, true>(a, 0, st);
  if (a.wfmt == W_MXFP4) return grouped ? go_mid_mx<true>(a, grid_items, st) : go_mid_mx<false>(a, 0, st);
  if (a.wfmt == W_UINT4_ZP)
    return grouped ? go_mid<true, true>(a, grid_items, st) : go_mid<true, false>(a, 0, st);
  return grouped ? go_mid<false, true>(a, grid_items, st) : go_mid<false, false>(a, 0, st);
}

}  // namespace hm
