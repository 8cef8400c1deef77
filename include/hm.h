/*
 * hm.h -- C ABI of the MI355X (gfx950) low-bit GEMM library.
 *
 * The library computes a linear layer Y[M,N] = X[M,K] . W_hat[N,K]^T whose
 * weights are stored in 4-bit form and dequantized inside the kernel, and the
 * grouped (MoE) variant in which every routed (token, expert) pair runs against
 * its expert's weights.  Sources, cited by page and section:
 *   - linear layer as X times W transposed, weights read once and reused over
 *     the M rows, about 2*M*N*K flops: ywsung.com note "How vLLM Humming
 *     computes 4 bits", section on one token vs many tokens;
 *   - 4-bit codes with a scale, q = round(w/s), restored as s*q, signed range
 *     -8..7, one 16-bit scale per 128 weights: same note, section on scales;
 *   - one common representation of weights, scales and zero points, then
 *     padding and re-ordering for the device, done once before inference
 *     (transform, then call the layer): same note, section on layout, and the
 *     aihaber.org article, Architecture;
 *   - the formats (INT4, MXFP4) and activation widths (16-bit, 8-bit):
 *     cocoloop.cn news item, format list; aihaber.org, hardware and format
 *     support; per-token FP8 activations: ywsung.com note, section on weight
 *     format / activation / backend;
 *   - tokens split per expert so that every expert's GEMM has its own M, and a
 *     grouped path over all experts: ywsung.com note, section on one token vs
 *     many tokens; aihaber.org, Performance.
 *
 * Conventions (every entry point):
 *   - Tensor pointers are DEVICE pointers unless stated; descriptors are host
 *     pointers.  The caller owns every buffer (weights, inputs, outputs,
 *     workspaces); the library allocates no device memory and keeps no state
 *     between calls.
 *   - Calls are asynchronous on `stream` (NULL = the default stream), never
 *     synchronize, and are safe to call from several host threads.
 *   - All argument checks happen before any launch.  On any error the call
 *     returns a non-zero hm_status and no kernel has been launched; outputs are
 *     untouched.  HM_ERR_HIP reports a failed launch.
 *   - Matrices are row-major and contiguous.  bf16 values are passed as their
 *     16-bit patterns (uint16_t).  Outputs are bf16, rounded to nearest even
 *     from an fp32 accumulator.
 *   - K must be a multiple of 128 for every format.  N is arbitrary.
 *   - Alignment: w_dev and workspaces 256 bytes, every other pointer 16 bytes
 *     (HM_ERR_ALIGN otherwise).
 *   - Inputs are finite; NaN or Inf in X, scales or weights gives unspecified
 *     (but memory-safe) results.
 */
#ifndef HM_H
#define HM_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define HM_ABI_VERSION 2

typedef enum hm_status {
  HM_OK = 0,
  HM_ERR_NULL = 1,        /* a required pointer is NULL */
  HM_ERR_SHAPE = 2,       /* bad size, group or count */
  HM_ERR_ALIGN = 3,       /* pointer not aligned as required */
  HM_ERR_UNSUPPORTED = 4, /* unknown weight format or format/activation pair */
  HM_ERR_WORKSPACE = 5,   /* buffer smaller than its size query */
  HM_ERR_HIP = 6,         /* a HIP launch failed */
  HM_ERR_ABI = 7,         /* descriptor abi field != HM_ABI_VERSION */
  HM_ERR_TUNING = 8       /* a tuning field out of range, or a forced kernel that cannot run this call */
} hm_status;

/* Weight number format (the "number format / scale unit / zero point" of the
 * quantization description, ywsung.com note, section on layout, figure on the
 * quantization description). */
typedef enum hm_wfmt {
  HM_W_INT4_SYM = 0, /* signed 4-bit two's complement q, bf16 scale per 128 along K: w = s*q */
  HM_W_UINT4_ZP = 1, /* unsigned 4-bit u, bf16 scale + 4-bit zero point per 128: w = s*(u-z) */
  HM_W_MXFP4 = 2,    /* E2M1 codes, E8M0 scale per 32 along K: w = e2m1(c) * 2^(b-127) */
  HM_W_MXINT4 = 3,   /* two's complement 4-bit q read as 1.2 fixed point, E8M0 scale per 32
                        along K: w = (q/4) * 2^(b-127); the format is named in the pages' lists
                        (cocoloop.cn item; aihaber.org article, hardware and format support)
                        without a definition, this is the MX-family reading */
  HM_W_UINT3_ZP = 4, /* unsigned 3-bit u, bf16 scale + 3-bit zero point per 128: w = s*(u-z) */
  HM_W_UINT2_ZP = 5, /* unsigned 2-bit u, bf16 scale + 2-bit zero point per 128: w = s*(u-z);
                        the pages list INT1..INT8 weights and name GPTQ INT3 as a compatibility
                        case (cocoloop.cn news item, format list and deployer section).  Both are
                        widened to the 4-bit zero-point device layout by hm_transform (exact; no
                        bandwidth saving over 4 bits) and run on every W4A16 kernel */
  HM_W_INT8_SYM = 6  /* signed 8-bit two's complement q, bf16 scale per 128 along K: w = s*q (own
                        device layout of 2 KiB tiles; the streaming (path 1) and 128 x 128
                        (path 4) kernels, and grouped streaming and 128-row units) */
} hm_wfmt;

/* Activation format (the compute option choosing A16, A8 or A4). */
typedef enum hm_afmt {
  HM_A_BF16 = 0,         /* X is bf16 [M,K]; x_scales unused (may be NULL) */
  HM_A_FP8_ROWSCALE = 1, /* X is OCP E4M3 bytes [M,K] with one fp32 scale per row: x = e4m3(c)*s[m] */
  HM_A_MXFP4 = 2         /* X is E2M1 codes [M][K/2] (value 2j in the low nibble of byte j) with E8M0
                            scale bytes [M][K/32] in x_scales: x = e2m1(c) * 2^(b-127) (W4A4) */
} hm_afmt;

/* Supported pairs: every weight format with HM_A_BF16 (W4A16: INT4_SYM,
 *                  UINT4_ZP, and MXFP4 / MXINT4, whose codes are scaled to
 *                  bf16 in the kernel; the pages list MXFP4 W4A16 among the
 *                  MoE results, aihaber.org article, performance section);
 *                  MXFP4 with HM_A_FP8_ROWSCALE (W4A8-MXFP4); MXFP4 with
 *                  HM_A_MXFP4 (W4A4: both operands E2M1 with E8M0 scales on
 *                  the scaled fp4 MFMA; the pages list W4A4 among the GEMM
 *                  types, cocoloop.cn news item, format list).  W4A4 runs on
 *                  the streaming kernel (path 1) and the 128 x 128 kernel
 *                  (path 4) only.
 * MXFP4 with bf16 rows requires every |w| < 2^128 (E8M0 scale bytes up to
 * 252 always satisfy it, up to 253 for MXINT4; larger products become inf,
 * and the row's sums NaN):
 * the dequantized weights enter the bf16 MFMA.  Subnormal products (scale
 * bytes 0..3) are kept exactly. */

/* Layer description (shapes, number format, group).  num_experts is 1 for a
 * dense layer.  group must be 128 for the INT4 formats and 32 for MXFP4. */
typedef struct hm_wdesc {
  int32_t abi;         /* HM_ABI_VERSION */
  int32_t wfmt;        /* hm_wfmt */
  int32_t group;       /* elements per scale along K */
  int32_t num_experts; /* >= 1 */
  int64_t n;           /* output features (rows of W), >= 1 */
  int64_t k;           /* input features, multiple of 128, >= 128 */
} hm_wdesc;

/* Explicit choices of one GEMM call (the pages' "Tuning Config": tile
 * shapes, launch shape and split of the work, chosen apart from the layer and
 * compute description; aihaber.org article, Architecture; ywsung.com note,
 * section on layout).  Pass NULL, or a zero-initialised struct with abi set,
 * for the library's default heuristic choice; any nonzero field overrides the
 * default for that one call (the library keeps no state).  Out-of-range
 * values, or a forced kernel that cannot run the call, give HM_ERR_TUNING
 * before any launch.  hm_gemm_plan / hm_moe_gemm_plan report what a given
 * tuning selects.  Every field has a documented default (0). */
typedef struct hm_tuning {
  int32_t abi;             /* HM_ABI_VERSION */
  int32_t path;            /* dense kernel: 0 default; 1 streaming (M <= 256); 2 128-row tiles
                              (W4A16 128 x 64 split over K, W4A8 64 x 128); 3 256 x 256 tiles;
                              4 128 x 128 tiles */
  int32_t stream_ks;       /* streaming: waves of a block splitting one column set's K: 0, 1, 2, 4, 8 */
  int32_t stream_nbw;      /* streaming: 16-column blocks per wave: 0, 1, 2 */
  int32_t stream_splits;   /* dense streaming: K split over blocks (fp32 partials): 0, 1 .. K/128 */
  int32_t stream_waves;    /* dense streaming: waves per block: 0, 4, 8 (8 needs stream_ks 2, 4 or 8) */
  int32_t moe_stream_rows; /* rows per grouped streaming unit: 0, 16, 32 */
  int32_t moe_stream_max;  /* largest expert (rows) taking streaming units: 0, 1 .. 4096 */
  int32_t moe_stream_nbw;  /* grouped streaming: 16-column blocks per wave: 0, 1, 2 */
  int32_t moe_stream_ks;   /* grouped streaming: waves splitting K: 0, 1, 2, 4 */
  int32_t moe_stream_lds_kb; /* grouped streaming: LDS per block in KiB: 0, 20 .. 159 */
  int32_t moe_big_min;     /* smallest expert remainder that takes a 256-row unit: 0, 1 .. 256;
                              -1: no 256-row units */
  int32_t moe_tile;        /* kernel of the up-to-128-row units: 0 default; 1 the 128-row tile
                              kernel of path 2; 2 the 128 x 128 kernel */
} hm_tuning;

/* ---------------------------------------------------------------- weights */

/* Bytes of the device weight buffer for `d` (all experts). */
hm_status hm_transform_size(const hm_wdesc* d, size_t* bytes);

/* Repack the standard format into the device layout (padding N to 16 and
 * re-ordering codes, scales and zero points so that each 64-lane wave reads
 * one 1 KiB tile of 16 columns x 128 K per 16-byte-per-lane load).  Run once
 * per weight, before inference.
 *   codes  [E][N][K/2] bytes, element k=2j in the low nibble of byte j,
 *          k=2j+1 in the high nibble (two's complement for INT4_SYM and
 *          MXINT4, unsigned for UINT4_ZP, E2M1 bits for MXFP4);
 *          UINT2_ZP: [E][N][K/4], element 4j+i at bits 2i..2i+1 of byte j;
 *          UINT3_ZP: [E][N][3K/8], element 8j+i at bits 3i..3i+2 of the
 *          little-endian 24-bit word of bytes 3j..3j+2;
 *          INT8_SYM: [E][N][K], one two's complement byte per element.
 *   scales INT4 formats: bf16 [E][N][K/128]; MXFP4, MXINT4: E8M0 bytes [E][N][K/32].
 *   zeros  zero-point formats only: bytes [E][N][K/128], the code's low 4 / 3 / 2
 *          bits used; else NULL.
 *   w_dev  output, w_bytes >= hm_transform_size.  Opaque; valid only for the
 *          same descriptor. */
hm_status hm_transform(const hm_wdesc* d, const uint8_t* codes, const void* scales,
                       const uint8_t* zeros, void* w_dev, size_t w_bytes, hipStream_t stream);

/* hm_transform of a gate_up weight (n = 2d rows: gate rows 0..d-1, up rows
 * d..2d-1, n a multiple of 32, else HM_ERR_SHAPE) into the gated device
 * layout that hm_moe_gemm_gated reads: device row 32 i + c holds gate row
 * 16 i + c and device row 32 i + 16 + c up row 16 i + c (c < 16), i.e. the
 * buffer equals hm_transform of the standard format with its rows so
 * permuted (hm_dequant of it returns the rows in that order).  Same size
 * (hm_transform_size) and arguments as hm_transform. */
hm_status hm_transform_gated(const hm_wdesc* d, const uint8_t* codes, const void* scales,
                             const uint8_t* zeros, void* w_dev, size_t w_bytes, hipStream_t stream);

/* Exact dequantization of one expert of a transformed buffer into fp32
 * out[N][K].  Every restored weight is exactly representable in fp32 for the
 * INT4 formats, and for MXFP4 with E8M0 scale bytes up to 252 (MXINT4: up to
 * 253); larger bytes give +-inf where the product leaves the fp32 range, and
 * byte 255 (the E8M0 NaN) gives NaN. */
hm_status hm_dequant(const hm_wdesc* d, const void* w_dev, size_t w_bytes, int32_t expert,
                     float* out, hipStream_t stream);

/* -------------------------------------------------------------- activations */

/* Per-token FP8: for each row m, s[m] = amax_k |x[m,k]| / 448 (fp32 division),
 * x8[m,k] = E4M3(x[m,k] / s[m]) with the division in fp32, round to nearest
 * even, saturating at +-448; a row of zeros gives s = 0 and zero codes.
 *   x bf16 [m][k]; x8 bytes [m][k]; row_scale fp32 [m].  k >= 1 (any k). */
hm_status hm_quant_fp8_rows(const uint16_t* x, int64_t m, int64_t k, uint8_t* x8,
                            float* row_scale, hipStream_t stream);

/* MXFP4 activation rows (the W4A4 pair: 4-bit weights with 4-bit
 * activations, cocoloop.cn news item, format list): per 32 consecutive values
 * of each row, the OCP MX rule -- shared exponent X = floor(log2 amax) - 2
 * clamped to [-127, 127], stored as the E8M0 byte X + 127 (0 for a zero
 * block), elements E2M1(x / 2^X) rounded to nearest even and saturated at
 * +-6 (negative values that round to zero keep the sign: code 8).
 *   x bf16 [m][k]; codes [m][k/2] bytes, value 2j in the low nibble of byte
 *   j; scales [m][k/32] E8M0 bytes.  k a multiple of 32; x and codes 16-byte
 *   aligned.  m = 0 is a no-op. */
hm_status hm_quant_mxfp4_rows(const uint16_t* x, int64_t m, int64_t k, uint8_t* codes, uint8_t* scales,
                              hipStream_t stream);

/* ---------------------------------------------------------------- dense GEMM */

/* Workspace bytes hm_gemm needs for this shape and tuning (may be 0). */
hm_status hm_gemm_workspace_size(const hm_wdesc* d, int32_t afmt, int64_t m, const hm_tuning* tune,
                                 size_t* bytes);

/* y[m][n] = bf16( sum_k x_hat[m,k] * w_hat[n,k] ), fp32 accumulation.
 *   w_dev      transformed weights (num_experts must be 1).
 *   x          bf16 [m][k] (HM_A_BF16), E4M3 bytes [m][k] (HM_A_FP8_ROWSCALE) or
 *              E2M1 codes [m][k/2] (HM_A_MXFP4).
 *   x_scales   fp32 [m] row scales for HM_A_FP8_ROWSCALE, E8M0 bytes [m][k/32]
 *              for HM_A_MXFP4 (4-byte aligned), else ignored.
 *   y          bf16 [m][n].
 *   ws         workspace of at least hm_gemm_workspace_size bytes (NULL if 0).
 *   tune       NULL for the default choice, else explicit choices (hm_tuning).
 * m = 0 is a no-op; m above 8388480 (65535 x 128) gives HM_ERR_SHAPE, here
 * and in the size and plan queries. */
hm_status hm_gemm(const hm_wdesc* d, const void* w_dev, int32_t afmt, const void* x,
                  const void* x_scales, int64_t m, uint16_t* y, void* ws, size_t ws_bytes,
                  const hm_tuning* tune, hipStream_t stream);

/* A short text naming the kernel path and tile configuration hm_gemm selects
 * for this shape and tuning (so a caller can confirm what actually runs). */
hm_status hm_gemm_plan(const hm_wdesc* d, int32_t afmt, int64_t m, const hm_tuning* tune, char* buf,
                       size_t buf_len);

/* ------------------------------------------------------------------- MoE */

/* Workspace bytes hm_moe_sort needs: 0 up to 4096 pairs (one workgroup),
 * else chunks x E x 4 for the per-chunk expert counts of the GPU-wide sort
 * (chunks of about 2048 pairs, at most 512 chunks: at most 1 MiB). */
hm_status hm_moe_sort_workspace_size(int64_t t, int32_t topk, int32_t num_experts, size_t* bytes);

/* Expert sort: pairs p = t*topk + j with ids topk_ids[t][j] (the expert
 * grouping of the MoE path: ywsung.com note, section on one token vs many
 * tokens; each expert's M follows its routing load).  Up to 4096 pairs one
 * workgroup counts and places them; more are cut into consecutive chunks,
 * one workgroup each: a counting pass writes every chunk's per-expert counts
 * to ws, and a placing pass gives each chunk its base positions from the
 * totals and the counts of the chunks before it.
 *   counts[e]        number of pairs routed to expert e        (int32 [E])
 *   offsets[e]       exclusive prefix sum, offsets[E] = pairs  (int32 [E+1])
 *   sorted_pairs[i]  pair ids grouped by expert, ascending within each
 *                    expert (stable)                           (int32 [t*topk])
 * Ids outside [0, E) are dropped (not counted, not placed); offsets[E] then
 * falls short of t*topk.  1 <= num_experts <= 512, topk <= num_experts,
 * t*topk < 2^31.  t = 0 is a no-op.  ws: hm_moe_sort_workspace_size bytes
 * (may be NULL when that is 0; HM_ERR_WORKSPACE when smaller), overwritten
 * by the call. */
hm_status hm_moe_sort(const int32_t* topk_ids, int64_t t, int32_t topk, int32_t num_experts,
                      int32_t* counts, int32_t* offsets, int32_t* sorted_pairs, void* ws,
                      size_t ws_bytes, hipStream_t stream);

/* Workspace bytes hm_moe_gemm needs for t tokens, topk and the tuning. */
hm_status hm_moe_gemm_workspace_size(const hm_wdesc* d, int32_t afmt, int64_t t, int32_t topk,
                                     const hm_tuning* tune, size_t* bytes);

/* Grouped GEMM over all experts in one call:
 *   y[p][:] = bf16( A_row(p) . W_hat_{e(p)}^T ) for every routed pair p,
 * where e(p) is the expert whose segment of sorted_pairs holds p.
 *   a            a_rows_are_pairs = 0: activations [t][k] and pair p uses row
 *                p / topk (gate/up projection);  = 1: [t*topk][k] and pair p
 *                uses row p (down projection).  bf16, or E4M3 bytes with
 *                a_scales (one fp32 per row of a) for HM_A_FP8_ROWSCALE, or
 *                E2M1 codes [rows][k/2] with E8M0 a_scales [rows][k/32] for
 *                HM_A_MXFP4.
 *   offsets, sorted_pairs  as produced by hm_moe_sort (device).
 *   y            bf16 [t*topk][n], rows in pair order; rows of dropped pairs
 *                are not written.
 *   ws           at least hm_moe_gemm_workspace_size bytes (the work lists
 *                of the schedule, written by the call).
 *   tune         NULL for the default choice, else explicit choices.
 * Activations of 4 GiB or more run their up-to-128-row units on the 128 x 128
 * kernel (64-bit row addressing) and take no 256-row units.
 * t = 0 is a no-op. */
hm_status hm_moe_gemm(const hm_wdesc* d, const void* w_dev, int32_t afmt, const void* a,
                      const void* a_scales, int32_t a_rows_are_pairs, int64_t t,
                      int32_t topk, const int32_t* offsets, const int32_t* sorted_pairs,
                      uint16_t* y, void* ws, size_t ws_bytes, const hm_tuning* tune,
                      hipStream_t stream);

/* A short text naming the unit kinds and kernels hm_moe_gemm schedules for
 * this call shape and tuning (no device access). */
hm_status hm_moe_gemm_plan(const hm_wdesc* d, int32_t afmt, int64_t t, int32_t topk,
                           int32_t a_rows_are_pairs, const hm_tuning* tune, char* buf, size_t buf_len);

/* The gate_up grouped GEMM with the gated activation in its epilogue (the
 * MoE feed-forward block of the pages: aihaber.org article on Humming, "what
 * problem does it solve"; ywsung.com note, section on one token vs many
 * tokens; the fusion is this library's, the formula that of hm_silu_mul):
 *   h[p][i] = bf16( silu(y[p][i]) * y[p][d + i] ),  y = hm_moe_gemm's bf16
 *   output for the same call, d = n / 2,
 * bit for bit what hm_moe_gemm followed by hm_silu_mul gives, without
 * writing or reading y.
 *   w_dev  from hm_transform_gated (same descriptor, n = 2d, n a multiple of
 *          32; HM_ERR_SHAPE otherwise): gate rows 0..d-1 and up rows
 *          d..2d-1 of the standard format, interleaved by 16-row blocks in
 *          the device layout so that a wave holds both halves of an output.
 *   h      bf16 [t*topk][n/2], rows in pair order; rows of dropped pairs are
 *          not written.
 *   ws     at least hm_moe_gemm_workspace_size bytes (the same schedule).
 * Other arguments and errors as hm_moe_gemm; the grouped streaming units
 * take two column blocks per wave (tune->moe_stream_nbw = 1 gives
 * HM_ERR_TUNING). */
hm_status hm_moe_gemm_gated(const hm_wdesc* d, const void* w_dev, int32_t afmt, const void* a,
                            const void* a_scales, int32_t a_rows_are_pairs, int64_t t,
                            int32_t topk, const int32_t* offsets, const int32_t* sorted_pairs,
                            uint16_t* h, void* ws, size_t ws_bytes, const hm_tuning* tune,
                            hipStream_t stream);

/* The plan text of hm_moe_gemm_gated (as hm_moe_gemm_plan). */
hm_status hm_moe_gemm_gated_plan(const hm_wdesc* d, int32_t afmt, int64_t t, int32_t topk,
                                 int32_t a_rows_are_pairs, const hm_tuning* tune, char* buf, size_t buf_len);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the same
 * grouped GEMM as hm_moe_gemm, with the schedule's work lists kept in a
 * static device array of hm_moe_gemm_static_max_workspace() bytes (4 MiB)
 * inside the library instead of a caller workspace.  Each GPU holds its own
 * array until the process ends; its address is resolved once per device on
 * the first call with that device current.  The call allocates nothing.
 * Calls whose work lists exceed the array (hm_moe_gemm_workspace_size >
 * the maximum, about three million routed pairs with the default tuning)
 * return HM_ERR_WORKSPACE before any launch.  All calls on one GPU share the
 * array: calls that overlap in time on one GPU (different streams, or host
 * threads) race and must be serialized by the caller.  Every other argument,
 * check and result is as for hm_moe_gemm. */
size_t hm_moe_gemm_static_max_workspace(void);
hm_status hm_moe_gemm_static(const hm_wdesc* d, const void* w_dev, int32_t afmt, const void* a,
                             const void* a_scales, int32_t a_rows_are_pairs, int64_t t, int32_t topk,
                             const int32_t* offsets, const int32_t* sorted_pairs, uint16_t* y,
                             const hm_tuning* tune, hipStream_t stream);

/* ------------------------------------------------------- MoE block steps */

/* Gated activation between the gate_up and down grouped GEMMs of an MoE
 * feed-forward block (tokens split per expert, each token activating only
 * some experts: aihaber.org article on Humming, "what problem does it solve";
 * ywsung.com note "How vLLM Humming computes 4 bits", section on one token vs
 * many tokens; the pages give no formula, the reading is the plainest one):
 *   h[r][i] = bf16( silu(gu[r][i]) * gu[r][d + i] ),  silu(x) = x / (1 + exp(-x)),
 * computed in fp32 from the bf16 inputs, rounded to nearest even.
 *   gu   bf16 [rows][2d], row-major: gate in columns 0..d-1, up in d..2d-1
 *        (hm_moe_gemm's gate_up output with n = 2d, pair order kept);
 *   h    bf16 [rows][d] (the down projection's input, a_rows_are_pairs = 1).
 * Device pointers, caller-owned, 16-byte aligned; gu and h must not overlap.
 * rows = 0 is a no-op.  HM_ERR_NULL for a null pointer when rows > 0,
 * HM_ERR_SHAPE for rows < 0 or d <= 0, HM_ERR_ALIGN for a misaligned pointer,
 * HM_ERR_HIP if the launch fails. */
hm_status hm_silu_mul(const uint16_t* gu, int64_t rows, int64_t d, uint16_t* h, hipStream_t stream);

/* The gated activation and the per-token FP8 quantization of its rows in one
 * pass, for an MoE block whose down projection takes FP8 rows (per-token FP8
 * activations: ywsung.com note, section on weight format / activation /
 * backend): h8 and h_scales are exactly what hm_silu_mul followed by
 * hm_quant_fp8_rows on its bf16 output give (h rounded to bf16 first, then
 * s = amax/448 and E4M3(h/s)), without writing or reading the bf16 h.
 *   gu bf16 [rows][2d]; h8 E4M3 bytes [rows][d]; h_scales fp32 [rows].
 * d a multiple of 8 and at most 8192 (HM_ERR_SHAPE otherwise); gu and h8
 * 16-byte aligned, h_scales 4-byte aligned.  rows = 0 is a no-op. */
hm_status hm_silu_mul_fp8(const uint16_t* gu, int64_t rows, int64_t d, uint8_t* h8, float* h_scales,
                          hipStream_t stream);

/* Top-k weighted combine of an MoE block (same pages; the reading: each
 * token's output is its routing-weighted sum of its experts' outputs):
 *   out[t][c] = bf16( sum_{j = 0..topk-1} w[t][j] * y[t*topk + j][c] ),
 * summed in fp32 in ascending j, rounded to nearest even.
 *   y    bf16 [t*topk][n], pair order (hm_moe_gemm's down output);
 *   w    fp32 [t][topk] routing weights;
 *   out  bf16 [t][n].
 * Device pointers, caller-owned; y and out 16-byte aligned, w 4-byte aligned;
 * out must not overlap y or w.  t = 0 is a no-op.  HM_ERR_NULL for a null
 * pointer when t > 0, HM_ERR_SHAPE for t < 0, n <= 0 or topk < 1,
 * HM_ERR_ALIGN for a misaligned pointer, HM_ERR_HIP if the launch fails. */
hm_status hm_moe_combine(const uint16_t* y, const float* w, int64_t t, int32_t topk, int64_t n,
                         uint16_t* out, hipStream_t stream);

/* ------------------------------------------------------------ measurement */

/* Plain-read reference: reads `bytes` bytes of `buf` once with the 16-byte
 * loads the decode GEMM uses for its weights, `unroll` loads in flight per
 * lane (1, 2, 4 or 8) over `blocks` blocks of 256 threads (1 .. 65535), and
 * writes one xor-fold word per block to out[blocks] (so no load is skipped).
 * Computes nothing of the GEMM: its time is the bandwidth floor the
 * weight-streaming kernel is compared against.  bytes a positive multiple of
 * 16; buf and out 16- and 4-byte aligned; HM_ERR_SHAPE / HM_ERR_NULL /
 * HM_ERR_ALIGN before any launch. */
hm_status hm_read_probe(const void* buf, int64_t bytes, int32_t blocks, int32_t unroll, uint32_t* out,
                        hipStream_t stream);

/* Human-readable name of a status code (static string). */
const char* hm_status_string(int32_t status);  /* any value; unknown ones named so */

#ifdef __cplusplus
}
#endif

#endif /* HM_H */
