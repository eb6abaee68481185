/*
 * mx.h -- C ABI of the MXFP4 (OCP Microscaling) training hot path for AMD
 * MI355X (gfx950): block quantizer, MXFP4 GEMMs, quantized linear layer and
 * the post-step weight de-oscillation pass.
 *
 * The operations follow these pages:
 *  [TJ]   "Oscillation-Reduced MXFP4 Training for Vision Transformers"
 *         (rebuttal, Question 2: Y = Q_D(X) Q_D(W^T), the STE weight gradient,
 *         1x32 / 32x1 group shapes and the double quantization Q_S(Q_D(X))).
 *  [ALTO] "ALTO MXFP4 training -- Weight de-oscillation -- What does it mean?"
 *         (Jargon: MXFP4, E2M1, Bin, RHT, Stochastic rounding; the ratio
 *         paragraph: window of 200 steps, d_w, d_Q, threshold 4.0, snap to
 *         the current bin centre, post-step hook).
 *  [OAS]  "Unveiling the Potential of Quantization with MXFP4" (abstract:
 *         power-of-two block scale).
 *  [MRG]  "Microscaling FP4 Quantization: MR-GPTQ ..." (section "FP4
 *         Quantization with Micro-Rotated GPTQ Algorithm": block-wise Hadamard).
 * Conventions the pages leave open follow the OCP MX v1.0 specification
 * (E2M1 values {0, .5, 1, 1.5, 2, 3, 4, 6}; shared exponent
 * floor(log2 amax) - 2 stored as an E8M0 byte with bias 127; values above 6
 * saturate to 6).
 *
 * Data layout
 *  - A "packed MXFP4 matrix" with B-element blocks along its last axis is two
 *    dense row-major arrays: codes [outer][inner/2] (element 2j in the low
 *    nibble of byte j, bit 3 = sign, bits 0-2 = index of the magnitude) and
 *    scales [outer][inner/32] (E8M0: value 2^(byte-127), 0xFF = NaN).
 *  - MX_ROW quantizes 1x32 blocks along the columns of a [rows, cols] input:
 *    codes [rows][cols/2], scales [rows][cols/32].
 *  - MX_COL quantizes 32x1 blocks along the rows and stores the result
 *    transposed: codes [cols][rows/2], scales [cols][rows/32].  So every GEMM
 *    operand is contiguous along its contraction axis.
 *  - Stochastic rounding rounds an element up iff floor(t * 2^22) + r22 >= 2^22,
 *    with t in [0, 1) the relative distance to the lower neighbour.  The
 *    elements 2i and 2i+1 of a block share output idx+1 of SplitMix64 started
 *    from `seed` (Steele, Lea & Flood, OOPSLA 2014), idx the logical row-major
 *    index of element 2i in the input: element 2i takes bits 42..63 as r22,
 *    element 2i+1 bits 9..30.  The result does not depend on tiling or launch
 *    shape.
 *
 * Ownership and execution
 *  - Every pointer argument is a DEVICE pointer owned by the caller, except
 *    `offs` of the grouped calls (host).  The library never allocates, frees or
 *    synchronizes; it keeps no state between calls, so every entry point is
 *    reentrant.  Work is enqueued on `stream` (a hipStream_t; NULL = default
 *    stream) and the call returns before it runs.
 *  - Input and output buffers must not overlap unless stated.
 *
 * Errors
 *  - Every entry point returns an mx_status.  Arguments are validated before
 *    any launch; on a validation error nothing is written and nothing is
 *    enqueued.  MX_ERR_HIP reports a failed launch (the stream may then hold
 *    earlier work of the same call).
 *  - Base pointers of device arrays must be 16-byte aligned (MX_ERR_ALIGN).
 */
#ifndef MX355_MX_H
#define MX355_MX_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MX_OK = 0,
  MX_ERR_NULL = 1,      /* a required pointer is NULL */
  MX_ERR_SHAPE = 2,     /* a size is negative, a block axis is not a multiple of 32, ... */
  MX_ERR_ALIGN = 3,     /* a device pointer is not 16-byte aligned */
  MX_ERR_ENUM = 4,      /* dtype / axis / rounding / flag out of range */
  MX_ERR_WORKSPACE = 5, /* workspace NULL or smaller than required */
  MX_ERR_HIP = 6        /* the HIP runtime rejected a launch */
} mx_status;

enum { MX_F32 = 0, MX_BF16 = 1 };   /* element types of unquantized tensors */
enum { MX_ROW = 0, MX_COL = 1 };    /* 1x32 blocks along cols / 32x1 blocks along rows */
enum { MX_RNE = 0, MX_SR = 1 };     /* Q_D: nearest, ties to even / Q_S: stochastic */

/* Largest number of groups mx_gemm_grouped accepts. */
#define MX_MAX_GROUPS 128

/* Human-readable name of a status code (static string). */
const char* mx_status_string(int status);

/* ------------------------------------------------------------------ quantizer
 * mx_quantize: MXFP4-quantize a [rows, cols] row-major tensor x (dtype MX_F32
 * or MX_BF16) -- [ALTO] Jargon "MXFP4", "E2M1", "Bin", "Stochastic rounding";
 * [TJ] Question 2 for the two group shapes.
 *  For each block of 32 values v (after the optional rotation):
 *    e = clamp(floor(log2 max|v|) - 2, -127, 127) (e = -127 for an all-zero
 *    block), scale byte = e + 127; a_i = |v_i| 2^-e; the magnitude is the
 *    nearest of {0,.5,1,1.5,2,3,4,6} with ties to the even code (MX_RNE) or
 *    one of the two neighbours chosen by stochastic rounding (MX_SR); a_i > 6
 *    gives 6; the sign bit is the sign bit of v_i (so -0 codes as 0x8).
 *    A block holding NaN or Inf gets scale byte 0xFF and zero codes.
 *  axis MX_ROW: cols % 32 == 0; writes codes [rows][cols/2], scales [rows][cols/32].
 *  axis MX_COL: rows % 32 == 0 and cols % 8 == 0; writes codes [cols][rows/2],
 *       scales [cols][rows/32] (transposed).
 *  hadamard != 0: each block is first rotated, v = H32 (s . x), H32 the
 *    unnormalised Sylvester Hadamard matrix (H H^T = 32 I) and s_j = -1 where
 *    bit j of sign_mask is set -- [ALTO] Jargon "Randomized Hadamard transform",
 *    [MRG] block-wise Hadamard.  Computed in float32 with butterfly stages
 *    h = 1, 2, 4, 8, 16.
 *  seed is used only by MX_SR.  rows or cols == 0 is a no-op.
 */
int mx_quantize(const void* x, int dtype, int64_t rows, int64_t cols, int axis, int round,
                uint64_t seed, int hadamard, uint32_t sign_mask,
                uint8_t* codes, uint8_t* scales, void* stream);

/* mx_quantize_ld: mx_quantize with the output's scale rows scale_ld bytes apart
 * (scale row r starts at scales + r * scale_ld; scale_ld >= the blocks per
 * output row, cols/32 for MX_ROW, rows/32 for MX_COL, else MX_ERR_SHAPE).  The
 * bytes of a scale row past its blocks are not written.  Codes are packed as
 * for mx_quantize.  Scale rows padded to a multiple of 16 bytes let the GEMMs
 * load the scales of four K-steps of a row at once (mx_gemm_ld,
 * mx_gemm_grouped_ld). */
int mx_quantize_ld(const void* x, int dtype, int64_t rows, int64_t cols, int axis, int round,
                   uint64_t seed, int hadamard, uint32_t sign_mask,
                   uint8_t* codes, uint8_t* scales, int64_t scale_ld, void* stream);

/* mx_quantize_dual: one read of a [rows, cols] tensor, two quantizations:
 * a MX_ROW one (codes_row [rows][cols/2], scales_row [rows][cols/32], seed
 * seed_row) and a MX_COL one (codes_col [cols][rows/2], scales_col
 * [cols][rows/32], seed seed_col), both with rounding `round`.  Equal,
 * bit for bit, to two mx_quantize calls.  This is the gradient dY of the
 * backward pass, which both backward GEMMs consume in different group
 * shapes ([TJ] Question 2 (2)).  rows % 32 == 0, cols % 32 == 0. */
int mx_quantize_dual(const void* x, int dtype, int64_t rows, int64_t cols, int round,
                     uint64_t seed_row, uint64_t seed_col,
                     uint8_t* codes_row, uint8_t* scales_row,
                     uint8_t* codes_col, uint8_t* scales_col, void* stream);

/* mx_quantize_pair: two MX_ROW quantizations in one launch -- the forward
 * layer's two operands Q_D(X) and Q_D(W) ([TJ] Question 2 (1): both 1x32 along
 * the contraction axis).  x0 [rows0, cols] and x1 [rows1, cols] (same dtype,
 * rounding, rotation and sign_mask) are quantized exactly as two mx_quantize
 * calls with axis MX_ROW and seeds seed0 / seed1 would (each tensor's
 * stochastic-rounding index starts at 0), writing codes0 [rows0][cols/2],
 * scales0 [rows0][cols/32] and codes1 / scales1 likewise.  cols % 32 == 0; a
 * tensor with 0 rows is skipped (its pointers may then be NULL). */
int mx_quantize_pair(const void* x0, int64_t rows0, const void* x1, int64_t rows1, int64_t cols,
                     int dtype, int round, uint64_t seed0, uint64_t seed1, int hadamard,
                     uint32_t sign_mask, uint8_t* codes0, uint8_t* scales0,
                     uint8_t* codes1, uint8_t* scales1, void* stream);

/* mx_quantize_dual_rht: mx_quantize_dual with the random-sign block Hadamard
 * ([ALTO] Jargon "Randomized Hadamard transform"; the "MXFP4 + RHT +
 * stochastic rounding" rows of its steps table) on both outputs: each row
 * block and each column block is rotated, y = H32 (s . x) with s from
 * sign_mask (bit j set: element j of the block negated), before it is
 * quantized -- equal, bit for bit, to two mx_quantize calls with hadamard = 1.
 * Arguments otherwise as mx_quantize_dual. */
int mx_quantize_dual_rht(const void* x, int dtype, int64_t rows, int64_t cols, int round,
                         uint64_t seed_row, uint64_t seed_col, uint32_t sign_mask,
                         uint8_t* codes_row, uint8_t* scales_row,
                         uint8_t* codes_col, uint8_t* scales_col, void* stream);

/* mx_requantize: double quantization Q(Q_D(X)) -- [TJ] Question 2 (2), the
 * double-quantized operand Q_S^(6)(Q_D^(1)(X)).  Input: a packed MX_ROW matrix
 * of logical shape [rows, cols] (codes_in [rows][cols/2], scales_in
 * [rows][cols/32]).  Its exact values are quantized again with 32x1 blocks
 * (MX_COL, output transposed: codes_out [cols][rows/2], scales_out
 * [cols][rows/32]) with rounding `round` and `seed`; the stochastic-rounding
 * index is the logical row-major index in [rows, cols].  Equal to
 * mx_quantize(dequantized input, MX_COL, ...).  rows % 32 == 0, cols % 32 == 0. */
int mx_requantize(const uint8_t* codes_in, const uint8_t* scales_in, int64_t rows, int64_t cols,
                  int round, uint64_t seed, uint8_t* codes_out, uint8_t* scales_out, void* stream);

/* mx_requantize_pair: two double quantizations in one launch -- the backward
 * layer's Q_S^(4)(Q_D(W)) and Q_S^(6)(Q_D(X)) ([TJ] Question 2 (2)).  The
 * packed MX_ROW inputs [rows0, cols] and [rows1, cols] are requantized exactly
 * as two mx_requantize calls with seeds seed0 / seed1 would, outputs transposed
 * (codes_out0 [cols][rows0/2], scales_out0 [cols][rows0/32], and likewise for
 * input 1).  rows0, rows1, cols multiples of 32; an input with 0 rows is skipped
 * (its pointers may then be NULL). */
int mx_requantize_pair(const uint8_t* codes_in0, const uint8_t* scales_in0, int64_t rows0,
                       const uint8_t* codes_in1, const uint8_t* scales_in1, int64_t rows1,
                       int64_t cols, int round, uint64_t seed0, uint64_t seed1,
                       uint8_t* codes_out0, uint8_t* scales_out0,
                       uint8_t* codes_out1, uint8_t* scales_out1, void* stream);

/* mx_requantize_rht: double quantization of an operand kept in the rotated
 * domain (the rotated layer's saved Q_D(H X), rotated along cols with
 * sign_mask): the input's row blocks are decoded and rotated back exactly as
 * mx_dequantize with hadamard = 1 does it (float32), then each 32x1 column
 * block is rotated with the same signs and quantized (output transposed, as
 * mx_requantize; the stochastic-rounding index is the logical row-major index
 * of the rotated position).  Equal to mx_quantize(mx_dequantize(in, MX_ROW,
 * hadamard = 1), MX_COL, hadamard = 1).  rows % 32 == 0, cols % 32 == 0. */
int mx_requantize_rht(const uint8_t* codes_in, const uint8_t* scales_in, int64_t rows,
                      int64_t cols, int round, uint64_t seed, uint32_t sign_mask,
                      uint8_t* codes_out, uint8_t* scales_out, void* stream);

/* mx_dequantize: exact values of a packed matrix -- [ALTO] Jargon "MXFP4" (each
 * block of 32 values shares one power-of-two scale, and an element's value is
 * its 4-bit E2M1 number times that scale) and "E2M1"; it is the deq(.) inside
 * every product of [TJ] Question 2 and the bin value q(w) of the
 * de-oscillation pass.  Input: a packed matrix of logical shape [rows, cols]
 * quantized along `axis` (the inverse layout of mx_quantize), written row-major
 * [rows, cols] as float32 or bf16 (out_dtype).  value = sign * E2M1[code & 7]
 * * 2^(byte - 127) (exact in both types), byte 0xFF gives NaN.  hadamard != 0
 * undoes the rotation: x = s . (H32 y) 2^-5 per block in float32 (bf16 output
 * then rounds to nearest even).  rows (MX_COL) or cols (MX_ROW) % 32 == 0;
 * rows or cols == 0 is a no-op.  Errors as for mx_quantize. */
int mx_dequantize(const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t cols,
                  int axis, int hadamard, uint32_t sign_mask, void* out, int out_dtype,
                  void* stream);

/* ------------------------------------------------------------------ GEMM
 * mx_gemm: C[m][n] = alpha * sum_k deq(A)[m][k] * deq(B)[n][k]  -- the MXFP4
 * matrix product of [TJ] Question 2 (1), (1x32) x (32x1) groups.
 *  A: packed MX_ROW [M, K] (a_codes [M][K/2], a_scales [M][K/32]);
 *  B: packed MX_ROW [N, K] (b_codes [N][K/2], b_scales [N][K/32]);
 *  C: float32 row-major, leading dimension ldc >= N (ldc % 4 == 0), overwritten.
 *  K % 32 == 0; M, N >= 0 (M or N == 0: no-op; K == 0: C = 0); M, N <= 2^31 and
 *  K < 2^31, else MX_ERR_SHAPE (the same bounds hold for every GEMM call below).
 *  Products of FP4 values and E8M0 scales are exact; sums are float32 in an
 *  unspecified order (error <= ~K/64 * 2^-24 * sum |a b|). */
int mx_gemm(const uint8_t* a_codes, const uint8_t* a_scales,
            const uint8_t* b_codes, const uint8_t* b_scales,
            int64_t M, int64_t N, int64_t K, float alpha, float* c, int64_t ldc, void* stream);

/* mx_gemm_grouped: per-group products for a mixture-of-experts layer ([ALTO]
 * news paragraph: the MoE model trained in MXFP4).  offs is a HOST array of
 * groups+1 non-decreasing row offsets with offs[0] == 0; rows
 * offs[g] .. offs[g+1]-1 of A and C use B_g, the g-th [N, K] matrix of b
 * (b_codes + g*N*K/2, b_scales + g*N*K/32).  C is [offs[groups]][N], ldc = N.
 * 1 <= groups <= MX_MAX_GROUPS, K % 32 == 0, N % 4 == 0. */
int mx_gemm_grouped(const uint8_t* a_codes, const uint8_t* a_scales,
                    const uint8_t* b_codes, const uint8_t* b_scales,
                    const int64_t* offs, int64_t groups, int64_t N, int64_t K, float alpha,
                    float* c, void* stream);

/* mx_gemm_ld / mx_gemm_grouped_ld: mx_gemm / mx_gemm_grouped with the scale
 * rows of A and of B a_scale_ld and b_scale_ld bytes apart (each >= K/32, else
 * MX_ERR_SHAPE; the bytes past K/32 in a row are never used as data); for the
 * grouped form, B_g's scales start at b_scales + g*N*b_scale_ld.  Codes are
 * packed as for mx_gemm.  Same results, bit for bit, as the packed calls on the
 * same values; pitches that are multiples of 16 (with 16-byte aligned scale
 * arrays) take the fastest scale loads whatever K is. */
int mx_gemm_ld(const uint8_t* a_codes, const uint8_t* a_scales, int64_t a_scale_ld,
               const uint8_t* b_codes, const uint8_t* b_scales, int64_t b_scale_ld,
               int64_t M, int64_t N, int64_t K, float alpha, float* c, int64_t ldc,
               void* stream);
int mx_gemm_grouped_ld(const uint8_t* a_codes, const uint8_t* a_scales, int64_t a_scale_ld,
                       const uint8_t* b_codes, const uint8_t* b_scales, int64_t b_scale_ld,
                       const int64_t* offs, int64_t groups, int64_t N, int64_t K, float alpha,
                       float* c, void* stream);

/* ------------------------------------------------------------------ token segments
 * The 32x1 quantizers of a grouped (mixture-of-experts) layer run per token
 * segment: segment g is rows offs[g] .. offs[g+1]-1 (offs: HOST array of
 * groups+1 non-decreasing offsets, offs[0] == 0, offs[groups] == rows, 1 <=
 * groups <= MX_MAX_GROUPS).  Blocks start at the segment's first row; the
 * segment's tail is zero-padded to a multiple of 128 rows, so the transposed
 * outputs have a padded row axis of P = mx_segments_padded_rows(offs, groups)
 * positions, segment g's starting at the sum of the padded lengths before it.
 * Padding blocks hold code 0 and scale byte 0.  The stochastic-rounding index
 * of a real element is its row-major index in [rows, cols]. */
int64_t mx_segments_padded_rows(const int64_t* offs, int64_t groups);

/* mx_quantize_segments: 32x1 blocks of x [rows, cols] (`dtype`) per segment:
 * codes [cols][P/2], scales [cols][P/32].  cols % 8 == 0. */
int mx_quantize_segments(const void* x, int dtype, int64_t rows, int64_t cols,
                         const int64_t* offs, int64_t groups, int round, uint64_t seed,
                         uint8_t* codes, uint8_t* scales, void* stream);

/* mx_requantize_segments: mx_requantize per segment -- the exact values of a
 * packed MX_ROW [rows, cols] matrix quantized with 32x1 blocks per segment:
 * codes_out [cols][P/2], scales_out [cols][P/32].  cols % 32 == 0. */
int mx_requantize_segments(const uint8_t* codes_in, const uint8_t* scales_in, int64_t rows,
                           int64_t cols, const int64_t* offs, int64_t groups, int round,
                           uint64_t seed, uint8_t* codes_out, uint8_t* scales_out, void* stream);

/* ------------------------------------------------------------------ linear layer
 * mx_linear_fwd: forward of the quantized linear layer, Y = Q_D(X) Q_D(W)^T
 * ([TJ] Question 2 (1)); X [M, K], W [N, K] (nn.Linear layout), both `dtype`;
 * Q_D is MX_ROW + MX_RNE along K.  Writes y [M][N] float32 and the packed
 * operands kept for the backward pass: xq_codes [M][K/2], xq_scales [M][K/32],
 * wq_codes [N][K/2], wq_scales [N][K/32].  M, N, K multiples of 32 and below 2^31,
 * N % 4 == 0 (else MX_ERR_SHAPE, before any launch).  M or N == 0: no-op;
 * K == 0: Y = 0 and nothing else is read or written (x, w and the packed
 * operands may then be NULL). */
int mx_linear_fwd(const void* x, const void* w, int dtype, int64_t M, int64_t N, int64_t K,
                  float* y, uint8_t* xq_codes, uint8_t* xq_scales,
                  uint8_t* wq_codes, uint8_t* wq_scales, void* stream);

/* Bytes of device workspace mx_linear_bwd needs for these sizes. */
size_t mx_linear_bwd_workspace_size(int64_t M, int64_t N, int64_t K);

/* mx_linear_bwd: backward of the quantized linear layer with straight-through
 * gradients ([TJ] Question 2 (1) and (2)):
 *   dX = Q_S^(3)(dY) . Q_S^(4)(Q_D(W))       contraction over N
 *   dW = Q_S^(5)(dY)^T . Q_S^(6)(Q_D(X))     contraction over M
 * Q^(3): dY 1x32 along N; Q^(5): dY 32x1 along M; Q^(4), Q^(6): double
 * quantization of the saved forward operands with 32x1 blocks along N and M.
 * Stochastic rounding; quantizer q uses seed + q.  dy [M][N] (`dtype`);
 * the saved operands are mx_linear_fwd's outputs; writes dx [M][K] and
 * dw [N][K] float32.  workspace: device buffer of at least
 * mx_linear_bwd_workspace_size(M, N, K) bytes, 16-byte aligned.
 * M, N, K multiples of 32 and below 2^31, K % 4 == 0.  K == 0: no-op.  M == 0 or
 * N == 0 (an empty contraction for one of the products): dx = 0 and dw = 0 are
 * written and nothing else is read (only dx, when M > 0, and dw, when N > 0,
 * are required). */
int mx_linear_bwd(const void* dy, int dtype, int64_t M, int64_t N, int64_t K,
                  const uint8_t* xq_codes, const uint8_t* xq_scales,
                  const uint8_t* wq_codes, const uint8_t* wq_scales,
                  uint64_t seed, float* dx, float* dw,
                  void* workspace, size_t workspace_bytes, void* stream);

/* mx_linear_bwd_noalloc: mx_linear_bwd for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): no workspace argument and no allocation of any kind; the
 * workspace is a file-scope device array of mx_linear_bwd_noalloc_max_workspace()
 * bytes (64 MiB) that each GPU the library runs on holds from library load until
 * the process ends.  Layers whose workspace (mx_linear_bwd_workspace_size) is
 * larger are rejected with MX_ERR_WORKSPACE before anything is enqueued (the
 * DeiT-S MLP layers need 36-43 MiB; the Llama-3-8B up-projection needs 166 MiB
 * and must use mx_linear_bwd).  Every call on one GPU shares that GPU's array,
 * so calls that may overlap on one GPU (on different streams, or from different
 * threads without ordering) race and give wrong results; calls on one stream are
 * ordered and safe.  Nothing in the array needs to start at zero.  The first call
 * on a device looks up the array's device address (MX_ERR_HIP if the runtime
 * cannot give it).  Arguments, results and other errors as mx_linear_bwd, bit
 * for bit. */
int mx_linear_bwd_noalloc(const void* dy, int dtype, int64_t M, int64_t N, int64_t K,
                          const uint8_t* xq_codes, const uint8_t* xq_scales,
                          const uint8_t* wq_codes, const uint8_t* wq_scales,
                          uint64_t seed, float* dx, float* dw, void* stream);
size_t mx_linear_bwd_noalloc_max_workspace(void);

/* mx_linear_fwd_rht / mx_linear_bwd_rht: the same layer with the random-sign
 * block Hadamard on every product ([ALTO] Jargon "Randomized Hadamard
 * transform", the "MXFP4 + RHT + stochastic rounding" rows of its steps
 * table): both operands of a product are rotated along that product's
 * contraction axis with the same signs (sign_mask), and since H H^T = 32 I the
 * product is scaled by alpha = 2^-5 (exact):
 *   Y  = 2^-5 Q_D(H_K X) Q_D(H_K W)^T
 *   dX = 2^-5 Q_S^(3)(H_N dY) . Q_S^(4)(H_N W~)      W~ = H_K^-1 deq(Q_D(H_K W))
 *   dW = 2^-5 Q_S^(5)(H_M dY)^T . Q_S^(6)(H_M X~)    X~ = H_K^-1 deq(Q_D(H_K X))
 * The saved operands (xq, wq) are in the K-rotated domain; the backward takes
 * them back before its own rotations (mx_requantize_rht).  Arguments, layouts,
 * seeds (seed + q), workspace (mx_linear_bwd_workspace_size) and errors as
 * mx_linear_fwd / mx_linear_bwd. */
int mx_linear_fwd_rht(const void* x, const void* w, int dtype, int64_t M, int64_t N, int64_t K,
                      uint32_t sign_mask, float* y, uint8_t* xq_codes, uint8_t* xq_scales,
                      uint8_t* wq_codes, uint8_t* wq_scales, void* stream);
int mx_linear_bwd_rht(const void* dy, int dtype, int64_t M, int64_t N, int64_t K,
                      const uint8_t* xq_codes, const uint8_t* xq_scales,
                      const uint8_t* wq_codes, const uint8_t* wq_scales,
                      uint64_t seed, uint32_t sign_mask, float* dx, float* dw,
                      void* workspace, size_t workspace_bytes, void* stream);

/* mx_grouped_linear_bwd: backward of a grouped (mixture-of-experts) linear
 * layer whose forward is mx_gemm_grouped(Q_D(X), Q_D(W)) ([ALTO] news
 * paragraph: the MoE model trained in MXFP4; the group shapes and double
 * quantization of [TJ] Question 2, per expert):
 *   dX[rows of e] = Q_S^(3)(dY)[rows of e] . Q_S^(4)(Q_D(W_e))  contraction over N
 *   dW_e          = Q_S^(5)(dY_e)^T . Q_S^(6)(Q_D(X_e))        contraction over e's tokens
 * Q^(3): 1x32 along N; Q^(4): 32x1 along N of each expert's [N, K] weight (the
 * index is that of the stacked [groups*N, K] weight); Q^(5), Q^(6): 32x1 along
 * the tokens of each expert (token segments, zero-padded tails).  Stochastic
 * rounding, quantizer q uses seed + q.  dy [R][N] (`dtype`, R = offs[groups]);
 * xq: Q_D(X) [R][K/2] + [R][K/32]; wq: the stacked Q_D(W) [groups*N][K/2] +
 * [groups*N][K/32].  Writes dx [R][K] and dw [groups][N][K] float32 (an expert
 * without tokens gets dW_e = 0).  N, K multiples of 32 and below 2^31, and the
 * workspace's token axis (each expert's tokens padded to a multiple of 512) below
 * 2^31 (else MX_ERR_SHAPE).  workspace: at least
 * mx_grouped_linear_bwd_workspace_size(offs, groups, N, K) bytes, 16-byte
 * aligned. */
size_t mx_grouped_linear_bwd_workspace_size(const int64_t* offs, int64_t groups, int64_t N,
                                            int64_t K);
int mx_grouped_linear_bwd(const void* dy, int dtype, const int64_t* offs, int64_t groups,
                          int64_t N, int64_t K, const uint8_t* xq_codes, const uint8_t* xq_scales,
                          const uint8_t* wq_codes, const uint8_t* wq_scales, uint64_t seed,
                          float* dx, float* dw, void* workspace, size_t workspace_bytes,
                          void* stream);

/* ------------------------------------------------------------------ de-oscillation
 * Weight de-oscillation as a post-optimizer-step pass ([ALTO] "How does ALTO
 * detect and fix oscillating weights?" and the ratio paragraph).  w is the
 * float32 master weight [rows, cols]; its bin value q(w) is the forward weight
 * quantizer's output deq(Q_D(w)) with 1x32 RNE blocks along cols.  The state is
 * three caller-owned float32 arrays of the same shape: w_prev (snapshot),
 * d_w (master-weight path length) and d_q (quantized path length).
 *
 * mx_deosc_init: w_prev = w, d_w = d_q = 0. */
int mx_deosc_init(const float* w, int64_t rows, int64_t cols,
                  float* w_prev, float* d_w, float* d_q, void* stream);

/* mx_deosc_step: call once after every optimizer step, in float32:
 *   d_w += |w - w_prev|;  d_q += |q(w) - q(w_prev)|;  w_prev = w.
 * If end_of_window != 0 (every P-th call, P = 200 on the page): flag =
 * d_q > threshold * d_w (threshold 4.0 on the page); flagged elements are
 * snapped, w = q(w); then w_prev = w and d_w = d_q = 0; flags (uint8 [rows][cols],
 * required then, else ignored) receives 1 for flagged elements, 0 otherwise.
 * cols % 32 == 0.  w is updated in place. */
int mx_deosc_step(float* w, int64_t rows, int64_t cols, float* w_prev, float* d_w, float* d_q,
                  int end_of_window, float threshold, uint8_t* flags, void* stream);

/* mx_deosc_step_quantize: mx_deosc_step, and in the same pass the next forward's
 * weight operand Q_D(w) of the updated w (1x32 blocks along cols, nearest
 * rounding), written to wq_codes [rows][cols/2] and wq_scales [rows][cols/32]
 * (caller-owned device memory; wq_codes 16-byte aligned) -- bit-identical to
 * mx_quantize(w, MX_F32, rows, cols, MX_ROW, MX_RNE, ...) after the step.  The
 * ALTO page runs the hook and the forward's weight quantization separately;
 * snapping to the bin value keeps every code and scale, so one pass gives both.
 * Arguments and errors otherwise as mx_deosc_step. */
int mx_deosc_step_quantize(float* w, int64_t rows, int64_t cols, float* w_prev, float* d_w,
                           float* d_q, int end_of_window, float threshold, uint8_t* flags,
                           uint8_t* wq_codes, uint8_t* wq_scales, void* stream);

/* mx_qema_step: Q-EMA post-step update ("Oscillation-Reduced MXFP4 Training for
 * Vision Transformers", rebuttal: Question 4 -- one EMA copy per linear weight;
 * the overhead answer -- it is updated with the parameters and it is what the
 * forward quantizes; the hyperparameter answer -- beta 0.998 by default).  In
 * float32, in this order:  ema = (beta * ema) + ((1 - beta) * w), 1 - beta
 * rounded to float32 first; then wq_codes / wq_scales = Q_D(ema) (1x32 blocks
 * along cols, nearest rounding), the next forward's weight operand.
 * w [rows][cols] float32 (read), ema [rows][cols] float32 (updated in place;
 * the caller starts it as a copy of w).  cols % 32 == 0; w, ema, wq_codes
 * 16-byte aligned device memory owned by the caller. */
int mx_qema_step(const float* w, float* ema, int64_t rows, int64_t cols, float beta,
                 uint8_t* wq_codes, uint8_t* wq_scales, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* MX355_MX_H */
