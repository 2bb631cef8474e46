/*
 * awq.h -- C ABI of the MI355X (gfx950) AWQ per-layer scale-search library.
 *
 * The library computes the activation-aware weight quantisation scale search
 * for one linear layer y = W x, W [N out, K in], on calibration activations
 * X [T tokens, K]:
 *
 *   1. a_j = mean_t |X[t, j]|                              (awq_act_stats)
 *   2. for every alpha on a grid: s_j = max(a_j, 1e-8)^alpha
 *   3. group-wise asymmetric round-to-nearest quantisation of W diag(s),
 *      dequantisation, division by s                     (awq_fake_quant)
 *   4. mean squared error of the layer output X W_hat^T against X W^T
 *   5. argmin over alpha                                  (awq_search_scales)
 *   and the final integer codes with per-group step and zero-point
 *                                                         (awq_quantize_pack)
 *
 * and the rows that build on it: the low-bit decode layer on the packed
 * codes (awq_lowbit_*), the mixed-precision ablation that motivates the
 * method (awq_salient_keep_loss), GPTQ error feedback after the scaling
 * (awq_gptq_*) and SmoothQuant W8A8 (awq_smooth_scales,
 * awq_quantize_rows_int8, awq_w8a8_loss).
 *
 * Sources (web pages on the method):
 *   [P1] "Как работает quantization-aware scaling в AWQ для защиты важных
 *        весов?" (aivaro.ru Q&A), sections 5, 6 and 9
 *   [P2] "AWQ: Activation-Aware Weight Quantization For On-Device LLM
 *        Compression AND Acceleration" (reading notes), section "Measures"
 *   [P3] "52 · AWQ, GPTQ và SmoothQuant", sections 2 to 5
 *   [P4] "GPTQ与AWQ" (study notes), sections "AWQ实现要点" and GPTQ
 *
 * Conventions shared by every entry point
 *   - Every tensor is a dense row-major buffer in device memory, allocated and
 *     owned by the caller; the library allocates no device memory.  Host
 *     buffers are named as such below.
 *   - Work is enqueued asynchronously on `stream` (NULL = the null stream);
 *     outputs are valid once the stream has been synchronised.  Calls that
 *     share a workspace must be ordered on one stream.
 *   - Arguments are validated before anything is enqueued.  A non-OK status
 *     enqueues nothing (AWQ_ERR_HIP: a launch failed; the stream may then hold
 *     part of the work).  awq_last_error() gives a message for the calling
 *     thread's last non-OK status.  No C++ exception crosses this ABI.
 *   - Element arithmetic of the quantiser is IEEE fp32 with round-to-nearest-
 *     even, correctly rounded division and no contraction, in the fixed order
 *     given at awq_fake_quant; codes, steps and zero-points are therefore
 *     bit-identical to any other IEEE implementation of that order.
 *   - W and X share one dtype.  fp16/bf16 layers use the MFMA path (fp32
 *     accumulation); fp32 layers use an fp32 vector-ALU path.
 *   - Sizes: every operand buffer must be below 4 GiB (byte offsets are
 *     32-bit inside the kernels); bits in [2, 8]; group a power of two in
 *     [32, 512] dividing K.
 */
#ifndef AWQ_MI355X_AWQ_H
#define AWQ_MI355X_AWQ_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* AWQ_DTYPE_MAX_ENUM is no dtype: it gives the enumeration the range of a
 * 32-bit int, so that whatever value a caller passes is a valid value for the
 * library to check (and refuse), in C and in C++ alike. */
typedef enum {
  AWQ_F32 = 0,
  AWQ_F16 = 1,
  AWQ_BF16 = 2,
  AWQ_DTYPE_MAX_ENUM = 0x7fffffff
} awq_dtype_t;

typedef enum {
  AWQ_OK = 0,
  AWQ_ERR_INVALID_ARG = -1,   /* null pointer, non-positive size, K % group != 0 ... */
  AWQ_ERR_UNSUPPORTED = -2,   /* valid but not handled: bits, group, dtype, size limit */
  AWQ_ERR_WORKSPACE = -3,     /* workspace missing or too small */
  AWQ_ERR_HIP = -4            /* a HIP runtime call or launch failed */
} awq_status_t;

/* Search flags: how a candidate's output error is formed.  Both give
 * sum_{t,i} (Y[t,i] - Yhat[t,i])^2 with Y = X W^T, Yhat = X W_hat^T. */
/* Default: the fake-quant pass writes D = W - W_hat (fp32 difference rounded
 * to the layer dtype) and the GEMM accumulates X D^T and squares it in the
 * epilogue; no reference output is formed or read.  Rounding hits D, whose
 * relative error stays at the dtype's half-ulp however small D is. */
#define AWQ_SEARCH_WEIGHT_DELTA 0u
/* The layer output W X is computed once into the workspace (fp32) and every
 * candidate GEMM on W_hat subtracts its output from it in the epilogue.
 * fp16 and fp32 layers only: rounding W_hat itself to bf16 perturbs the
 * up-scaled salient channels by more than the 1e-3 loss tolerance, so bf16
 * returns AWQ_ERR_UNSUPPORTED.  With fp16 the rounding of W_hat still limits
 * the loss accuracy at high bit widths (about 1e-3 relative at INT4 on narrow
 * layers, several 1e-3 at INT8); the default form has no such limit. */
#define AWQ_SEARCH_REFERENCE_OUTPUT 1u

/* awq_fake_quant output selection. */
#define AWQ_FQ_WEIGHT_HAT 0u     /* out = W_hat */
#define AWQ_FQ_WEIGHT_DELTA 1u   /* out = W - W_hat */

/* Library version string, e.g. "awq-mi355x 0.1". */
const char* awq_version(void);

/* Message for the calling thread's last non-OK status ("" if none). */
const char* awq_last_error(void);

/* ------------------------------------------------------------------------ *
 * Step 1: per-input-channel activation magnitude ([P2] "Measures";
 * [P4] "AWQ实现要点" item 2).
 *
 *   a_out[j] = fp32( (sum_{t<T} |X[t, j]|) / T ),  the sum in fp64.
 *
 * X: [T, K] of x_dtype.  a_out: [K] fp32.  workspace: device scratch of at
 * least awq_act_stats_workspace_size(T, K) bytes (fp64 partial sums), may be
 * NULL when that size is 0.  The summation order is fixed, so the result is
 * reproducible run to run.
 * ------------------------------------------------------------------------ */
size_t awq_act_stats_workspace_size(int64_t T, int64_t K);
awq_status_t awq_act_stats(const void* X, awq_dtype_t x_dtype, int64_t T, int64_t K,
                           float* a_out, void* workspace, size_t workspace_bytes,
                           hipStream_t stream);

/* ------------------------------------------------------------------------ *
 * Step 2: the scale table ([P2] "Measures": s = a^alpha per input channel).
 *
 *   s_out[k, j] = fp32( pow( fp64(max(a[j], 1e-8f)), fp64(alphas[k]) ) )
 *
 * a: [K] fp32 device.  alphas: [n_alpha] fp32 HOST array.  s_out:
 * [n_alpha, K] fp32 device.  (awq_search_scales builds the same table
 * internally; this entry point exposes it on its own.)
 * ------------------------------------------------------------------------ */
awq_status_t awq_scale_table(const float* a, int64_t K, const float* alphas, int n_alpha,
                             float* s_out, hipStream_t stream);

/* ------------------------------------------------------------------------ *
 * Step 3: group-wise asymmetric fake quantisation of W diag(s)
 * ([P1] sections 5 and 9: round-to-nearest over groups, zero_point,
 * q_group_size, w_bit; [P2] "Measures": scale, then quantise group-wise).
 *
 * For one scale vector s_k (row k of s, n_s rows) and every output row i and
 * group g of `group` consecutive input channels, in fp32 and in this order:
 *   w'    = W[i, j] * s[j]
 *   mx,mn = max, min of w' over the group
 *   delta = max((mx - mn) / (2^bits - 1), 1e-10f)
 *   z     = clamp(rint(-mn / delta), 0, 2^bits - 1)
 *   c     = clamp(rint(w' / delta) + z, 0, 2^bits - 1)     (rint: ties to even)
 *   W_hat = ((c - z) * delta) / s[j]
 * Output out[k, i, j] = W_hat rounded (nearest-even) to out_dtype, or, with
 * flags = AWQ_FQ_WEIGHT_DELTA, fp32(W[i, j] - W_hat) rounded to out_dtype.
 * W: [N, K] of w_dtype; s: [n_s, K] fp32 device; out: [n_s, N, K] of out_dtype (AWQ_F16/AWQ_BF16 only for fp16/bf16 W, AWQ_F32
 * only for fp32 W).
 * ------------------------------------------------------------------------ */
awq_status_t awq_fake_quant(const void* W, awq_dtype_t w_dtype, int64_t N, int64_t K,
                            const float* s, int n_s, int bits, int group, uint32_t flags,
                            void* out, awq_dtype_t out_dtype, hipStream_t stream);

/* ------------------------------------------------------------------------ *
 * Steps 2-5: the whole search ([P2] "Measures": statistics, then for each
 * alpha scale, group-quantise and measure the error, keep the best;
 * [P1] section 6: the criterion is the output mean squared error).
 *
 * Inputs: W [N, K] and X [T, K] of `dtype`; a [K] fp32 device (from
 * awq_act_stats); alphas [n_alpha] fp32 HOST array; bits; group; flags
 * (AWQ_SEARCH_WEIGHT_DELTA, the default, or AWQ_SEARCH_REFERENCE_OUTPUT).
 * Outputs (device): losses_out [n_alpha] fp64,
 *   losses_out[k] = sum_{t,i} (Y[t,i] - Yhat_k[t,i])^2 / (T N),
 *   Y = X W^T, Yhat_k = X W_hat_k^T with W_hat_k from awq_fake_quant; the
 *   GEMM takes X and D = W - W_hat_k (or W_hat_k) in the layer dtype and
 *   accumulates in fp32;
 * best_idx_out [1] int32 = lowest k with the smallest loss;
 * s_best_out [K] fp32 = row best_idx of the scale table (the factors the
 * caller folds into the operator that produces X, dividing it).
 *
 * workspace: device scratch laid out as awq_search_layout() reports for the
 * same arguments and workspace_bytes.  With the full size (layout with
 * workspace_bytes = 0) every alpha is fake-quantised in one batch (one launch,
 * W read once); a smaller workspace (at least one alpha's W_hat) makes the
 * library process the grid in batches of layout.alpha_batch.  A batch's
 * fp16/bf16 candidate GEMMs run in launches of 4 rounds of the persistent grid
 * (4 x 256 output tiles of 256 x 256 on 256 compute units), the last launch
 * of a batch taking the rest.  Losses do not depend on either.  After the
 * call the workspace holds the scale table, the reference output
 * (REFERENCE_OUTPUT form), the tiled copy of X, the last batch's D (or W_hat)
 * and the per-tile partial sums, at the reported offsets.
 *
 * Tiled layout (fp16/bf16 GEMM operands): rows padded with zeros to a multiple
 * of 256, K split in stages of 32.  Element (row, k) of a [rows, K] matrix
 * sits at element index ((t * K/32 + s) * 256 + r) * 32 + 8 * (c ^ ((r >> 1) & 3))
 * + k % 8 with t = row / 256, r = row % 256, s = k / 32, c = (k % 32) / 8:
 * each 256 x 32 block is one contiguous 16 KB unit, pre-swizzled for the
 * GEMM's LDS fragment reads.
 *
 * Fragment layout (the fp16/bf16 reference output at y_ref_offset): whole
 * 256 x 256 output tiles, Tp x Np floats in all (T and N rounded up to
 * multiples of 256).  Output (t, n) with tm = t / 256, tn = n / 256, a = t %
 * 256, b = n % 256 sits at float index
 * ((((tm * tiles_n + tn) * 8 + w) * 32 + i * 4 + j) * 64 + l) * 4 + r with
 * w = (a / 128) * 4 + b / 64, i = (a % 128) / 16, j = (b % 64) / 16,
 * l = ((a % 16) / 4) * 16 + b % 16, r = a % 4: the accumulator order of the
 * GEMM's waves, so that its squared-error epilogue reads the reference in
 * contiguous 1 KB pieces.  Entries past T or N hold the product of the zero
 * padding.
 * ------------------------------------------------------------------------ */
typedef struct {
  size_t total_bytes;       /* bytes the call uses */
  size_t s_table_offset;    /* fp32 [n_alpha][K] scale table, followed by fp32
                               [n_alpha][K] of its reciprocals RN(1/s) */
  size_t y_ref_offset;      /* fp32 reference output X W^T: fp16/bf16 in the fragment
                               layout below (Tp x Np floats), fp32 [T][N]; SIZE_MAX in
                               the WEIGHT_DELTA form */
  size_t x_tiled_offset;    /* fp16/bf16: X in the tiled layout below, Tp = T rounded
                               up to a multiple of 256 rows; SIZE_MAX for fp32 */
  size_t w_hat_offset;      /* alpha_batch consecutive matrices D = W - W_hat (or
                               W_hat): fp16/bf16 tiled [Np = N rounded up to 256][K],
                               fp32 row-major [N][K] */
  size_t partials_offset;   /* fp64 [n_alpha][tiles_m][tiles_n]: sum of squared
                               errors of output tile (m, n) = rows
                               [m*tile_m, +tile_m) x cols [n*tile_n, +tile_n) */
  int32_t alpha_batch;      /* alphas fake-quantised and scored per pass */
  int32_t tile_m, tile_n;   /* output tile of the GEMM (tokens x out channels) */
  int32_t tiles_m, tiles_n; /* ceil(T / tile_m), ceil(N / tile_n) */
} awq_search_layout_t;

/* Host-only query (no device work).  workspace_bytes = 0 asks for the layout
 * that fake-quantises every alpha in one batch; otherwise the largest batch
 * that fits in workspace_bytes.  AWQ_ERR_WORKSPACE if not even one alpha
 * fits. */
awq_status_t awq_search_layout(awq_dtype_t dtype, int64_t N, int64_t K, int64_t T,
                               int n_alpha, uint32_t flags, size_t workspace_bytes,
                               awq_search_layout_t* layout_out);

/* Host-only query: workspace bytes that let awq_search_scales fake-quantise
 * all n_alpha candidates of a W [N, K], X [T, K] layer in one batch with the
 * default form (AWQ_SEARCH_WEIGHT_DELTA), whatever the layer dtype: the
 * largest layout.total_bytes that awq_search_layout reports over AWQ_F32,
 * AWQ_F16 and AWQ_BF16 for workspace_bytes = 0.  0 when a size is
 * < 1 or n_alpha is outside [1, 4096].  The reference-output form needs
 * awq_search_layout's figure, which adds the fp32 [T][N] layer output. */
size_t awq_search_workspace_size(int64_t N, int64_t K, int64_t T, int n_alpha);

awq_status_t awq_search_scales(const void* W, const void* X, awq_dtype_t dtype,
                               int64_t N, int64_t K, int64_t T,
                               const float* a, int bits, int group,
                               const float* alphas, int n_alpha, uint32_t flags,
                               double* losses_out, float* s_best_out,
                               int32_t* best_idx_out,
                               void* workspace, size_t workspace_bytes,
                               hipStream_t stream);

/* ------------------------------------------------------------------------ *
 * Step 5b: final quantisation and packing ([P2] "Measures", last step: save
 * the low-bit weights with their quantisation metadata; [P1] section 9).
 *
 * Same arithmetic as awq_fake_quant for one scale vector s [K] (device).
 * codes_out: uint32 [N, bits*K/32]; the code of column j sits at bits
 * [bits*j, bits*j + bits) of its row's little-endian bitstream (bit p of a
 * row in word p/32, bit p%32).  scales_out: fp32 [N, K/group] = delta.
 * zeros_out: uint8 [N, K/group] = z.  With s = 1 this is plain
 * round-to-nearest quantisation.
 * ------------------------------------------------------------------------ */
awq_status_t awq_quantize_pack(const void* W, awq_dtype_t w_dtype, int64_t N, int64_t K,
                               const float* s, int bits, int group,
                               uint32_t* codes_out, float* scales_out, uint8_t* zeros_out,
                               hipStream_t stream);

/* ------------------------------------------------------------------------ *
 * The mixed-precision ablation that motivates the method ([P2] "Measures":
 * keeping 1% of the weights in FP16 chosen by activation magnitude recovers
 * most of the quantisation loss, chosen by weight magnitude it does not;
 * [P1] section 4: rank the input channels by the activation statistic and
 * keep the top 1% in FP16; section 5 item 4: round the other weights to
 * nearest over groups; [P4] "AWQ实现要点": k = int(0.01 * in_features)).
 *
 * score: [K] fp32 device, the ranking statistic (awq_act_stats of X for
 *   "by activation"; awq_act_stats applied to W, i.e. mean_i |W[i, j]|, for
 *   "by weight").  The n_keep channels with the largest score (ties: lower
 *   index first) keep their full-precision weights; every other weight is
 *   quantised round-to-nearest (s = 1, the quantiser of awq_fake_quant),
 *   with each group's min and max taken over its quantised weights only.
 * loss_out [1] fp64 device = sum_{t,i} (Y - Y_mix)^2 / (T N), formed like the
 *   search's default weight-delta form.  keep_out [K] uint8 device (may be
 *   NULL) = the chosen mask.  fp16/bf16 layers; workspace of
 *   awq_salient_keep_workspace_size(dtype, N, K, T) bytes, 256-byte aligned;
 *   it begins with the regions of awq_search_layout(dtype, N, K, T, 1,
 *   AWQ_SEARCH_WEIGHT_DELTA, 0), and after the call its w_hat region holds
 *   D = W - W_mix (tiled, in the layer dtype).
 * ------------------------------------------------------------------------ */
size_t awq_salient_keep_workspace_size(awq_dtype_t dtype, int64_t N, int64_t K, int64_t T);
awq_status_t awq_salient_keep_loss(const void* W, const void* X, awq_dtype_t dtype, int64_t N,
                                   int64_t K, int64_t T, const float* score, int64_t n_keep,
                                   int bits, int group, double* loss_out, uint8_t* keep_out,
                                   void* workspace, size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------ *
 * Using the packed weights: the low-bit linear layer for decode-shaped
 * inputs ([P2] "Tiny Chat": dequantise on the fly inside the kernel, never
 * write the dequantised weights back, reorder the low-bit weights offline so
 * the kernel unpacks them cheaply; [P2] "Measures": the layer computes
 * (W diag(s)) (diag(s)^-1 x), so it receives activations already divided by
 * s, which [P1] section 5 folds into the operator that produces them).
 *
 * awq_lowbit_repack: one-off reordering of awq_quantize_pack's output.
 *   codes [N, bits*K/32] uint32, scales [N, K/group] fp32, zeros
 *   [N, K/group] uint8 (device) ->
 *   codes_t uint32 [K/32][N][bits]: the `bits` words of chunk j (columns
 *     32j .. 32j+31) of row n at word ((j*N) + n)*bits, same bit order;
 *   meta_t  [K/group][N] pairs of fp32 (delta, z) (8 bytes each).
 * awq_lowbit_gemv: Y [M, N] fp32 = Xs W'^T, Xs [M, K] of x_dtype (the
 *   activations divided by s), W'[n, k] = fp32((c[n,k] - z) * delta) of k's
 *   group: exactly the quantiser's dequantised value, applied as
 *   y = sum_g delta_g * sum_{k in g} x_k (c_k - z_g) with the integer
 *   differences and their products exact and the sums in fp32, added in a fixed
 *   order, so results are reproducible: K is split over workgroups whose
 *   partial sums go to the workspace (awq_lowbit_gemv_workspace_size(x_dtype,
 *   M, N, K) bytes, possibly 0, then the workspace may be NULL) and are added by a
 *   second kernel in split order.  Xs must be 16-byte aligned.  The kernel follows M and x_dtype:
 *   fp32 activations, or 1 to 4 rows, take a vector kernel (the packed weights read once per 8
 *   rows); from 5 fp16 / bf16 rows a matrix-core kernel unpacks every code once per tile of up
 *   to 96 rows; beyond 1024 rows, or from 65 rows once ceil(N/128) * ceil(M/256) >= 200,
 *   awq_lowbit_gemm's kernels run (no workspace used).  All of them sum exact products in
 *   fp32; the vector and small-M kernels multiply each group's sum by its delta once, within
 *   (K + 2) 2^-24 sum_k |x_k w'_k| of the exact y, and awq_lowbit_gemm's kernels stay within
 *   (K + 2 K/group + 2) 2^-24 sum_k |x_k w'_k|; their summation orders differ.  The workspace
 *   size is that of the kernel the dtype and sizes select.
 * ------------------------------------------------------------------------ */
awq_status_t awq_lowbit_repack(const uint32_t* codes, const float* scales, const uint8_t* zeros,
                               int64_t N, int64_t K, int bits, int group,
                               uint32_t* codes_t, void* meta_t, hipStream_t stream);
size_t awq_lowbit_gemv_workspace_size(awq_dtype_t x_dtype, int64_t M, int64_t N, int64_t K);
awq_status_t awq_lowbit_gemv(const void* X, awq_dtype_t x_dtype, int64_t M, int64_t K,
                             const uint32_t* codes_t, const void* meta_t, int64_t N, int bits,
                             int group, float* Y, void* workspace, size_t workspace_bytes,
                             hipStream_t stream);
/* awq_lowbit_gemv_noalloc: awq_lowbit_gemv for callers that cannot allocate
 *   device memory (code under HIP graph capture, tight serving loops,
 *   harnesses that forbid allocation).  Same arguments, kernels, results (bit
 *   for bit) and workspace-free cases as awq_lowbit_gemv; the k-split partial
 *   sums go to a static array of AWQ_LOWBIT_STATIC_SCRATCH_BYTES that the
 *   library keeps on each GPU it runs on until the process ends, instead of a
 *   caller workspace.  The call allocates nothing (no hipMalloc, no library
 *   allocation); the first call on a device looks the array's address up.
 *   Sizes whose partial sums (awq_lowbit_gemv_workspace_size) exceed the
 *   array return AWQ_ERR_UNSUPPORTED before anything is enqueued.  Every call
 *   on one GPU shares that GPU's array: calls that overlap in time on one GPU
 *   (other streams, other host threads) race and must not be issued.  The
 *   array keeps the last call's partial sums; no call depends on its earlier
 *   contents. */
#define AWQ_LOWBIT_STATIC_SCRATCH_BYTES (32u << 20)
awq_status_t awq_lowbit_gemv_noalloc(const void* X, awq_dtype_t x_dtype, int64_t M, int64_t K,
                                     const uint32_t* codes_t, const void* meta_t, int64_t N,
                                     int bits, int group, float* Y, hipStream_t stream);
/* awq_lowbit_gemm: the same layer for many activation rows (prefill, M from
 *   a few tens up): the same Y, the same repacked operands, the same exact
 *   products x (c - z) summed in fp32 on the matrix cores; awq_lowbit_gemv
 *   itself calls it for large fp16 / bf16 inputs, below that its own kernels
 *   are the faster ones.  Each workgroup dequantises a tile of the packed
 *   weights into on-chip memory once and uses it for 256 activation rows; the
 *   dequantised weights never reach device memory.  Two kernels, chosen by
 *   the number of tiles: 256 x 128 output tiles whose group sums are scaled
 *   by delta once per group and output (within (K + 2) 2^-24 sum |x w'| of
 *   the exact y), and, when the layer needs at least about 1.5 times fewer
 *   rounds of the chip's compute units that way, 256 x 256 tiles whose
 *   running sums are kept in units of the current group's delta and rescaled
 *   by the quotient of consecutive non-zero deltas at each group start (within
 *   (K + 2 K/group + 2) 2^-24 sum |x w'|; deltas must be finite, and those of
 *   one output row within a factor 2^100 of each other, or the scaled sums
 *   may overflow).  x_dtype AWQ_F16 or AWQ_BF16 only (AWQ_ERR_UNSUPPORTED
 *   otherwise); Xs 16-byte aligned; M <= 8388480, K <= 4194304; no workspace.
 *   Results are reproducible. */
awq_status_t awq_lowbit_gemm(const void* X, awq_dtype_t x_dtype, int64_t M, int64_t K,
                             const uint32_t* codes_t, const void* meta_t, int64_t N, int bits,
                             int group, float* Y, hipStream_t stream);

/* ------------------------------------------------------------------------ *
 * GPTQ error feedback after the scaling (AWQ + GPTQ).  [P3] section 4: the
 * weights are rounded one column at a time and each column's rounding error
 * is moved onto the columns not yet rounded, weighted by the second-order
 * statistics of real inputs; [P4] GPTQ section: Hessian-guided compensation
 * column by column with a Cholesky factorisation done once; [P2]
 * "Experiment": AWQ's scaling and GPTQ's compensation are complementary.
 *
 * Operates on W' = W diag(s) with inputs X' = X diag(s)^-1 (s [K] fp32
 * device; s = 1 gives plain GPTQ):
 *   H = X'^T X' (fp64); channels with H[j][j] = 0 get H[j][j] = 1 and W'[:, j]
 *   = 0; then damp * mean(diag H) is added to the diagonal (damp >= 0, e.g.
 *   0.01; with damp = 0 and a singular H the result is undefined);
 *   U upper triangular with U^T U = H^-1 (fp64);
 *   for j = 0 .. K-1, every row independently: at the first column of a
 *   group, its step and zero-point come from the group's current values
 *   (fp64 rounded to fp32) exactly as in awq_quantize_pack; the current
 *   value is rounded to fp32 and quantised the same way, q = (c - z) delta;
 *   e = (w_j - q) / U[j][j] and w_k -= e U[j][k] for k > j (fp64).
 * Outputs in awq_quantize_pack's format: codes_out uint32 [N, bits*K/32],
 * scales_out fp32 [N, K/group], zeros_out uint8 [N, K/group] (device).
 * W and X of dtype; K <= 32768.  Workspace: awq_gptq_workspace_size(N, K, T)
 * bytes, 256-byte aligned.  After the call the workspace begins with the
 * factor matrix, fp64 with leading dimension awq_gptq_factor_ld(K) (K rounded
 * up to 128): its upper triangle (column >= row) over the first K rows and
 * columns holds U; the rest is scratch.
 * Arithmetic: H, the factorisation and the error updates run in fp64 (MFMA
 * and FMA), so codes agree with any exact-arithmetic GPTQ except where a
 * current value lies within fp64 rounding of a quantisation boundary.
 * ------------------------------------------------------------------------ */
size_t awq_gptq_workspace_size(int64_t N, int64_t K, int64_t T);
int64_t awq_gptq_factor_ld(int64_t K);
awq_status_t awq_gptq_quantize(const void* W, const void* X, awq_dtype_t dtype, int64_t N,
                               int64_t K, int64_t T, const float* s, int bits, int group,
                               double damp, uint32_t* codes_out, float* scales_out,
                               uint8_t* zeros_out, void* workspace, size_t workspace_bytes,
                               hipStream_t stream);

/* ------------------------------------------------------------------------ *
 * SmoothQuant: 8-bit weights and activations ([P3] section 5: divide every
 * activation channel by a factor and multiply the matching weights by it,
 * s_j = sqrt(max|X_j| / max|W_j|), so both sides have moderate ranges and
 * the product can run in INT8).
 *
 * awq_smooth_scales: absmax_out [2K] fp32 device = max_t |X[t, j]| then
 *   max_i |W[i, j]|; s_out [K] = fp32 sqrt(fp32 division), 1 where either
 *   maximum is 0.  Exact (maxima) and correctly rounded, so bit-identical
 *   to any IEEE evaluation.
 * awq_quantize_rows_int8: A [R, K] (dtype; K a multiple of 64), smoothed per
 *   channel by s [K] (multiply != 0: A * s, as for weights; else A / s, as
 *   for activations; s NULL: no smoothing), then symmetric per row:
 *   step_out[r] = max_k |v[r, k]| / 127 (1 for an all-zero row),
 *   q_out[r, k] = clamp(rint(v / step), -127, 127), int8 row-major [R, K].
 * awq_w8a8_loss: the W8A8 layer's output error: activations quantised per
 *   token (A / s), weights per output channel (W * s) as above, their exact
 *   int32 product rescaled to y = fp32(fp32(fp32(acc) * step_x[t]) *
 *   step_w[n]) (the int8 MFMA GEMM), loss_out [1] fp64 device = mean over T N
 *   outputs of (Y - y)^2 with Y = X W^T from the fp16/bf16 MFMA GEMM (fp32
 *   accumulation).  y_out (device fp32 [T, N], may be NULL) receives y.
 *   fp16/bf16; K a multiple of 64; workspace of awq_w8a8_workspace_size(N, K,
 *   T) bytes, 256-byte aligned.
 * ------------------------------------------------------------------------ */
awq_status_t awq_smooth_scales(const void* X, const void* W, awq_dtype_t dtype, int64_t T,
                               int64_t N, int64_t K, float* absmax_out, float* s_out,
                               hipStream_t stream);
awq_status_t awq_quantize_rows_int8(const void* A, awq_dtype_t dtype, int64_t R, int64_t K,
                                    const float* s, int multiply, int8_t* q_out,
                                    float* step_out, hipStream_t stream);
size_t awq_w8a8_workspace_size(int64_t N, int64_t K, int64_t T);
awq_status_t awq_w8a8_loss(const void* W, const void* X, awq_dtype_t dtype, int64_t N,
                           int64_t K, int64_t T, const float* s, double* loss_out, float* y_out,
                           void* workspace, size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------ *
 * Kernel timing.  While enabled, every kernel the library launches (or, after
 * awq_profile_select(prefix), every kernel whose name starts with prefix) is
 * bracketed by a pair of HIP events on its stream; each event pair adds a few
 * microseconds between launches.  awq_profile_read() synchronises on them and
 * returns, for kernels whose name starts with `prefix` (NULL or "" = all),
 * the launch count and the summed elapsed milliseconds.  Kernel names:
 * awq_act_stats_partial, awq_act_stats_finish, awq_scale_table, awq_tile_rows,
 * awq_fake_quant, awq_gemm_ref_output, awq_gemm_sse, awq_loss_argmin,
 * awq_quantize_pack, awq_keep_mask, awq_lowbit_repack, awq_lowbit_gemv, awq_lowbit_gemm,
 * awq_lowbit_reduce.  GPTQ is timed by phase, one event pair around all the
 * launches of each: awq_gptq_hessian, awq_gptq_prep, awq_gptq_cholesky,
 * awq_gptq_inverse, awq_gptq_columns, awq_gptq_pack.  SmoothQuant: awq_smooth_scales,
 * awq_quant_rows_int8, awq_gemm_w8a8_sse (the INT8 GEMM with the squared-error
 * epilogue), awq_gemm_w8a8_store (the INT8 GEMM writing y).
 * awq_profile_reset() drops the records.  Thread-safe.
 * ------------------------------------------------------------------------ */
awq_status_t awq_profile_enable(int enable);
awq_status_t awq_profile_select(const char* prefix);
awq_status_t awq_profile_read(const char* prefix, int64_t* launches, double* total_ms);
awq_status_t awq_profile_reset(void);

#ifdef __cplusplus
}
#endif
#endif /* AWQ_MI355X_AWQ_H */
