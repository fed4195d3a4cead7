/*
 * awq.h - C ABI of the MI355X (gfx950) AWQ activation-aware scale search and INT4
 * group quantization library (libawq_mi355x.so).
 *
 * The method, as the pages define it:
 *   act_mean[c] = mean over tokens i of |X[i,c]|
 *       (bjdmk.com.cn AWQ article, section "显著权重的识别", the S_X equation;
 *        msModelSlim "AWQ：激活感知权重量化算法说明", 原理 / 算法公式).
 *   for k = 0 .. n_grid-1, r = k / n_grid:  s = max(act_mean^r, 1e-4);  s /= sqrt(max(s)*min(s))
 *       (msModelSlim 算法公式; the grid covers [0, 1) in steps of 1/n_grid).
 *   W is scaled by s per input channel, quantized to asymmetric INT4 in groups of 128
 *   consecutive input channels of a row: step = max((max-min)/15, 1e-8),
 *   zero = round(-min/step), q = clamp(round(y/step) + zero, 0, 15), dequantized as
 *   (q - zero)*step and divided by s again
 *       (gsyq.cn "AWQ 离群激活平滑实操：逐通道等价缩放与 4-bit 精度无损转换", section 二,
 *        pseudo_quantize_int4 and search_smooth_scaling_factors).
 *   Each ratio is scored by mean((X W^T - X What^T)^2) (gsyq section 二; bjdmk L(s)),
 *   the first strict minimum is chosen (gsyq section 二, best_loss / best_scale = ones),
 *   and W*s* is exported as packed INT4 codes with per-group steps and zero points
 *   (qqiyuan.cn "基于awq 4-bit量化技术的大模型推理优化实战", group_quantize;
 *    bjdmk section "GPU 硬件级反量化算子内联融合": two 4-bit values per uint8).
 *
 * Conventions shared by every entry point
 *   - Every tensor argument is DEVICE memory owned by the caller; the library never
 *     allocates, frees or keeps a pointer after the call returns. Host-side arrays are
 *     marked "host" (the list of weight-part pointers and their row counts).
 *   - Matrices are row-major. X is [n_tokens, d_in] with row pitch ld_x elements
 *     (ld_x >= d_in, ld_x a multiple of 8). W is [d_out, d_in], contiguous; a fused set
 *     of linears that share the input (q/k/v, gate/up) is passed as up to
 *     AWQ_MAX_PARTS parts whose rows are stacked in order (total rows d_out), and every
 *     per-row output follows that stacked order.
 *   - dtype selects the storage type of X, W and the delta buffer: AWQ_DTYPE_BF16
 *     (uint16 bfloat16 bit patterns) or AWQ_DTYPE_F32. Statistics, scales and losses
 *     are float64; exported steps are float32, zero points int32, codes uint8.
 *   - Device pointers must be 16-byte aligned (256-byte for workspaces).
 *   - stream is a hipStream_t (NULL = the default stream). Calls only enqueue work and
 *     return without synchronising; results are ready when the stream reaches them.
 *   - Argument errors are detected on the host before anything is enqueued; the call
 *     then returns a non-zero awq_status and enqueues nothing. AWQ_ERR_HIP reports a
 *     failed HIP runtime call or kernel launch. awq_last_error() gives the detail for
 *     the calling thread. No entry point aborts the process.
 *   - Inputs are never modified. Calls that share a workspace must not overlap.
 *   - group_size must be 128 (the only group the GPU kernels implement).
 */
#ifndef AWQ_MI355X_H
#define AWQ_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(__GNUC__)
#define AWQ_API __attribute__((visibility("default")))
#else
#define AWQ_API
#endif

#define AWQ_ABI_VERSION 5
#define AWQ_MAX_PARTS 8
#define AWQ_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20) /* device scratch of awq_search_scales_noalloc */
#define AWQ_GROUP_SIZE 128
#define AWQ_MAX_RATIOS 64

typedef enum {
  AWQ_OK = 0,
  AWQ_ERR_NULL = 1,        /* a required pointer is NULL */
  AWQ_ERR_SHAPE = 2,       /* a size is negative or zero where it must be positive, sizes
                              disagree, or d_in is not a multiple of group_size */
  AWQ_ERR_NO_TOKENS = 3,   /* n_tokens == 0: there is no activation mean to search with
                              (msModelSlim FAQ, "No activation mean for target module") */
  AWQ_ERR_ARG = 4,         /* n_grid < 1, bad candidate range, ld_x < d_in, too many parts */
  AWQ_ERR_UNSUPPORTED = 5, /* unknown dtype, group_size != 128, misaligned pointer or pitch,
                              or a size beyond the kernels' 32-bit tile offsets (256 rows of
                              ld_x or d_in elements must span at most 2^31 - 1 bytes) */
  AWQ_ERR_WORKSPACE = 6,   /* workspace missing or smaller than the matching query returns */
  AWQ_ERR_HIP = 7          /* a HIP runtime call or kernel launch failed */
} awq_status;

typedef enum {
  AWQ_DTYPE_F32 = 0,
  AWQ_DTYPE_BF16 = 1,
  AWQ_DTYPE_F16 = 2 /* float16 (uint16 bit patterns): activations of awq_w4a16_gemm only */
} awq_dtype;

/* Candidate-scale formulas (awq_candidate_scales_ex), a = act_mean, r = a ratio of the list. */
typedef enum {
  AWQ_FORMULA_MSMODELSLIM = 0, /* max(a^r, 1e-4) / sqrt(max * min)            (msModelSlim 算法公式) */
  AWQ_FORMULA_RMS = 1,         /* v = max(a, 1e-5)^r; max(v / sqrt(mean(v^2)), 1e-4)   (gsyq 二) */
  AWQ_FORMULA_DUO = 2          /* v = max(a^r / (wm^(1-r) + 1e-6), 1e-4); v / sqrt(max * min),
                                  wm = mean over output rows of |W|  (bjdmk AWQChannelScaler) */
} awq_formula;

/* Weight quantizers of the delta step (awq_quant_delta_ex). */
typedef enum {
  AWQ_QUANT_INT4_GROUP = 0,   /* asymmetric INT4, groups of 128 (the main quantizer, gsyq 二) */
  AWQ_QUANT_INT4_ROW = 1,     /* per row: step = (max - min)/15, restored round(y/(step+1e-6))*step,
                                 no zero point, no clamp (bjdmk AWQChannelScaler) */
  AWQ_QUANT_INT8_ROW_SYM = 2  /* per row: step = max(max|y|/127, 1e-8),
                                 restored clip(round(y/step), -127, 127)*step
                                 (msModelSlim weight_qconfig: per-channel int8 symmetric min-max) */
} awq_quantizer;

/* Flag bits of best_info[1] (written on the device by awq_loss_argmin / awq_search_scales). */
#define AWQ_INFO_ALL_NONFINITE 1 /* no loss was below +inf: k* = 0 and best_scales are all 1 */

/* ------------------------------------------------------------------ library */

/* Returns AWQ_ABI_VERSION of the built library. */
AWQ_API int awq_abi_version(void);

/* Static, human-readable name of a status code. Never NULL. */
AWQ_API const char* awq_status_string(int status);

/* Detail of the last non-OK status returned on the calling thread ("" if none). The string
 * stays valid until the next call into the library on this thread. */
AWQ_API const char* awq_last_error(void);

/* ------------------------------------------------------------------ a1: activation statistic */

/* Workspace bytes awq_act_stats needs for this shape (0 on invalid sizes). */
AWQ_API size_t awq_act_stats_workspace_bytes(int dtype, int64_t n_tokens, int64_t d_in);

/* act_mean[c] = (1/n_tokens) * sum_i |X[i,c]|, accumulated in float64 in a fixed order
 * (bjdmk S_X equation; msModelSlim 算法公式, act_mean = mean(abs(act))).
 *   x         device, [n_tokens, ld_x] of dtype.
 *   act_mean  device, float64 [d_in], written.
 *   workspace device, >= awq_act_stats_workspace_bytes(dtype, n_tokens, d_in) bytes.
 * n_tokens == 0 returns AWQ_ERR_NO_TOKENS. NaN/Inf inputs propagate into their channel. */
AWQ_API int awq_act_stats(const void* x, int dtype, int64_t n_tokens, int64_t d_in, int64_t ld_x,
                  double* act_mean, void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------ a2: candidate scales */

/* For k = 0 .. n_grid-1 and r = k/n_grid:
 *   cand_scales[k, c] = max(act_mean[c]^r, 1e-4) / sqrt(max_c(.) * min_c(.))   (float64)
 * (msModelSlim 算法公式, both lines; grid step 1/n_grid over [0, 1)).
 *   act_mean    device, float64 [d_in].
 *   cand_scales device, float64 [n_grid, d_in], written. Row 0 is exactly 1.
 * A NaN in act_mean makes every row with r > 0 NaN, as the formula implies. */
AWQ_API int awq_candidate_scales(const double* act_mean, int64_t d_in, int n_grid, double* cand_scales,
                         void* stream);

/* ------------------------------------------------------------------ a3: quantize -> delta */

/* For each of n_cand candidate scale rows s (float64 [n_cand, d_in], consecutive):
 *   y = W * s (per input channel), asymmetric INT4 group quantization of y (groups of 128
 *   consecutive channels of a row, gsyq section 二), dequantize, divide by s, and write
 *   delta[j, o, c] = What[o, c] - W[o, c]   in dtype (bfloat16 rounds to nearest even).
 * Every quantizer decision (step, zero point, code) equals the float64 definition's; delta is
 * within 1e-5 * step / s of the float64 value before its rounding to dtype (float32 evaluation:
 * 8.6e-6 * step from the residual, plus the two float32 roundings of the unscaling).
 *   w_parts    host array of n_parts device pointers; part p is [part_rows[p], d_in] of dtype.
 *   part_rows  host array of n_parts row counts (d_out = their sum).
 *   cand_scales device, float64 [n_cand, d_in], 16-byte aligned (AWQ_ERR_UNSUPPORTED otherwise).
 *   delta      device, [n_cand, d_out, d_in] of dtype, written. */
AWQ_API int awq_quant_delta(const void* const* w_parts, const int64_t* part_rows, int n_parts, int dtype,
                    int64_t d_in, int group_size, const double* cand_scales, int n_cand,
                    void* delta, void* stream);

/* ------------------------------------------------------------------ a4: error GEMM + SSE */

/* Number of 256x256 output tiles per candidate: ceil(n_tokens/256) * ceil(d_out/256). */
AWQ_API int64_t awq_error_tiles(int64_t n_tokens, int64_t d_out);

/* Per-tile sums of squares of E_j = X * delta_j^T, the output error of candidate j, which by
 * linearity equals X W^T - X What_j^T (gsyq section 二 target_out - actual_out; bjdmk L(s)).
 * E_j is never written out: each 256x256 tile of it is squared and summed in the GEMM's
 * epilogue. Products are exact bf16 (or f32) matrix-core products with float32
 * accumulation; tile sums are float64.
 *   x        device, [n_tokens, ld_x] of dtype.
 *   delta    device, [n_cand, d_out, d_in] of dtype (as written by awq_quant_delta).
 *   tile_sse device, float64 [n_cand, awq_error_tiles(n_tokens, d_out)], written; within a
 *            candidate the tiles are ordered token-tile major, row-tile minor. */
AWQ_API int awq_error_sse(const void* x, int64_t ld_x, const void* delta, int dtype, int64_t n_tokens,
                  int64_t d_in, int64_t d_out, int n_cand, double* tile_sse, void* stream);

/* ------------------------------------------------------------------ a4 in the Gram form */

/* The same losses through the Gram matrix of the activations. By linearity the loss of a ratio is
 * sum_o ||X delta[o]^T||^2 / (N d_out) (gsyq section 二 target_out - actual_out; bjdmk L(s)), and
 * ||X v||^2 = v G v^T with G = X^T X: with G formed once, and G's symmetry leaving only its
 * 256-blocks on and above the diagonal to multiply, each ratio costs about d_out d_in (d_in + 256)
 * flops instead of 2 N d_in d_out, about half when tokens and input channels are as many. G is
 * accumulated in float32 by the matrix cores from the bfloat16 activations; both operands of the
 * quadratic form are float16, each scaled by a power of two into float16's range (exact, removed
 * exactly from the float64 tile sums). awq_search_scales uses this form by itself where it pays
 * (awq_search_loss_form). */
typedef enum { AWQ_LOSS_DIRECT = 0, AWQ_LOSS_GRAM = 1 } awq_loss_form;

/* The loss form awq_search_scales (and awq_search_scales_ex, with any quantizer) uses for
 * these sizes: AWQ_LOSS_GRAM for bfloat16 activations with n_tokens >= d_in when G's upper tiles
 * plus the n_grid quadratic forms, d_in (d_in + 256) (n_pad + n_grid d_out) flops with n_pad =
 * ceil(n_tokens / 64) * 64, take under 0.85 of the direct products' 2 n_tokens d_in d_out n_grid
 * (and 256 * n_pad * 2 < 2^31), else AWQ_LOSS_DIRECT. Host-only. */
AWQ_API int awq_search_loss_form(int dtype, int64_t n_tokens, int64_t d_in, int64_t d_out, int n_grid);

/* Workspace bytes of awq_gram: X^T padded to a multiple of 64 tokens (bfloat16) and G in float32.
 * 0 on invalid sizes. */
AWQ_API size_t awq_gram_workspace_bytes(int64_t n_tokens, int64_t d_in);

/* G = X^T X for bfloat16 activations, written as float16(G * 2^gram_exp[0]); gram_exp[0] is chosen
 * so that G's largest entry (on its diagonal) scales to at most 2^14. The 256 x 256 blocks on the
 * diagonal (rows and columns 256 I .. 256 I + 255) hold those float16 values times 1/2 (a float16
 * product: exact but for values below float16's normal range, under 2^-26 of G's largest entry), the
 * form awq_gram_error_sse takes.
 *   x          device, bfloat16 [n_tokens, ld_x] (the rules of awq_act_stats).
 *   gram       device, float16 bits [d_in, d_in], 16-byte aligned, written.
 *   gram_exp   device, int32 [1], written.
 *   workspace  device, >= awq_gram_workspace_bytes(n_tokens, d_in) bytes, 256-byte aligned.
 * AWQ_ERR_UNSUPPORTED when 256 rows of the padded X^T exceed 32-bit byte offsets. */
AWQ_API int awq_gram(const void* x, int64_t ld_x, int64_t n_tokens, int64_t d_in, uint16_t* gram,
                     int32_t* gram_exp, void* workspace, size_t workspace_bytes, void* stream);

/* awq_quant_delta for bfloat16 weights with delta written as float16(delta * 2^delta_exp[k]). Every
 * quantizer decision is awq_quant_delta's. delta_exp[k] makes a proven bound on |delta_k|,
 * (1.5 max|W| max(s_k) + 1e-8) / min(s_k) + max|W|, scale to at most 2^14.
 *   delta      device, float16 bits [n_cand, d_out, d_in], 16-byte aligned, written.
 *   delta_exp  device, int32 [n_cand + 1], written (the last entry is scratch: max|W|).
 *   the other arguments as awq_quant_delta (dtype bfloat16). */
AWQ_API int awq_quant_delta_f16(const void* const* w_parts, const int64_t* part_rows, int n_parts, int64_t d_in,
                                int group_size, const double* cand_scales, int n_cand, uint16_t* delta,
                                int32_t* delta_exp, void* stream);

/* Per-tile shares of candidate j's sum_o delta_j[o] G delta_j[o]^T (float16 operands, float32
 * accumulation, float64 tile sums, the scales removed), laid out as awq_error_sse's tile_sse so
 * that awq_loss_argmin gives the losses: candidate j's ceil(d_in/256) * ceil(d_out/256) tile sums
 * then zeros, awq_error_tiles(n_tokens, d_out) entries per candidate (n_tokens >= d_in, else
 * AWQ_ERR_SHAPE). Tile (I, t) holds, over output rows t, delta_I G_II delta_I^T + 2 sum_{J>I}
 * delta_I G_IJ delta_J^T for the 256-blocks I, J of d_in: only G's blocks on and above the diagonal
 * are read. G's diagonal blocks enter halved, as awq_gram stores them, and the tile's sum doubled.
 *   gram, gram_exp    as written by awq_gram.
 *   delta, delta_exp  as written by awq_quant_delta_f16.
 *   tile_sse          device, float64 [n_cand, awq_error_tiles(n_tokens, d_out)], written. */
AWQ_API int awq_gram_error_sse(const uint16_t* gram, const int32_t* gram_exp, const uint16_t* delta,
                               const int32_t* delta_exp, int n_cand, int64_t n_tokens, int64_t d_in,
                               int64_t d_out, double* tile_sse, void* stream);

/* ------------------------------------------------------------------ a5: losses and argmin */

/* losses[k] = (sum of tile_sse[k, :], float64, fixed order) / (n_tokens * d_out): the output
 * MSE of ratio k. k* = the first k with the smallest loss among losses below +inf (a strict
 * "<" scan starting from +inf), or 0 when there is none (gsyq section 二).
 *   tile_sse    device, float64 [n_grid, tiles_per_cand].
 *   cand_scales device, float64 [n_grid, d_in].
 *   losses      device, float64 [n_grid], written.
 *   best_scales device, float64 [d_in], written with cand_scales[k*, :], or with ones when no
 *               loss is below +inf (the search's starting scales).
 *   best_info   device, int32 [2], written: {k*, flags (AWQ_INFO_*)}. */
AWQ_API int awq_loss_argmin(const double* tile_sse, int64_t tiles_per_cand, int n_grid, int64_t n_tokens,
                    int64_t d_out, const double* cand_scales, int64_t d_in, double* losses,
                    double* best_scales, int32_t* best_info, void* stream);

/* ------------------------------------------------------------------ a2..a5 composed */

/* Workspace bytes awq_search_scales needs when it evaluates cand_per_pass candidates per
 * GEMM launch (1 <= cand_per_pass <= n_grid; larger passes fill the GPU better and need a
 * delta buffer of cand_per_pass * d_out * d_in elements), including the Gram form's buffers
 * (float16 G, X^T and float32 G) when awq_search_loss_form chooses it. 0 on invalid sizes. */
AWQ_API size_t awq_search_workspace_bytes(int dtype, int64_t n_tokens, int64_t d_in, int64_t d_out,
                                  int group_size, int n_grid, int cand_per_pass);

/* The whole grid search for one layer (or fused set): a2, then a3 + a4 for every pass of
 * cand_per_pass candidates, then a5 (msModelSlim 缩放因子搜索流程, in that order). a4 is the
 * direct error GEMM or the Gram form, as awq_search_loss_form says for these sizes.
 *   x, ld_x, w_parts, part_rows, n_parts, dtype: as above.
 *   act_mean    device, float64 [d_in] (from awq_act_stats).
 *   cand_scales device, float64 [n_grid, d_in], 16-byte aligned, written (all candidates).
 *   losses, best_scales, best_info: as awq_loss_argmin.
 *   workspace   device, >= awq_search_workspace_bytes(...) bytes. */
AWQ_API int awq_search_scales(const void* x, int64_t ld_x, const void* const* w_parts,
                      const int64_t* part_rows, int n_parts, int dtype, int64_t n_tokens,
                      int64_t d_in, const double* act_mean, int group_size, int n_grid,
                      int cand_per_pass, double* cand_scales, double* losses,
                      double* best_scales, int32_t* best_info, void* workspace,
                      size_t workspace_bytes, void* stream);

/* The same search for callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): no workspace argument and no allocation.
 * Its temporaries live in a fixed device scratch of AWQ_NOALLOC_SCRATCH_BYTES (64 MiB) inside the
 * library, one per GPU, held from the first use on that GPU until the process ends: the tile sums
 * of all candidates, then the delta of one candidate for a chunk of whole 256-row tiles of the
 * stacked rows (all rows when they fit), chunk after chunk. Slower than awq_search_scales with a
 * full workspace (one quantize->delta and one error-GEMM launch per candidate and chunk). Calls that
 * overlap on one GPU (on any streams) share the scratch and race; serialise them.
 *   Arguments as awq_search_scales, without cand_per_pass and the workspace.
 *   AWQ_ERR_WORKSPACE when n_grid * awq_error_tiles(n_tokens, d_out) float64 sums and 256 rows of
 *   delta (d_in * element size bytes each; fewer when d_out is smaller) do not fit the scratch. */
AWQ_API int awq_search_scales_noalloc(const void* x, int64_t ld_x, const void* const* w_parts,
                                      const int64_t* part_rows, int n_parts, int dtype, int64_t n_tokens,
                                      int64_t d_in, const double* act_mean, int group_size, int n_grid,
                                      double* cand_scales, double* losses, double* best_scales,
                                      int32_t* best_info, void* stream);

/* ------------------------------------------------------------------ a6: final quantize + pack */

/* Quantize y = W * s with the same quantizer and emit, per row o and group j:
 *   codes[o, c/2]  = q[o, c] | (q[o, c+1] << 4) for even c (uint8, [d_out, d_in/2]),
 *   qscales[o, j]  = step (float32, [d_out, d_in/128]; within 1e-6 relative of the float64
 *                    step),
 *   zeros[o, j]    = zero point (int32, [d_out, d_in/128]; not clamped to [0,15],
 *                    saturated to the int32 range),
 * so that W*s ~= (q - zero) * step. s is usually best_scales from the search; the caller
 * divides the layer input by s (folds diag(s)^-1 into the previous op, gsyq section 四).
 *   s  device, float64 [d_in], 16-byte aligned (AWQ_ERR_UNSUPPORTED otherwise). */
AWQ_API int awq_quantize_pack(const void* const* w_parts, const int64_t* part_rows, int n_parts, int dtype,
                      int64_t d_in, int group_size, const double* s, uint8_t* codes,
                      float* qscales, int32_t* zeros, void* stream);

/* ------------------------------------------------------------------ around the search */

/* The statistic over several calibration batches (msModelSlim 预处理阶段: hooks gather the
 * per-channel mean of |activation| while the batches run): sums[c] += sum_i |X[i,c]| over this
 * batch's rows, float64 in a fixed order. The caller zeroes sums before the first batch and keeps
 * the total token count for awq_act_stats_finalize.
 *   x, dtype, n_tokens, d_in, ld_x, workspace: as awq_act_stats.
 *   sums   device, float64 [d_in], read and written. */
AWQ_API int awq_act_stats_accumulate(const void* x, int dtype, int64_t n_tokens, int64_t d_in, int64_t ld_x,
                             double* sums, void* workspace, size_t workspace_bytes, void* stream);

/* act_mean[c] = sums[c] / total_tokens (float64). total_tokens == 0 returns AWQ_ERR_NO_TOKENS.
 * sums and act_mean may be the same buffer. */
AWQ_API int awq_act_stats_finalize(const double* sums, int64_t d_in, int64_t total_tokens, double* act_mean,
                           void* stream);

/* Source-side fold of the inverse scales (msModelSlim 支持的子图类型: after the search the norm
 * of norm-linear, linear1 of linear-linear, v_proj of ov and up_proj of up-down get the inverse
 * scaling; gsyq section 四): for the rows r of the source operator that produce input channel r
 * of the searched linears,
 *   dst[r, j] = src[r, j] / s[r]   (quotient in float64, rounded to float32, then to dtype,
 *                                   nearest even at each step)
 * — a norm weight or a bias is one column, a source linear's weight is [d_in, cols].
 *   src, dst  device, [rows, ld_src] / [rows, ld_dst] of dtype; dst may equal src (in place).
 *   s         device, float64 [rows] (usually best_scales). */
AWQ_API int awq_fold_scales(const void* src, int64_t ld_src, int dtype, int64_t rows, int64_t cols,
                    const double* s, void* dst, int64_t ld_dst, void* stream);

/* Output-value subgraph with grouped KV heads (msModelSlim 支持的子图类型, OVSubgraph: MHA, MQA and
 * GQA; o_proj gets the forward scaling, v_proj the inverse). o_proj input channel h * head_dim + d
 * is the attention output of query head h, which mixes the value rows of KV head h / g
 * (g = n_heads / n_kv_heads; consecutive query heads share a KV head). Dividing v_proj row
 * kv * head_dim + d by one scale therefore reaches the g channels (kv * g + j) * head_dim + d,
 * j < g, and the o_proj scales must be equal across them. The search runs on a tied statistic:
 *   tied[(kv * g + j) * head_dim + d] = (sum over j' < g, in order, of
 *                                        act_mean[(kv * g + j') * head_dim + d]) / g   (float64)
 * for every j < g. Passed to awq_search_scales as its act_mean, it gives tied candidate scales
 * (the formula is per channel, and the normaliser's max and min are unchanged by repeating values).
 *   act_mean, tied  device, float64 [n_heads * head_dim]; tied may equal act_mean.
 * n_heads must be a positive multiple of n_kv_heads (AWQ_ERR_SHAPE); MHA (n_kv_heads == n_heads)
 * copies act_mean. */
AWQ_API int awq_tie_heads(const double* act_mean, int64_t n_heads, int64_t n_kv_heads, int64_t head_dim,
                          double* tied, void* stream);

/* The v_proj side of the same fold: s_kv[kv * head_dim + d] = s[(kv * g) * head_dim + d], the tied
 * o_proj scale of the group's first query head (all g are equal after awq_tie_heads); then
 * awq_fold_scales(v_proj weight [n_kv_heads * head_dim, d_model] (and its bias), s_kv) divides each
 * v_proj row by its scale.
 *   s     device, float64 [n_heads * head_dim] (usually best_scales of the tied search).
 *   s_kv  device, float64 [n_kv_heads * head_dim], written. */
AWQ_API int awq_head_group_scales(const double* s, int64_t n_heads, int64_t n_kv_heads, int64_t head_dim,
                                  double* s_kv, void* stream);

/* Deployment form of an export from awq_quantize_pack (bjdmk "GPU 硬件级反量化算子内联融合":
 * FP16 per-group scales, 4-bit values two per byte), for [rows, n_groups] qscales / zeros:
 *   steps_f16[o, j]  = qscales[o, j] rounded to float16 (nearest even), as uint16 bits;
 *   zeros_u4[o, j/2] = zero points clipped to [0, 15], even j in the low nibble
 *                      (uint8, [rows, ceil(n_groups / 2)]);
 *   counts[0]       += zero points outside [0, 15] (only one-signed groups have them; the packed
 *                      form cannot hold them, the int32 zero points stay exact),
 *   counts[1]       += steps whose float16 value is not a normal number (zero, subnormal,
 *                      infinite or NaN).
 *   counts  device, int32 [2], accumulated (the caller zeroes it). */
AWQ_API int awq_export_fp16(const float* qscales, const int32_t* zeros, int64_t rows, int64_t n_groups,
                    uint16_t* steps_f16, uint8_t* zeros_u4, int32_t* counts, void* stream);

/* ------------------------------------------------------------------ grid and quantizer variants */

/* wm[c] = (1/d_out) * sum_o |W[o, c]| over the stacked rows of the parts, float64 in a fixed order
 * (bjdmk AWQChannelScaler, weight_mean = mean of |weight| over the output dimension): the
 * second statistic of AWQ_FORMULA_DUO.
 *   w_parts, part_rows, n_parts, dtype, d_in: as awq_quant_delta.
 *   w_mean    device, float64 [d_in], written.
 *   workspace device, >= awq_act_stats_workspace_bytes(dtype, max_p part_rows[p], d_in) bytes. */
AWQ_API int awq_weight_mean(const void* const* w_parts, const int64_t* part_rows, int n_parts, int dtype,
                    int64_t d_in, double* w_mean, void* workspace, size_t workspace_bytes, void* stream);

/* cand_scales[k, :] = the formula's scales at ratio ratios[k], k = 0 .. n_ratios-1 (float64).
 *   act_mean  device, float64 [d_in].
 *   w_mean    device, float64 [d_in] (from awq_weight_mean); read only by AWQ_FORMULA_DUO, may be
 *             NULL otherwise.
 *   ratios    HOST, float64 [n_ratios], each in [0, 1]; 1 <= n_ratios <= AWQ_MAX_RATIOS. The
 *             pages' grids: k/n for k < n (msModelSlim), k/(n-1) for k < n (bjdmk linspace),
 *             0.0, 0.1, ..., 1.0 (gsyq).
 *   cand_scales device, float64 [n_ratios, d_in], written.
 * NaN in a statistic makes the rows that depend on it NaN, as the formulas imply. */
AWQ_API int awq_candidate_scales_ex(const double* act_mean, const double* w_mean, int64_t d_in,
                            const double* ratios, int n_ratios, int formula, double* cand_scales,
                            void* stream);

/* awq_quant_delta with a choice of quantizer (awq_quantizer). AWQ_QUANT_INT4_GROUP is exactly
 * awq_quant_delta. The per-row quantizers take every rounding decision as the float64
 * definition does and write delta = restored / s - W rounded from float64 to float32 (then to
 * bfloat16 for AWQ_DTYPE_BF16), nearest even. Weights must be finite. d_in a multiple of 128. */
AWQ_API int awq_quant_delta_ex(const void* const* w_parts, const int64_t* part_rows, int n_parts, int dtype,
                       int64_t d_in, int quantizer, const double* cand_scales, int n_cand, void* delta,
                       void* stream);

/* awq_search_scales over an explicit ratio list with a scale formula and a quantizer:
 * awq_candidate_scales_ex, then awq_quant_delta_ex + the error GEMM per pass of cand_per_pass
 * candidates, then awq_loss_argmin (k* indexes the list). Where awq_search_loss_form says so, the
 * loss takes the Gram form as in awq_search_scales, each quantizer's delta written in float16 with
 * a power-of-two scale from a proven bound on |delta| (the symmetric INT8 quantizer's step floor
 * widens that bound by 1.27e-6 / min(s_k)).
 *   w_mean     device, float64 [d_in]; read only by AWQ_FORMULA_DUO, may be NULL otherwise.
 *   ratios, n_ratios, formula: as awq_candidate_scales_ex.  quantizer: as awq_quant_delta_ex.
 *   workspace  device, >= awq_search_workspace_bytes(dtype, n_tokens, d_in, d_out, 128, n_ratios,
 *              cand_per_pass) bytes.
 *   the other arguments as awq_search_scales. */
AWQ_API int awq_search_scales_ex(const void* x, int64_t ld_x, const void* const* w_parts,
                         const int64_t* part_rows, int n_parts, int dtype, int64_t n_tokens,
                         int64_t d_in, const double* act_mean, const double* w_mean,
                         const double* ratios, int n_ratios, int formula, int quantizer,
                         int cand_per_pass, double* cand_scales, double* losses, double* best_scales,
                         int32_t* best_info, void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------ the export's consumer */

/* Y = X * W_hat^T with W_hat dequantized on the fly from the deployment form written by
 * awq_quantize_pack + awq_export_fp16 (bjdmk "GPU 硬件级反量化算子内联融合": packed 4-bit weights
 * unpacked and scaled per group in registers and fed to the matrix units with 16-bit activations;
 * the 16-bit weights are never written to memory). For input c of output row o, in group
 * g = c / 128:
 *   W_hat[o, c] = (q[o, c] - zero[o, g]) * step[o, g]   (qqiyuan dequantize),
 * exact in float32 and rounded once, to nearest even, to the activations' type; products are
 * accumulated in float32. X is usually the layer input divided by the searched scales (the fold of
 * gsyq section 四), so that Y approximates X_orig * W^T.
 *   x         device, [n_tokens, ld_x] of x_dtype (AWQ_DTYPE_BF16 or AWQ_DTYPE_F16); ld_x >= d_in,
 *             ld_x a multiple of 8.
 *   codes     device, uint8 [d_out, d_in / 2] (element 2j in the low 4 bits of byte j), 16-byte
 *             aligned.
 *   steps_f16 device, uint16 [d_out, d_in / 128], float16 bit patterns.
 *   zeros_u4  device, uint8 [d_out, ceil(d_in / 256)], groups 2i / 2i+1 in the low / high 4 bits.
 *   y         device, [n_tokens, ld_y] of y_dtype (AWQ_DTYPE_F32, or x_dtype: rounded to nearest
 *             even), ld_y >= d_out; written.
 * d_in must be a multiple of 128. n_tokens == 0 returns AWQ_ERR_NO_TOKENS. One token (d_in up to
 * 32768) uses a kernel whose waves stream whole weight rows; up to 32 tokens one that streams the
 * weights once per 16 tokens; more use kernels that stage activations in LDS (16 output rows per
 * wave up to 512 tokens, 64 up to 1023, 256 x 256 tiles from 1024); the order of the float32
 * additions differs between these kernels. */
AWQ_API int awq_w4a16_gemm(const void* x, int64_t ld_x, int x_dtype, const uint8_t* codes,
                   const uint16_t* steps_f16, const uint8_t* zeros_u4, int64_t n_tokens, int64_t d_in,
                   int64_t d_out, void* y, int64_t ld_y, int y_dtype, void* stream);

/* ------------------------------------------------------------------ block-level objective */

/* Activations of the gated MLP block (awq_search_scales_mlp). */
typedef enum { AWQ_ACT_SILU = 0, AWQ_ACT_RELU = 1 } awq_act;

/* The gated MLP's gate and up outputs with the original weights (the float reference of the
 * block, msModelSlim 缩放因子搜索流程):
 *   g_ref = X * w_gate^T, u_ref = X * w_up^T   (float32 [n_tokens, d_ff], row pitch d_ff; written)
 *   x       device, bfloat16 [n_tokens, ld_x] (ld_x >= d_in, a multiple of 8).
 *   w_gate, w_up  device, bfloat16 [d_ff, d_in].
 * d_in and d_ff multiples of 128. */
AWQ_API int awq_mlp_hidden_ref(const void* x, int64_t ld_x, const void* w_gate, const void* w_up, int64_t n_tokens,
                       int64_t d_in, int64_t d_ff, float* g_ref, float* u_ref, void* stream);

/* The change of the MLP's hidden activations when gate and up are replaced by their quantized
 * versions W + dW (dW as awq_quant_delta writes it):
 *   dh = act(g_ref) * u_ref - act(g_ref + X dw_gate^T) * (u_ref + X dw_up^T)
 * float32 arithmetic, rounded to bfloat16 [n_tokens, d_ff] (row pitch d_ff; written). Since the down
 * projection is linear, the block's output error is dh * w_down^T, whose sum of squares
 * awq_error_sse gives (x = dh, delta = w_down).
 *   act  AWQ_ACT_SILU (v / (1 + e^-v)) or AWQ_ACT_RELU. */
AWQ_API int awq_mlp_hidden_delta(const void* x, int64_t ld_x, const void* dw_gate, const void* dw_up,
                         const float* g_ref, const float* u_ref, int act, int64_t n_tokens, int64_t d_in,
                         int64_t d_ff, void* dh, void* stream);

/* Workspace bytes of awq_search_scales_mlp (0 on invalid sizes). */
AWQ_API size_t awq_search_workspace_bytes_mlp(int64_t n_tokens, int64_t d_in, int64_t d_ff, int64_t d_model,
                                      int n_grid, int cand_per_pass);

/* The search for the gate/up pair of a gated MLP y = down(act(x gate^T) * (x up^T)), scored at the
 * block's output — the lowest common ancestor of the two searched linears (msModelSlim 关键特性,
 * block-level error; 缩放因子搜索流程). For k = 0 .. n_grid-1 the msModelSlim scales s_k are applied
 * to gate and up together (one fused set), both are quantized (INT4, groups of 128) and unscaled,
 * and losses[k] = mean over tokens and d_model outputs of (y_ref - y_k)^2, accumulated as the fixed
 * order sum of per-tile float64 sums of squares of dh_k * w_down^T; k* as awq_loss_argmin.
 *   x          device, bfloat16 [n_tokens, ld_x] (the block's input after the norm).
 *   w_gate, w_up  device, bfloat16 [d_ff, d_in];  w_down  device, bfloat16 [d_model, d_ff].
 *   act_mean   device, float64 [d_in] (awq_act_stats of x).
 *   act        AWQ_ACT_SILU or AWQ_ACT_RELU.
 *   cand_scales, losses, best_scales, best_info: as awq_search_scales.
 *   workspace  device, >= awq_search_workspace_bytes_mlp(...) bytes, 256-byte aligned.
 * d_in and d_ff multiples of 128. */
AWQ_API int awq_search_scales_mlp(const void* x, int64_t ld_x, const void* w_gate, const void* w_up,
                          const void* w_down, int64_t n_tokens, int64_t d_in, int64_t d_ff, int64_t d_model,
                          const double* act_mean, int act, int n_grid, int cand_per_pass, double* cand_scales,
                          double* losses, double* best_scales, int32_t* best_info, void* workspace,
                          size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* AWQ_MI355X_H */
