/*
 * awq.h - C ABI of the AWQ per-linear-layer library for AMD MI355X (gfx950).
 *
 * The library implements, for one linear layer Y = X·W with calibration
 * activations X [N x D_in] and weights W [D_in x D_out], the activation-aware
 * weight quantisation search and the W4A16 inference product described in:
 *   [CA] compassingai, "AWQ (Activation-aware Weight Quantization)"
 *   [MR] mudrobot, "【论文笔记】AWQ" (notes on the MLSys 2024 AWQ paper)
 *   [LQ] laojiahuo2003, "LLM Quantization（大模型量化）：GPTQ、AWQ、SmoothQuant 的核心思路"
 *
 * Conventions shared by every entry point
 *   - Tensors are dense, row-major (C order), caller-owned device memory,
 *     16-byte aligned.  Only `alphas` (awq_search_layer) is a host array.
 *   - Every call is asynchronous on `stream` (a hipStream_t; NULL means the
 *     legacy default stream).  Outputs are valid once the caller has
 *     synchronised that stream.  The library never allocates device memory:
 *     scratch comes from the caller's `workspace`.
 *   - Arguments are validated on the host before any HIP call.  On failure
 *     the function returns a negative awq_status, launches nothing and
 *     leaves every output untouched; awq_last_error() then describes the
 *     problem (thread-local string).  Launch failures return AWQ_ERR_HIP.
 *   - No global mutable device state: calls on different streams may run
 *     concurrently as long as they do not share outputs or workspace.
 */
#ifndef AWQ_MI355X_H
#define AWQ_MI355X_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* The enumerations are int-sized in both languages.  In C++ they take int as
 * their fixed underlying type, so that any int a caller passes (from C, or
 * through a foreign-function layer) is a value of the type and the library
 * can reject it, rather than holding an out-of-range enumeration value. */
#ifdef __cplusplus
#define AWQ_ENUM_INT : int
#else
#define AWQ_ENUM_INT
#endif

typedef enum AWQ_ENUM_INT {
    AWQ_OK = 0,
    AWQ_ERR_ARG = -1,        /* NULL pointer, bad bits/group/alpha, misalignment */
    AWQ_ERR_SHAPE = -2,      /* sizes inconsistent or out of the supported range  */
    AWQ_ERR_DTYPE = -3,      /* unsupported element type                           */
    AWQ_ERR_WORKSPACE = -4,  /* workspace NULL or smaller than required            */
    AWQ_ERR_NONFINITE = -5,  /* awq_search_status: the search met a NaN or Inf     */
    AWQ_ERR_HIP = -6         /* a HIP runtime call or kernel launch failed         */
} awq_status;

typedef enum AWQ_ENUM_INT {
    AWQ_F32 = 0,   /* IEEE binary32                      */
    AWQ_BF16 = 1,  /* bfloat16 (1 sign, 8 exp, 7 frac)   */
    AWQ_F16 = 2    /* IEEE binary16; only for stored steps (awq_w4a16_gemm_ex) */
} awq_dtype;

/* Largest supported alpha-grid length. */
#define AWQ_MAX_ALPHAS 64

/* Thread-local description of the last failure in this thread ("" if none). */
const char *awq_last_error(void);

/* Library version string. */
const char *awq_version(void);

/*
 * awq_act_stats - per-input-channel activation magnitude.
 *   a[j] = mean over n of |X[n, j]|                     [CA] 重要通道識別的統計依據
 * (the mean statistic named by [MR] 搜索最优比例).  Accumulated in float64 and
 * rounded once to float32.
 *   X    device, [N x D_in], element type xt (AWQ_F32 or AWQ_BF16).
 *   a    device, [D_in] float32, written.
 * Requires N >= 1, D_in >= 1.
 */
awq_status awq_act_stats(const void *X, awq_dtype xt, int64_t N, int64_t D_in,
                         float *a, hipStream_t stream);

/* Activation statistics the pages allow as the saliency measure. */
typedef enum AWQ_ENUM_INT {
    AWQ_STAT_MEAN_ABS = 0,   /* mean_n |X[n, j]|  ([CA] 重要通道識別的統計依據; [MR] 搜索最优比例) */
    AWQ_STAT_MAX_ABS = 1     /* max_n |X[n, j]|   ([CA] 重要通道識別的統計依據 "or max";
                                                   [CA] 二、縮放因子的搜尋: s_j = (max|X_j|)^α) */
} awq_statistic;

/*
 * awq_act_stats_ex - awq_act_stats with a choice of statistic.
 *   AWQ_STAT_MEAN_ABS: identical to awq_act_stats.
 *   AWQ_STAT_MAX_ABS:  a[j] = max over n of |X[n, j]|, exact (no rounding);
 *                      a NaN in column j makes a[j] NaN.
 * Arguments and requirements as for awq_act_stats; an unknown `stat` is
 * AWQ_ERR_ARG.
 */
awq_status awq_act_stats_ex(const void *X, awq_dtype xt, int64_t N, int64_t D_in,
                            awq_statistic stat, float *a, hipStream_t stream);

/*
 * awq_weight_stats - per-input-channel weight magnitude.
 *   b[j] = mean over o of |W[j, o]|       [LQ] 4.4 怎么做：不是留 FP16，而是「缩放」
 * (mean|W_j| of the weights input channel j feeds: row j of W as stored
 * here).  Accumulated in float64 and rounded once to float32.
 *   W    device, [D_in x D_out], element type wt (AWQ_F32 or AWQ_BF16).
 *   b    device, [D_in] float32, written.
 * Requires D_in >= 1, D_out >= 1.
 */
awq_status awq_weight_stats(const void *W, awq_dtype wt, int64_t D_in, int64_t D_out,
                            float *b, hipStream_t stream);

/*
 * awq_search_workspace_size - bytes of device workspace with which
 * awq_search_layer (and every awq_search_layer* variant) runs in one pass
 * over the output columns (0 if the arguments are invalid; awq_last_error()
 * says why).  The size grows with n_alpha * D_in * D_out: every candidate's
 * error weights are formed before one loss contraction runs over all
 * candidates at once.  On layers that may take the bf16 matrix path (16-bit
 * path, 2048 <= D_in <= 16384) it also covers that path's 64 correction rows
 * and channel maps, whichever path the size rule or the flags of
 * awq_search_layer_flags then choose.
 */
size_t awq_search_workspace_size(int64_t N, int64_t D_in, int64_t D_out, awq_dtype xt,
                                 int bits, int group, int n_alpha);

/*
 * awq_search_workspace_min_size - the smallest workspace the search accepts
 * (0 if the arguments are invalid).  With a workspace of at least this size
 * but less than awq_search_workspace_size, the search forms the error
 * weights and runs the loss contraction over the output columns in chunks
 * (whole 256-column tiles; as many columns per chunk as the workspace holds),
 * one pair of launches per chunk.  The loss L is a sum over output columns
 * and quantisation groups never cross columns ([CA] 縮放因子最佳化的完整流程
 * step 4; [MR] 搜索最优比例), so every output is identical, bit for bit, to
 * the one-pass result: each tile's partial loss is computed the same way and
 * reduced in the same fixed order.
 */
size_t awq_search_workspace_min_size(int64_t N, int64_t D_in, int64_t D_out, awq_dtype xt,
                                     int bits, int group, int n_alpha);

/*
 * awq_search_layer - the activation-aware scale search for one layer.
 *
 * For each grid value alphas[k] ([CA] 縮放因子最佳化的完整流程; [MR] 搜索最优比例):
 *   s_j      = a_j ^ alpha_k  (float64 pow rounded once to float32; a channel
 *              with a_j == 0 or a_j < FLT_MIN keeps s_j = 1)
 *   W'       = diag(s)·W                     (float32 products)
 *   per group of `group` consecutive input rows of one output column:
 *   step     = max|W'| / (2^(bits-1) - 1)    (IEEE float32 division)
 *   q        = round_half_even(W' / step) clamped to ±(2^(bits-1) - 1);
 *              an all-zero group has step 0 and q 0   [CA] 量化數學基礎
 *   L_k      = || (X·S⁻¹)·(q·step) − X·W ||²   (sum over all N x D_out outputs)
 * then best = the first k with the smallest L_k.
 *
 * Inputs
 *   X        device, [N x D_in], type xt.  AWQ_BF16 inputs with at least
 *            2^16 outputs (N * D_out) run the loss contraction on 16-bit
 *            matrix cores with float32 accumulation: bf16 for 2048 <= D_in
 *            <= 16384 and N * D_in * D_out >= 2^39, where the error weights
 *            of the 64 channels with the largest a_j also carry their bf16
 *            rounding residual as 64 extra contraction rows; fp16 otherwise
 *            (both operands prescaled by exact powers of two).  AWQ_F32
 *            inputs and smaller layers use float32 matrix cores.
 *   W        device, [D_in x D_out], type wt (AWQ_F32 or AWQ_BF16).
 *   a        device, [D_in] float32, e.g. from awq_act_stats.
 *   alphas   HOST, [n_alpha] float32, each in [0, 1]; 1 <= n_alpha <= 64.
 *   bits     2..8.   group: multiple of 8 dividing D_in.
 * Outputs (device)
 *   losses   [n_alpha] float64: L_k.
 *   best     [1] int32: argmin index, or -1 if any loss is not finite (then
 *            s_best/scales/codes are left unwritten; awq_search_status
 *            reports it as AWQ_ERR_NONFINITE once the stream is done).
 *   s_best   [D_in] float32: s at alpha[best].
 *   scales   [D_in/group x D_out] float32: step at alpha[best].
 *   codes    [D_in x D_out] int8: q at alpha[best]; may be NULL.
 * Workspace: device, 256-byte aligned, at least
 * awq_search_workspace_min_size(...) bytes (awq_search_workspace_size(...)
 * for one pass over the columns); its contents on entry are ignored.
 */
awq_status awq_search_layer(const void *X, awq_dtype xt, int64_t N, int64_t D_in,
                            const void *W, awq_dtype wt, int64_t D_out,
                            const float *a, const float *alphas, int n_alpha,
                            int bits, int group,
                            double *losses, int32_t *best, float *s_best,
                            float *scales, int8_t *codes,
                            void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * awq_search_status - the synchronising check of a search's result.
 * Waits for `stream` (the stream the search ran on), reads the search's
 * device `best` word and returns
 *   AWQ_OK             best >= 0: every loss finite, outputs written;
 *   AWQ_ERR_NONFINITE  best == -1: X, W or a loss held a NaN or Inf
 *                      ([CA] 縮放因子最佳化的完整流程 step 5 picks a minimum,
 *                      which a non-finite loss does not have); s_best, scales,
 *                      codes (and zeros) were left unwritten;
 *   AWQ_ERR_HIP        the wait or the read failed (an earlier asynchronous
 *                      failure on the stream is reported here too).
 * The search calls themselves stay asynchronous, so they cannot return
 * AWQ_ERR_NONFINITE; this call is where that status surfaces.
 *   best      device, [1] int32: the `best` output of any awq_search_layer*
 *             call on `stream`.
 *   best_out  HOST, [1] int32, may be NULL: receives the index.
 */
awq_status awq_search_status(const int32_t *best, hipStream_t stream, int32_t *best_out);

/*
 * awq_search_layer_ex - awq_search_layer with phase timing.
 *   Identical arguments and results, plus `events`: NULL, or an array of
 *   n_events == AWQ_SEARCH_EVENTS hipEvent_t handles created by the caller.
 *   They are recorded on `stream` at the phase boundaries:
 *     [0] start; [1] after max|X|, max|W|, the scale tables and the X layout;
 *     [2] after the all-alpha quantiser and error-weight pass;
 *     [3] after the loss contraction (the dominant kernel);
 *   With a workspace below awq_search_workspace_size the error weights and
 *   the contraction alternate per column chunk: [2] is then recorded after
 *   the first chunk's error weights and [3] after the last chunk's
 *   contraction.
 *     [4] after the loss reduction, argmin and final quantisation.
 *   Any other n_events with non-NULL events is AWQ_ERR_ARG.
 */
#define AWQ_SEARCH_EVENTS 5
awq_status awq_search_layer_ex(const void *X, awq_dtype xt, int64_t N, int64_t D_in,
                               const void *W, awq_dtype wt, int64_t D_out,
                               const float *a, const float *alphas, int n_alpha,
                               int bits, int group,
                               double *losses, int32_t *best, float *s_best,
                               float *scales, int8_t *codes,
                               void *workspace, size_t workspace_bytes, hipStream_t stream,
                               hipEvent_t *events, int n_events);

/*
 * awq_search_layer_wscale - awq_search_layer with the weight-term candidate
 * scales of [LQ] 4.4 怎么做：不是留 FP16，而是「缩放」:
 *   s_j = a_j ^ alpha_k / b_j ^ (1 - alpha_k)
 * (both powers and the quotient in float64, 1 - alpha exact, rounded once to
 * float32; a channel with a_j or b_j zero or below FLT_MIN keeps s_j = 1).
 *   b    device, [D_in] float32, non-NULL, e.g. from awq_weight_stats.
 * Every other argument, the quantiser, the loss, the argmin and the outputs
 * are exactly those of awq_search_layer (same workspace size).  At alpha = 1
 * the result equals awq_search_layer's; at alpha = 0, s = 1/b.
 */
awq_status awq_search_layer_wscale(const void *X, awq_dtype xt, int64_t N, int64_t D_in,
                                   const void *W, awq_dtype wt, int64_t D_out,
                                   const float *a, const float *b, const float *alphas,
                                   int n_alpha, int bits, int group,
                                   double *losses, int32_t *best, float *s_best,
                                   float *scales, int8_t *codes,
                                   void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * awq_search_layer_zp - the search with zero-point (asymmetric) codes.
 *                                      [CA] 三、量化方案細節 (symmetric or asymmetric)
 * As awq_search_layer (b may be NULL, or a weight statistic as in
 * awq_search_layer_wscale), with the group quantiser replaced by
 *   lo = min(min W', 0), hi = max(max W', 0)      over the group
 *   step = fl32(fl32(hi − lo) / (2^bits − 1))      (IEEE division)
 *   z    = round_half_even(fl32(−lo / step))       in [0, 2^bits − 1]
 *   q    = clamp(round_half_even(W'/step) + z, 0, 2^bits − 1)
 * and dequantisation (q − z)·step in the loss; an all-zero group has step 0,
 * z 0 and q 0.  Zero is exactly representable.
 *   scales   [D_in/group x D_out] float32: step at alpha[best].
 *   zeros    [D_in/group x D_out] uint8, non-NULL: z at alpha[best].
 *   codes    [D_in x D_out] uint8 (values 0 .. 2^bits − 1); may be NULL.
 * bits 2..8; workspace as for awq_search_layer.
 */
awq_status awq_search_layer_zp(const void *X, awq_dtype xt, int64_t N, int64_t D_in,
                               const void *W, awq_dtype wt, int64_t D_out,
                               const float *a, const float *b, const float *alphas,
                               int n_alpha, int bits, int group,
                               double *losses, int32_t *best, float *s_best,
                               float *scales, uint8_t *zeros, uint8_t *codes,
                               void *workspace, size_t workspace_bytes, hipStream_t stream);

/* Flags of awq_search_layer_flags. */
#define AWQ_SEARCH_ZERO_POINT 1u   /* zero-point codes, as awq_search_layer_zp        */
#define AWQ_SEARCH_FP16_STEPS 2u   /* steps rounded to and stored in FP16            */
#define AWQ_SEARCH_MATRIX_BF16 4u  /* loss contraction on bf16 matrix cores (below)  */
#define AWQ_SEARCH_MATRIX_FP16 8u  /* loss contraction on fp16 matrix cores (below)  */

/*
 * awq_search_layer_flags - the search with any combination of the variants.
 *   b        weight statistic or NULL (awq_search_layer_wscale).
 *   flags    AWQ_SEARCH_ZERO_POINT: as awq_search_layer_zp (zeros non-NULL,
 *            codes uint8).  AWQ_SEARCH_FP16_STEPS ([MR] 通过激活感知缩放保护
 *            显著权重: the scaling factors are kept in FP16): every step is
 *            rounded to the nearest binary16 value (ties to even) before the
 *            codes are taken against it, in the loss and in the outputs, and
 *            `scales` receives FP16 bits (uint16 [D_in/group x D_out]).  The
 *            steps must lie in FP16's range; smaller ones lose precision or
 *            become 0, larger ones overflow.
 *            AWQ_SEARCH_MATRIX_BF16 / AWQ_SEARCH_MATRIX_FP16 (not both): for
 *            a layer on the 16-bit path with 2048 <= D_in <= 16384, run the
 *            loss contraction on bf16 matrix cores with the 64 correction
 *            rows, or on fp16 matrix cores, instead of choosing by the size
 *            rule of awq_search_layer; other layers ignore them.  Codes,
 *            steps and s at a given alpha are the same with either.  The
 *            bf16 losses rely on averaging over the layer's output columns:
 *            on a narrow layer whose activation energy spreads over many
 *            more than 64 strongly correlated channels they can miss the
 *            1e-4 loss tolerance (200 identical x50 channels, 520 columns:
 *            1.5e-4), which the size rule avoids by taking bf16 only from
 *            2^39 multiply-adds per alpha.
 *   scales   float32, or FP16 bits with AWQ_SEARCH_FP16_STEPS.
 *   zeros    uint8, used only with AWQ_SEARCH_ZERO_POINT (else may be NULL).
 *   codes    int8 (uint8 with AWQ_SEARCH_ZERO_POINT); may be NULL.
 * Other arguments, workspace and results as for awq_search_layer; unknown
 * flags are AWQ_ERR_ARG.
 */
awq_status awq_search_layer_flags(const void *X, awq_dtype xt, int64_t N, int64_t D_in,
                                  const void *W, awq_dtype wt, int64_t D_out,
                                  const float *a, const float *b, const float *alphas,
                                  int n_alpha, int bits, int group, unsigned flags,
                                  double *losses, int32_t *best, float *s_best,
                                  void *scales, uint8_t *zeros, void *codes,
                                  void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * awq_clip_workspace_size - bytes of device workspace awq_clip_search needs:
 * the Gram matrices H_g (D_in/group x group x group float32) and their
 * per-chunk partials (ceil(N/256) times that), each rounded up to 256.
 * 0 if the arguments are invalid (awq_last_error() says why).
 */
size_t awq_clip_workspace_size(int64_t N, int64_t D_in, int group);

/*
 * awq_clip_search - per-group weight-clipping search with fixed scales.
 *                                                   [MR] 搜索最优比例 (weight clipping)
 * For every group g (group consecutive input rows) of every output column o
 * and every ratio r_k of the grid:
 *   W'       = diag(s)·W                   (float32 products)
 *   m_r      = fl32(r_k · max|W'_g|),  step = fl32(m_r / (2^(bits-1) - 1))
 *   q        = round_half_even(W' / step) clamped to ±(2^(bits-1) - 1)
 *              (weights beyond the threshold saturate; step 0 gives q 0)
 *   E_k[g,o] = sum_n ( sum_{j in g} X[n, j] · (q_j·step / s_j − W[j, o]) )²
 * (the search loss of [CA] 縮放因子最佳化的完整流程 step 4c restricted to one
 * group), evaluated as dᵀ·(X_gᵀX_g)·d on the matrix cores in float32;
 * ratio_idx[g,o] = the first k with the smallest E_k.  r = 1 is the plain
 * quantiser of awq_search_layer.
 *   X, xt, N, D_in, W, wt, D_out   as for awq_search_layer.
 *   s        device, [D_in] float32: the scales (e.g. s_best of the search).
 *   ratios   HOST, [n_ratio] float32, each in (0, 1]; 1 <= n_ratio <= 64.
 *   bits     2..8.  group: 32, 64, 128 or 256, dividing D_in.
 * Outputs (device)
 *   ratio_idx [D_in/group x D_out] int32.
 *   scales    [D_in/group x D_out] float32: step at the chosen ratio.
 *   codes     [D_in x D_out] int8 at the chosen ratio; may be NULL.
 *   errors    [n_ratio x D_in/group x D_out] float32: E_k; may be NULL.
 * Workspace: device, at least awq_clip_workspace_size(N, D_in, group) bytes,
 * 16-byte aligned; contents on entry are ignored.  Inputs must be finite.
 */
awq_status awq_clip_search(const void *X, awq_dtype xt, int64_t N, int64_t D_in,
                           const void *W, awq_dtype wt, int64_t D_out,
                           const float *s, const float *ratios, int n_ratio, int bits, int group,
                           int32_t *ratio_idx, float *scales, int8_t *codes, float *errors,
                           void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * awq_pack - pack signed codes into 4-bit words.         [MR] SIMD 感知权重打包
 *   word[kw, o] = sum_{i<8} (codes[8·kw + P[i], o] + 8) << (4·i),
 *   P = (0, 2, 4, 6, 1, 3, 5, 7): least-significant nibble first.
 *   codes   device, [D_in x D_out] int8, values in ±(2^(bits-1) - 1).
 *   packed  device, [D_in/8 x D_out] uint32, written.
 * Requires bits in 2..4 and D_in % 8 == 0.  Codes outside the range are
 * packed modulo 16 (not checked on the device).
 */
awq_status awq_pack(const int8_t *codes, int64_t D_in, int64_t D_out, int bits,
                    uint32_t *packed, hipStream_t stream);

/*
 * awq_pack_ex - awq_pack for either code kind.
 *   zero_point_codes == 0: signed codes, nibble = code + 8 (awq_pack).
 *   zero_point_codes != 0: unsigned codes of awq_search_layer_zp (passed as
 *                          the same bytes), nibble = code.
 */
awq_status awq_pack_ex(const int8_t *codes, int64_t D_in, int64_t D_out, int bits,
                       int zero_point_codes, uint32_t *packed, hipStream_t stream);

/*
 * awq_w4a16_workspace_size - bytes of device workspace awq_w4a16_gemm needs.
 * Decode regime (see awq_w4a16_gemm): room for the activations in the
 * product's own layout (M * D_in * 2 bytes, rounded up to 256; formed once
 * per call, scaled by inv_s when given) plus, when the k axis of a pass (of
 * at most 32 rows) is split across workgroups to fill the GPU, one float32
 * partial [splits x rows x D_out] (splits chosen from D_in and D_out; the
 * size covers the largest split over every pass, group size and code kind,
 * so one workspace serves all of them).
 * Prefill regime: the activations as FP16 fragments, rows padded to 256 and
 * k to 64 (ceil(M/256)*256 * ceil(D_in/64)*64 * 2 bytes), one float per
 * output column, 1024 partial maxima and one scalar (each rounded up to 256),
 * and, for grids of fewer than 256 output tiles (k split 2 or 4 ways), a
 * float32 partial [splits x M x D_out]; where at least 256 tiles leave a
 * last round of at most 128, whose last column tiles run split 2 ways along
 * k, a float32 partial [2 x M x those columns] (the larger of the two).
 * has_inv_s is accepted for symmetry; the size does not depend on it.
 */
size_t awq_w4a16_workspace_size(int64_t M, int64_t D_in, int64_t D_out, int has_inv_s);

/*
 * awq_w4a16_gemm - Y = (X·diag(inv_s))·Dequant(packed, scales)
 *                                       [CA] 推論時的等效實現; [MR] 即时权重反量化
 *   X       device, [M x D_in] bfloat16.
 *   packed  device, [D_in/8 x D_out] uint32 (awq_pack layout).
 *   scales  device, [D_in/group x D_out] float32.
 *   inv_s   device, [D_in] float32, or NULL when 1/s has been folded into the
 *           producer of X.  When given, X·inv_s is formed in float32 and
 *           rounded once to bfloat16 before the product.
 *   Y       device, [M x D_out], type yt (AWQ_F32 or AWQ_BF16), written.
 *   workspace  device, >= awq_w4a16_workspace_size(M, D_in, D_out,
 *           inv_s != NULL) bytes, 16-byte aligned; its contents on entry do
 *           not matter.  The k-range partials are summed in a fixed order, so
 *           results are deterministic.
 * Dequant[j, o] = (nibble - 8) · scales[j / group, o].  Two regimes:
 *  - decode (M < 192, or fewer than 64 output tiles of 256 x 256): rows are
 *    processed 32 at a time, the weights re-read once per 32 rows; the
 *    integer codes enter the matrix cores exactly and each group's float32
 *    partial sum is scaled by its step.
 *  - prefill (M >= 192 and at least 64 tiles): [MR] 即时权重反量化, the
 *    codes are dequantised to FP16 in registers, q · fp16(kw_o · step)
 *    rounded once more to FP16 ([MR] 为什么 AWQ 能加速本地设备上的 LLM: this
 *    stage is compute-bound), against kx · bf16(X·inv_s) in FP16 (exact,
 *    except below FP16's normal range); kx and kw_o
 *    are powers of two (from max|X·inv_s| and each column's largest step)
 *    divided out exactly in the float32 result.
 * Requires M >= 1, group = 32 * 2^k, D_in % group == 0, D_out % 4 == 0.
 */
awq_status awq_w4a16_gemm(const void *X, int64_t M, int64_t D_in, int64_t D_out,
                          const uint32_t *packed, const float *scales, int group,
                          const float *inv_s, void *Y, awq_dtype yt,
                          void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * awq_w4a16_gemm_noalloc - awq_w4a16_gemm without a caller workspace, for
 * callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc.
 *   Arguments, results and kernels are those of awq_w4a16_gemm minus
 *   `workspace`/`workspace_bytes`.  The kernels' scratch memory is a static
 *   device array inside the library, awq_w4a16_noalloc_scratch_bytes() bytes
 *   (32 MiB) on each GPU that loads the library, held until the process ends.
 *   A shape whose awq_w4a16_workspace_size(M, D_in, D_out, inv_s != NULL)
 *   exceeds that is rejected with AWQ_ERR_WORKSPACE before anything runs
 *   (every decode shape up to M = 32 at D_in x D_out = 8192 x 28672 fits).
 *   The call allocates nothing.  The first call on a device, with that device
 *   current, looks up the array's device address (AWQ_ERR_HIP if that fails).
 *   Every call on one GPU shares that GPU's array: calls that overlap on one
 *   GPU (several streams or host threads) race and must be serialised by the
 *   caller.  Nothing in the array needs to start at zero.
 */
size_t awq_w4a16_noalloc_scratch_bytes(void);
awq_status awq_w4a16_gemm_noalloc(const void *X, int64_t M, int64_t D_in, int64_t D_out,
                                  const uint32_t *packed, const float *scales, int group,
                                  const float *inv_s, void *Y, awq_dtype yt, hipStream_t stream);

/*
 * awq_w4a16_gemm_zp - awq_w4a16_gemm for zero-point codes.
 *   packed  words of awq_pack_ex(..., zero_point_codes = 1, ...): nibble n = q.
 *   zeros   device, [D_in/group x D_out] uint8, non-NULL, 16-byte aligned.
 * Dequant[j, o] = (n − zeros[j / group, o]) · scales[j / group, o]; every
 * other argument, the workspace size and the two regimes as for
 * awq_w4a16_gemm (with group 32 the decode regime serves every M).
 */
awq_status awq_w4a16_gemm_zp(const void *X, int64_t M, int64_t D_in, int64_t D_out,
                             const uint32_t *packed, const float *scales, const uint8_t *zeros,
                             int group, const float *inv_s, void *Y, awq_dtype yt,
                             void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * awq_w4a16_workspace_size_ex - workspace of awq_w4a16_gemm_ex: that of
 * awq_w4a16_gemm with inv_s; with AWQ_F16 steps in the prefill regime's
 * shapes, that size rounded up to 256 plus one float32 per step (the
 * regime's float32 copy of the steps).  0 if the arguments are invalid.
 */
size_t awq_w4a16_workspace_size_ex(int64_t M, int64_t D_in, int64_t D_out, int group,
                                   awq_dtype scale_type);

/*
 * awq_w4a16_gemm_ex - the product with any step storage and code kind.
 *   scales      device, [D_in/group x D_out], type scale_type: AWQ_F32, or
 *               AWQ_F16 (FP16 bits, e.g. from AWQ_SEARCH_FP16_STEPS; the
 *               decode regime reads them as such, the prefill regime first
 *               widens them to float32 in the workspace; the values are the
 *               same either way, so results equal AWQ_F32 with the widened
 *               steps).
 *   zeros       NULL for signed codes (awq_w4a16_gemm), else as
 *               awq_w4a16_gemm_zp.
 *   workspace   >= awq_w4a16_workspace_size_ex(M, D_in, D_out, group,
 *               scale_type) bytes.
 * Everything else as for awq_w4a16_gemm.
 */
awq_status awq_w4a16_gemm_ex(const void *X, int64_t M, int64_t D_in, int64_t D_out,
                             const uint32_t *packed, const void *scales, awq_dtype scale_type,
                             const uint8_t *zeros, int group, const float *inv_s, void *Y,
                             awq_dtype yt, void *workspace, size_t workspace_bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* AWQ_MI355X_H */
