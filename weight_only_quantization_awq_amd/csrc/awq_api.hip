// C ABI of the AWQ library: host-side argument validation, workspace
// sizing and kernel launches.  See include/awq.h for the contract.
#include "awq.h"  // include/awq.h (on the -I path)

#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include "awq_internal.h"

namespace {

thread_local char g_err[512] = "";

awq_status fail(awq_status code, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return code;
}

awq_status hip_status(hipError_t e, const char *what) {
    if (e == hipSuccess) return AWQ_OK;
    return fail(AWQ_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool valid_dtype(int t) { return t == AWQ_F32 || t == AWQ_BF16; }

// Bounds that keep every index of every kernel inside int64 and every grid
// dimension inside the hardware limits.
constexpr int64_t kMaxDim = int64_t(1) << 24;
constexpr int64_t kMinF16Outputs = int64_t(1) << 16;

awq_status check_search_shape(int64_t N, int64_t D_in, int64_t D_out, int xt, int bits, int group, int n_alpha,
                              awq::SearchShape *sh, unsigned matrix = 0) {
    if (!valid_dtype(xt)) return fail(AWQ_ERR_DTYPE, "unsupported activation dtype %d", xt);
    if (N < 1 || D_in < 1 || D_out < 1) return fail(AWQ_ERR_SHAPE, "N, D_in, D_out must be >= 1");
    if (N > kMaxDim || D_in > kMaxDim || D_out > kMaxDim)
        return fail(AWQ_ERR_SHAPE, "dimension above %lld", static_cast<long long>(kMaxDim));
    if (bits < 2 || bits > 8) return fail(AWQ_ERR_ARG, "bits must be in 2..8 (got %d)", bits);
    if (group < 8 || group % 8 != 0) return fail(AWQ_ERR_ARG, "group must be a positive multiple of 8 (got %d)", group);
    if (D_in % group != 0) return fail(AWQ_ERR_SHAPE, "D_in (%lld) must be a multiple of group (%d)",
                                       static_cast<long long>(D_in), group);
    if (n_alpha < 1 || n_alpha > AWQ_MAX_ALPHAS) return fail(AWQ_ERR_ARG, "n_alpha must be in 1..%d", AWQ_MAX_ALPHAS);
    awq::SearchShape s{};
    s.N = N;
    s.D_in = D_in;
    s.D_out = D_out;
    s.Mp = awq::round_up(N, awq::kTileM);
    s.Kq = awq::round_up(D_in, awq::kTileK);
    s.Np = awq::round_up(D_out, awq::kTileN);
    // bf16 activations run the loss contraction on 16-bit matrix cores.  Its
    // relative error shrinks like 2^-11 / sqrt(number of outputs) with fp16
    // error weights; below 2^16 outputs the float32 matrix path (exact X,
    // float32 error weights) is used so that small layers also meet a 1e-4
    // relative loss error.  Layers of 2048 to 16384 input channels with at
    // least 2^39 multiply-adds per alpha use bf16 matrix cores, which sustain
    // about 7% more on full-entropy operands; the error weights of the 64
    // channels with the largest activation statistic then also carry their
    // bf16 rounding residual as 64 extra contraction rows, so that a few
    // dominant channels cannot concentrate the coarser bf16 rounding in the
    // loss.  Below 2^39 the costs of that path (choosing the channels, the
    // gathers, the residual stores and the quantiser's two-wave groups, which
    // run slower while W stays in the Infinity Cache) outweighed the faster
    // contraction: whole searches at N = 4096 on 4096 x 11008 / 11008 x 4096
    // (2^37.4) took 6.62 / 6.24 ms against 6.47 / 6.23 ms on fp16, 8192 x
    // 28672 (2^39.8) 31.90 against 33.02 ms.
    // `matrix` (AWQ_SEARCH_MATRIX_BF16 / _FP16, or 0) overrides the size rule
    // for the layers that may take the bf16 path.
    s.f16 = (xt == AWQ_BF16) && (N * D_out >= kMinF16Outputs);
    const bool eligible = s.f16 && D_in >= awq::kMinBf16Rows && D_in <= awq::kMaxBf16Rows;
    if (matrix == AWQ_SEARCH_MATRIX_BF16)
        s.bf16 = eligible;
    else if (matrix == AWQ_SEARCH_MATRIX_FP16)
        s.bf16 = false;
    else
        s.bf16 = eligible && static_cast<double>(N) * static_cast<double>(D_in) * static_cast<double>(D_out) >=
                                 awq::kMinBf16Macs;
    s.Kc = s.bf16 ? awq::kCorrRows : 0;
    s.Kp = s.Kq + s.Kc;
    s.MB = s.Mp / 16;
    s.KB = s.Kp / 32;
    s.NB = s.Np / 16;
    s.MB32 = s.Mp / 32;
    s.KB64 = s.Kp / 64;
    s.NB32 = s.Np / 32;
    s.tiles_m = s.Mp / awq::kTileM;
    s.tiles_n = s.Np / awq::kTileN;
    s.group = group;
    s.bits = bits;
    s.n_alpha = n_alpha;
    awq::set_search_chunk(s, 0, s.Np);
    const int64_t blocks = s.tiles_m * s.tiles_n * n_alpha;
    if (blocks >= (int64_t(1) << 31)) return fail(AWQ_ERR_SHAPE, "problem too large for one launch");
    if (D_in / group >= 65535) return fail(AWQ_ERR_SHAPE, "too many groups per column");
    *sh = s;
    return AWQ_OK;
}

// Output columns per error-weight chunk that `bytes` of workspace hold: all
// Np columns when the whole layer fits, else the largest multiple of 256
// that does (0 if not even 256 columns fit).  The layout's only
// column-dependent region is the error weights, whose size is a multiple of
// 256 bytes for any multiple of 256 columns.
int64_t search_chunk_cols(const awq::SearchShape &sh, size_t bytes) {
    if (bytes >= awq::search_workspace_layout(sh, sh.Np).total) return sh.Np;
    const size_t fixed = awq::search_workspace_layout(sh, 0).total;
    if (bytes < fixed) return 0;
    const size_t per_col = static_cast<size_t>(sh.n_alpha) * static_cast<size_t>(sh.Kp) * (sh.f16 ? 2 : 4);
    const int64_t cols = static_cast<int64_t>((bytes - fixed) / per_col) / 256 * 256;
    return cols < sh.Np ? cols : sh.Np;
}

awq_status search_impl(const void *X, awq_dtype xt, int64_t N, int64_t D_in, const void *W, awq_dtype wt,
                       int64_t D_out, const float *a, const float *b, const float *alphas, int n_alpha, int bits,
                       int group, double *losses, int32_t *best, float *s_best, float *scales, int8_t *codes,
                       void *workspace, size_t workspace_bytes, hipStream_t stream, hipEvent_t *events,
                       int n_events, uint8_t *zeros = nullptr, bool f16_steps = false, unsigned matrix = 0) {
    g_err[0] = 0;
    if (events && n_events != AWQ_SEARCH_EVENTS)
        return fail(AWQ_ERR_ARG, "events needs exactly %d handles (got %d)", AWQ_SEARCH_EVENTS, n_events);
    awq::SearchShape sh{};
    awq_status s = check_search_shape(N, D_in, D_out, xt, bits, group, n_alpha, &sh, matrix);
    if (s != AWQ_OK) return s;
    if (!valid_dtype(wt)) return fail(AWQ_ERR_DTYPE, "unsupported weight dtype %d", static_cast<int>(wt));
    if (!X || !W || !a || !alphas || !losses || !best || !s_best || !scales)
        return fail(AWQ_ERR_ARG, "only `codes` may be NULL");
    const void *dev[] = {X, W, a, losses, best, s_best, scales};
    for (const void *p : dev)
        if (!aligned16(p)) return fail(AWQ_ERR_ARG, "device pointers must be 16-byte aligned");
    if (codes && !aligned16(codes)) return fail(AWQ_ERR_ARG, "codes must be 16-byte aligned");
    if (b && !aligned16(b)) return fail(AWQ_ERR_ARG, "b must be 16-byte aligned");
    sh.asym = zeros != nullptr;
    sh.f16_steps = f16_steps;
    if (zeros && !aligned16(zeros)) return fail(AWQ_ERR_ARG, "zeros must be 16-byte aligned");
    awq::AlphaGrid grid{};
    for (int k = 0; k < n_alpha; ++k) {
        const float v = alphas[k];
        if (!(v >= 0.0f && v <= 1.0f)) return fail(AWQ_ERR_ARG, "alphas[%d] = %g is outside [0, 1]", k, v);
        grid.v[k] = v;
    }
    const int64_t chunk = search_chunk_cols(sh, workspace_bytes);
    if (!workspace)
        return fail(AWQ_ERR_WORKSPACE, "workspace is NULL (need %zu bytes, at least %zu)",
                    awq::search_workspace_layout(sh, sh.Np).total, awq::search_workspace_layout(sh, 256).total);
    if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
        return fail(AWQ_ERR_WORKSPACE, "workspace must be 256-byte aligned");
    if (chunk < 256)
        return fail(AWQ_ERR_WORKSPACE, "workspace too small: %zu < %zu bytes (the minimum, one 256-column chunk)",
                    workspace_bytes, awq::search_workspace_layout(sh, 256).total);
    return hip_status(awq::launch_search(X, xt, W, wt, a, b, zeros, grid, sh, losses, best, s_best, scales, codes,
                                         static_cast<unsigned char *>(workspace), chunk, stream, events),
                      "awq_search_layer launch");
}

awq_status gemm_impl(const void *X, int64_t M, int64_t D_in, int64_t D_out, const uint32_t *packed,
                     const void *scales, bool steps_f16, const uint8_t *zeros, int group, const float *inv_s,
                     void *Y, awq_dtype yt, void *workspace, size_t workspace_bytes, hipStream_t stream);

}  // namespace

namespace awq {

int report_error(int code, const char *msg) { return fail(static_cast<awq_status>(code), "%s", msg); }

}  // namespace awq

extern "C" {

const char *awq_last_error(void) { return g_err; }

const char *awq_version(void) { return "awq-mi355x 0.1 (gfx950)"; }

awq_status awq_act_stats_ex(const void *X, awq_dtype xt, int64_t N, int64_t D_in, awq_statistic stat, float *a,
                            hipStream_t stream) {
    g_err[0] = 0;
    if (!valid_dtype(xt)) return fail(AWQ_ERR_DTYPE, "unsupported dtype %d", static_cast<int>(xt));
    if (stat != AWQ_STAT_MEAN_ABS && stat != AWQ_STAT_MAX_ABS)
        return fail(AWQ_ERR_ARG, "unknown statistic %d", static_cast<int>(stat));
    if (!X || !a) return fail(AWQ_ERR_ARG, "X and a must be non-NULL");
    if (!aligned16(X) || !aligned16(a)) return fail(AWQ_ERR_ARG, "X and a must be 16-byte aligned");
    if (N < 1 || D_in < 1) return fail(AWQ_ERR_SHAPE, "N and D_in must be >= 1");
    if (N > (int64_t(1) << 31) || D_in > kMaxDim) return fail(AWQ_ERR_SHAPE, "shape too large");
    return hip_status(awq::launch_act_stats(X, xt, N, D_in, static_cast<int>(stat), a, stream),
                      "awq_act_stats launch");
}

awq_status awq_act_stats(const void *X, awq_dtype xt, int64_t N, int64_t D_in, float *a, hipStream_t stream) {
    return awq_act_stats_ex(X, xt, N, D_in, AWQ_STAT_MEAN_ABS, a, stream);
}

awq_status awq_weight_stats(const void *W, awq_dtype wt, int64_t D_in, int64_t D_out, float *b, hipStream_t stream) {
    g_err[0] = 0;
    if (!valid_dtype(wt)) return fail(AWQ_ERR_DTYPE, "unsupported dtype %d", static_cast<int>(wt));
    if (!W || !b) return fail(AWQ_ERR_ARG, "W and b must be non-NULL");
    if (!aligned16(W) || !aligned16(b)) return fail(AWQ_ERR_ARG, "W and b must be 16-byte aligned");
    if (D_in < 1 || D_out < 1) return fail(AWQ_ERR_SHAPE, "D_in and D_out must be >= 1");
    if (D_in > (int64_t(1) << 31) - 1 || D_out > kMaxDim) return fail(AWQ_ERR_SHAPE, "shape too large");
    return hip_status(awq::launch_weight_stats(W, wt, D_in, D_out, b, stream), "awq_weight_stats launch");
}

size_t awq_search_workspace_size(int64_t N, int64_t D_in, int64_t D_out, awq_dtype xt, int bits, int group,
                                 int n_alpha) {
    g_err[0] = 0;
    awq::SearchShape sh{};
    // sized for the bf16 path wherever a layer may take it (AWQ_SEARCH_MATRIX_BF16)
    if (check_search_shape(N, D_in, D_out, xt, bits, group, n_alpha, &sh, AWQ_SEARCH_MATRIX_BF16) != AWQ_OK) return 0;
    return awq::search_workspace_layout(sh, sh.Np).total;
}

size_t awq_search_workspace_min_size(int64_t N, int64_t D_in, int64_t D_out, awq_dtype xt, int bits, int group,
                                     int n_alpha) {
    g_err[0] = 0;
    awq::SearchShape sh{};
    if (check_search_shape(N, D_in, D_out, xt, bits, group, n_alpha, &sh, AWQ_SEARCH_MATRIX_BF16) != AWQ_OK) return 0;
    return awq::search_workspace_layout(sh, 256).total;
}

awq_status awq_search_layer(const void *X, awq_dtype xt, int64_t N, int64_t D_in, const void *W, awq_dtype wt,
                            int64_t D_out, const float *a, const float *alphas, int n_alpha, int bits, int group,
                            double *losses, int32_t *best, float *s_best, float *scales, int8_t *codes,
                            void *workspace, size_t workspace_bytes, hipStream_t stream) {
    return search_impl(X, xt, N, D_in, W, wt, D_out, a, nullptr, alphas, n_alpha, bits, group, losses, best, s_best,
                       scales, codes, workspace, workspace_bytes, stream, nullptr, 0);
}

awq_status awq_search_status(const int32_t *best, hipStream_t stream, int32_t *best_out) {
    g_err[0] = 0;
    if (!best) return fail(AWQ_ERR_ARG, "best must be non-NULL");
    int32_t h = -1;
    hipError_t e = hipMemcpyAsync(&h, best, sizeof(h), hipMemcpyDeviceToHost, stream);
    if (e == hipSuccess) e = hipStreamSynchronize(stream);
    if (e != hipSuccess) return hip_status(e, "awq_search_status");
    if (best_out) *best_out = h;
    if (h < 0) return fail(AWQ_ERR_NONFINITE, "the search met a NaN or Inf (best = %d)", static_cast<int>(h));
    return AWQ_OK;
}

awq_status awq_search_layer_ex(const void *X, awq_dtype xt, int64_t N, int64_t D_in, const void *W, awq_dtype wt,
                               int64_t D_out, const float *a, const float *alphas, int n_alpha, int bits, int group,
                               double *losses, int32_t *best, float *s_best, float *scales, int8_t *codes,
                               void *workspace, size_t workspace_bytes, hipStream_t stream, hipEvent_t *events,
                               int n_events) {
    return search_impl(X, xt, N, D_in, W, wt, D_out, a, nullptr, alphas, n_alpha, bits, group, losses, best, s_best,
                       scales, codes, workspace, workspace_bytes, stream, events, n_events);
}

awq_status awq_search_layer_zp(const void *X, awq_dtype xt, int64_t N, int64_t D_in, const void *W, awq_dtype wt,
                               int64_t D_out, const float *a, const float *b, const float *alphas, int n_alpha,
                               int bits, int group, double *losses, int32_t *best, float *s_best, float *scales,
                               uint8_t *zeros, uint8_t *codes, void *workspace, size_t workspace_bytes,
                               hipStream_t stream) {
    if (!zeros) {
        g_err[0] = 0;
        return fail(AWQ_ERR_ARG, "zeros must be non-NULL");
    }
    return search_impl(X, xt, N, D_in, W, wt, D_out, a, b, alphas, n_alpha, bits, group, losses, best, s_best,
                       scales, reinterpret_cast<int8_t *>(codes), workspace, workspace_bytes, stream, nullptr, 0,
                       zeros);
}

awq_status awq_search_layer_flags(const void *X, awq_dtype xt, int64_t N, int64_t D_in, const void *W,
                                  awq_dtype wt, int64_t D_out, const float *a, const float *b, const float *alphas,
                                  int n_alpha, int bits, int group, unsigned flags, double *losses, int32_t *best,
                                  float *s_best, void *scales, uint8_t *zeros, void *codes, void *workspace,
                                  size_t workspace_bytes, hipStream_t stream) {
    g_err[0] = 0;
    if (flags & ~static_cast<unsigned>(AWQ_SEARCH_ZERO_POINT | AWQ_SEARCH_FP16_STEPS | AWQ_SEARCH_MATRIX_BF16 |
                                       AWQ_SEARCH_MATRIX_FP16))
        return fail(AWQ_ERR_ARG, "unknown flags 0x%x", flags);
    const unsigned matrix = flags & (AWQ_SEARCH_MATRIX_BF16 | AWQ_SEARCH_MATRIX_FP16);
    if (matrix == (AWQ_SEARCH_MATRIX_BF16 | AWQ_SEARCH_MATRIX_FP16))
        return fail(AWQ_ERR_ARG, "AWQ_SEARCH_MATRIX_BF16 and AWQ_SEARCH_MATRIX_FP16 exclude each other");
    const bool zp = (flags & AWQ_SEARCH_ZERO_POINT) != 0;
    if (zp && !zeros) return fail(AWQ_ERR_ARG, "zeros must be non-NULL with AWQ_SEARCH_ZERO_POINT");
    return search_impl(X, xt, N, D_in, W, wt, D_out, a, b, alphas, n_alpha, bits, group, losses, best, s_best,
                       static_cast<float *>(scales), static_cast<int8_t *>(codes), workspace, workspace_bytes,
                       stream, nullptr, 0, zp ? zeros : nullptr, (flags & AWQ_SEARCH_FP16_STEPS) != 0, matrix);
}

awq_status awq_search_layer_wscale(const void *X, awq_dtype xt, int64_t N, int64_t D_in, const void *W,
                                   awq_dtype wt, int64_t D_out, const float *a, const float *b, const float *alphas,
                                   int n_alpha, int bits, int group, double *losses, int32_t *best, float *s_best,
                                   float *scales, int8_t *codes, void *workspace, size_t workspace_bytes,
                                   hipStream_t stream) {
    if (!b) {
        g_err[0] = 0;
        return fail(AWQ_ERR_ARG, "b must be non-NULL");
    }
    return search_impl(X, xt, N, D_in, W, wt, D_out, a, b, alphas, n_alpha, bits, group, losses, best, s_best,
                       scales, codes, workspace, workspace_bytes, stream, nullptr, 0);
}

size_t awq_clip_workspace_size(int64_t N, int64_t D_in, int group) {
    g_err[0] = 0;
    if (!awq::clip_group_supported(group)) {
        fail(AWQ_ERR_ARG, "clip search supports group 32, 64, 128 or 256 (got %d)", group);
        return 0;
    }
    if (N < 1 || D_in < group || D_in % group != 0 || D_in > kMaxDim || N > (int64_t(1) << 31)) {
        fail(AWQ_ERR_SHAPE, "bad shape N=%lld D_in=%lld group=%d", static_cast<long long>(N),
             static_cast<long long>(D_in), group);
        return 0;
    }
    return awq::clip_workspace_bytes(N, D_in, group);
}

awq_status awq_clip_search(const void *X, awq_dtype xt, int64_t N, int64_t D_in, const void *W, awq_dtype wt,
                           int64_t D_out, const float *s, const float *ratios, int n_ratio, int bits, int group,
                           int32_t *ratio_idx, float *scales, int8_t *codes, float *errors, void *workspace,
                           size_t workspace_bytes, hipStream_t stream) {
    g_err[0] = 0;
    if (!valid_dtype(xt) || !valid_dtype(wt)) return fail(AWQ_ERR_DTYPE, "unsupported dtype");
    if (!awq::clip_group_supported(group))
        return fail(AWQ_ERR_ARG, "clip search supports group 32, 64, 128 or 256 (got %d)", group);
    if (bits < 2 || bits > 8) return fail(AWQ_ERR_ARG, "bits must be in 2..8 (got %d)", bits);
    if (N < 1 || D_in < group || D_out < 1 || D_in % group != 0)
        return fail(AWQ_ERR_SHAPE, "need N >= 1, D_out >= 1 and D_in a positive multiple of group");
    if (N > (int64_t(1) << 31) || D_in > kMaxDim || D_out > kMaxDim) return fail(AWQ_ERR_SHAPE, "shape too large");
    if ((D_out + 63) / 64 >= 65536) return fail(AWQ_ERR_SHAPE, "too many output columns");
    if (n_ratio < 1 || n_ratio > AWQ_MAX_ALPHAS)
        return fail(AWQ_ERR_ARG, "n_ratio must be in 1..%d (got %d)", AWQ_MAX_ALPHAS, n_ratio);
    if (!X || !W || !s || !ratios || !ratio_idx || !scales)
        return fail(AWQ_ERR_ARG, "only `codes` and `errors` may be NULL");
    const void *dev[] = {X, W, s, ratio_idx, scales};
    for (const void *p : dev)
        if (!aligned16(p)) return fail(AWQ_ERR_ARG, "device pointers must be 16-byte aligned");
    if ((codes && !aligned16(codes)) || (errors && !aligned16(errors)))
        return fail(AWQ_ERR_ARG, "codes and errors must be 16-byte aligned");
    awq::AlphaGrid grid{};
    for (int k = 0; k < n_ratio; ++k) {
        const float v = ratios[k];
        if (!(v > 0.0f && v <= 1.0f)) return fail(AWQ_ERR_ARG, "ratios[%d] = %g is outside (0, 1]", k, v);
        grid.v[k] = v;
    }
    const size_t need = awq::clip_workspace_bytes(N, D_in, group);
    if (!workspace) return fail(AWQ_ERR_WORKSPACE, "workspace is NULL (need %zu bytes)", need);
    if (!aligned16(workspace)) return fail(AWQ_ERR_WORKSPACE, "workspace must be 16-byte aligned");
    if (workspace_bytes < need)
        return fail(AWQ_ERR_WORKSPACE, "workspace too small: %zu < %zu bytes", workspace_bytes, need);
    return hip_status(awq::launch_clip(X, xt, N, D_in, W, wt, D_out, s, grid, n_ratio, bits, group, ratio_idx,
                                       scales, codes, errors, workspace, stream),
                      "awq_clip_search launch");
}

awq_status awq_pack(const int8_t *codes, int64_t D_in, int64_t D_out, int bits, uint32_t *packed,
                    hipStream_t stream) {
    return awq_pack_ex(codes, D_in, D_out, bits, 0, packed, stream);
}

awq_status awq_pack_ex(const int8_t *codes, int64_t D_in, int64_t D_out, int bits, int zero_point_codes,
                       uint32_t *packed, hipStream_t stream) {
    g_err[0] = 0;
    if (!codes || !packed) return fail(AWQ_ERR_ARG, "codes and packed must be non-NULL");
    if (!aligned16(codes) || !aligned16(packed)) return fail(AWQ_ERR_ARG, "pointers must be 16-byte aligned");
    if (bits < 2 || bits > 4) return fail(AWQ_ERR_ARG, "packing needs bits in 2..4 (got %d)", bits);
    if (D_in < 8 || D_out < 1) return fail(AWQ_ERR_SHAPE, "D_in must be >= 8 and D_out >= 1");
    if (D_in % 8 != 0) return fail(AWQ_ERR_SHAPE, "D_in must be a multiple of 8");
    if (D_in > kMaxDim || D_out > kMaxDim) return fail(AWQ_ERR_SHAPE, "shape too large");
    return hip_status(awq::launch_pack(codes, D_in, D_out, zero_point_codes ? 0 : 8, packed, stream),
                      "awq_pack launch");
}

size_t awq_w4a16_workspace_size(int64_t M, int64_t D_in, int64_t D_out, int has_inv_s) {
    g_err[0] = 0;
    if (M < 1 || D_in < 1 || D_out < 1) {
        fail(AWQ_ERR_SHAPE, "M, D_in and D_out must be >= 1");
        return 0;
    }
    return awq::w4a16_workspace_bytes(M, D_in, D_out, has_inv_s != 0);
}

awq_status awq_w4a16_gemm(const void *X, int64_t M, int64_t D_in, int64_t D_out, const uint32_t *packed,
                          const float *scales, int group, const float *inv_s, void *Y, awq_dtype yt,
                          void *workspace, size_t workspace_bytes, hipStream_t stream) {
    g_err[0] = 0;
    return gemm_impl(X, M, D_in, D_out, packed, scales, false, nullptr, group, inv_s, Y, yt, workspace, workspace_bytes,
                     stream);
}

size_t awq_w4a16_workspace_size_ex(int64_t M, int64_t D_in, int64_t D_out, int group, awq_dtype scale_type) {
    g_err[0] = 0;
    if (M < 1 || D_in < 1 || D_out < 1 || group < 1 || D_in % group != 0) {
        fail(AWQ_ERR_SHAPE, "need M, D_in, D_out >= 1 and D_in a multiple of group");
        return 0;
    }
    if (scale_type != AWQ_F32 && scale_type != AWQ_F16) {
        fail(AWQ_ERR_DTYPE, "scale type must be AWQ_F32 or AWQ_F16");
        return 0;
    }
    return awq::w4a16_workspace_bytes_ex(M, D_in, D_out, group, scale_type == AWQ_F16);
}

awq_status awq_w4a16_gemm_ex(const void *X, int64_t M, int64_t D_in, int64_t D_out, const uint32_t *packed,
                             const void *scales, awq_dtype scale_type, const uint8_t *zeros, int group,
                             const float *inv_s, void *Y, awq_dtype yt, void *workspace, size_t workspace_bytes,
                             hipStream_t stream) {
    g_err[0] = 0;
    if (scale_type != AWQ_F32 && scale_type != AWQ_F16)
        return fail(AWQ_ERR_DTYPE, "scale type must be AWQ_F32 or AWQ_F16");
    if (zeros && !aligned16(zeros)) return fail(AWQ_ERR_ARG, "zeros must be 16-byte aligned");
    return gemm_impl(X, M, D_in, D_out, packed, scales, scale_type == AWQ_F16, zeros, group, inv_s, Y, yt,
                     workspace, workspace_bytes, stream);
}

awq_status awq_w4a16_gemm_zp(const void *X, int64_t M, int64_t D_in, int64_t D_out, const uint32_t *packed,
                             const float *scales, const uint8_t *zeros, int group, const float *inv_s, void *Y,
                             awq_dtype yt, void *workspace, size_t workspace_bytes, hipStream_t stream) {
    g_err[0] = 0;
    if (!zeros) return fail(AWQ_ERR_ARG, "zeros must be non-NULL");
    if (!aligned16(zeros)) return fail(AWQ_ERR_ARG, "zeros must be 16-byte aligned");
    return gemm_impl(X, M, D_in, D_out, packed, scales, false, zeros, group, inv_s, Y, yt, workspace, workspace_bytes,
                     stream);
}

}  // extern "C"

namespace {

awq_status gemm_impl(const void *X, int64_t M, int64_t D_in, int64_t D_out, const uint32_t *packed,
                     const void *scales, bool steps_f16, const uint8_t *zeros, int group, const float *inv_s,
                     void *Y, awq_dtype yt, void *workspace, size_t workspace_bytes, hipStream_t stream) {
    if (!valid_dtype(yt)) return fail(AWQ_ERR_DTYPE, "unsupported output dtype %d", static_cast<int>(yt));
    if (!X || !packed || !scales || !Y) return fail(AWQ_ERR_ARG, "only inv_s and workspace may be NULL");
    const void *dev[] = {X, packed, scales, Y};
    for (const void *p : dev)
        if (!aligned16(p)) return fail(AWQ_ERR_ARG, "device pointers must be 16-byte aligned");
    if (inv_s && !aligned16(inv_s)) return fail(AWQ_ERR_ARG, "inv_s must be 16-byte aligned");
    if (M < 1 || D_in < 1 || D_out < 1) return fail(AWQ_ERR_SHAPE, "M, D_in, D_out must be >= 1");
    if (M > (int64_t(1) << 31) || D_in > kMaxDim || D_out > kMaxDim) return fail(AWQ_ERR_SHAPE, "shape too large");
    if (group < 32 || group % 32 != 0 || ((group / 32) & (group / 32 - 1)) != 0)
        return fail(AWQ_ERR_ARG, "group must be 32 times a power of two (got %d)", group);
    if (D_in % group != 0) return fail(AWQ_ERR_SHAPE, "D_in must be a multiple of group");
    if (D_out % 4 != 0) return fail(AWQ_ERR_SHAPE, "D_out must be a multiple of 4");
    const size_t need = steps_f16 ? awq::w4a16_workspace_bytes_ex(M, D_in, D_out, group, true)
                                  : awq::w4a16_workspace_bytes(M, D_in, D_out, inv_s != nullptr);
    if (need > 0) {
        if (!workspace) return fail(AWQ_ERR_WORKSPACE, "workspace is NULL (need %zu bytes)", need);
        if (!aligned16(workspace)) return fail(AWQ_ERR_WORKSPACE, "workspace must be 16-byte aligned");
        if (workspace_bytes < need)
            return fail(AWQ_ERR_WORKSPACE, "workspace too small: %zu < %zu bytes", workspace_bytes, need);
    }
    return hip_status(awq::launch_w4a16_gemm(X, M, D_in, D_out, packed, scales, steps_f16, zeros, group, inv_s,
                                             Y, yt, workspace, stream),
                      "awq_w4a16_gemm launch");
}

}  // namespace
