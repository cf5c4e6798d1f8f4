// Activation statistics: a_j = mean_n |X[n, j]| or max_n |X[n, j]|, and the
// weight statistic b_j = mean_o |W[j, o]|.
//
// [CA] "重要通道識別的統計依據": activation_scale[j] = mean(|X_calib[:, j]|), or
// the max; [MR] "搜索最优比例": s_X is the per-channel mean activation
// magnitude; [CA] "二、縮放因子的搜尋": s_j = (max|X_j|)^α; [LQ] "4.4 怎么做：
// 不是留 FP16，而是「缩放」": the weight term mean|W_j| of input channel j.
//
// The max is exact in any order; a NaN in a column makes that channel's
// maximum NaN (the comparisons below keep a NaN once it appears).
//
// Bound by HBM: N·D_in·elt bytes read, D_in·4 bytes written.  Every sum is
// accumulated in float64 in a fixed order (per-thread running sums, then a
// fixed butterfly and a fixed cross-wave order), so the result does not
// depend on scheduling; a_j = float32(sum / N).
//
// Main kernel (rows 16-byte aligned): one workgroup owns one 16-byte run of
// columns (8 bf16 or 4 fp32) over all rows; thread t reads rows t, t + 256,
// ... with eight loads in flight.  Consecutive column runs share 128-byte
// lines, so workgroups are renumbered to give each XCD (workgroups are
// dispatched round-robin over the 8 XCDs, each with its own L2) one
// contiguous range of runs: every line is then fetched into one L2 only.
// Fallback (unaligned rows): 64 columns x 16 row phases per workgroup.
#include "awq_internal.h"

namespace awq {

__device__ __forceinline__ float load_elem(const void *p, int xt, int64_t i) {
    if (xt == 1) {
        const uint16_t v = static_cast<const uint16_t *>(p)[i];
        return __uint_as_float(static_cast<uint32_t>(v) << 16);
    }
    return static_cast<const float *>(p)[i];
}

constexpr int kStatCols = 64;
constexpr int kStatPhases = 16;

// combine for the two statistics: sum, or a maximum that keeps NaN
template <bool MAX>
__device__ __forceinline__ double stat_comb(double acc, double v) {
    if constexpr (MAX)
        return (v > acc || v != v) ? v : acc;
    else
        return acc + v;
}

template <bool MAX>
__global__ __launch_bounds__(kStatCols *kStatPhases) void act_stats_kernel(
    const void *__restrict__ X, int xt, int64_t N, int64_t D_in, float *__restrict__ a) {
    const int lane = threadIdx.x % kStatCols;
    const int ph = threadIdx.x / kStatCols;
    const int64_t col = static_cast<int64_t>(blockIdx.x) * kStatCols + lane;
    double acc = 0.0;
    if (col < D_in) {
        int64_t n = ph;
        // four independent loads in flight per lane
        for (; n + 3 * kStatPhases < N; n += 4 * kStatPhases) {
            const float v0 = load_elem(X, xt, n * D_in + col);
            const float v1 = load_elem(X, xt, (n + kStatPhases) * D_in + col);
            const float v2 = load_elem(X, xt, (n + 2 * kStatPhases) * D_in + col);
            const float v3 = load_elem(X, xt, (n + 3 * kStatPhases) * D_in + col);
            acc = stat_comb<MAX>(acc, fabs(static_cast<double>(v0)));
            acc = stat_comb<MAX>(acc, fabs(static_cast<double>(v1)));
            acc = stat_comb<MAX>(acc, fabs(static_cast<double>(v2)));
            acc = stat_comb<MAX>(acc, fabs(static_cast<double>(v3)));
        }
        for (; n < N; n += kStatPhases)
            acc = stat_comb<MAX>(acc, fabs(static_cast<double>(load_elem(X, xt, n * D_in + col))));
    }
    __shared__ double red[kStatPhases][kStatCols];
    red[ph][lane] = acc;
    __syncthreads();
    if (ph == 0 && col < D_in) {
        double s = 0.0;
        for (int p = 0; p < kStatPhases; ++p) s = stat_comb<MAX>(s, red[p][lane]);
        a[col] = static_cast<float>(MAX ? s : s / static_cast<double>(N));
    }
}

template <bool BF16, bool MAX>
__global__ __launch_bounds__(256) void act_stats_run_kernel(const void *__restrict__ X, int64_t N, int64_t D_in,
                                                            float *__restrict__ a) {
    constexpr int C = BF16 ? 8 : 4;   // columns per 16-byte run
    const int64_t runs = D_in / C;
    // XCD-contiguous renumbering of the workgroups
    const unsigned total = gridDim.x, bid = blockIdx.x;
    const unsigned xcd = bid % 8u, local = bid / 8u, q = total / 8u, r = total % 8u;
    const int64_t run = static_cast<int64_t>(xcd * q + (xcd < r ? xcd : r) + local);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const unsigned char *base = static_cast<const unsigned char *>(X) + run * 16;
    const int64_t pitch = D_in * (BF16 ? 2 : 4);
    double acc[C];
#pragma unroll
    for (int c = 0; c < C; ++c) acc[c] = 0.0;
    auto add = [&](const uint4 &u) {
        const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            if constexpr (BF16) {
                acc[2 * p] = stat_comb<MAX>(acc[2 * p], fabs(static_cast<double>(__uint_as_float(w[p] << 16))));
                acc[2 * p + 1] =
                    stat_comb<MAX>(acc[2 * p + 1], fabs(static_cast<double>(__uint_as_float(w[p] & 0xFFFF0000u))));
            } else {
                acc[p] = stat_comb<MAX>(acc[p], fabs(static_cast<double>(__uint_as_float(w[p]))));
            }
        }
    };
    int64_t n = tid;
    // eight loads in flight per thread (a 2048-row slab is one round trip)
    for (; n + 7 * 256 < N; n += 8 * 256) {
        uint4 u[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) u[i] = *reinterpret_cast<const uint4 *>(base + (n + i * 256) * pitch);
#pragma unroll
        for (int i = 0; i < 8; ++i) add(u[i]);
    }
    for (; n < N; n += 256) add(*reinterpret_cast<const uint4 *>(base + n * pitch));
    __shared__ double red[4][C];
#pragma unroll
    for (int c = 0; c < C; ++c) {
        double v = acc[c];
        for (int off = 32; off > 0; off >>= 1) v = stat_comb<MAX>(v, __shfl_xor(v, off));
        if (lane == 0) red[wave][c] = v;
    }
    __syncthreads();
    if (tid < C && run < runs) {
        const double s = stat_comb<MAX>(stat_comb<MAX>(stat_comb<MAX>(red[0][tid], red[1][tid]), red[2][tid]),
                                        red[3][tid]);
        a[run * C + tid] = static_cast<float>(MAX ? s : s / static_cast<double>(N));
    }
}

template <bool MAX>
static hipError_t launch_act_stats_t(const void *X, int xt, int64_t N, int64_t D_in, float *a, hipStream_t st) {
    const int C = xt == 1 ? 8 : 4;
    if (D_in % C == 0) {
        const int64_t runs = D_in / C;
        if (xt == 1)
            hipLaunchKernelGGL((act_stats_run_kernel<true, MAX>), dim3(static_cast<unsigned>(runs)), dim3(256), 0, st,
                               X, N, D_in, a);
        else
            hipLaunchKernelGGL((act_stats_run_kernel<false, MAX>), dim3(static_cast<unsigned>(runs)), dim3(256), 0, st,
                               X, N, D_in, a);
        return hipGetLastError();
    }
    const int64_t blocks = (D_in + kStatCols - 1) / kStatCols;
    hipLaunchKernelGGL((act_stats_kernel<MAX>), dim3(static_cast<unsigned>(blocks)), dim3(kStatCols * kStatPhases), 0,
                       st, X, xt, N, D_in, a);
    return hipGetLastError();
}

hipError_t launch_act_stats(const void *X, int xt, int64_t N, int64_t D_in, int stat, float *a, hipStream_t st) {
    return stat == 1 ? launch_act_stats_t<true>(X, xt, N, D_in, a, st) : launch_act_stats_t<false>(X, xt, N, D_in, a, st);
}

// b_j = mean_o |W[j, o]|: one workgroup per row of W, float64 partial sums per
// thread over columns t, t + 256, ... (four loads in flight), then a fixed
// butterfly and a fixed cross-wave order; b_j = float32(sum / D_out).  Rows
// are contiguous, so each load instruction of a wave covers one 128-byte
// (bf16) or 256-byte (fp32) run.
__global__ __launch_bounds__(256) void weight_stats_kernel(const void *__restrict__ W, int wt, int64_t D_in,
                                                           int64_t D_out, float *__restrict__ b) {
    const int64_t j = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t base = j * D_out;
    double acc = 0.0;
    int64_t o = tid;
    for (; o + 768 < D_out; o += 1024) {
        const float v0 = load_elem(W, wt, base + o);
        const float v1 = load_elem(W, wt, base + o + 256);
        const float v2 = load_elem(W, wt, base + o + 512);
        const float v3 = load_elem(W, wt, base + o + 768);
        acc += fabs(static_cast<double>(v0));
        acc += fabs(static_cast<double>(v1));
        acc += fabs(static_cast<double>(v2));
        acc += fabs(static_cast<double>(v3));
    }
    for (; o < D_out; o += 256) acc += fabs(static_cast<double>(load_elem(W, wt, base + o)));
    for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
    __shared__ double red[4];
    if (lane == 0) red[wave] = acc;
    __syncthreads();
    if (tid == 0) b[j] = static_cast<float>((((red[0] + red[1]) + red[2]) + red[3]) / static_cast<double>(D_out));
}

hipError_t launch_weight_stats(const void *W, int wt, int64_t D_in, int64_t D_out, float *b, hipStream_t st) {
    hipLaunchKernelGGL(weight_stats_kernel, dim3(static_cast<unsigned>(D_in)), dim3(256), 0, st, W, wt, D_in, D_out, b);
    return hipGetLastError();
}

}  // namespace awq
