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
// Main kernel (rows 16-byte aligned): one 512-thread workgroup per slice of
// columns over all rows (described at the kernel).  Fallback (unaligned
// rows): 64 columns x 16 row phases per workgroup.
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

// Main kernel (rows 16-byte aligned): one workgroup of 512 threads owns R
// consecutive 16-byte column runs (8 bf16 or 4 fp32 columns each) over all N
// rows.  Thread t reads run t % R of rows t / R, t / R + 512 / R, ... with
// eight 16-byte loads in flight (the last batch clamps its rows and masks
// the repeats out of the sums), so a wave's load covers 64 / R rows of R·16
// contiguous bytes and a workgroup keeps 64 KiB in flight, with no
// cross-workgroup reduction.  R is the largest of 8, 4, 2, 1 that leaves at
// least 128 workgroups.  Launch shapes measured with a copy of this kernel
// (bf16, HIP events per call, X resident / X rotating over 8 copies):
// 4096 x 8192: 16.9 / 22.4 us with 512 threads and 8 loads in flight against
// 19.6 / 24.3 us with 1024 threads and 16 (and 18.3-20.7 us warm for the
// other mixes of 512 / 1024 threads, R = 4 / 8 and 8 / 12 / 16 loads);
// 2048 x 4096: 9.3-10.4 / 10.3 us against 10.4-11.9 / 10.9-11.6 us.  Summing
// with xor instead of float64 left every shape within 4%, and splitting the
// rows over up to 64 workgroups per column slice with a second fixed-order
// pass over float64 partials, or reading 512-byte and 1 KiB row segments per
// workgroup, gave 18-31 us at 4096 x 8192: none reached the 12.7 us of a
// plain linear read of the same bytes.  The per-thread float64 sums are
// combined over the threads of the same run by a fixed butterfly, then over
// the 8 waves in wave order.  Workgroups are renumbered so that each XCD
// (workgroups are dispatched round-robin over the 8 XCDs, each with its own
// L2) gets one contiguous range of runs: a 128-byte line shared by
// neighbouring workgroups is then fetched into one L2 only.
constexpr int kStatThreads = 512;

template <bool BF16, bool MAX, int R>
__global__ __launch_bounds__(kStatThreads) void act_stats_run_kernel(const void *__restrict__ X, int64_t N,
                                                                     int64_t D_in, float *__restrict__ a) {
    constexpr int C = BF16 ? 8 : 4;   // columns per 16-byte run
    constexpr int P = kStatThreads / R;   // row phases
    const int64_t runs = D_in / C;
    const unsigned total = gridDim.x, bid = blockIdx.x;
    const unsigned xcd = bid % 8u, local = bid / 8u, q = total / 8u, rem = total % 8u;
    const int64_t wg = static_cast<int64_t>(xcd * q + (xcd < rem ? xcd : rem) + local);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int r = tid % R;
    const int64_t run = wg * R + r;
    const bool live = run < runs;
    const int64_t runc = live ? run : runs - 1;   // in-bounds loads for a ragged last workgroup
    const unsigned char *base = static_cast<const unsigned char *>(X) + runc * 16;
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
    constexpr int U = 8;   // loads in flight per thread
    for (int64_t n0 = tid / R; n0 < N; n0 += U * P) {
        uint4 u[U];
#pragma unroll
        for (int i = 0; i < U; ++i) {
            const int64_t n = n0 + i * P;
            u[i] = *reinterpret_cast<const uint4 *>(base + (n < N ? n : N - 1) * pitch);
        }
#pragma unroll
        for (int i = 0; i < U; ++i) {
            // rows past N repeat row N - 1: zero them (|x| = 0 leaves both statistics unchanged)
            if (n0 + i * P >= N) u[i] = make_uint4(0u, 0u, 0u, 0u);
            add(u[i]);
        }
    }
    __shared__ double red[kStatThreads / 64][R * C];
#pragma unroll
    for (int c = 0; c < C; ++c) {
        double v = acc[c];
        // lanes lane, lane ^ R, ... hold the same run: fixed butterfly over them
        for (int off = 32; off >= R; off >>= 1) v = stat_comb<MAX>(v, __shfl_xor(v, off));
        if (lane < R) red[wave][lane * C + c] = v;
    }
    __syncthreads();
    if (tid < R * C) {
        const int rr = tid / C;
        const int64_t col = (wg * R + rr) * C + tid % C;
        double s = red[0][tid];
#pragma unroll
        for (int w = 1; w < kStatThreads / 64; ++w) s = stat_comb<MAX>(s, red[w][tid]);
        if (wg * R + rr < runs) a[col] = static_cast<float>(MAX ? s : s / static_cast<double>(N));
    }
}

template <bool BF16, bool MAX, int R>
static void launch_runs(const void *X, int64_t N, int64_t D_in, float *a, hipStream_t st) {
    const int64_t runs = D_in / (BF16 ? 8 : 4);
    const dim3 grid(static_cast<unsigned>((runs + R - 1) / R));
    hipLaunchKernelGGL((act_stats_run_kernel<BF16, MAX, R>), grid, dim3(kStatThreads), 0, st, X, N, D_in, a);
}

// Runs per workgroup: the largest of 8, 4, 2 that still leaves 128
// workgroups, else 1.
static int runs_per_workgroup(int64_t runs) {
    for (int R = 8; R > 1; R >>= 1)
        if (runs / R >= 128) return R;
    return 1;
}

template <bool MAX>
static hipError_t launch_act_stats_t(const void *X, int xt, int64_t N, int64_t D_in, float *a, hipStream_t st) {
    const int C = xt == 1 ? 8 : 4;
    if (D_in % C == 0) {
        const int R = runs_per_workgroup(D_in / C);
#define AWQ_STAT_R(BF)                                                  \
    do {                                                                \
        switch (R) {                                                    \
        case 8: launch_runs<BF, MAX, 8>(X, N, D_in, a, st); break;      \
        case 4: launch_runs<BF, MAX, 4>(X, N, D_in, a, st); break;      \
        case 2: launch_runs<BF, MAX, 2>(X, N, D_in, a, st); break;      \
        default: launch_runs<BF, MAX, 1>(X, N, D_in, a, st); break;     \
        }                                                               \
    } while (0)
        if (xt == 1)
            AWQ_STAT_R(true);
        else
            AWQ_STAT_R(false);
#undef AWQ_STAT_R
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
