// Activation statistics: a_j = mean_n |X[n, j]|.
//
// [CA] "重要通道識別的統計依據": activation_scale[j] = mean(|X_calib[:, j]|);
// [MR] "搜索最优比例": s_X is the per-channel mean activation magnitude.
//
// Bound by HBM: N·D_in·elt bytes read, D_in·4 bytes written.  Every sum is
// accumulated in float64 in a fixed order (per-thread running sums, then a
// fixed butterfly and a fixed cross-wave order), so the result does not
// depend on scheduling; a_j = float32(sum / N).
//
// Main kernel (rows 16-byte aligned): one workgroup owns one 16-byte run of
// columns (8 bf16 or 4 fp32) over all rows; thread t reads rows t, t + 256,
// ... with four loads in flight.  Consecutive column runs share 128-byte
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
            acc += fabs(static_cast<double>(v0));
            acc += fabs(static_cast<double>(v1));
            acc += fabs(static_cast<double>(v2));
            acc += fabs(static_cast<double>(v3));
        }
        for (; n < N; n += kStatPhases) acc += fabs(static_cast<double>(load_elem(X, xt, n * D_in + col)));
    }
    __shared__ double red[kStatPhases][kStatCols];
    red[ph][lane] = acc;
    __syncthreads();
    if (ph == 0 && col < D_in) {
        double s = 0.0;
        for (int p = 0; p < kStatPhases; ++p) s += red[p][lane];
        a[col] = static_cast<float>(s / static_cast<double>(N));
    }
}

template <bool BF16>
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
                acc[2 * p] += fabs(static_cast<double>(__uint_as_float(w[p] << 16)));
                acc[2 * p + 1] += fabs(static_cast<double>(__uint_as_float(w[p] & 0xFFFF0000u)));
            } else {
                acc[p] += fabs(static_cast<double>(__uint_as_float(w[p])));
            }
        }
    };
    int64_t n = tid;
    for (; n + 768 < N; n += 1024) {
        const uint4 u0 = *reinterpret_cast<const uint4 *>(base + n * pitch);
        const uint4 u1 = *reinterpret_cast<const uint4 *>(base + (n + 256) * pitch);
        const uint4 u2 = *reinterpret_cast<const uint4 *>(base + (n + 512) * pitch);
        const uint4 u3 = *reinterpret_cast<const uint4 *>(base + (n + 768) * pitch);
        add(u0);
        add(u1);
        add(u2);
        add(u3);
    }
    for (; n < N; n += 256) add(*reinterpret_cast<const uint4 *>(base + n * pitch));
    __shared__ double red[4][C];
#pragma unroll
    for (int c = 0; c < C; ++c) {
        double v = acc[c];
        for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
        if (lane == 0) red[wave][c] = v;
    }
    __syncthreads();
    if (tid < C && run < runs) {
        const double s = ((red[0][tid] + red[1][tid]) + red[2][tid]) + red[3][tid];
        a[run * C + tid] = static_cast<float>(s / static_cast<double>(N));
    }
}

hipError_t launch_act_stats(const void *X, int xt, int64_t N, int64_t D_in, float *a, hipStream_t st) {
    const int C = xt == 1 ? 8 : 4;
    if (D_in % C == 0) {
        const int64_t runs = D_in / C;
        if (xt == 1)
            hipLaunchKernelGGL(act_stats_run_kernel<true>, dim3(static_cast<unsigned>(runs)), dim3(256), 0, st, X, N,
                               D_in, a);
        else
            hipLaunchKernelGGL(act_stats_run_kernel<false>, dim3(static_cast<unsigned>(runs)), dim3(256), 0, st, X, N,
                               D_in, a);
        return hipGetLastError();
    }
    const int64_t blocks = (D_in + kStatCols - 1) / kStatCols;
    hipLaunchKernelGGL(act_stats_kernel, dim3(static_cast<unsigned>(blocks)), dim3(kStatCols * kStatPhases), 0,
                       st, X, xt, N, D_in, a);
    return hipGetLastError();
}

}  // namespace awq
