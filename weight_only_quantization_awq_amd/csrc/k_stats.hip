// Activation statistics: a_j = mean_n |X[n, j]|.
//
// [CA] "重要通道識別的統計依據": activation_scale[j] = mean(|X_calib[:, j]|);
// [MR] "搜索最优比例": s_X is the per-channel mean activation magnitude.
//
// One workgroup owns 64 consecutive columns and 16 row phases: a wavefront
// reads 64 consecutive elements of one row (coalesced along D_in) and each
// lane keeps a float64 running sum.  The 16 phase sums are combined in a fixed
// order through LDS, so the result does not depend on scheduling.  Bound by
// HBM: N·D_in·elt bytes read, D_in·4 bytes written.
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

hipError_t launch_act_stats(const void *X, int xt, int64_t N, int64_t D_in, float *a, hipStream_t st) {
    const int64_t blocks = (D_in + kStatCols - 1) / kStatCols;
    hipLaunchKernelGGL(act_stats_kernel, dim3(static_cast<unsigned>(blocks)), dim3(kStatCols * kStatPhases), 0,
                       st, X, xt, N, D_in, a);
    return hipGetLastError();
}

}  // namespace awq
