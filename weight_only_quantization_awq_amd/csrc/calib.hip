// Calibration probes for roofline reporting (not part of the AWQ path):
//   * a plain device-to-device copy of known size, whose rocprofv3
//     FETCH_SIZE / WRITE_SIZE readings give the counter-to-bytes factor and
//     whose duration gives the achievable HBM bandwidth;
//   * an MFMA issue loop (independent accumulator chains, no memory traffic)
//     that measures the achievable matrix-core rate for one instruction.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <type_traits>

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

__global__ __launch_bounds__(256) void calib_copy_kernel(const uint4 *__restrict__ src, uint4 *__restrict__ dst,
                                                         int64_t n) {
    const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += stride) dst[i] = src[i];
}

// Write-only and read-only streams (4 x 16 B per thread per iteration).
// NT: streaming (nontemporal) stores instead of ordinary cached ones.
template <bool NT>
__global__ __launch_bounds__(256) void calib_fill_kernel(uint4 *__restrict__ dst, int64_t n) {
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
    const uint4 v = make_uint4(threadIdx.x, 1u, 2u, 3u);
    const u32x4 vv = {v.x, v.y, v.z, v.w};
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += stride) {
        if constexpr (NT)
            __builtin_nontemporal_store(vv, reinterpret_cast<u32x4 *>(dst + i));
        else
            dst[i] = v;
    }
}

__global__ __launch_bounds__(256) void calib_read_kernel(const uint4 *__restrict__ src, int64_t n,
                                                         unsigned *__restrict__ out) {
    const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
    unsigned acc = 0;
    int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    for (; i + 3 * stride < n; i += 4 * stride) {
        const uint4 a = src[i], b = src[i + stride], c = src[i + 2 * stride], d = src[i + 3 * stride];
        acc ^= a.x ^ b.y ^ c.z ^ d.w;
    }
    for (; i < n; i += stride) acc ^= src[i].x;
    if (acc == 0x12345678u) out[0] = acc;  // keeps the loads alive; practically never true
}

// Pseudo-random FP16 values in [-1, 1) from a lane-dependent seed (integer
// hash), so that the operands of the operand-sensitivity probe below have
// full-entropy mantissas.
__device__ __forceinline__ half8 calib_rand_half8(uint32_t seed) {
    half8 h;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        uint32_t x = seed * 2654435761u + static_cast<uint32_t>(i) * 40503u;
        x ^= x >> 13;
        x *= 0x5bd1e995u;
        x ^= x >> 15;
        h[i] = static_cast<_Float16>(static_cast<float>(x & 0xFFFFu) * (2.0f / 65536.0f) - 1.0f);
    }
    return h;
}

// The same values rounded to bf16.
__device__ __forceinline__ bf16x8 calib_rand_bf16x8(uint32_t seed) {
    const half8 h = calib_rand_half8(seed);
    bf16x8 v;
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = static_cast<__bf16>(static_cast<float>(h[i]));
    return v;
}

// v_mfma_f32_32x32x16_f16 (BF: v_mfma_f32_32x32x16_bf16) with 16 independent
// accumulators per wave (the loss contraction's count) and the operands
// cycling through 4 register sets: pseudo-random values (ZERO = false) or all
// zeros (ZERO = true).  The sustained rate depends on the operand values on
// this part.
template <bool ZERO, bool BF = false>
__global__ __launch_bounds__(256, 1) void calib_mfma_operands_kernel(float *__restrict__ out, int iters) {
    const uint32_t lane = threadIdx.x;
    typedef typename std::conditional<BF, bf16x8, half8>::type vec8;
    vec8 a[4], b[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        if constexpr (BF) {
            a[j] = ZERO ? bf16x8{} : calib_rand_bf16x8(lane * 7u + j + blockIdx.x);
            b[j] = ZERO ? bf16x8{} : calib_rand_bf16x8(lane * 13u + 3u * j + blockIdx.x);
        } else {
            a[j] = ZERO ? half8{} : calib_rand_half8(lane * 7u + j + blockIdx.x);
            b[j] = ZERO ? half8{} : calib_rand_half8(lane * 13u + 3u * j + blockIdx.x);
        }
    }
    floatx16 c[16];
#pragma unroll
    for (int m = 0; m < 16; ++m)
#pragma unroll
        for (int i = 0; i < 16; ++i) c[m][i] = 0.f;
    for (int it = 0; it < iters; ++it)
#pragma unroll
        for (int m = 0; m < 16; ++m)
            if constexpr (BF)
                c[m] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[m & 3], b[(m >> 2) & 3], c[m], 0, 0, 0);
            else
                c[m] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[m & 3], b[(m >> 2) & 3], c[m], 0, 0, 0);
    float s = 0.f;
#pragma unroll
    for (int m = 0; m < 16; ++m)
#pragma unroll
        for (int i = 0; i < 16; ++i) s += c[m][i];
    out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// kind 0: v_mfma_f32_16x16x32_f16, 1: v_mfma_f32_32x32x16_f16, 2: v_mfma_f32_16x16x4_f32
// (kinds 3 and 4: calib_mfma_operands_kernel, random and zero operands;
// kind 5: the same loop on v_mfma_f32_32x32x16_bf16 with random operands)
template <int KIND>
__global__ __launch_bounds__(256) void calib_mfma_kernel(float *__restrict__ out, int iters, float seed) {
    const int lane = threadIdx.x & 63;
    if constexpr (KIND == 0) {
        half8 a, b;
        for (int i = 0; i < 8; ++i) {
            a[i] = static_cast<_Float16>(seed * (lane + i));
            b[i] = static_cast<_Float16>(seed * (lane - i));
        }
        floatx4 c[8];
        for (int j = 0; j < 8; ++j) c[j] = floatx4{0.f, 0.f, 0.f, 0.f};
        for (int it = 0; it < iters; ++it)
#pragma unroll
            for (int j = 0; j < 8; ++j) c[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c[j], 0, 0, 0);
        float s = 0.f;
        for (int j = 0; j < 8; ++j) s += c[j][0] + c[j][1] + c[j][2] + c[j][3];
        out[blockIdx.x * blockDim.x + threadIdx.x] = s;
    } else if constexpr (KIND == 1) {
        half8 a, b;
        for (int i = 0; i < 8; ++i) {
            a[i] = static_cast<_Float16>(seed * (lane + i));
            b[i] = static_cast<_Float16>(seed * (lane - i));
        }
        floatx16 c[4];
        for (int j = 0; j < 4; ++j)
            for (int i = 0; i < 16; ++i) c[j][i] = 0.f;
        for (int it = 0; it < iters; ++it)
#pragma unroll
            for (int j = 0; j < 4; ++j) c[j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c[j], 0, 0, 0);
        float s = 0.f;
        for (int j = 0; j < 4; ++j)
            for (int i = 0; i < 16; ++i) s += c[j][i];
        out[blockIdx.x * blockDim.x + threadIdx.x] = s;
    } else {
        const float a = seed * lane, b = seed * (64 - lane);
        floatx4 c[8];
        for (int j = 0; j < 8; ++j) c[j] = floatx4{0.f, 0.f, 0.f, 0.f};
        for (int it = 0; it < iters; ++it)
#pragma unroll
            for (int j = 0; j < 8; ++j) c[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c[j], 0, 0, 0);
        float s = 0.f;
        for (int j = 0; j < 8; ++j) s += c[j][0] + c[j][1] + c[j][2] + c[j][3];
        out[blockIdx.x * blockDim.x + threadIdx.x] = s;
    }
}

extern "C" {

// Copies `bytes` (a multiple of 16) from src to dst on `stream`.
int awq_calib_copy(const void *src, void *dst, int64_t bytes, hipStream_t stream) {
    if (!src || !dst || bytes <= 0 || (bytes % 16) != 0) return -1;
    const int64_t n = bytes / 16;
    hipLaunchKernelGGL(calib_copy_kernel, dim3(4096), dim3(256), 0, stream, static_cast<const uint4 *>(src),
                       static_cast<uint4 *>(dst), n);
    return hipGetLastError() == hipSuccess ? 0 : -6;
}

// Writes `bytes` (multiple of 16) to dst; mode 1: reads them from src instead;
// mode 2: writes them with streaming (nontemporal) stores.
int awq_calib_stream(void *buf, int64_t bytes, int mode, unsigned *sink, hipStream_t stream) {
    if (!buf || bytes <= 0 || (bytes % 16) != 0 || !sink || mode < 0 || mode > 2) return -1;
    const int64_t n = bytes / 16;
    if (mode == 0)
        hipLaunchKernelGGL(calib_fill_kernel<false>, dim3(4096), dim3(256), 0, stream, static_cast<uint4 *>(buf), n);
    else if (mode == 2)
        hipLaunchKernelGGL(calib_fill_kernel<true>, dim3(4096), dim3(256), 0, stream, static_cast<uint4 *>(buf), n);
    else
        hipLaunchKernelGGL(calib_read_kernel, dim3(4096), dim3(256), 0, stream, static_cast<const uint4 *>(buf), n,
                           sink);
    return hipGetLastError() == hipSuccess ? 0 : -6;
}

// Runs `blocks` workgroups of 4 waves, each wave issuing iters x 8 (kind 0, 2),
// iters x 4 (kind 1) or iters x 16 (kinds 3, 4, 5) MFMAs.  `out` needs
// blocks*256 floats.
// FLOP per launch: kind 0: blocks*4*iters*8*16384, kind 1: blocks*4*iters*4*32768,
// kind 2: blocks*4*iters*8*2048, kinds 3, 4 and 5: blocks*4*iters*16*32768.
int awq_calib_mfma(float *out, int kind, int blocks, int iters, hipStream_t stream) {
    if (!out || blocks < 1 || iters < 1) return -1;
    switch (kind) {
        case 0:
            hipLaunchKernelGGL(calib_mfma_kernel<0>, dim3(blocks), dim3(256), 0, stream, out, iters, 1e-3f);
            break;
        case 1:
            hipLaunchKernelGGL(calib_mfma_kernel<1>, dim3(blocks), dim3(256), 0, stream, out, iters, 1e-3f);
            break;
        case 2:
            hipLaunchKernelGGL(calib_mfma_kernel<2>, dim3(blocks), dim3(256), 0, stream, out, iters, 1e-3f);
            break;
        case 3:
            hipLaunchKernelGGL(calib_mfma_operands_kernel<false>, dim3(blocks), dim3(256), 0, stream, out, iters);
            break;
        case 4:
            hipLaunchKernelGGL(calib_mfma_operands_kernel<true>, dim3(blocks), dim3(256), 0, stream, out, iters);
            break;
        case 5:
            hipLaunchKernelGGL((calib_mfma_operands_kernel<false, true>), dim3(blocks), dim3(256), 0, stream, out,
                               iters);
            break;
        default:
            return -1;
    }
    return hipGetLastError() == hipSuccess ? 0 : -6;
}

}  // extern "C"
