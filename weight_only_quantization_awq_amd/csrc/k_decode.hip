// W4A16 inference product Y = (X·diag(inv_s))·Dequant(W_q).
//
// [CA] "推論時的等效實現": online, Y = (X·diag(1/s*))·Dequant(W_quantized), the
// activation scaling fused into the kernel.  [MR] "即时权重反量化": INT4 weights
// are dequantised on the fly inside the main loop, and "为什么 AWQ 能加速本地设备上
// 的 LLM": at decode batch sizes the product is bound by weight traffic, which
// 4-bit storage cuts to a quarter.
//
// Design for CDNA4.  Each wavefront owns 64 output columns and a contiguous
// range of quantisation groups; the four waves of a workgroup split the
// groups of the same 64 columns and meet in LDS at the end.  Per 32-row k
// step, lane (c, n) = (lane/16, lane%16) loads one 16-byte vector holding the
// packed words of rows 8c..8c+7 for columns 4n..4n+3: a wave reads 1 KiB in
// four 256-byte runs.  Word t becomes the B operand of MFMA t with two ALU
// ops per register pair, (w >> 4d) & 0x000F000F | 0x43004300 = bf16(136 + q);
// the constant offset is removed by one extra MFMA against bf16(136)
// (136·sum X per row), and the per-group step is applied to the float32
// group partial, so no per-weight multiply is needed.
#include "awq_internal.h"

namespace awq {

__device__ __forceinline__ uint32_t bf16_rne_bits(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
}

template <int MT, bool HAS_INV, bool OUT_BF16>
__global__ __launch_bounds__(256) void w4a16_kernel(const uint16_t *__restrict__ X, int64_t M, int64_t D_in,
                                                    int64_t D_out, const uint32_t *__restrict__ packed,
                                                    const float *__restrict__ scales, int group,
                                                    const float *__restrict__ inv_s, void *__restrict__ Y) {
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int c = lane >> 4, n = lane & 15;
    const int64_t o0 = static_cast<int64_t>(blockIdx.x) * 64;
    const int64_t oc = o0 + 4 * n;  // first of this lane's four columns
    const bool col_ok = oc < D_out;
    const int64_t G = D_in / group;
    const int64_t g0 = G * wave / 4, g1 = G * (wave + 1) / 4;
    const int ksteps = group / 32;

    floatx4 ytot[MT][4];
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int t = 0; t < 4; ++t) ytot[m][t] = floatx4{0.f, 0.f, 0.f, 0.f};

    bf16x8 ones;
    {
        const uint32_t k136 = 0x43084308u;  // bf16(136) twice
        uint32_t tmp[4] = {k136, k136, k136, k136};
        ones = *reinterpret_cast<bf16x8 *>(tmp);
    }

    for (int64_t g = g0; g < g1; ++g) {
        floatx4 acc[MT][4], acc1[MT];
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            acc1[m] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int t = 0; t < 4; ++t) acc[m][t] = floatx4{0.f, 0.f, 0.f, 0.f};
        }
        for (int ks = 0; ks < ksteps; ++ks) {
            const int64_t kbase = g * group + ks * 32;
            uint4 wv = make_uint4(0x88888888u, 0x88888888u, 0x88888888u, 0x88888888u);
            if (col_ok) wv = *reinterpret_cast<const uint4 *>(packed + (kbase / 8 + c) * D_out + oc);
            // A fragments: row m*16 + n, k = kbase + 8c .. +7
            bf16x8 av[MT];
#pragma unroll
            for (int m = 0; m < MT; ++m) {
                const int64_t row = m * 16 + n;
                uint4 xv = make_uint4(0u, 0u, 0u, 0u);
                if (row < M) {
                    xv = *reinterpret_cast<const uint4 *>(X + row * D_in + kbase + 8 * c);
                    if (HAS_INV) {
                        const float4 i0 = *reinterpret_cast<const float4 *>(inv_s + kbase + 8 * c);
                        const float4 i1 = *reinterpret_cast<const float4 *>(inv_s + kbase + 8 * c + 4);
                        const float iv[8] = {i0.x, i0.y, i0.z, i0.w, i1.x, i1.y, i1.z, i1.w};
                        uint32_t xw[4] = {xv.x, xv.y, xv.z, xv.w};
#pragma unroll
                        for (int p = 0; p < 4; ++p) {
                            const float lo = __uint_as_float(xw[p] << 16) * iv[2 * p];
                            const float hi = __uint_as_float(xw[p] & 0xFFFF0000u) * iv[2 * p + 1];
                            xw[p] = bf16_rne_bits(lo) | (bf16_rne_bits(hi) << 16);
                        }
                        xv = make_uint4(xw[0], xw[1], xw[2], xw[3]);
                    }
                }
                av[m] = *reinterpret_cast<bf16x8 *>(&xv);
            }
            const uint32_t words[4] = {wv.x, wv.y, wv.z, wv.w};
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const uint32_t w = words[t];
                uint32_t b[4];
#pragma unroll
                for (int d = 0; d < 4; ++d) b[d] = ((w >> (4 * d)) & 0x000F000Fu) | 0x43004300u;
                const bf16x8 bv = *reinterpret_cast<bf16x8 *>(b);
#pragma unroll
                for (int m = 0; m < MT; ++m)
                    acc[m][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[m], bv, acc[m][t], 0, 0, 0);
            }
#pragma unroll
            for (int m = 0; m < MT; ++m) acc1[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[m], ones, acc1[m], 0, 0, 0);
        }
        float4 sc = make_float4(0.f, 0.f, 0.f, 0.f);
        if (col_ok) sc = *reinterpret_cast<const float4 *>(scales + g * D_out + oc);
        const float scv[4] = {sc.x, sc.y, sc.z, sc.w};
#pragma unroll
        for (int m = 0; m < MT; ++m)
#pragma unroll
            for (int t = 0; t < 4; ++t)
#pragma unroll
                for (int i = 0; i < 4; ++i) ytot[m][t][i] += scv[t] * (acc[m][t][i] - acc1[m][i]);
    }

    // combine the four waves' group ranges
    __shared__ float red[4][MT * 16][64];
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i) red[wave][(m * 4 + t) * 4 + i][lane] = ytot[m][t][i];
    __syncthreads();
    for (int item = tid; item < MT * 16 * 64; item += 256) {
        const int slot = item / 64, l = item % 64;
        const int m = slot / 16, t = (slot / 4) % 4, i = slot % 4;
        const float v = ((red[0][slot][l] + red[1][slot][l]) + red[2][slot][l]) + red[3][slot][l];
        // MFMA C layout: lane l holds rows 4*(l/16)+i, column l%16 of the tile
        const int64_t row = m * 16 + 4 * (l >> 4) + i;
        const int64_t col = o0 + 4 * (l & 15) + t;
        if (row < M && col < D_out) {
            if (OUT_BF16)
                static_cast<uint16_t *>(Y)[row * D_out + col] = static_cast<uint16_t>(bf16_rne_bits(v));
            else
                static_cast<float *>(Y)[row * D_out + col] = v;
        }
    }
}

template <int MT>
static hipError_t launch_mt(const void *X, int64_t M, int64_t D_in, int64_t D_out, const uint32_t *packed,
                            const float *scales, int group, const float *inv_s, void *Y, int yt, hipStream_t st) {
    const dim3 grid(static_cast<unsigned>((D_out + 63) / 64));
    const uint16_t *Xb = static_cast<const uint16_t *>(X);
    if (inv_s) {
        if (yt == 1)
            hipLaunchKernelGGL((w4a16_kernel<MT, true, true>), grid, dim3(256), 0, st, Xb, M, D_in, D_out, packed,
                               scales, group, inv_s, Y);
        else
            hipLaunchKernelGGL((w4a16_kernel<MT, true, false>), grid, dim3(256), 0, st, Xb, M, D_in, D_out, packed,
                               scales, group, inv_s, Y);
    } else {
        if (yt == 1)
            hipLaunchKernelGGL((w4a16_kernel<MT, false, true>), grid, dim3(256), 0, st, Xb, M, D_in, D_out, packed,
                               scales, group, inv_s, Y);
        else
            hipLaunchKernelGGL((w4a16_kernel<MT, false, false>), grid, dim3(256), 0, st, Xb, M, D_in, D_out, packed,
                               scales, group, inv_s, Y);
    }
    return hipGetLastError();
}

hipError_t launch_w4a16_gemm(const void *X, int64_t M, int64_t D_in, int64_t D_out, const uint32_t *packed,
                             const float *scales, int group, const float *inv_s, void *Y, int yt, hipStream_t st) {
    const size_t ybytes = yt == 1 ? 2 : 4;
    for (int64_t m0 = 0; m0 < M; m0 += 64) {
        const int64_t mc = (M - m0) < 64 ? (M - m0) : 64;
        const void *Xc = static_cast<const uint16_t *>(X) + m0 * D_in;
        void *Yc = static_cast<unsigned char *>(Y) + static_cast<size_t>(m0 * D_out) * ybytes;
        hipError_t e;
        if (mc <= 16)
            e = launch_mt<1>(Xc, mc, D_in, D_out, packed, scales, group, inv_s, Yc, yt, st);
        else if (mc <= 32)
            e = launch_mt<2>(Xc, mc, D_in, D_out, packed, scales, group, inv_s, Yc, yt, st);
        else if (mc <= 48)
            e = launch_mt<3>(Xc, mc, D_in, D_out, packed, scales, group, inv_s, Yc, yt, st);
        else
            e = launch_mt<4>(Xc, mc, D_in, D_out, packed, scales, group, inv_s, Yc, yt, st);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace awq
