// Weight clipping after the scale search: per group of every output column,
// the clip ratio r of a grid that minimises the group's own output error.
//
// [MR] "搜索最优比例": besides the scale search, weight clipping is applied to
// lower the mean squared quantisation error.  Reading (the pages give one
// sentence): with s fixed, group g of column o and ratio r quantise
// W' = s·W with the clipped maximum m_r = fl(r·max|W'_g|), step = fl(m_r /
// qmax), q = clamp(rint(W'/step), ±qmax), and
//   E_g,o(r) = sum_n ( sum_{k in g} X[n, k] · (q_k·step / s_k − W[k, o]) )²
//            = d_gᵀ · H_g · d_g,   H_g = X_gᵀ X_g  (group x group),
// the loss of [CA] "縮放因子最佳化的完整流程" step 4c restricted to the group.
// The first ratio with the smallest E is kept.
//
// Design for CDNA4:
//  * The Gram matrices H_g (group² floats per group) replace the N-row
//    activation block: the per-ratio work is 2·group² FLOP per column instead
//    of 2·N·group, 16x less at N = 2048, group = 128.
//  * gram_kernel: one workgroup per (group, 256-row chunk) on
//    v_mfma_f32_16x16x4f32 (exact products for bf16 activations, float32
//    accumulation); gram_reduce_kernel sums the chunks in a fixed order in
//    float64.
//  * clip_kernel: one workgroup per (group, 64 columns) with H_g, W' and the
//    error-weight tile in LDS.  Per ratio: the quantiser (round half to even
//    of the IEEE quotient, clamp) writes d = (q·step − W')/s into LDS, the
//    matrix cores form P = H_g·D (wave w: 16 columns, all rows), and the
//    epilogue reduces E = colsum(D ⊙ P).  The codes and step of the chosen
//    ratio are written at the end.  (A variant holding H in registers with a
//    double-buffered tile measured 1.24 ms against 0.82 ms at 4096², 11
//    ratios: the compiler placed the next ratio's quantiser ahead of the
//    matrix block instead of between its MFMAs.)
#include "awq_internal.h"

namespace awq {

namespace {

constexpr int kClipCols = 64;    // output columns per clip workgroup
constexpr int kGramRows = 256;   // calibration rows per Gram chunk

template <bool XB>
__device__ __forceinline__ float ld_x(const void *p, int64_t i) {
    if constexpr (XB) return __uint_as_float(static_cast<uint32_t>(static_cast<const uint16_t *>(p)[i]) << 16);
    else return static_cast<const float *>(p)[i];
}

// Partial Gram matrix of group g over rows [c·256, c·256 + 256): part[c][g]
// (GR x GR floats, row-major).  A = X_gᵀ (channel i, row n), B = X_g; wave w
// owns channel blocks w·RB .. w·RB + RB − 1 (RB = NB/4 rounded up) and all
// column blocks.  16x16x4 layout: operand lane l holds (row l%16, k l/16);
// result register r of lane l holds (row 4·(l/16) + r, column l%16).
template <int NB, bool XB>
__global__ __launch_bounds__(256) void gram_kernel(const void *__restrict__ X, int64_t N, int64_t D_in,
                                                   float *__restrict__ part) {
    constexpr int GR = NB * 16;
    constexpr int RB = (NB + 3) / 4;
    const int g = blockIdx.x, c = blockIdx.y, G = gridDim.x;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    __shared__ float xs[64][GR + 4];
    floatx4 acc[RB][NB];
#pragma unroll
    for (int a = 0; a < RB; ++a)
#pragma unroll
        for (int b = 0; b < NB; ++b) acc[a][b] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
    const int64_t n0 = static_cast<int64_t>(c) * kGramRows;
    const int64_t n1 = n0 + kGramRows < N ? n0 + kGramRows : N;
    for (int64_t nb0 = n0; nb0 < n1; nb0 += 64) {
        __syncthreads();
        for (int i = tid; i < 64 * GR; i += 256) {
            const int r = i / GR, k = i % GR;
            const int64_t n = nb0 + r;
            xs[r][k] = n < n1 ? ld_x<XB>(X, n * D_in + static_cast<int64_t>(g) * GR + k) : 0.0f;
        }
        __syncthreads();
#pragma unroll 4
        for (int ks = 0; ks < 16; ++ks) {
            const int r = ks * 4 + (lane >> 4);
            float bv[NB];
#pragma unroll
            for (int jb = 0; jb < NB; ++jb) bv[jb] = xs[r][jb * 16 + (lane & 15)];
#pragma unroll
            for (int a = 0; a < RB; ++a) {
                const int ib = wave * RB + a;
                if (ib < NB) {
                    const float av = xs[r][ib * 16 + (lane & 15)];
#pragma unroll
                    for (int jb = 0; jb < NB; ++jb)
                        acc[a][jb] = __builtin_amdgcn_mfma_f32_16x16x4f32(av, bv[jb], acc[a][jb], 0, 0, 0);
                }
            }
        }
    }
    float *dst = part + (static_cast<int64_t>(c) * G + g) * GR * GR;
#pragma unroll
    for (int a = 0; a < RB; ++a) {
        const int ib = wave * RB + a;
        if (ib < NB) {
#pragma unroll
            for (int jb = 0; jb < NB; ++jb)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    dst[(ib * 16 + 4 * (lane >> 4) + r) * GR + jb * 16 + (lane & 15)] = acc[a][jb][r];
        }
    }
}

// H[g] = sum over chunks of part[c][g], float64 in chunk order, one rounding.
__global__ __launch_bounds__(256) void gram_reduce_kernel(const float *__restrict__ part, int chunks,
                                                          int64_t n_elem, float *__restrict__ H) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    if (i >= n_elem) return;
    double sum = 0.0;
    for (int c = 0; c < chunks; ++c) sum += static_cast<double>(part[static_cast<int64_t>(c) * n_elem + i]);
    H[i] = static_cast<float>(sum);
}

struct ClipArgs {
    int64_t D_in, D_out;
    int G, bits, n_ratio;
    AlphaGrid ratios;   // clip ratios, each in (0, 1]
};

// q = clamp(rint(fl(wp / step)), ±qmax) without a division in the common
// case: t = fl(wp · fl(1/step)) is within |wp/step|·(2^-23 + 2^-48) of the
// quotient, and the IEEE quotient within 2^-24·|wp/step|.  For |t| >= qmax + 1
// both clamp to ±qmax; below that, when t lies farther than
// (qmax + 1)·2^-20 from every half-integer both round to the same integer.
// Otherwise (rare) the true quotient is taken.  step = 0 gives 0.
__device__ __forceinline__ float clip_code(float wp, float step, float rstep, float qmax, float thr) {
    if (!(step > 0.0f)) return 0.0f;
    const float t = wp * rstep;
    if (fabsf(t) >= qmax + 1.0f) return copysignf(qmax, t);
    float q = rintf(t);
    if (!(fabsf(t - q) < thr)) q = rintf(wp / step);
    return fminf(fmaxf(q, -qmax), qmax);
}

// One workgroup: group g = blockIdx.x, columns [64·blockIdx.y, +64).
// Thread t: column t%64 and row quarter t/64 for the quantiser; wave w:
// columns 16w..16w+15, all rows, for the matrix product and the error.
// H_g, W' and the error-weight tile sit in LDS.
template <int NB, bool WB>
__global__ __launch_bounds__(256) void clip_kernel(const void *__restrict__ W, const float *__restrict__ s,
                                                   const float *__restrict__ H, ClipArgs ca,
                                                   int32_t *__restrict__ ratio_idx, float *__restrict__ scales,
                                                   int8_t *__restrict__ codes, float *__restrict__ errors) {
    constexpr int GR = NB * 16;
    constexpr int RQ = GR / 4;   // rows per quarter
    const int g = blockIdx.x;
    const int64_t o0 = static_cast<int64_t>(blockIdx.y) * kClipCols;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
    const int col = tid & 63, quarter = wave;
    const int64_t o = o0 + col;
    const bool live = o < ca.D_out;

    __shared__ float Hs[GR][GR + 1];
    __shared__ float Wp[GR][kClipCols + 1];
    __shared__ float Dt[GR][kClipCols + 1];
    __shared__ float rs[GR];
    __shared__ float mred[4][kClipCols];
    __shared__ int bsel[kClipCols];

    const float *Hg = H + static_cast<int64_t>(g) * GR * GR;
    for (int i = tid; i < GR * GR; i += 256) Hs[i / GR][i % GR] = Hg[i];
    const int64_t j0 = static_cast<int64_t>(g) * GR;
    for (int i = tid; i < GR; i += 256) rs[i] = 1.0f / s[j0 + i];
    // W' = fl(s·w) of this thread's quarter of its column; its absmax
    float m = 0.0f;
    for (int k = quarter * RQ; k < quarter * RQ + RQ; ++k) {
        float wp = 0.0f;
        if (live) {
            const float w = WB ? __uint_as_float(static_cast<uint32_t>(
                                     static_cast<const uint16_t *>(W)[(j0 + k) * ca.D_out + o]) << 16)
                               : static_cast<const float *>(W)[(j0 + k) * ca.D_out + o];
            wp = s[j0 + k] * w;
        }
        Wp[k][col] = wp;
        m = fmaxf(m, fabsf(wp));
    }
    mred[quarter][col] = m;
    __syncthreads();
    const float mcol = fmaxf(fmaxf(mred[0][col], mred[1][col]), fmaxf(mred[2][col], mred[3][col]));
    const float qmax = static_cast<float>((1 << (ca.bits - 1)) - 1);
    const float thr = 0.5f - (qmax + 1.0f) * 0x1p-20f;

    float best_e = INFINITY;   // lanes 0-15 of wave w: column 16w + lane
    int best_i = 0;
    for (int ri = 0; ri < ca.n_ratio; ++ri) {
        // quantiser at this ratio: error weights of this thread's quarter
        const float step = (ca.ratios.v[ri] * mcol) / qmax;
        const float rstep = step > 0.0f ? 1.0f / step : 0.0f;
        for (int k = quarter * RQ; k < quarter * RQ + RQ; ++k) {
            const float wp = Wp[k][col];
            const float q = clip_code(wp, step, rstep, qmax, thr);
            Dt[k][col] = fmaf(q, step, -wp) * rs[k];
        }
        __syncthreads();
        // P = H_g · D for columns 16·wave .. +16, then E = sum_k D[k]·P[k]
        floatx4 acc[NB];
#pragma unroll
        for (int rb = 0; rb < NB; ++rb) acc[rb] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
        const int cb = wave * 16 + (lane & 15);
#pragma unroll 4
        for (int ks = 0; ks < GR / 4; ++ks) {
            const int kk = ks * 4 + (lane >> 4);
            const float bv = Dt[kk][cb];
#pragma unroll
            for (int rb = 0; rb < NB; ++rb)
                acc[rb] = __builtin_amdgcn_mfma_f32_16x16x4f32(Hs[rb * 16 + (lane & 15)][kk], bv, acc[rb], 0, 0, 0);
        }
        float e = 0.0f;
#pragma unroll
        for (int rb = 0; rb < NB; ++rb)
#pragma unroll
            for (int r = 0; r < 4; ++r) e = fmaf(acc[rb][r], Dt[rb * 16 + 4 * (lane >> 4) + r][cb], e);
        e += __shfl_xor(e, 16);
        e += __shfl_xor(e, 32);
        const int64_t oc = o0 + cb;
        if (lane < 16 && oc < ca.D_out) {
            if (errors) errors[(static_cast<int64_t>(ri) * ca.G + g) * ca.D_out + oc] = e;
            if (e < best_e) {
                best_e = e;
                best_i = ri;
            }
        }
        __syncthreads();   // Dt is rewritten by the next ratio
    }
    if (lane < 16) bsel[wave * 16 + lane] = best_i;
    __syncthreads();
    if (!live) return;
    const int bi = bsel[col];
    const float step = (ca.ratios.v[bi] * mcol) / qmax;
    const float rstep = step > 0.0f ? 1.0f / step : 0.0f;
    for (int k = quarter * RQ; k < quarter * RQ + RQ; ++k) {
        const float q = clip_code(Wp[k][col], step, rstep, qmax, thr);
        if (codes) codes[(j0 + k) * ca.D_out + o] = static_cast<int8_t>(q);
    }
    if (quarter == 0) {
        scales[static_cast<int64_t>(g) * ca.D_out + o] = step;
        ratio_idx[static_cast<int64_t>(g) * ca.D_out + o] = bi;
    }
}

struct ClipLayout {
    size_t off_h, off_part, total;
    int chunks;
};

ClipLayout clip_layout(int64_t N, int64_t D_in, int group) {
    auto up = [](size_t b) { return (b + 255) / 256 * 256; };
    ClipLayout L{};
    const int64_t G = D_in / group;
    L.chunks = static_cast<int>((N + kGramRows - 1) / kGramRows);
    const size_t hbytes = static_cast<size_t>(G) * group * group * 4;
    L.off_h = 0;
    L.off_part = up(hbytes);
    L.total = L.off_part + up(hbytes * static_cast<size_t>(L.chunks));
    return L;
}

template <int NB>
hipError_t launch_clip_nb(const void *X, int xt, int64_t N, int64_t D_in, const void *W, int wt, int64_t D_out,
                          const float *s, const AlphaGrid &ratios, int n_ratio, int bits, int32_t *ratio_idx,
                          float *scales, int8_t *codes, float *errors, unsigned char *ws, hipStream_t st) {
    constexpr int GR = NB * 16;
    const ClipLayout L = clip_layout(N, D_in, GR);
    const int G = static_cast<int>(D_in / GR);
    float *H = reinterpret_cast<float *>(ws + L.off_h);
    float *part = reinterpret_cast<float *>(ws + L.off_part);
    const dim3 gg(static_cast<unsigned>(G), static_cast<unsigned>(L.chunks));
    if (xt == 1)
        hipLaunchKernelGGL((gram_kernel<NB, true>), gg, dim3(256), 0, st, X, N, D_in, part);
    else
        hipLaunchKernelGGL((gram_kernel<NB, false>), gg, dim3(256), 0, st, X, N, D_in, part);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t n_elem = static_cast<int64_t>(G) * GR * GR;
    hipLaunchKernelGGL(gram_reduce_kernel, dim3(static_cast<unsigned>((n_elem + 255) / 256)), dim3(256), 0, st,
                       part, L.chunks, n_elem, H);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    ClipArgs ca{};
    ca.D_in = D_in;
    ca.D_out = D_out;
    ca.G = G;
    ca.bits = bits;
    ca.n_ratio = n_ratio;
    ca.ratios = ratios;
    const dim3 cg(static_cast<unsigned>(G), static_cast<unsigned>((D_out + kClipCols - 1) / kClipCols));
    if (wt == 1)
        hipLaunchKernelGGL((clip_kernel<NB, true>), cg, dim3(256), 0, st, W, s, H, ca, ratio_idx, scales, codes,
                           errors);
    else
        hipLaunchKernelGGL((clip_kernel<NB, false>), cg, dim3(256), 0, st, W, s, H, ca, ratio_idx, scales, codes,
                           errors);
    return hipGetLastError();
}

}  // namespace

bool clip_group_supported(int group) { return group == 32 || group == 64 || group == 128; }

size_t clip_workspace_bytes(int64_t N, int64_t D_in, int group) { return clip_layout(N, D_in, group).total; }

hipError_t launch_clip(const void *X, int xt, int64_t N, int64_t D_in, const void *W, int wt, int64_t D_out,
                       const float *s, const AlphaGrid &ratios, int n_ratio, int bits, int group, int32_t *ratio_idx,
                       float *scales, int8_t *codes, float *errors, void *ws, hipStream_t st) {
    unsigned char *w = static_cast<unsigned char *>(ws);
    switch (group) {
        case 32:
            return launch_clip_nb<2>(X, xt, N, D_in, W, wt, D_out, s, ratios, n_ratio, bits, ratio_idx, scales, codes,
                                     errors, w, st);
        case 64:
            return launch_clip_nb<4>(X, xt, N, D_in, W, wt, D_out, s, ratios, n_ratio, bits, ratio_idx, scales, codes,
                                     errors, w, st);
        default:
            return launch_clip_nb<8>(X, xt, N, D_in, W, wt, D_out, s, ratios, n_ratio, bits, ratio_idx, scales, codes,
                                     errors, w, st);
    }
}

}  // namespace awq
