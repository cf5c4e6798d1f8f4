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
#include <cfloat>

#include "awq_internal.h"

namespace awq {

namespace {

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

// bf16 activations: the same partial Gram matrix on v_mfma_f32_32x32x16_bf16
// (bf16 products are exact in float32, accumulation in float32 as above).
// Each 64-row slab of X_g is transposed into LDS ([channel][row], 16-byte
// k runs), so that one lane's A or B fragment (8 consecutive rows of one
// channel) is a single 16-byte read.  Output blocks of 32 x 32: wave w owns
// row block w and every column block (group 128), block w (group 64), or
// the only block (group 32, wave 0); for group 256, 8 waves of 8 blocks each.
constexpr int gram_threads(int GR) { return GR <= 128 ? 256 : 512; }

template <int GR>
__global__ __launch_bounds__(gram_threads(GR)) void gram_bf16_kernel(const uint16_t *__restrict__ X, int64_t N,
                                                                     int64_t D_in, float *__restrict__ part) {
    constexpr int NT = gram_threads(GR);
    constexpr int NWg = NT / 64;
    constexpr int RB = GR / 32;                  // 32-blocks per side
    constexpr int BPW = RB * RB >= NWg ? RB * RB / NWg : 1;   // blocks per wave
    constexpr int XS = 64 + 8;                   // row stride of the transposed slab (144 B)
    const int g = blockIdx.x, c = blockIdx.y, G = gridDim.x;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool active = wave * BPW < RB * RB;
    __shared__ __align__(16) uint16_t xt[GR][XS];
    floatx16 acc[BPW];
#pragma unroll
    for (int b = 0; b < BPW; ++b)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[b][i] = 0.0f;
    const int64_t n0 = static_cast<int64_t>(c) * kGramRows;
    const int64_t n1 = n0 + kGramRows < N ? n0 + kGramRows : N;
    for (int64_t nb0 = n0; nb0 < n1; nb0 += 64) {
        __syncthreads();
        // slab rows nb0 .. +64 (zero past n1), 8 channels per load, transposed
        for (int i = tid; i < 64 * (GR / 8); i += NT) {
            const int r = i % 64, c8 = i / 64;
            const int64_t n = nb0 + r;
            uint4 v = make_uint4(0u, 0u, 0u, 0u);
            if (n < n1) v = *reinterpret_cast<const uint4 *>(X + n * D_in + static_cast<int64_t>(g) * GR + c8 * 8);
            const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                xt[c8 * 8 + 2 * e][r] = static_cast<uint16_t>(w4[e] & 0xFFFFu);
                xt[c8 * 8 + 2 * e + 1][r] = static_cast<uint16_t>(w4[e] >> 16);
            }
        }
        __syncthreads();
        if (active) {
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                const int kofs = ks * 16 + 8 * (lane >> 5);
#pragma unroll
                for (int b = 0; b < BPW; ++b) {
                    const int blk = wave * BPW + b;
                    const int ib = blk / RB, jb = blk % RB;
                    const bf16x8 av = *reinterpret_cast<const bf16x8 *>(&xt[ib * 32 + (lane & 31)][kofs]);
                    const bf16x8 bv = *reinterpret_cast<const bf16x8 *>(&xt[jb * 32 + (lane & 31)][kofs]);
                    acc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bv, acc[b], 0, 0, 0);
                }
            }
        }
    }
    if (!active) return;
    // 32x32 C layout: register r holds row 8·(r/4) + 4·(lane/32) + r%4, column lane%32
    float *dst = part + (static_cast<int64_t>(c) * G + g) * GR * GR;
#pragma unroll
    for (int b = 0; b < BPW; ++b) {
        const int blk = wave * BPW + b;
        const int ib = blk / RB, jb = blk % RB;
#pragma unroll
        for (int r = 0; r < 16; ++r)
            dst[(ib * 32 + 8 * (r / 4) + 4 * (lane >> 5) + r % 4) * GR + jb * 32 + (lane & 31)] = acc[b][r];
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

// Power of two 2^e with v·2^e in [2^(top-1), 2^top) (v > 0 and finite),
// else 1; the exponent is clamped so that 2^e and 2^-e stay normal.
__device__ __forceinline__ int pow2_exp(float v, int top) {
    if (!(v > 0.0f) || !(v <= FLT_MAX)) return 0;
    int e = 0;
    frexpf(v, &e);
    const int k = top - e;
    return k < -100 ? -100 : (k > 100 ? 100 : k);
}

// hi/lo FP16 split of x (|x| < 2^15): hi = fp16(x), lo = fp16(x − hi); the
// difference is exact in float32, so hi + lo holds x to about 22 bits.
__device__ __forceinline__ void split16(float x, _Float16 &hi, _Float16 &lo) {
    hi = static_cast<_Float16>(x);
    lo = static_cast<_Float16>(x - static_cast<float>(hi));
}

// clip_code's common case without branches.  t is first clamped to
// ±(qmax + 1/4) (one v_med3): where |t| >= qmax + 1/4 the quotient is at
// least qmax + 1/4 − (qmax + 1)·2^-22 in magnitude, so clip_code gives ±qmax,
// and so does rint of the clamped t (which lies 1/4 from ±qmax, inside the
// margin); below that the argument of clip_code applies unchanged, and
// |rint(t)| <= qmax needs no clamp.  Sets `bad` where t lies within thr of a
// half-integer; the caller then takes clip_code for that run (rare).
__device__ __forceinline__ float clip_code_fast(float wp, float rstep, float qmax, float thr, bool &bad) {
    const float lim = qmax + 0.25f;
    const float t = __builtin_amdgcn_fmed3f(wp * rstep, -lim, lim);
    const float q = rintf(t);
    bad |= !(fabsf(t - q) < thr);
    return q;
}

// One workgroup: group g = blockIdx.x (GR rows), C columns (blockIdx.y): C =
// 8192 / GR with 4 waves for groups up to 128, and C = 64 with 8 waves for
// group 256.  Quantiser: thread t takes column t % C and the 32 rows
// 32·(t / C) .. +32 (the row part is uniform over a wave).  Matrix work: the
// GR x C product T = H_g·D on v_mfma_f32_32x32x16_f16 as output blocks of
// 32 x 32, two per wave (wave w: row block w % RBn, two column blocks), so
// that each wave keeps the fragments of one row block of H_g in registers.
//
// Precision: H_g·2^a and each column of D·2^b_o (powers of two; |H_g·2^a| <
// 2^15 since |H_ij| <= max_i H_ii, |D·2^b| < 2^14 from the bound
// |d_k| <= 2·m/s_k) are split into FP16 hi + lo parts and
// T = Hh·Dh + Hh·Dl + Hl·Dh (float32 accumulation; the dropped Hl·Dl term
// is 2^-22 relative).  E_o = 2^-(a+b_o) · sum_k d_k·T_k with d in float32.
// H_g's fragments stay in registers for all ratios; D's fragments and the
// float32 error weights go through LDS.  Two workgroups share a CU, so one's
// quantiser runs while the other's matrix work does.
constexpr int clip_cols(int GR) { return GR <= 128 ? 64 * (128 / GR) : 64; }
constexpr int clip_threads(int GR) { return GR <= 128 ? 256 : 512; }
constexpr int clip_min_blocks(int GR) { return GR <= 128 ? 2 : 1; }   // workgroups per CU

template <int GR, bool WB>
__global__ __launch_bounds__(clip_threads(GR), clip_min_blocks(GR)) void clip_kernel(
    const void *__restrict__ W, const float *__restrict__ s, const float *__restrict__ H, ClipArgs ca,
    int32_t *__restrict__ ratio_idx, float *__restrict__ scales, int8_t *__restrict__ codes,
    float *__restrict__ errors) {
    constexpr int C = clip_cols(GR);     // columns per workgroup
    constexpr int NT = clip_threads(GR);
    constexpr int NW = NT / 64;          // waves
    constexpr int RBn = GR / 32;         // row blocks of T
    constexpr int CBn = C / 32;          // column blocks of T
    constexpr int KS = GR / 16;          // k steps of 16
    constexpr int PARTS = NT / C;        // 32-row parts per column
    constexpr int DS = GR + 4;           // float32 error-weight row stride (16-byte reads without conflicts)
    static_assert(PARTS * 32 == GR && RBn * CBn == 2 * NW, "tile shape");
    const int g = blockIdx.x;
    const int64_t o0 = static_cast<int64_t>(blockIdx.y) * C;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col = tid % C;
    const int part = __builtin_amdgcn_readfirstlane(tid / C);   // C is a multiple of 64
    const int r0 = part * 32;
    const int64_t o = o0 + col;
    const bool live = o < ca.D_out;
    const int64_t j0 = static_cast<int64_t>(g) * GR;

    __shared__ half8 Bh[CBn * KS * 64];   // D·2^b hi parts, B-fragment order
    __shared__ half8 Bl[CBn * KS * 64];   // lo parts
    __shared__ __align__(16) float Dw[C][DS];   // float32 error weights, [column][row]
    __shared__ float Ep[RBn][C];          // per-row-block partial errors
    __shared__ float mred[PARTS][C];
    __shared__ float pre[2][NW];
    __shared__ int bsel[C];

    // group statistics: max_i H_ii (scale of H) and max_k fl(1/s_k)
    float hd = 0.0f, rsm = 0.0f;
    if (tid < GR) {
        hd = H[static_cast<int64_t>(g) * GR * GR + tid * (GR + 1)];
        rsm = 1.0f / s[j0 + tid];
    }
    for (int off = 32; off > 0; off >>= 1) {
        hd = fmaxf(hd, __shfl_xor(hd, off));
        rsm = fmaxf(rsm, __shfl_xor(rsm, off));
    }
    if (lane == 0) {
        pre[0][wave] = hd;
        pre[1][wave] = rsm;
    }
    // W' = fl(s·w) of this thread's 32 rows, and their absmax.  Columns past
    // D_out load a valid column and use 0, so that the 32 loads issue
    // back to back.
    float wp[32];
    float m = 0.0f;
    const int64_t oc = live ? o : ca.D_out - 1;
    const uint32_t keep = live ? 0xFFFFFFFFu : 0u;   // a mask, not a branch around the load
#pragma unroll
    for (int i = 0; i < 32; ++i) {
        const int64_t j = j0 + r0 + i;
        const uint32_t wb = WB ? static_cast<uint32_t>(static_cast<const uint16_t *>(W)[j * ca.D_out + oc]) << 16
                               : __float_as_uint(static_cast<const float *>(W)[j * ca.D_out + oc]);
        wp[i] = s[j] * __uint_as_float(wb & keep);
        m = fmaxf(m, fabsf(wp[i]));
    }
    mred[part][col] = m;
    __syncthreads();
    float hmax = pre[0][0], rsmax = pre[1][0];
#pragma unroll
    for (int w = 1; w < NW; ++w) {
        hmax = fmaxf(hmax, pre[0][w]);
        rsmax = fmaxf(rsmax, pre[1][w]);
    }
    float mcol = 0.0f;
#pragma unroll
    for (int p = 0; p < PARTS; ++p) mcol = fmaxf(mcol, mred[p][col]);
    const int ea = pow2_exp(hmax, 15);
    const int eb = pow2_exp(2.01f * mcol * rsmax, 14);   // |d·2^eb| < 2^14
    const float sa = ldexpf(1.0f, ea), sb = ldexpf(1.0f, eb);
    // fl(1/s) of this thread's 32 rows (uniform over a wave): in registers,
    // or for group 256 in LDS, where the registers are needed for H_g
    constexpr bool kRsLds = GR > 128;
    __shared__ float rsl[kRsLds ? GR : 1];
    float rsv[kRsLds ? 1 : 32];
    if constexpr (kRsLds) {
        if (tid < GR) rsl[tid] = 1.0f / s[j0 + tid];
        __syncthreads();
    } else {
#pragma unroll
        for (int i = 0; i < 32; ++i) rsv[i] = 1.0f / s[j0 + r0 + i];
    }
    auto rs_at = [&](int i) -> float {
        if constexpr (kRsLds) return rsl[r0 + i];
        else return rsv[i];
    };

    // this wave's A fragments (row block rb, every k step), split hi/lo
    const int rb = wave % RBn;
    const int cb0 = (wave / RBn) * 2;
    half8 Ah[KS], Al[KS];
    {
        const float *hrow = H + static_cast<int64_t>(g) * GR * GR + static_cast<int64_t>(rb * 32 + (lane & 31)) * GR;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const float4 v0 = *reinterpret_cast<const float4 *>(hrow + ks * 16 + 8 * (lane >> 5));
            const float4 v1 = *reinterpret_cast<const float4 *>(hrow + ks * 16 + 8 * (lane >> 5) + 4);
            const float hv[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                _Float16 hi, lo;
                split16(hv[e] * sa, hi, lo);
                Ah[ks][e] = hi;
                Al[ks][e] = lo;
            }
        }
    }

    const float qmax = static_cast<float>((1 << (ca.bits - 1)) - 1);
    const float thr = 0.5f - (qmax + 1.0f) * 0x1p-20f;
    float best_e = INFINITY;   // kept by the part-0 thread of each column
    int best_i = 0;
    for (int ri = 0; ri < ca.n_ratio; ++ri) {
        // quantiser at this ratio: error weights of this thread's 32 rows
        const float step = (ca.ratios.v[ri] * mcol) / qmax;
        const float rstep = step > 0.0f ? 1.0f / step : 0.0f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            float d[8], q[8];
            half8 hh, hl;
            bool bad = false;
#pragma unroll
            for (int e = 0; e < 8; ++e) q[e] = clip_code_fast(wp[8 * j + e], rstep, qmax, thr, bad);
            if (bad) {
#pragma unroll
                for (int e = 0; e < 8; ++e) q[e] = clip_code(wp[8 * j + e], step, rstep, qmax, thr);
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int i = 8 * j + e;
                d[e] = fmaf(q[e], step, -wp[i]) * rs_at(i);
                _Float16 hi, lo;
                split16(d[e] * sb, hi, lo);
                hh[e] = hi;
                hl[e] = lo;
            }
            *reinterpret_cast<float4 *>(&Dw[col][r0 + 8 * j]) = float4{d[0], d[1], d[2], d[3]};
            *reinterpret_cast<float4 *>(&Dw[col][r0 + 8 * j + 4]) = float4{d[4], d[5], d[6], d[7]};
            const int krun = (r0 >> 3) + j;   // 8-row run index
            const int f = ((col >> 5) * KS + (krun >> 1)) * 64 + (col & 31) + 32 * (krun & 1);
            Bh[f] = hh;
            Bl[f] = hl;
        }
        __syncthreads();
        // T blocks (rb, cb0) and (rb, cb0 + 1), interleaved (two independent
        // accumulation chains); then the row block's share of E
        floatx16 acc[2];
#pragma unroll
        for (int jb = 0; jb < 2; ++jb)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[jb][i] = 0.0f;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            half8 bh[2], bl[2];
#pragma unroll
            for (int jb = 0; jb < 2; ++jb) {
                bh[jb] = Bh[((cb0 + jb) * KS + ks) * 64 + lane];
                bl[jb] = Bl[((cb0 + jb) * KS + ks) * 64 + lane];
            }
#pragma unroll
            for (int jb = 0; jb < 2; ++jb) acc[jb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(Ah[ks], bh[jb], acc[jb], 0, 0, 0);
#pragma unroll
            for (int jb = 0; jb < 2; ++jb) acc[jb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(Ah[ks], bl[jb], acc[jb], 0, 0, 0);
#pragma unroll
            for (int jb = 0; jb < 2; ++jb) acc[jb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(Al[ks], bh[jb], acc[jb], 0, 0, 0);
        }
        // 32x32 C layout: register r holds row 8·(r/4) + 4·(lane/32) + r%4, column lane%32
#pragma unroll
        for (int jb = 0; jb < 2; ++jb) {
            const int cc = (cb0 + jb) * 32 + (lane & 31);
            float e = 0.0f;
#pragma unroll
            for (int qd = 0; qd < 4; ++qd) {
                const float4 dv = *reinterpret_cast<const float4 *>(&Dw[cc][rb * 32 + 8 * qd + 4 * (lane >> 5)]);
                e = fmaf(acc[jb][4 * qd + 0], dv.x, e);
                e = fmaf(acc[jb][4 * qd + 1], dv.y, e);
                e = fmaf(acc[jb][4 * qd + 2], dv.z, e);
                e = fmaf(acc[jb][4 * qd + 3], dv.w, e);
            }
            e += __shfl_xor(e, 32);
            if (lane < 32) Ep[rb][cc] = e;
        }
        __syncthreads();
        if (part == 0) {
            float e = 0.0f;
#pragma unroll
            for (int b = 0; b < RBn; ++b) e += Ep[b][col];
            e = ldexpf(e, -(ea + eb));   // exact
            if (live) {
                if (errors) errors[(static_cast<int64_t>(ri) * ca.G + g) * ca.D_out + o] = e;
                if (e < best_e) {
                    best_e = e;
                    best_i = ri;
                }
            }
        }
    }
    if (part == 0) bsel[col] = best_i;
    __syncthreads();
    if (!live) return;
    const int bi = bsel[col];
    const float step = (ca.ratios.v[bi] * mcol) / qmax;
    const float rstep = step > 0.0f ? 1.0f / step : 0.0f;
    if (codes) {
#pragma unroll
        for (int i = 0; i < 32; ++i)
            codes[(j0 + r0 + i) * ca.D_out + o] = static_cast<int8_t>(clip_code(wp[i], step, rstep, qmax, thr));
    }
    if (part == 0) {
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
        hipLaunchKernelGGL((gram_bf16_kernel<GR>), gg, dim3(gram_threads(GR)), 0, st, static_cast<const uint16_t *>(X),
                           N, D_in, part);
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
    constexpr int C = clip_cols(GR);   // columns per clip workgroup
    const dim3 cg(static_cast<unsigned>(G), static_cast<unsigned>((D_out + C - 1) / C));
    if (wt == 1)
        hipLaunchKernelGGL((clip_kernel<GR, true>), cg, dim3(clip_threads(GR)), 0, st, W, s, H, ca, ratio_idx,
                           scales, codes, errors);
    else
        hipLaunchKernelGGL((clip_kernel<GR, false>), cg, dim3(clip_threads(GR)), 0, st, W, s, H, ca, ratio_idx,
                           scales, codes, errors);
    return hipGetLastError();
}

}  // namespace

bool clip_group_supported(int group) { return group == 32 || group == 64 || group == 128 || group == 256; }

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
        case 256:
            return launch_clip_nb<16>(X, xt, N, D_in, W, wt, D_out, s, ratios, n_ratio, bits, ratio_idx, scales,
                                      codes, errors, w, st);
        default:
            return launch_clip_nb<8>(X, xt, N, D_in, W, wt, D_out, s, ratios, n_ratio, bits, ratio_idx, scales, codes,
                                     errors, w, st);
    }
}

}  // namespace awq
