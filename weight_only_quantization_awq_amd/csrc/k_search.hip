// The per-layer alpha grid search of AWQ on one MI355X.
//
// [CA] "縮放因子最佳化的完整流程": for every grid value alpha, s = a^alpha,
// W' = diag(s)·W, per-group quantisation to Ŵ', L(alpha) = ||X·S⁻¹·Ŵ' − X·W||²,
// alpha* = argmin L, record s* = a^alpha*.  [MR] "搜索最优比例" states the same
// objective and one-dimensional search space.
//
// Pipeline (all on the caller's stream, scratch in the caller's workspace):
//   1. absmax     max|X| and max|W| (HBM pass)            -> power-of-two prescales
//   2. scale_tab  s_j(alpha), 1/s_j(alpha), per-alpha error-weight prescale
//   3. prep_x     X -> MFMA fragment order (fp16·2^kx, or fp32), zero padded
//   4. quant_all  for every alpha and (group, column): exact float32
//                 quantiser, then the error weight D = Ŵ'/s − W, written in
//                 fragment order (fp16·2^kd, or fp32)
//   5. loss_gemm  E = X·D for all alphas in one launch on the matrix cores;
//                 the epilogue squares and sums the 256x256 tile in float64
//   6. reduce     fixed-order float64 sum of tile partials -> L(alpha); first
//                 argmin; non-finite check; s* copy
//   7. select     re-run the quantiser at alpha* -> int8 codes and steps
//
// Error-weight form.  Because (X·S⁻¹)·Ŵ' − X·W = X·(S⁻¹·Ŵ' − W) exactly, the
// contraction runs on the small difference D (a quantisation residual) and
// never forms Ŵ' or X·W.  Rounding D to the 16-bit matrix-core format then
// perturbs L only at the 1e-6..1e-5 level, while rounding X·S⁻¹ or Ŵ' before a
// subtraction of two large products would bias L by ~1e-3.
#include "awq_internal.h"

#include <float.h>

#pragma clang fp contract(off)

namespace awq {

// ---------------------------------------------------------------- helpers --

__device__ __forceinline__ float ld_f(const void *p, int dt, int64_t i) {
    if (dt == 1) {
        const uint16_t v = static_cast<const uint16_t *>(p)[i];
        return __uint_as_float(static_cast<uint32_t>(v) << 16);
    }
    return static_cast<const float *>(p)[i];
}

__global__ void init_state_kernel(SearchState *st) {
    if (threadIdx.x == 0) {
        st->max_abs_x_bits = 0u;
        st->max_abs_w_bits = 0u;
        st->kx = 0;
    }
    if (threadIdx.x < 64) st->kd[threadIdx.x] = 0;
}

// max|v| over a buffer; NaN or Inf anywhere yields +Inf (flagged later).
__global__ __launch_bounds__(256) void absmax_kernel(const void *__restrict__ p, int dt, int64_t count,
                                                     unsigned int *__restrict__ out) {
    float m = 0.0f;
    const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
    int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (dt == 1) {
        const int64_t n8 = count / 8;
        const uint4 *p4 = static_cast<const uint4 *>(p);
        for (int64_t v = i; v < n8; v += stride) {
            const uint4 u = p4[v];
            const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
            for (int h = 0; h < 4; ++h) {
                const float lo = fabsf(__uint_as_float(w[h] << 16));
                const float hi = fabsf(__uint_as_float(w[h] & 0xFFFF0000u));
                m = (lo > m || lo != lo) ? (lo != lo ? INFINITY : lo) : m;
                m = (hi > m || hi != hi) ? (hi != hi ? INFINITY : hi) : m;
            }
        }
        for (int64_t v = n8 * 8 + i; v < count; v += stride) {
            const float x = fabsf(ld_f(p, 1, v));
            m = (x > m || x != x) ? (x != x ? INFINITY : x) : m;
        }
    } else {
        const int64_t n4 = count / 4;
        const float4 *p4 = static_cast<const float4 *>(p);
        for (int64_t v = i; v < n4; v += stride) {
            const float4 u = p4[v];
            const float w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
            for (int h = 0; h < 4; ++h) {
                const float x = fabsf(w[h]);
                m = (x > m || x != x) ? (x != x ? INFINITY : x) : m;
            }
        }
        for (int64_t v = n4 * 4 + i; v < count; v += stride) {
            const float x = fabsf(ld_f(p, 0, v));
            m = (x > m || x != x) ? (x != x ? INFINITY : x) : m;
        }
    }
    // wave then block reduction (max is order independent)
    for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
    __shared__ float red[4];
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
    __syncthreads();
    if (threadIdx.x == 0) {
        float b = red[0];
        for (int w = 1; w < static_cast<int>(blockDim.x >> 6); ++w) b = fmaxf(b, red[w]);
        atomicMax(out, __float_as_uint(b));
    }
}

// Candidate scales for one alpha per workgroup, plus the error-weight
// prescale.  |D_jo| = |Ŵ'_jo/s_j − w_jo| <= step_go/(2 s_j) and
// step_go <= max_{i in g} s_i · max|W| / qmax, so
// |D| <= max|W| · max_g(max_{i in g} s_i / min_{j in g} s_j) / (2 qmax).
// Scaling D by 2^kd with that bound below 2^14 keeps fp16 far from overflow
// and keeps the significant part of D in the fp16 normal range.
__global__ __launch_bounds__(256) void scale_table_kernel(const float *__restrict__ a, AlphaGrid alphas,
                                                          int64_t D_in, int group, int bits, bool f16,
                                                          float *__restrict__ s_tab,
                                                          float *__restrict__ invp_tab,
                                                          SearchState *__restrict__ st) {
    const int k = blockIdx.x;
    const double alpha = static_cast<double>(alphas.v[k]);
    const int64_t G = D_in / group;
    float *s_row = s_tab + k * D_in;
    float *invp_row = invp_tab + k * D_in;
    for (int64_t j = threadIdx.x; j < D_in; j += blockDim.x) {
        const float aj = a[j];
        // dead channel (zero or below the smallest normal float) keeps s = 1
        s_row[j] = (aj >= FLT_MIN) ? static_cast<float>(pow(static_cast<double>(aj), alpha)) : 1.0f;
    }
    __syncthreads();  // s_row written by this workgroup is now visible to it
    double rmax = 1.0;
    for (int64_t g = threadIdx.x; g < G; g += blockDim.x) {
        float smax = 0.0f, smin = INFINITY;
        for (int r = 0; r < group; ++r) {
            const float s = s_row[g * group + r];
            smax = fmaxf(smax, s);
            smin = fminf(smin, s);
        }
        const double r = static_cast<double>(smax) / static_cast<double>(smin);
        rmax = (r > rmax || r != r) ? r : rmax;
    }
    for (int off = 32; off > 0; off >>= 1) {
        const double o = __shfl_xor(rmax, off);
        rmax = (o > rmax || o != o) ? o : rmax;
    }
    __shared__ double red[4];
    __shared__ int kd_sh;
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = rmax;
    __syncthreads();
    if (threadIdx.x == 0) {
        double R = red[0];
        for (int w = 1; w < static_cast<int>(blockDim.x >> 6); ++w) R = (red[w] > R || red[w] != red[w]) ? red[w] : R;
        int kd = 0;
        if (f16) {
            const double wmax = static_cast<double>(__uint_as_float(st->max_abs_w_bits));
            const double qmax = static_cast<double>((1 << (bits - 1)) - 1);
            const double B = wmax * R / (2.0 * qmax) * 1.01;
            if (B > 0.0 && B <= DBL_MAX) {
                int e = 0;
                frexp(B, &e);
                kd = 14 - e;
            }
            kd = kd < -120 ? -120 : (kd > 120 ? 120 : kd);
        }
        st->kd[k] = kd;
        kd_sh = kd;
        if (k == 0) {
            int kx = 0;
            if (f16) {
                const float xm = __uint_as_float(st->max_abs_x_bits);
                if (xm > 0.0f && xm <= FLT_MAX) {
                    int e = 0;
                    frexpf(xm, &e);
                    kx = 14 - e;
                }
                kx = kx < -120 ? -120 : (kx > 120 ? 120 : kx);
            }
            st->kx = kx;
        }
    }
    __syncthreads();
    // 2^kd / s_j: folds the error-weight prescale into the per-row factor
    const float pre = ldexpf(1.0f, kd_sh);
    for (int64_t j = threadIdx.x; j < D_in; j += blockDim.x) invp_row[j] = pre / s_row[j];
}

// X -> fragment order.  fp16 path: one thread per (row, 64-k block); rows
// vary fastest across a wave so that each 16-byte store lands next to its
// neighbour's inside the same 1 KiB chunk.
__global__ __launch_bounds__(256) void prep_x_f16_kernel(const uint16_t *__restrict__ X, SearchShape sh,
                                                         const SearchState *__restrict__ st,
                                                         half8 *__restrict__ Xf) {
    const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (idx >= sh.Mp * sh.KB64) return;
    const int64_t row = idx % sh.Mp;
    const int64_t kb = idx / sh.Mp;
    const float scale = ldexpf(1.0f, st->kx);
    const int64_t mb = row / 32, r = row % 32;
#pragma unroll
    for (int run = 0; run < 8; ++run) {
        const int64_t k0 = kb * 64 + run * 8;
        half8 h;
        if (row < sh.N && k0 < sh.D_in) {
            const uint4 u = *reinterpret_cast<const uint4 *>(X + row * sh.D_in + k0);
            const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                h[2 * p] = static_cast<_Float16>(__uint_as_float(w[p] << 16) * scale);
                h[2 * p + 1] = static_cast<_Float16>(__uint_as_float(w[p] & 0xFFFF0000u) * scale);
            }
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) h[i] = static_cast<_Float16>(0.0f);
        }
        const int64_t kq = run / 2, c = run % 2;
        Xf[((kb * sh.MB32 + mb) * 4 + kq) * 64 + c * 32 + r] = h;
    }
}

// fp32 path: one thread per element.
__global__ __launch_bounds__(256) void prep_x_f32_kernel(const void *__restrict__ X, int xt, SearchShape sh,
                                                         float *__restrict__ Xf) {
    const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (idx >= sh.Mp * sh.Kp) return;
    const int64_t row = idx / sh.Kp, k = idx % sh.Kp;
    const float v = (row < sh.N && k < sh.D_in) ? ld_f(X, xt, row * sh.D_in + k) : 0.0f;
    const int64_t kb = k / 32, ks = (k % 32) / 4, c = k % 4, mb = row / 16, r = row % 16;
    Xf[((kb * sh.MB + mb) * 8 + ks) * 64 + c * 16 + r] = v;
}

// ------------------------------------------------------------ quantiser ----
// [CA] "量化數學基礎": per group, step = max|w| / (2^(b-1)-1) and
// w_q = round(w / step) clipped to ±(2^(b-1)-1).  Float32 IEEE: the product
// s·w, true division twice, round half to even; an all-zero group has step 0.

// fp16 error-weight fragment slot (in half8 units) of rows [j, j+8), column o.
__device__ __forceinline__ int64_t f16_dchunk(int64_t j, int64_t o, const SearchShape &sh) {
    const int64_t kb = j / 64, kq = (j % 64) / 16, c = (j % 16) / 8;
    const int64_t nb = o / 32, n = o % 32;
    return ((kb * sh.NB32 + nb) * 4 + kq) * 64 + c * 32 + n;
}

// Writes the error weights of rows [j, j + ROWS) of column o for one alpha,
// given the group's step.  ROWS is a multiple of 8.
// Exact quantiser for 8 values of one group: q_i = clamp(rint(fl(wp_i/step)),
// ±qmax) with the IEEE float32 quotient, step > 0.
// Fast path: t = fl(wp · rstep) with rstep = fl(1/step).  Then
// |t − wp/step| <= |wp/step|·(2^-23 + 2^-48), and the IEEE quotient is within
// 2^-24·|wp/step| of wp/step, so whenever t is farther than |t|·2^-20 from
// every half-integer both round to the same integer (and neither is a tie).
// Otherwise (about one value in 10^5, or a non-finite t) the 8 values are
// recomputed with true division.  t − rint(t) is exact (Sterbenz).
__device__ __forceinline__ void quant8(const float *wp, float step, float rstep, float qmax, float *q) {
    bool exact_needed = false;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float t = wp[i] * rstep;
        const float qt = rintf(t);
        exact_needed |= !(fabsf(t - qt) < fmaf(-fabsf(t), 0x1p-20f, 0.5f));
        q[i] = qt;
    }
    if (exact_needed) {
#pragma unroll
        for (int i = 0; i < 8; ++i) q[i] = rintf(wp[i] / step);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) q[i] = fminf(fmaxf(q[i], -qmax), qmax);
}

// Writes the error weights of rows [j, j + ROWS) of column o for one alpha,
// given the group's step.  ROWS is a multiple of 8.
// Writes the error weights of rows [j, j + ROWS) of column o for one alpha,
// given the group's step.  ROWS is a multiple of 8.  With W' = s·w and
// Ŵ' = q·step, (Ŵ'/s − w)·2^kd = (q·step − W')·(2^kd/s) up to the float32
// rounding of W' (2^-24 relative to w, far below the error weight itself).
template <bool F16, int ROWS>
__device__ __forceinline__ void emit_rows(const float *w, const float *__restrict__ s, const float *__restrict__ invp,
                                          float step, float qmax, int64_t j, int64_t o,
                                          const SearchShape &sh, void *__restrict__ Dk) {
    const int64_t nb = o / 16, n = o % 16;
    const float rstep = 1.0f / step;
#pragma unroll
    for (int r0 = 0; r0 < ROWS; r0 += 8) {
        float wp[8], q[8], d[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            // recompute s·w here rather than keep the max pass's products
            // live (an opaque copy of s stops the compiler from reusing them)
            float sv = s[r0 + i];
            asm volatile("" : "+s"(sv));
            wp[i] = sv * w[r0 + i];
        }
        if (step > 0.0f) {
            quant8(wp, step, rstep, qmax, q);
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) q[i] = 0.0f;
        }
        // tolerance path, not bit-exact
#pragma unroll
        for (int i = 0; i < 8; ++i) d[i] = fmaf(q[i], step, -wp[i]) * invp[r0 + i];
        const int64_t jj = j + r0;
        const int64_t kb = jj / 32;
        if constexpr (F16) {
            half8 h;
#pragma unroll
            for (int i = 0; i < 8; ++i) h[i] = static_cast<_Float16>(d[i]);
            static_cast<half8 *>(Dk)[f16_dchunk(jj, o, sh)] = h;
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int64_t ji = jj + i;
                const int64_t ks = (ji % 32) / 4, c = ji % 4;
                static_cast<float *>(Dk)[((kb * sh.NB + nb) * 8 + ks) * 64 + c * 16 + n] = d[i];
            }
        }
    }
}

template <bool F16>
__device__ __forceinline__ void emit_zero(int64_t j0, int rows, int64_t o, const SearchShape &sh, void *Dk) {
    const int64_t nb = o / 16, n = o % 16;
    for (int r0 = 0; r0 < rows; r0 += 8) {
        const int64_t j = j0 + r0;
        const int64_t kb = j / 32;
        if constexpr (F16) {
            half8 h;
#pragma unroll
            for (int i = 0; i < 8; ++i) h[i] = static_cast<_Float16>(0.0f);
            static_cast<half8 *>(Dk)[f16_dchunk(j, o, sh)] = h;
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int64_t ji = j + i;
                const int64_t ks = (ji % 32) / 4, c = ji % 4;
                static_cast<float *>(Dk)[((kb * sh.NB + nb) * 8 + ks) * 64 + c * 16 + n] = 0.0f;
            }
        }
    }
}

// One thread per (group, column) covering every alpha: W is read once.
// GC > 0: the group size is a compile-time constant and the column slice
// lives in registers; GC == 0: any multiple of 8, re-read through the cache.
template <bool F16, int GC>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3))) void quant_all_kernel(const void *__restrict__ W, int wt, SearchShape sh,
                                                        const float *__restrict__ s_tab,
                                                        const float *__restrict__ invp_tab,
                                                        const SearchState *__restrict__ st,
                                                        void *__restrict__ Df) {
    const int64_t o = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    const int64_t g = blockIdx.y;
    if (o >= sh.Np) return;
    const int group = GC > 0 ? GC : sh.group;
    const int64_t j0 = g * group;
    const int64_t G = sh.D_in / group;
    const size_t dstride = static_cast<size_t>(sh.Kp) * static_cast<size_t>(sh.Np) * (F16 ? 2 : 4);
    const float qmax = static_cast<float>((1 << (sh.bits - 1)) - 1);
    unsigned char *D0 = static_cast<unsigned char *>(Df);
    if (o >= sh.D_out) {
        for (int k = 0; k < sh.n_alpha; ++k) emit_zero<F16>(j0, group, o, sh, D0 + k * dstride);
    } else {
        if constexpr (GC > 0) {
            float w[GC];
#pragma unroll
            for (int r = 0; r < GC; ++r) w[r] = ld_f(W, wt, (j0 + r) * sh.D_out + o);
            for (int k = 0; k < sh.n_alpha; ++k) {
                const float *s = s_tab + k * sh.D_in + j0;
                const float *invp = invp_tab + k * sh.D_in + j0;
                float m = 0.0f;
#pragma unroll
                for (int r = 0; r < GC; ++r) m = fmaxf(m, fabsf(s[r] * w[r]));
                const float step = m / qmax;
                emit_rows<F16, GC>(w, s, invp, step, qmax, j0, o, sh, D0 + k * dstride);
            }
        } else {
            for (int k = 0; k < sh.n_alpha; ++k) {
                const float *s = s_tab + k * sh.D_in + j0;
                const float *invp = invp_tab + k * sh.D_in + j0;
                float m = 0.0f;
                for (int r = 0; r < group; ++r) m = fmaxf(m, fabsf(s[r] * ld_f(W, wt, (j0 + r) * sh.D_out + o)));
                const float step = m / qmax;
                for (int r0 = 0; r0 < group; r0 += 8) {
                    float w8[8];
#pragma unroll
                    for (int i = 0; i < 8; ++i) w8[i] = ld_f(W, wt, (j0 + r0 + i) * sh.D_out + o);
                    emit_rows<F16, 8>(w8, s + r0, invp + r0, step, qmax, j0 + r0, o, sh, D0 + k * dstride);
                }
            }
        }
    }
    // zero the k padding below the last group
    if (g == G - 1 && sh.Kp > sh.D_in) {
        for (int k = 0; k < sh.n_alpha; ++k)
            emit_zero<F16>(sh.D_in, static_cast<int>(sh.Kp - sh.D_in), o, sh, D0 + k * dstride);
    }
}

// ------------------------------------------------------- loss contraction --

// Tile scheduling.  Workgroups are dispatched round-robin over the 8 XCDs
// (blockIdx % 8), each with its own L2.  Logical tiles are renumbered so that
// every XCD receives one contiguous range, and inside that range tiles are
// walked in groups of 4 row-tiles x all column-tiles: the ~32 workgroups an
// XCD runs at once then share a few X row-blocks and error-weight column
// strips in their L2 instead of each streaming its own from HBM.
__device__ __forceinline__ void map_tile(const SearchShape &sh, int &L, int &alpha, int &tm, int &tn) {
    const unsigned tiles = static_cast<unsigned>(sh.tiles_m * sh.tiles_n);
    const unsigned total = tiles * static_cast<unsigned>(sh.n_alpha);
    const unsigned bid = blockIdx.x;
    const unsigned xcd = bid % 8u, local = bid / 8u, q = total / 8u, r = total % 8u;
    const unsigned Lu = xcd * q + (xcd < r ? xcd : r) + local;
    L = static_cast<int>(Lu);
    alpha = static_cast<int>(Lu / tiles);
    const unsigned t = Lu % tiles;
    constexpr unsigned GM = 4;
    const unsigned tiles_m = static_cast<unsigned>(sh.tiles_m);
    const unsigned per_group = GM * static_cast<unsigned>(sh.tiles_n);
    const unsigned first_m = (t / per_group) * GM;
    const unsigned gm = (tiles_m - first_m) < GM ? (tiles_m - first_m) : GM;
    const unsigned in_group = t % per_group;
    tm = static_cast<int>(first_m + in_group % gm);
    tn = static_cast<int>(in_group / gm);
}

__device__ __forceinline__ double wave_sum(double v) {
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
    return v;
}

// fp16 path.  E = X·D over one 256x256 output tile of one alpha with
// v_mfma_f32_32x32x16_f16.  Four waves; wave w owns columns [64w, 64w+64)
// of the tile and all 256 rows (8 x 2 accumulator blocks of 32x32 = 256
// accumulation registers).  Per 64-k stage the workgroup copies the 32 KiB
// X block straight into LDS (global_load_lds, no register staging; four
// buffers, the next three stages in flight while the current one feeds the
// matrix cores) and each wave loads its own 8 KiB of error weights into
// registers three stages ahead.  One barrier per stage.
__global__ __launch_bounds__(kThreads, 1) void loss_gemm_f16_kernel(const half8 *__restrict__ Xf,
                                                                    const half8 *__restrict__ Df,
                                                                    double *__restrict__ partials, SearchShape sh) {
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    int L, alpha, tm, tn;
    map_tile(sh, L, alpha, tm, tn);

    // four distinct LDS objects (4 x 32 KiB), so the compiler can tell the
    // copies into one buffer from the reads of another
    __shared__ half8 As0[32 * 64];
    __shared__ half8 As1[32 * 64];
    __shared__ half8 As2[32 * 64];
    __shared__ half8 As3[32 * 64];
    const int64_t xstride = sh.MB32 * 4 * 64;          // half8 per 64-k stage of X
    const int64_t dstride = sh.NB32 * 4 * 64;          // half8 per 64-k stage of D
    const half8 *xsrc = Xf + (static_cast<int64_t>(tm) * 8 + wave * 2) * 4 * 64 + lane;  // this wave's 8 chunks
    const half8 *dsrc = Df + (static_cast<int64_t>(alpha) * sh.KB64 * sh.NB32 + tn * 8 + wave * 2) * 4 * 64 + lane;

    floatx16 acc[8][2];
#pragma unroll
    for (int m = 0; m < 8; ++m)
#pragma unroll
        for (int n = 0; n < 2; ++n)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[m][n][i] = 0.0f;

    half8 b0[8], b1[8], b2[8], b3[8];

    auto load_a = [&](int64_t kb, int buf) {
        const half8 *src = xsrc + kb * xstride;
#pragma unroll
        for (int i = 0; i < 8; ++i)
            __builtin_amdgcn_global_load_lds(
                (const __attribute__((address_space(1))) void *)(src + i * 64),
                (__attribute__((address_space(3))) void *)((buf == 0 ? As0 : (buf == 1 ? As1 : (buf == 2 ? As2 : As3))) + (wave * 8 + i) * 64), 16, 0,
                0);
    };
    auto load_b = [&](int64_t kb, half8 *b) {
        const half8 *src = dsrc + kb * dstride;
#pragma unroll
        for (int i = 0; i < 8; ++i) b[i] = src[i * 64];
    };
    // One stage = 4 k-steps of 16.  The 8 A fragments of k-step kq+1 are read
    // from LDS while the 16 MFMAs of k-step kq run (two register sets), one
    // read per two MFMAs, so LDS latency hides behind matrix work.
    auto read_a = [&](int buf, int kq, half8 *a) {
        const half8 *base = (buf == 0 ? As0 : (buf == 1 ? As1 : (buf == 2 ? As2 : As3))) + kq * 64 + lane;
#pragma unroll
        for (int m = 0; m < 8; ++m) a[m] = base[m * 4 * 64];
    };
    auto mma_step = [&](const half8 *a, const half8 *b, int kq, int buf, half8 *a_next) {
#pragma unroll
        for (int m = 0; m < 8; ++m) {
            acc[m][0] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[m], b[kq], acc[m][0], 0, 0, 0);
            acc[m][1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[m], b[4 + kq], acc[m][1], 0, 0, 0);
            if (a_next)
                a_next[m] = (buf == 0 ? As0 : (buf == 1 ? As1 : (buf == 2 ? As2 : As3)))[(m * 4 + kq + 1) * 64 + lane];
        }
    };
    // Scheduling pattern of one stage (one scheduling region after the stage
    // barrier): the 8 LDS reads of k-step 0, then 16 units of
    // "2 MFMA, 1 LDS read, 2 MFMA, 1 LDS read, 1 global copy" (LDS reads only
    // while k-steps 1..3 still need them).  Spreading the 16 copies of the
    // stage three ahead over the matrix work keeps the CU's single texture
    // address path from stalling every wave at once, as a burst after the
    // barrier does.
    auto pin_schedule = [&]() {
        __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
            if (u < 12) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
            if (u < 12) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);
        }
    };
    auto compute = [&](int buf, const half8 *b) {
        half8 a0[8], a1[8];
        read_a(buf, 0, a0);
        mma_step(a0, b, 0, buf, a1);
        mma_step(a1, b, 1, buf, a0);
        mma_step(a0, b, 2, buf, a1);
        mma_step(a1, b, 3, buf, nullptr);
    };

    // Four-stage ring: stages s, s+1 and s+2 are in flight while stage s is
    // consumed, so each copy has three stages of matrix work (~3 us) to land;
    // shallower rings leave the matrix cores waiting on L2 misses.  After the
    // barrier of stage s the copies of stage s+3 are issued and pinned there
    // (sched_barrier), then stage s feeds the matrix cores.  Each stage is 16
    // vector-memory operations per wave (8 LDS copies + 8 register loads), so
    // "stage s has landed" is vmcnt <= 32.  Past the end, the last stage is
    // re-loaded into the idle buffer instead of branching.
    const int64_t KB = sh.KB64;
    const int64_t last = KB - 1;
    auto clampk = [&](int64_t k) { return k < last ? k : last; };
    load_a(0, 0);
    load_b(0, b0);
    load_a(clampk(1), 1);
    load_b(clampk(1), b1);
    load_a(clampk(2), 2);
    load_b(clampk(2), b2);
    // Stage barrier without a memory fence: a fenced __syncthreads would wait
    // for every copy in flight (vmcnt(0)), collapsing the ring.  Each wave
    // waits for its own stage-s copies and its LDS reads, then all waves meet.
    auto stage_barrier = [&]() {
        __builtin_amdgcn_s_waitcnt(0x8070);  // vmcnt(32) lgkmcnt(0)
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
    };
    int64_t kb = 0;
    for (; kb + 4 <= KB; kb += 4) {
        stage_barrier();  // stage kb landed everywhere; buffer 3 is free
        __builtin_amdgcn_sched_barrier(0);
        load_a(clampk(kb + 3), 3);
        load_b(clampk(kb + 3), b3);
        compute(0, b0);
        pin_schedule();
        __builtin_amdgcn_sched_barrier(0);
        stage_barrier();
        __builtin_amdgcn_sched_barrier(0);
        load_a(clampk(kb + 4), 0);
        load_b(clampk(kb + 4), b0);
        compute(1, b1);
        pin_schedule();
        __builtin_amdgcn_sched_barrier(0);
        stage_barrier();
        __builtin_amdgcn_sched_barrier(0);
        load_a(clampk(kb + 5), 1);
        load_b(clampk(kb + 5), b1);
        compute(2, b2);
        pin_schedule();
        __builtin_amdgcn_sched_barrier(0);
        stage_barrier();
        __builtin_amdgcn_sched_barrier(0);
        load_a(clampk(kb + 6), 2);
        load_b(clampk(kb + 6), b2);
        compute(3, b3);
        pin_schedule();
        __builtin_amdgcn_sched_barrier(0);
    }
    // 0..3 stages remain, in buffers 0, 1, 2
    __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (kb < KB) compute(0, b0);
    if (kb + 1 < KB) compute(1, b1);
    if (kb + 2 < KB) compute(2, b2);

    double ssum = 0.0;
#pragma unroll
    for (int m = 0; m < 8; ++m)
#pragma unroll
        for (int n = 0; n < 2; ++n)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const double v = static_cast<double>(acc[m][n][i]);
                ssum += v * v;
            }
    ssum = wave_sum(ssum);
    __shared__ double wred[4];
    if (lane == 0) wred[wave] = ssum;
    __syncthreads();
    if (tid == 0) partials[L] = ((wred[0] + wred[1]) + wred[2]) + wred[3];
}

// fp32 path (small layers, fp32 inputs): v_mfma_f32_16x16x4_f32, wave w owns
// columns [64w, 64w+64) and all 256 rows of the tile; X staged through LDS.
__global__ __launch_bounds__(kThreads, 1) void loss_gemm_f32_kernel(const float *__restrict__ Xf,
                                                                    const float *__restrict__ Df,
                                                                    double *__restrict__ partials, SearchShape sh) {
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    int L, alpha, tm, tn;
    map_tile(sh, L, alpha, tm, tn);

    floatx4 acc[16][4];
#pragma unroll
    for (int i = 0; i < 16; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};

    __shared__ float Af[16 * 8 * 64];
    for (int64_t kb = 0; kb < sh.KB; ++kb) {
        const float4 *src = reinterpret_cast<const float4 *>(Xf + (kb * sh.MB + static_cast<int64_t>(tm) * 16) * 512);
        __syncthreads();
#pragma unroll
        for (int i = 0; i < 8; ++i) reinterpret_cast<float4 *>(Af)[tid + i * 256] = src[tid + i * 256];
        __syncthreads();
#pragma unroll 2
        for (int ks = 0; ks < 8; ++ks) {
            float b[4];
#pragma unroll
            for (int nt = 0; nt < 4; ++nt)
                b[nt] = Df[(((static_cast<int64_t>(alpha) * sh.KB + kb) * sh.NB + tn * 16 + wave * 4 + nt) * 8 + ks) * 64 + lane];
#pragma unroll
            for (int mt = 0; mt < 16; ++mt) {
                const float av = Af[(mt * 8 + ks) * 64 + lane];
#pragma unroll
                for (int nt = 0; nt < 4; ++nt)
                    acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x4f32(av, b[nt], acc[mt][nt], 0, 0, 0);
            }
        }
    }

    double ssum = 0.0;
#pragma unroll
    for (int mt = 0; mt < 16; ++mt)
#pragma unroll
        for (int nt = 0; nt < 4; ++nt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const double v = static_cast<double>(acc[mt][nt][i]);
                ssum += v * v;
            }
    ssum = wave_sum(ssum);
    __shared__ double wred[4];
    if (lane == 0) wred[wave] = ssum;
    __syncthreads();
    if (tid == 0) partials[L] = ((wred[0] + wred[1]) + wred[2]) + wred[3];
}

// L(alpha) = sum of partials (fixed order) · 2^-2(kx+kd); alpha* = first argmin.
__global__ __launch_bounds__(256) void reduce_argmin_kernel(const double *__restrict__ partials, int64_t tiles,
                                                            int n_alpha, const SearchState *__restrict__ st,
                                                            const float *__restrict__ s_tab, int64_t D_in,
                                                            double *__restrict__ losses, int32_t *__restrict__ best,
                                                            float *__restrict__ s_best) {
    __shared__ double red[256];
    __shared__ double L[64];
    __shared__ int bsel;
    const int tid = threadIdx.x;
    for (int k = 0; k < n_alpha; ++k) {
        double s = 0.0;
        for (int64_t i = tid; i < tiles; i += 256) s += partials[k * tiles + i];
        red[tid] = s;
        __syncthreads();
        for (int w = 128; w > 0; w >>= 1) {
            if (tid < w) red[tid] += red[tid + w];
            __syncthreads();
        }
        if (tid == 0) {
            const double v = ldexp(red[0], -2 * (st->kx + st->kd[k]));
            L[k] = v;
            losses[k] = v;
        }
        __syncthreads();
    }
    if (tid == 0) {
        bool finite = st->max_abs_x_bits < 0x7f800000u && st->max_abs_w_bits < 0x7f800000u;
        int b = 0;
        for (int k = 0; k < n_alpha; ++k) {
            if (!(L[k] <= DBL_MAX)) finite = false;
            if (L[k] < L[b]) b = k;
        }
        bsel = finite ? b : -1;
        best[0] = bsel;
    }
    __syncthreads();
    const int b = bsel;
    if (b >= 0)
        for (int64_t j = tid; j < D_in; j += 256) s_best[j] = s_tab[b * D_in + j];
}

// Quantiser at alpha*: codes (int8, row-major [D_in x D_out]) and steps.
template <int GC>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3))) void quant_select_kernel(const void *__restrict__ W, int wt, SearchShape sh,
                                                           const float *__restrict__ s_tab,
                                                           const int32_t *__restrict__ best,
                                                           int8_t *__restrict__ codes, float *__restrict__ scales) {
    const int k = best[0];
    if (k < 0) return;
    const int64_t o = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    const int64_t g = blockIdx.y;
    if (o >= sh.D_out) return;
    const int group = GC > 0 ? GC : sh.group;
    const int64_t j0 = g * group;
    const float *s = s_tab + static_cast<int64_t>(k) * sh.D_in + j0;
    const float qmax = static_cast<float>((1 << (sh.bits - 1)) - 1);
    auto wp_at = [&](int r) { return s[r] * ld_f(W, wt, (j0 + r) * sh.D_out + o); };
    float m = 0.0f;
    if constexpr (GC > 0) {
        float wp[GC];
#pragma unroll
        for (int r = 0; r < GC; ++r) {
            wp[r] = wp_at(r);
            m = fmaxf(m, fabsf(wp[r]));
        }
        const float step = m / qmax;
        scales[g * sh.D_out + o] = step;
        if (codes) {
            const float rstep = 1.0f / step;
#pragma unroll
            for (int r0 = 0; r0 < GC; r0 += 8) {
                float q[8];
                if (step > 0.0f) {
                    quant8(wp + r0, step, rstep, qmax, q);
                } else {
#pragma unroll
                    for (int i = 0; i < 8; ++i) q[i] = 0.0f;
                }
#pragma unroll
                for (int i = 0; i < 8; ++i) codes[(j0 + r0 + i) * sh.D_out + o] = static_cast<int8_t>(q[i]);
            }
        }
    } else {
        for (int r = 0; r < group; ++r) m = fmaxf(m, fabsf(wp_at(r)));
        const float step = m / qmax;
        scales[g * sh.D_out + o] = step;
        if (codes) {
            const float rstep = 1.0f / step;
            for (int r0 = 0; r0 < group; r0 += 8) {
                float wp[8], q[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) wp[i] = wp_at(r0 + i);
                if (step > 0.0f) {
                    quant8(wp, step, rstep, qmax, q);
                } else {
#pragma unroll
                    for (int i = 0; i < 8; ++i) q[i] = 0.0f;
                }
#pragma unroll
                for (int i = 0; i < 8; ++i) codes[(j0 + r0 + i) * sh.D_out + o] = static_cast<int8_t>(q[i]);
            }
        }
    }
}

// ------------------------------------------------------------- launcher ----

SearchWorkspace search_workspace_layout(const SearchShape &sh) {
    auto al = [](size_t x) { return (x + 255) / 256 * 256; };
    const size_t elt = sh.f16 ? 2 : 4;
    SearchWorkspace w{};
    size_t off = 0;
    w.off_state = off;
    off += al(sizeof(SearchState));
    w.off_s = off;
    off += al(static_cast<size_t>(sh.n_alpha) * sh.D_in * 4);
    w.off_invp = off;
    off += al(static_cast<size_t>(sh.n_alpha) * sh.D_in * 4);
    w.off_x = off;
    off += al(static_cast<size_t>(sh.Mp) * sh.Kp * elt);
    w.off_d = off;
    off += al(static_cast<size_t>(sh.n_alpha) * sh.Kp * sh.Np * elt);
    w.off_part = off;
    off += al(static_cast<size_t>(sh.n_alpha) * sh.tiles_m * sh.tiles_n * 8);
    w.total = off;
    return w;
}

#define AWQ_LAUNCH_CHECK()                          \
    do {                                            \
        hipError_t e__ = hipGetLastError();         \
        if (e__ != hipSuccess) return e__;          \
    } while (0)

hipError_t launch_search(const void *X, int xt, const void *W, int wt, const float *a, const AlphaGrid &alphas,
                         const SearchShape &sh, double *losses, int32_t *best, float *s_best, float *scales,
                         int8_t *codes, unsigned char *ws, hipStream_t st, hipEvent_t *events) {
    const SearchWorkspace L = search_workspace_layout(sh);
    SearchState *state = reinterpret_cast<SearchState *>(ws + L.off_state);
    float *s_tab = reinterpret_cast<float *>(ws + L.off_s);
    float *invp_tab = reinterpret_cast<float *>(ws + L.off_invp);
    void *Xf = ws + L.off_x;
    void *Df = ws + L.off_d;
    double *partials = reinterpret_cast<double *>(ws + L.off_part);
    const int64_t G = sh.D_in / sh.group;
    auto mark = [&](int i) -> hipError_t { return events ? hipEventRecord(events[i], st) : hipSuccess; };
#define AWQ_MARK(i)                              \
    do {                                         \
        hipError_t e__ = mark(i);                \
        if (e__ != hipSuccess) return e__;       \
    } while (0)

    AWQ_MARK(0);
    hipLaunchKernelGGL(init_state_kernel, dim3(1), dim3(64), 0, st, state);
    AWQ_LAUNCH_CHECK();
    hipLaunchKernelGGL(absmax_kernel, dim3(1024), dim3(256), 0, st, X, xt, sh.N * sh.D_in, &state->max_abs_x_bits);
    AWQ_LAUNCH_CHECK();
    hipLaunchKernelGGL(absmax_kernel, dim3(2048), dim3(256), 0, st, W, wt, sh.D_in * sh.D_out,
                       &state->max_abs_w_bits);
    AWQ_LAUNCH_CHECK();
    hipLaunchKernelGGL(scale_table_kernel, dim3(sh.n_alpha), dim3(256), 0, st, a, alphas, sh.D_in, sh.group, sh.bits,
                       sh.f16, s_tab, invp_tab, state);
    AWQ_LAUNCH_CHECK();
    if (sh.f16) {
        const int64_t n = sh.Mp * sh.KB64;
        hipLaunchKernelGGL(prep_x_f16_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, st,
                           static_cast<const uint16_t *>(X), sh, state, static_cast<half8 *>(Xf));
    } else {
        const int64_t n = sh.Mp * sh.Kp;
        hipLaunchKernelGGL(prep_x_f32_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, st, X, xt,
                           sh, static_cast<float *>(Xf));
    }
    AWQ_LAUNCH_CHECK();
    AWQ_MARK(1);
    {
        const dim3 grid(static_cast<unsigned>((sh.Np + 255) / 256), static_cast<unsigned>(G));
        if (sh.f16) {
            if (sh.group == 128)
                hipLaunchKernelGGL((quant_all_kernel<true, 128>), grid, dim3(256), 0, st, W, wt, sh, s_tab, invp_tab,
                                   state, Df);
            else
                hipLaunchKernelGGL((quant_all_kernel<true, 0>), grid, dim3(256), 0, st, W, wt, sh, s_tab, invp_tab,
                                   state, Df);
        } else {
            if (sh.group == 128)
                hipLaunchKernelGGL((quant_all_kernel<false, 128>), grid, dim3(256), 0, st, W, wt, sh, s_tab,
                                   invp_tab, state, Df);
            else
                hipLaunchKernelGGL((quant_all_kernel<false, 0>), grid, dim3(256), 0, st, W, wt, sh, s_tab, invp_tab,
                                   state, Df);
        }
    }
    AWQ_LAUNCH_CHECK();
    AWQ_MARK(2);
    {
        const int64_t blocks = sh.tiles_m * sh.tiles_n * sh.n_alpha;
        if (sh.f16)
            hipLaunchKernelGGL(loss_gemm_f16_kernel, dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0, st,
                               static_cast<const half8 *>(Xf), static_cast<const half8 *>(Df), partials, sh);
        else
            hipLaunchKernelGGL(loss_gemm_f32_kernel, dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0, st,
                               static_cast<const float *>(Xf), static_cast<const float *>(Df), partials, sh);
    }
    AWQ_LAUNCH_CHECK();
    AWQ_MARK(3);
    hipLaunchKernelGGL(reduce_argmin_kernel, dim3(1), dim3(256), 0, st, partials, sh.tiles_m * sh.tiles_n,
                       sh.n_alpha, state, s_tab, sh.D_in, losses, best, s_best);
    AWQ_LAUNCH_CHECK();
    {
        const dim3 grid(static_cast<unsigned>((sh.D_out + 255) / 256), static_cast<unsigned>(G));
        if (sh.group == 128)
            hipLaunchKernelGGL(quant_select_kernel<128>, grid, dim3(256), 0, st, W, wt, sh, s_tab, best, codes, scales);
        else
            hipLaunchKernelGGL(quant_select_kernel<0>, grid, dim3(256), 0, st, W, wt, sh, s_tab, best, codes, scales);
    }
    AWQ_LAUNCH_CHECK();
    AWQ_MARK(4);
#undef AWQ_MARK
    return hipSuccess;
}

}  // namespace awq
