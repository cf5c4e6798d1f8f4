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

typedef unsigned short ushort2v __attribute__((ext_vector_type(2)));

// Bits of max|v| over one grid-strided slice of a buffer.  For non-negative
// floats the integer order of the bit patterns is the numeric order and every
// NaN pattern lies above +Inf's, so a NaN or Inf anywhere leaves the result
// >= 0x7F800000 (flagged as non-finite later).  Four 16-byte loads in flight.
__device__ __forceinline__ uint32_t absmax_bits(const void *p, int dt, int64_t count, int64_t i, int64_t stride) {
    const uint4 *p4 = static_cast<const uint4 *>(p);
    if (dt == 1) {
        const int64_t n8 = count / 8;
        ushort2v h = {0, 0};
        auto fold = [&](const uint4 &u) {
            h = __builtin_elementwise_max(h, __builtin_bit_cast(ushort2v, u.x & 0x7FFF7FFFu));
            h = __builtin_elementwise_max(h, __builtin_bit_cast(ushort2v, u.y & 0x7FFF7FFFu));
            h = __builtin_elementwise_max(h, __builtin_bit_cast(ushort2v, u.z & 0x7FFF7FFFu));
            h = __builtin_elementwise_max(h, __builtin_bit_cast(ushort2v, u.w & 0x7FFF7FFFu));
        };
        int64_t v = i;
        for (; v + 3 * stride < n8; v += 4 * stride) {
            const uint4 a = p4[v], b = p4[v + stride], c = p4[v + 2 * stride], d = p4[v + 3 * stride];
            fold(a);
            fold(b);
            fold(c);
            fold(d);
        }
        for (; v < n8; v += stride) fold(p4[v]);
        uint32_t m = h.x > h.y ? h.x : h.y;
        const uint16_t *p2 = static_cast<const uint16_t *>(p);
        for (int64_t t = n8 * 8 + i; t < count; t += stride) {
            const uint32_t b = p2[t] & 0x7FFFu;
            m = b > m ? b : m;
        }
        return m << 16;
    }
    const int64_t n4 = count / 4;
    uint32_t m = 0u;
    auto fold = [&](const uint4 &u) {
        const uint32_t a = max(u.x & 0x7FFFFFFFu, u.y & 0x7FFFFFFFu);
        const uint32_t b = max(u.z & 0x7FFFFFFFu, u.w & 0x7FFFFFFFu);
        m = max(m, max(a, b));
    };
    int64_t v = i;
    for (; v + 3 * stride < n4; v += 4 * stride) {
        const uint4 a = p4[v], b = p4[v + stride], c = p4[v + 2 * stride], d = p4[v + 3 * stride];
        fold(a);
        fold(b);
        fold(c);
        fold(d);
    }
    for (; v < n4; v += stride) fold(p4[v]);
    const uint32_t *p1 = static_cast<const uint32_t *>(p);
    for (int64_t t = n4 * 4 + i; t < count; t += stride) m = max(m, p1[t] & 0x7FFFFFFFu);
    return m;
}

// max|X| and max|W| in one launch: workgroups [0, bx) scan X, the rest W;
// each posts its own maximum (part_x / part_w, reduced by the next launch:
// no atomics on two shared words).  Workgroup 0 also clears the state that
// the scale tables then merge into.
__global__ __launch_bounds__(256) void absmax_kernel(const void *__restrict__ X, int xt, int64_t nx,
                                                     const void *__restrict__ W, int wt, int64_t nw, int bx,
                                                     SearchState *__restrict__ st) {
    if (blockIdx.x == 0 && threadIdx.x < 64) {
        st->kd[threadIdx.x] = 0;
        st->sminbits[threadIdx.x] = 0x7F800000u;   // +inf: merged with atomicMin
        if (threadIdx.x == 0) {
            st->kx = 0;
            st->pad0 = 0;
        }
    }
    const bool isx = static_cast<int>(blockIdx.x) < bx;
    const int64_t b = isx ? blockIdx.x : blockIdx.x - bx;
    const int64_t nb = isx ? bx : gridDim.x - bx;
    uint32_t m = isx ? absmax_bits(X, xt, nx, b * 256 + threadIdx.x, nb * 256)
                     : absmax_bits(W, wt, nw, b * 256 + threadIdx.x, nb * 256);
    for (int off = 32; off > 0; off >>= 1) m = max(m, static_cast<uint32_t>(__shfl_xor(static_cast<int>(m), off)));
    __shared__ uint32_t red[4];
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
    __syncthreads();
    if (threadIdx.x == 0) {
        const uint32_t r = max(max(red[0], red[1]), max(red[2], red[3]));
        (isx ? st->part_x : st->part_w)[b] = r;
    }
}

// max over the posted per-workgroup maxima (order independent), by one
// workgroup of the scale-table launch, for every later launch.
__device__ __forceinline__ void reduce_absmax(SearchState *st, int nbx, int nbw) {
    uint32_t mx = 0u, mw = 0u;
    for (int i = threadIdx.x; i < nbx; i += 256) mx = max(mx, st->part_x[i]);
    for (int i = threadIdx.x; i < nbw; i += 256) mw = max(mw, st->part_w[i]);
    for (int off = 32; off > 0; off >>= 1) {
        mx = max(mx, static_cast<uint32_t>(__shfl_xor(static_cast<int>(mx), off)));
        mw = max(mw, static_cast<uint32_t>(__shfl_xor(static_cast<int>(mw), off)));
    }
    __shared__ uint32_t rx[4], rw[4];
    if ((threadIdx.x & 63) == 0) {
        rx[threadIdx.x >> 6] = mx;
        rw[threadIdx.x >> 6] = mw;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        st->max_abs_x_bits = max(max(rx[0], rx[1]), max(rx[2], rx[3]));
        st->max_abs_w_bits = max(max(rw[0], rw[1]), max(rw[2], rw[3]));
    }
}

// Power-of-two prescales of the fp16 path (exact in binary floating point).
// X·2^kx keeps max|X|·2^kx in [2^13, 2^14).
// Error weights: |D_jo| = |Ŵ'_jo/s_j − w_jo| = |q·step − W'_jo| / s_j, and
// q·step is the representable value nearest to W' (rounding, or the end of
// the code range that lies between 0 and W' when the code saturates), while
// 0 is itself representable (code 0, or q = z with zero points).  So
// |q·step − W'| <= |W'| and |D| <= |w|·(1 + 2^-22) after float32 rounding,
// for either code kind and for FP16 steps.  kd puts B = max|W|·(1 + 2^-20)
// just below 2^14: D·2^kd stays far from fp16 overflow and its significant
// part in the fp16 normal range, independently of how the scales of one
// group compare.  The per-row factor 2^kd/s_j must stay finite for the
// smallest scale of the alpha (s >= FLT_MIN: dead channels keep 1), so kd is
// also capped at 126 + e(s_min), which bounds 2^kd/s_min by 2^127.
__device__ __forceinline__ int kx_from_state(const SearchState *st, bool f16) {
    if (!f16) return 0;
    const float xm = __uint_as_float(st->max_abs_x_bits);
    int kx = 0;
    if (xm > 0.0f && xm <= FLT_MAX) {
        int e = 0;
        frexpf(xm, &e);
        kx = 14 - e;
    }
    return kx < -120 ? -120 : (kx > 120 ? 120 : kx);
}

__device__ __forceinline__ int kd_from_state(const SearchState *st, int k, bool f16) {
    if (!f16) return 0;
    const double B = static_cast<double>(__uint_as_float(st->max_abs_w_bits)) * (1.0 + 0x1p-20);
    int kd = 0;
    if (B > 0.0 && B <= DBL_MAX) {
        int e = 0;
        frexp(B, &e);
        kd = 14 - e;
    }
    const float smin = __uint_as_float(st->sminbits[k]);
    if (smin > 0.0f && smin <= FLT_MAX) {
        int es = 0;
        frexpf(smin, &es);
        kd = kd < 126 + es ? kd : 126 + es;
    }
    return kd < -120 ? -120 : (kd > 120 ? 120 : kd);
}

// Candidate scales s_j(alpha) for alpha k = blockIdx.y over a run of whole
// groups (blockIdx.x; gpw groups of at most 256 channels, or one larger
// group), and the smallest scale of that run, merged into sminbits[k] with
// atomicMin on its float bits (positive floats order like their bits, so the
// result is exact and independent of order).  A dead channel (magnitude
// zero, below the smallest normal float or NaN) keeps s = 1.
__global__ __launch_bounds__(256) void scale_table_kernel(const float *__restrict__ a, const float *__restrict__ b,
                                                          AlphaGrid alphas, int64_t D_in, int group, int gpw,
                                                          float *__restrict__ s_tab, SearchState *__restrict__ st,
                                                          int nbx, int nbw) {
    if (blockIdx.x == 0 && blockIdx.y == 0) reduce_absmax(st, nbx, nbw);   // uniform branch
    const int k = blockIdx.y;
    const double alpha = static_cast<double>(alphas.v[k]);
    const int tid = threadIdx.x;
    const int64_t c0 = static_cast<int64_t>(blockIdx.x) * gpw * group;
    const int64_t c1 = c0 + static_cast<int64_t>(gpw) * group < D_in ? c0 + static_cast<int64_t>(gpw) * group : D_in;
    float *s_row = s_tab + static_cast<int64_t>(k) * D_in;
    // s = a^α, or a^α / b^(1−α) with a weight statistic ([LQ] "4.4 怎么做"):
    // float64 powers and quotient, one rounding; dead channels keep 1
    auto scale_of = [&](int64_t j) {
        const float aj = a[j];
        if (!(aj >= FLT_MIN)) return 1.0f;
        if (!b) return static_cast<float>(pow(static_cast<double>(aj), alpha));
        const float bj = b[j];
        if (!(bj >= FLT_MIN)) return 1.0f;
        return static_cast<float>(pow(static_cast<double>(aj), alpha) / pow(static_cast<double>(bj), 1.0 - alpha));
    };
    __shared__ float rmn[4];
    float smin = INFINITY;
    for (int64_t j = c0 + tid; j < c1; j += 256) {
        const float s = scale_of(j);
        s_row[j] = s;
        smin = fminf(smin, s);
    }
    for (int off = 32; off > 0; off >>= 1) smin = fminf(smin, __shfl_xor(smin, off));
    if ((tid & 63) == 0) rmn[tid >> 6] = smin;
    __syncthreads();
    if (tid == 0) {
        const float mn = fminf(fminf(rmn[0], rmn[1]), fminf(rmn[2], rmn[3]));
        atomicMin(&st->sminbits[k], __float_as_uint(mn));
    }
}

// Last step of the scale tables, run by extra workgroups of the X preparation
// launch (after every ratio is known): kd per alpha and the per-row factor
// 2^kd / s_j that turns a quantisation residual into a scaled error weight.
__device__ __forceinline__ void finish_tables(int64_t b, int64_t D_in, bool f16, SearchState *st,
                                              const float *__restrict__ s_tab, float *__restrict__ invp_tab) {
    const int64_t per = (D_in + 255) / 256;
    const int k = static_cast<int>(b / per);
    const int64_t j = (b % per) * 256 + threadIdx.x;
    const int kd = kd_from_state(st, k, f16);
    if (b % per == 0 && threadIdx.x == 0) st->kd[k] = kd;
    if (j < D_in) invp_tab[k * D_in + j] = ldexpf(1.0f, kd) / s_tab[k * D_in + j];
}

// bf16 bits of v rounded to nearest even (one v_cvt_pk_bf16_f32), and the
// exact bf16 bits of a float that a bf16 value times a power of two formed.
__device__ __forceinline__ uint16_t bf16_bits_rne(float v) {
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
    const f32x2 f = {v, 0.0f};
    return static_cast<uint16_t>(__builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2v)));
}
__device__ __forceinline__ uint32_t bf16_pair_bits_rne(float lo, float hi) {
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
    const f32x2 f = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2v));
}
__device__ __forceinline__ _Float16 bf16_slot(uint16_t bits) { return __builtin_bit_cast(_Float16, bits); }
// Bit r of word r/32: row j0 + r is a correction row's source (sel[j0 + r] >= 0).
template <int ROWS>
__device__ __forceinline__ void sel_mask(const int *__restrict__ sel, int64_t j0, uint32_t *m) {
#pragma unroll
    for (int w = 0; w < (ROWS + 31) / 32; ++w) m[w] = 0u;
#pragma unroll
    for (int r = 0; r < ROWS; ++r) m[r / 32] |= (sel[j0 + r] >= 0 ? 1u : 0u) << (r % 32);
}
__device__ __forceinline__ uint16_t bf16_bits_exact(float v) { return static_cast<uint16_t>(__float_as_uint(v) >> 16); }

// Correction rows of the bf16 path: the kCorrRows input channels with the
// largest activation statistic a_j (a non-finite or negative a_j counts as
// 0; ties go to the lower channel index).  A radix select on the float bits
// (non-negative floats order like their bits) finds the kCorrRows-th largest
// key t; every channel above t is taken, then the lowest-indexed channels
// equal to t.  sel_pos[j] = the channel's correction row (0 .. kCorrRows-1,
// in channel order) or -1; sel_idx[p] = the channel of correction row p.
// One workgroup; thread t holds the keys of channels [t·per, t·per + per)
// in registers (per <= kSelPer, loaded once, four at a time), so thread
// order is channel order; every count is an integer, so the result does not
// depend on scheduling.  Requires kCorrRows <= D_in <= kSelThreads·kSelPer.
constexpr int kSelThreads = 1024;
constexpr int kSelPer = 16;
static_assert(kSelThreads * kSelPer >= kMaxBf16Rows, "selection covers the bf16 path's D_in");
__device__ __forceinline__ uint32_t sel_key(float v) { return (v >= 0.0f && v <= FLT_MAX) ? __float_as_uint(v) : 0u; }

__global__ __launch_bounds__(kSelThreads) void select_rows_kernel(const float *__restrict__ a, int64_t D_in,
                                                                  int *__restrict__ sel_pos, int *__restrict__ sel_idx) {
    __shared__ unsigned hist[256];
    __shared__ unsigned bcast[2];
    __shared__ int wsum[kSelThreads / 64];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    // channels per thread: a multiple of 4 (16-byte loads; D_in is a multiple of 8)
    const int per = static_cast<int>(((D_in + kSelThreads - 1) / kSelThreads + 3) / 4 * 4);
    const int64_t c0 = static_cast<int64_t>(tid) * per;
    uint32_t key[kSelPer];
#pragma unroll
    for (int q = 0; q < kSelPer / 4; ++q) {
        const int64_t j = c0 + 4 * q;
        float4 v = make_float4(-1.0f, -1.0f, -1.0f, -1.0f);
        if (4 * q < per && j < D_in) v = *reinterpret_cast<const float4 *>(a + j);
        key[4 * q] = sel_key(v.x);
        key[4 * q + 1] = sel_key(v.y);
        key[4 * q + 2] = sel_key(v.z);
        key[4 * q + 3] = sel_key(v.w);
    }
    // number of this thread's channels that exist (its run may pass D_in)
    const int cnt = c0 >= D_in ? 0 : (c0 + per <= D_in ? per : static_cast<int>(D_in - c0));
    uint32_t prefix = 0u, mask = 0u;
    unsigned need = kCorrRows;   // channels still to take among those matching prefix under mask
    for (int shift = 24; shift >= 0; shift -= 8) {
        if (tid < 256) hist[tid] = 0u;
        __syncthreads();
#pragma unroll
        for (int i = 0; i < kSelPer; ++i)
            if (i < cnt && (key[i] & mask) == prefix) atomicAdd(&hist[(key[i] >> shift) & 255u], 1u);
        __syncthreads();
        // the largest digit d with (count above d) < need <= (count at or
        // above d): thread d (of the first 4 waves) forms the count at or
        // above its digit by a suffix sum over the 256 bins, within its wave
        // and then over the later waves; exactly one digit qualifies.
        unsigned own = 0u, suf = 0u;
        if (tid < 256) {
            own = hist[tid];
            suf = own;
            for (int off = 1; off < 64; off <<= 1) {
                const unsigned t = __shfl_down(suf, off);
                if (lane + off < 64) suf += t;
            }
            if (lane == 0) wsum[wave] = static_cast<int>(suf);
        }
        __syncthreads();
        if (tid < 256) {
            for (int w = wave + 1; w < 4; ++w) suf += static_cast<unsigned>(wsum[w]);
            const unsigned above = suf - own;
            if (above < need && need <= suf) {
                bcast[0] = static_cast<unsigned>(tid);
                bcast[1] = need - above;
            }
        }
        __syncthreads();
        prefix |= bcast[0] << shift;
        mask |= 255u << shift;
        need = bcast[1];   // channels equal to the final key still to take
        __syncthreads();
    }
    // exclusive prefix sum over threads in thread order
    auto block_scan = [&](int v) {
        int incl = v;
        for (int off = 1; off < 64; off <<= 1) {
            const int t = __shfl_up(incl, off);
            if (lane >= off) incl += t;
        }
        if (lane == 63) wsum[wave] = incl;
        __syncthreads();
        int base = 0;
        for (int w = 0; w < wave; ++w) base += wsum[w];
        __syncthreads();
        return base + incl - v;
    };
    int eq = 0;
#pragma unroll
    for (int i = 0; i < kSelPer; ++i) eq += (i < cnt && key[i] == prefix) ? 1 : 0;
    const int eq_base = block_scan(eq);
    uint32_t take = 0u;   // bit i: channel c0 + i is taken
    int r = eq_base, taken = 0;
#pragma unroll
    for (int i = 0; i < kSelPer; ++i) {
        bool t = false;
        if (i < cnt) {
            if (key[i] > prefix) t = true;
            else if (key[i] == prefix) t = static_cast<unsigned>(r++) < need;
        }
        take |= (t ? 1u : 0u) << i;
        taken += t ? 1 : 0;
    }
    int slot = block_scan(taken);
#pragma unroll
    for (int i = 0; i < kSelPer; ++i) {
        if (i < cnt) {
            const int64_t j = c0 + i;
            if (take & (1u << i)) {
                sel_idx[slot] = static_cast<int>(j);
                sel_pos[j] = slot++;
            } else {
                sel_pos[j] = -1;
            }
        }
    }
}

// X -> fragment order, fp16 path.  One workgroup per 32-row block and
// kPrepKB 64-k blocks: each wave load reads one 1 KiB row segment (a lane per
// 16-byte run), the values go to FP16·2^kx in an LDS tile (rows padded by 16
// bytes), and each thread then writes one 16-byte fragment entry per 64-k
// block, so that a block's 256 entries (4 KiB) leave as four contiguous
// 1 KiB wave stores.  (One thread per row and block, rows fastest across a
// wave, read 16 bytes of 64 rows 2·D_in bytes apart per load and fetched
// about four times X past L2.)  Workgroups from nprep on finish the scale
// tables.  BF: the same layout holds bf16·2^kx (exact), and the correction
// stage after the Kq quantised rows holds X[:, sel_idx[p]] as its row p.
constexpr int kPrepKB = 8;
template <bool BF>
__global__ __launch_bounds__(256) void prep_x_f16_kernel(const uint16_t *__restrict__ X, SearchShape sh,
                                                         SearchState *__restrict__ st, half8 *__restrict__ Xf,
                                                         int64_t nprep, const float *__restrict__ s_tab,
                                                         float *__restrict__ invp_tab, const int *__restrict__ sel_idx) {
    if (static_cast<int64_t>(blockIdx.x) >= nprep) {
        finish_tables(blockIdx.x - nprep, sh.D_in, true, st, s_tab, invp_tab);
        return;
    }
    __shared__ __align__(16) uint16_t tile[32][kPrepKB * 64 + 8];
    const int tid = threadIdx.x;
    const int kx = kx_from_state(st, true);
    if (blockIdx.x == 0 && tid == 0) st->kx = kx;
    const int64_t nkc = (sh.KB64 + kPrepKB - 1) / kPrepKB;
    const int64_t mb = blockIdx.x / nkc, kc = blockIdx.x % nkc;
    const float scale = ldexpf(1.0f, kx);
    const int run = tid % 64;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int r = tid / 64 + 4 * i;
        const int64_t row = mb * 32 + r, k0 = (kc * kPrepKB * 64) + run * 8;
        half8 h;
        if (row < sh.N && k0 < sh.D_in) {
            const uint4 u = *reinterpret_cast<const uint4 *>(X + row * sh.D_in + k0);
            const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                const float lo = __uint_as_float(w[p] << 16) * scale, hi = __uint_as_float(w[p] & 0xFFFF0000u) * scale;
                if constexpr (BF) {
                    h[2 * p] = bf16_slot(bf16_bits_exact(lo));
                    h[2 * p + 1] = bf16_slot(bf16_bits_exact(hi));
                } else {
                    h[2 * p] = static_cast<_Float16>(lo);
                    h[2 * p + 1] = static_cast<_Float16>(hi);
                }
            }
        } else if (BF && row < sh.N && k0 >= sh.Kq && k0 < sh.Kp) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int64_t j = sel_idx[k0 - sh.Kq + e];
                h[e] = bf16_slot(bf16_bits_exact(__uint_as_float(static_cast<uint32_t>(X[row * sh.D_in + j]) << 16) * scale));
            }
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) h[e] = static_cast<_Float16>(0.0f);
        }
        *reinterpret_cast<half8 *>(&tile[r][run * 8]) = h;
    }
    __syncthreads();
    // entry tid of each 64-k block: ((kb·MB32 + mb)·4 + kq)·64 + c·32 + r holds
    // row r, k = kb·64 + (2·kq + c)·8 .. +7
    const int kq = tid / 64, c = (tid / 32) % 2, r = tid % 32;
#pragma unroll
    for (int b = 0; b < kPrepKB; ++b) {
        const int64_t kb = kc * kPrepKB + b;
        if (kb >= sh.KB64) break;
        Xf[((kb * sh.MB32 + mb) * 4 + kq) * 64 + c * 32 + r] =
            *reinterpret_cast<const half8 *>(&tile[r][b * 64 + (2 * kq + c) * 8]);
    }
}

// fp32 path: one thread per element.
__global__ __launch_bounds__(256) void prep_x_f32_kernel(const void *__restrict__ X, int xt, SearchShape sh,
                                                         float *__restrict__ Xf, SearchState *__restrict__ st,
                                                         int64_t nprep, const float *__restrict__ s_tab,
                                                         float *__restrict__ invp_tab) {
    if (static_cast<int64_t>(blockIdx.x) >= nprep) {
        finish_tables(blockIdx.x - nprep, sh.D_in, false, st, s_tab, invp_tab);
        return;
    }
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

template <bool WB>
__device__ __forceinline__ float ld_w(const void *p, int64_t i) {
    if constexpr (WB) return __uint_as_float(static_cast<uint32_t>(static_cast<const uint16_t *>(p)[i]) << 16);
    else return static_cast<const float *>(p)[i];
}

// ld_w of an in-bounds element, kept where keep = ~0 and +0 where keep = 0:
// a mask rather than a select, so that the compiler issues the load
// unconditionally (a select lets it branch around each load and wait for it).
template <bool WB>
__device__ __forceinline__ float ld_w_masked(const void *p, int64_t i, uint32_t keep) {
    return __uint_as_float(__float_as_uint(ld_w<WB>(p, i)) & keep);
}

// Exact quantiser for 8 values of one group:
// q_i = rint(fl(wp_i / step)) (IEEE float32 quotient, ties to even), and
// q_i = 0 for an all-zero group (step = 0, passed as rstep = 0).
// Fast path: t = fl(wp · rstep) with rstep = fl(1/step).  Then
// |t − wp/step| <= |wp/step|·(2^-23 + 2^-48), and the IEEE quotient is within
// 2^-24·|wp/step| of wp/step, so whenever t is farther than |t|·2^-20 from
// every half-integer both round to the same integer (and neither is a tie).
// Since |wp| <= max|W'| = qmax·step·(1 + O(2^-24)), |t| < qmax + 1, and the
// test uses the uniform margin thr = 0.5 − (qmax + 1)·2^-20.  Otherwise
// (about one value in 10^5, or a non-finite t) the 8 values are recomputed
// with true division.  t − rint(t) is exact (Sterbenz).  The same bound gives
// |q| <= qmax for finite inputs, so no clamp is needed for the codes' range.
__device__ __forceinline__ void quant8(const float *wp, float step, float rstep, float thr, float *q) {
    bool exact_needed = false;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float t = wp[i] * rstep;
        const float qt = rintf(t);
        exact_needed |= !(fabsf(t - qt) < thr);
        q[i] = qt;
    }
    if (exact_needed) {
#pragma unroll
        for (int i = 0; i < 8; ++i) q[i] = step > 0.0f ? rintf(wp[i] / step) : 0.0f;
    }
}

// Zero-point codes: q = clamp(rint(fl(wp/step)) + z, 0, qhi).  |wp| <= hi − lo
// = (2^b − 1)·step·(1 + O(2^-24)), so quant8's argument holds with
// qmax = 2^b − 1 in the margin.
__device__ __forceinline__ void quant8z(const float *wp, float step, float rstep, float thr, float zf, float qhi,
                                        float *q) {
    quant8(wp, step, rstep, thr, q);
#pragma unroll
    for (int i = 0; i < 8; ++i) q[i] = fminf(fmaxf(q[i] + zf, 0.0f), qhi);
}

__device__ __forceinline__ float quant_margin(float qmax) { return 0.5f - (qmax + 1.0f) * 0x1p-20f; }
__device__ __forceinline__ float recip_step(float step) { return step > 0.0f ? 1.0f / step : 0.0f; }

// Writes the error weights of rows [j, j + ROWS) of one column for one alpha,
// given the group's step.  ROWS is a multiple of 8.  With W' = s·w and
// Ŵ' = q·step, (Ŵ'/s − w)·2^kd = (q·step − W')·(2^kd/s) up to the float32
// rounding of W' (2^-24 relative to w, far below the error weight itself).
// `dk` is the (uniform) error-weight block of this alpha, `lane_off` the byte
// offset of this column's slot in it.
// The blocks are written with streaming (nontemporal) stores: all alphas'
// blocks together exceed the Infinity Cache and the contraction reads them
// back oldest first, so allocating them in the caches saves no reads, and
// the streaming stores raised the quantiser's write rate from about 3.6 to
// 4.6 TB/s (4096 x 4096, 21 alphas: 194 -> 153 us).
// `qmax` is the largest code: 2^(b-1) − 1, or 2^b − 1 with ASYM, where the
// codes carry the zero point zf (in [0, qmax]) and the error weight is
// ((q − zf)·step − W')·(2^kd/s).
// Byte offset of correction row p inside an error-weight block of the bf16
// path (the stage after the Kq quantised rows), before the lane's column
// offset: row p sits in k-step p/16, half (p%16)/8, element p%8.
__device__ __forceinline__ int64_t corr_slot_bytes(const SearchShape &sh, int p) {
    return ((sh.Kq / 64 * sh.NB32c * 4 + p / 16) * 64 + ((p % 16) / 8) * 32) * 16 + (p % 8) * 2;
}

// BF (bf16 path): the error weights are rounded to bf16, and a row j that
// sel[j] >= 0 names also stores its rounding residual, rounded to bf16, as
// correction row sel[j] of the same column.  selmask holds one bit per row
// of the ROWS rows (bit r of word r/32: sel[j + r] >= 0), the same for every
// lane, so each 8-row block costs one uniform test.
template <bool F16, int ROWS, bool ASYM = false, bool BF = false>
__device__ __forceinline__ void emit_rows(const float *w, const float *__restrict__ s, const float *__restrict__ invp,
                                          float step, float thr, int64_t j, const SearchShape &sh,
                                          unsigned char *__restrict__ dk, uint32_t lane_off, float qmax, float zf = 0.0f,
                                          const int *__restrict__ sel = nullptr, const uint32_t *selmask = nullptr) {
    const float rstep = recip_step(step);
#pragma unroll
    for (int r0 = 0; r0 < ROWS; r0 += 8) {
        float wp[8], q[8], d[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) wp[i] = s[r0 + i] * w[r0 + i];
        if constexpr (ASYM) {
            quant8z(wp, step, rstep, thr, zf, qmax, q);
#pragma unroll
            for (int i = 0; i < 8; ++i) q[i] -= zf;
        } else {
            quant8(wp, step, rstep, thr, q);
            // A step rounded to FP16 can lie below max|W'|/qmax by more than
            // quant8's margin when it is subnormal, so the quotient can pass
            // qmax + 1/2: clamp as the stored codes are clamped.
            if (sh.f16_steps) {
#pragma unroll
                for (int i = 0; i < 8; ++i) q[i] = fminf(fmaxf(q[i], -qmax), qmax);
            }
        }
        // error weight (tolerance path, not bit-exact)
#pragma unroll
        for (int i = 0; i < 8; ++i) d[i] = fmaf(q[i], step, -wp[i]) * invp[r0 + i];
        const int64_t jj = j + r0;
        if constexpr (F16) {
            half8 h;
            if constexpr (BF) {
                uint32_t hw[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) hw[i] = bf16_pair_bits_rne(d[2 * i], d[2 * i + 1]);
#pragma unroll
                for (int i = 0; i < 8; ++i) h[i] = bf16_slot(static_cast<uint16_t>(hw[i / 2] >> (16 * (i % 2))));
                const uint32_t m8 = (selmask[r0 / 32] >> (r0 % 32)) & 0xFFu;   // uniform
                if (m8) {
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        if (m8 & (1u << i)) {
                            const int p = sel[jj + i];
                            // d − bf16(d) is exact in float32
                            const float back = __uint_as_float((hw[i / 2] << (16 * (1 - i % 2))) & 0xFFFF0000u);
                            const uint16_t rb = bf16_bits_rne(d[i] - back);
                            __builtin_nontemporal_store(rb,
                                                        reinterpret_cast<uint16_t *>(dk + corr_slot_bytes(sh, p) + lane_off));
                        }
                    }
                }
            } else {
#pragma unroll
                for (int i = 0; i < 8; ++i) h[i] = static_cast<_Float16>(d[i]);
            }
            // uniform part of the fragment slot: ((kb·NB32 + nb)·4 + kq)·64 + c·32 + n
            const int64_t kb = jj / 64, kq = (jj % 64) / 16, c = (jj % 16) / 8;
            unsigned char *base = dk + ((kb * sh.NB32c * 4 + kq) * 64 + c * 32) * 16;
            __builtin_nontemporal_store(h, reinterpret_cast<half8 *>(base + lane_off));
        } else {
            const int64_t kb = jj / 32;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int64_t ji = jj + i;
                const int64_t ks = (ji % 32) / 4, c = ji % 4;
                unsigned char *base = dk + ((kb * sh.NBc * 8 + ks) * 64 + c * 16) * 4;
                __builtin_nontemporal_store(d[i], reinterpret_cast<float *>(base + lane_off));
            }
        }
    }
}

// Byte offset of column o's slot inside an error-weight block.
template <bool F16>
__device__ __forceinline__ uint32_t dlane_bytes(int64_t o) {
    if constexpr (F16) return static_cast<uint32_t>(((o / 32) * 4 * 64 + (o % 32)) * 16);   // nb32·4·64 + n
    else return static_cast<uint32_t>(((o / 16) * 8 * 64 + (o % 16)) * 4);                  // nb16·8·64 + n
}

// Zero error weights for rows j0 .. j0+rows-1 (padding columns or the k
// padding); with sel (bf16 path), the correction rows those rows own are
// zeroed as well.
template <bool F16>
__device__ __forceinline__ void emit_zero(int64_t j0, int rows, const SearchShape &sh, unsigned char *dk,
                                          uint32_t lane_off, const int *__restrict__ sel = nullptr) {
    for (int r0 = 0; r0 < rows; r0 += 8) {
        const int64_t j = j0 + r0;
        if constexpr (F16) {
            half8 h;
#pragma unroll
            for (int i = 0; i < 8; ++i) h[i] = static_cast<_Float16>(0.0f);
            if (sel) {
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const int p = sel[j + i];
                    if (p >= 0)
                        __builtin_nontemporal_store(static_cast<uint16_t>(0),
                                                    reinterpret_cast<uint16_t *>(dk + corr_slot_bytes(sh, p) + lane_off));
                }
            }
            const int64_t kb = j / 64, kq = (j % 64) / 16, c = (j % 16) / 8;
            __builtin_nontemporal_store(h, reinterpret_cast<half8 *>(dk + ((kb * sh.NB32c * 4 + kq) * 64 + c * 32) * 16 + lane_off));
        } else {
            const int64_t kb = j / 32;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int64_t ji = j + i;
                const int64_t ks = (ji % 32) / 4, c = ji % 4;
                __builtin_nontemporal_store(0.0f, reinterpret_cast<float *>(dk + ((kb * sh.NBc * 8 + ks) * 64 + c * 16) * 4 + lane_off));
            }
        }
    }
}

// Alphas handled by one thread of quant_all.  The grid's z dimension splits
// the alphas into slices of equal size, and each slice reads W again.
// While the W columns of the pass fit well inside the 256 MB Infinity Cache
// the re-reads are cheap and 7-alpha slices give more waves for the
// arithmetic (4096 x 4096, 21 alphas, groups 32 / 64 / 128: 0.146 / 0.144 /
// 0.169 ms with three slices against 0.166 / 0.153 / 0.219 ms with one;
// 4096 x 11008 and 11008 x 4096 within 3% for one to three slices).  A
// larger W is re-read from HBM, so the alphas are then split only as far as
// needed for about kQuantMinWorkgroups workgroups (two rounds of the 768
// that fit at three waves per SIMD): 8192 x 28672, 21 alphas, 7168
// workgroups per slice, one slice 2.33 ms against 2.59 / 2.68 ms with 2 / 3.
constexpr int kAlphaSliceCached = 7;
constexpr int64_t kQuantCachedWBytes = int64_t(128) << 20;
constexpr int64_t kQuantMinWorkgroups = 1536;
static int quant_alpha_slice(int64_t workgroups_per_slice, int n_alpha, int64_t w_bytes) {
    if (w_bytes <= kQuantCachedWBytes) return kAlphaSliceCached;
    int64_t slices = (kQuantMinWorkgroups + workgroups_per_slice - 1) / workgroups_per_slice;
    slices = slices < 1 ? 1 : (slices > n_alpha ? n_alpha : slices);
    return static_cast<int>((n_alpha + slices - 1) / slices);
}

// One thread per (group, column) and slice of alphas: W is read once per
// slice.  GC > 0: the group's rows live in registers, GC per thread; with P
// = 1 a workgroup covers 256 columns, with P = 2 or 4 every P consecutive
// waves hold the P GC-row parts of one group for the same 64 columns (group
// = P·GC) and combine the group's extremes through LDS, so that
// row-dependent operands (s, 1/s) stay wave-uniform while fewer rows per
// lane leave registers for more waves.  GC == 0: any multiple of 8, re-read
// through the cache.  WB: W is bf16.
// Zero-point statistics of one group: lo = min(min W', 0), hi = max(max W',
// 0), step = fl((hi − lo)/qu), z = clamp(rint(fl(−lo/step)), 0, qu).
__device__ __forceinline__ float f16_step(float step) { return static_cast<float>(static_cast<_Float16>(step)); }

__device__ __forceinline__ void zp_step(float lo, float hi, float qu, bool f16s, float &step, float &zf) {
    step = (hi - lo) / qu;
    if (f16s) step = f16_step(step);   // the step is stored in FP16: codes follow the stored value
    zf = step > 0.0f ? fminf(fmaxf(rintf(-lo / step), 0.0f), qu) : 0.0f;
}

// Extremes of a group whose rows are split over P consecutive waves of a
// workgroup (same lane = same column): each wave posts its partial maximum
// (and, for zero points, minimum) and reads back those of its P.  Two LDS
// slots by parity, so one barrier per use suffices: a wave can only
// overwrite a slot after every wave has passed the barrier that follows the
// reads of its previous use.
template <int P>
struct GroupXchg {
    float v[2][2][4][64];
    __device__ __forceinline__ void combine(int parity, int wave, int lane, float &mx, float &mn) {
        v[parity][0][wave][lane] = mx;
        v[parity][1][wave][lane] = mn;
        __syncthreads();
        const int w0 = wave - wave % P;
#pragma unroll
        for (int q = 0; q < P; ++q) {
            mx = fmaxf(mx, v[parity][0][w0 + q][lane]);
            mn = fminf(mn, v[parity][1][w0 + q][lane]);
        }
    }
};

template <bool F16, int GC, bool WB, bool ASYM, int P, bool BF>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3))) void quant_all_kernel(
    const void *__restrict__ W, SearchShape sh, const float *__restrict__ s_tab, const float *__restrict__ invp_tab,
    void *__restrict__ Df, int alpha_slice, const int *__restrict__ sel_pos) {
    static_assert(P == 1 || ((P == 2 || P == 4) && GC > 0), "waves per group");
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int part = wave % P;
    // column of the chunk's error-weight block, and of the layer
    const int64_t oc = static_cast<int64_t>(blockIdx.x) * (256 / P) + (wave / P) * 64 + lane;
    const int64_t o = sh.col0 + oc;
    const int64_t g = blockIdx.y;
    if (oc >= sh.Nc) return;   // P > 1: never (the grid covers Nc exactly), so every wave meets each barrier
    const int k0 = static_cast<int>(blockIdx.z) * alpha_slice;
    const int k1 = k0 + alpha_slice < sh.n_alpha ? k0 + alpha_slice : sh.n_alpha;
    const int group = GC > 0 ? GC * P : sh.group;
    const int64_t j0 = g * group + part * GC;   // this lane's first row
    const int64_t G = sh.D_in / group;
    const size_t dstride = static_cast<size_t>(sh.Kp) * static_cast<size_t>(sh.Nc) * (F16 ? 2 : 4);
    const float qmax = ASYM ? static_cast<float>((1 << sh.bits) - 1) : static_cast<float>((1 << (sh.bits - 1)) - 1);
    const float thr = quant_margin(qmax);
    unsigned char *D0 = static_cast<unsigned char *>(Df);
    const uint32_t lo = dlane_bytes<F16>(oc);
    // P > 1: padding columns run the same code on w = 0 (whose error weights
    // are 0), so that no wave leaves the barriers
    if (P == 1 && o >= sh.D_out) {
        for (int k = k0; k < k1; ++k) emit_zero<F16>(j0, group, sh, D0 + k * dstride, lo, BF ? sel_pos : nullptr);
    } else {
        if constexpr (GC > 0) {
            __shared__ GroupXchg<P> xchg;
            uint32_t selm[(GC + 31) / 32];
            if constexpr (BF) sel_mask<GC>(sel_pos, j0, selm);
            float w[GC];
            const bool live = o < sh.D_out;
            const int oi = static_cast<int>(live ? o : sh.D_out - 1);   // in-bounds loads
            const uint32_t keep = live ? 0xFFFFFFFFu : 0u;
#pragma unroll
            for (int r = 0; r < GC; ++r) {
                // uniform row base + 32-bit lane offset
                const unsigned char *row = static_cast<const unsigned char *>(W) + (j0 + r) * sh.D_out * (WB ? 2 : 4);
                w[r] = ld_w_masked<WB>(row, oi, keep);
            }
            for (int k = k0; k < k1; ++k) {
                const float *s = s_tab + k * sh.D_in + j0;
                const float *invp = invp_tab + k * sh.D_in + j0;
                // group maximum from s·|w| = |s·w| (s > 0): a different product
                // from the s·w formed again below, so the compiler does not keep
                // all of the group's products alive between the two passes
                if constexpr (ASYM) {
                    float wlo = 0.0f, whi = 0.0f;
#pragma unroll
                    for (int r = 0; r < GC; ++r) {
                        const float p = s[r] * w[r];
                        wlo = fminf(wlo, p);
                        whi = fmaxf(whi, p);
                    }
                    if constexpr (P > 1) xchg.combine(k & 1, wave, lane, whi, wlo);
                    float step, zf;
                    zp_step(wlo, whi, qmax, sh.f16_steps, step, zf);
                    emit_rows<F16, GC, true, BF>(w, s, invp, step, thr, j0, sh, D0 + k * dstride, lo, qmax, zf,
                                                 sel_pos, selm);
                } else {
                    float m = 0.0f;
#pragma unroll
                    for (int r = 0; r < GC; ++r) m = fmaxf(m, s[r] * fabsf(w[r]));
                    if constexpr (P > 1) {
                        float unused = 0.0f;
                        xchg.combine(k & 1, wave, lane, m, unused);
                    }
                    float step = m / qmax;
                    if (sh.f16_steps) step = f16_step(step);
                    emit_rows<F16, GC, false, BF>(w, s, invp, step, thr, j0, sh, D0 + k * dstride, lo, qmax, 0.0f,
                                                  sel_pos, selm);
                }
            }
        } else {
            for (int k = k0; k < k1; ++k) {
                const float *s = s_tab + k * sh.D_in + j0;
                const float *invp = invp_tab + k * sh.D_in + j0;
                float step, zf = 0.0f;
                if constexpr (ASYM) {
                    float wlo = 0.0f, whi = 0.0f;
                    for (int r = 0; r < group; ++r) {
                        const float p = s[r] * ld_w<WB>(W, (j0 + r) * sh.D_out + o);
                        wlo = fminf(wlo, p);
                        whi = fmaxf(whi, p);
                    }
                    zp_step(wlo, whi, qmax, sh.f16_steps, step, zf);
                } else {
                    float m = 0.0f;
                    for (int r = 0; r < group; ++r) m = fmaxf(m, s[r] * fabsf(ld_w<WB>(W, (j0 + r) * sh.D_out + o)));
                    step = m / qmax;
                    if (sh.f16_steps) step = f16_step(step);
                }
                for (int r0 = 0; r0 < group; r0 += 8) {
                    float w8[8];
#pragma unroll
                    for (int i = 0; i < 8; ++i) w8[i] = ld_w<WB>(W, (j0 + r0 + i) * sh.D_out + o);
                    uint32_t selm[1] = {0u};
                    if constexpr (BF) sel_mask<8>(sel_pos, j0 + r0, selm);
                    emit_rows<F16, 8, ASYM, BF>(w8, s + r0, invp + r0, step, thr, j0 + r0, sh, D0 + k * dstride, lo,
                                                qmax, zf, sel_pos, selm);
                }
            }
        }
    }
    // zero the k padding below the last group (the correction rows of the
    // bf16 path after it are written by the rows they correct)
    if (g == G - 1 && part == 0 && sh.Kq > sh.D_in) {
        for (int k = k0; k < k1; ++k)
            emit_zero<F16>(sh.D_in, static_cast<int>(sh.Kq - sh.D_in), sh, D0 + k * dstride, lo);
    }
}

// ------------------------------------------------------- loss contraction --

// Tile scheduling.  Workgroups are dispatched round-robin over the 8 XCDs
// (blockIdx % 8), each with its own L2.  Logical tiles are renumbered so that
// every XCD receives one contiguous range, and inside that range each alpha's
// tiles are walked in column groups of CG = 4 column tiles; inside a column
// group, in blocks of RG = 8 row tiles x the group's column tiles (row tile
// fastest), one block after the other down the rows.  The 32 workgroups an
// XCD runs at once then cover 8 row tiles x 4 column tiles and share those
// X row blocks and error-weight column strips through their L2; the next
// block reuses the same 4 strips at once, from the Infinity Cache.  Per
// alpha of the 8192 x 28672 layer (N = 4096: 16 row tiles, 112 column tiles)
// this reads 448 X strips and 224 error-weight strips past L2 (112 from
// HBM), against 896 + 112 for blocks of 16 row tiles x 2 column tiles.
// Measured on that layer, alternating in one process: 30.33 against 30.51 ms
// and 32.00 against 32.24 ms on two boxes for blocks of 16 x 2, and 33.25 ms
// for blocks of 4 x 8 (the strips then re-read 4 times); earlier, 16 row tiles
// x all column tiles measured 30.15 ms against 30.25-30.53 / 30.85 / 32.77
// ms for 8 / 4 / 2 row tiles x all column tiles (8: each strip fetched twice
// from HBM).  The order is applied to the tiles of the current column chunk;
// `pidx` is the partial's index in the whole layer's numbering (alpha-major,
// then groups of GM = 16 row tiles x all column tiles, column-major inside a
// group), which does not depend on the walk or the chunking, so neither
// changes the partials or the losses the fixed-order reduction forms from
// them.
__device__ __forceinline__ unsigned grouped_tile(unsigned tm, unsigned tn, unsigned tiles_m, unsigned tiles_n,
                                                 unsigned GM) {
    const unsigned first_m = (tm / GM) * GM;
    const unsigned gm = (tiles_m - first_m) < GM ? (tiles_m - first_m) : GM;
    return first_m * tiles_n + tn * gm + (tm - first_m);
}

__device__ __forceinline__ void map_tile(const SearchShape &sh, int &pidx, int &alpha, int &tm, int &tn) {
    constexpr unsigned GM = 16;
    const unsigned tiles_m = static_cast<unsigned>(sh.tiles_m);
    const unsigned tiles = static_cast<unsigned>(sh.tiles_m * sh.tiles_nc);
    const unsigned total = tiles * static_cast<unsigned>(sh.n_alpha);
    const unsigned bid = blockIdx.x;
    const unsigned xcd = bid % 8u, local = bid / 8u, q = total / 8u, r = total % 8u;
    const unsigned Lu = xcd * q + (xcd < r ? xcd : r) + local;
    alpha = static_cast<int>(Lu / tiles);
    const unsigned t = Lu % tiles;
    constexpr unsigned RG = 8, CG = 4;
    const unsigned tiles_nc = static_cast<unsigned>(sh.tiles_nc);
    const unsigned per_cg = tiles_m * CG;   // tiles of one full column group
    const unsigned cgi = t / per_cg;
    const unsigned first_n = cgi * CG;
    const unsigned cg = (tiles_nc - first_n) < CG ? (tiles_nc - first_n) : CG;
    const unsigned in_cg = t - cgi * per_cg;
    const unsigned rgi = in_cg / (RG * cg);   // blocks before this one are full
    const unsigned first_m = rgi * RG;
    const unsigned rg = (tiles_m - first_m) < RG ? (tiles_m - first_m) : RG;
    const unsigned in_blk = in_cg - rgi * RG * cg;
    tm = static_cast<int>(first_m + in_blk % rg);
    tn = static_cast<int>(first_n + in_blk / rg);   // column tile inside the chunk
    const unsigned tn_layer = static_cast<unsigned>(sh.col0 / kTileN) + static_cast<unsigned>(tn);
    pidx = static_cast<int>(static_cast<unsigned>(alpha) * static_cast<unsigned>(sh.tiles_m * sh.tiles_n) +
                            grouped_tile(static_cast<unsigned>(tm), tn_layer, tiles_m,
                                         static_cast<unsigned>(sh.tiles_n), GM));
}

__device__ __forceinline__ double wave_sum(double v) {
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
    return v;
}

// 16-bit path.  E = X·D over one 256x256 output tile of one alpha with
// v_mfma_f32_32x32x16_f16, or v_mfma_f32_32x32x16_bf16 (BF: the fragments
// hold bf16 bits in the same layout).  Four waves; wave w owns columns [64w, 64w+64)
// of the tile and all 256 rows (8 x 2 accumulator blocks of 32x32 = 256
// accumulation registers).  Per 64-k stage the workgroup copies the 32 KiB
// X block straight into LDS (global_load_lds, no register staging; four
// buffers, the next three stages in flight while the current one feeds the
// matrix cores) and each wave loads its own 8 KiB of error weights into
// registers three stages ahead.  One barrier per stage.
template <bool BF>
__global__ __launch_bounds__(kThreads, 1) void loss_gemm_f16_kernel(const half8 *__restrict__ Xf,
                                                                    const half8 *__restrict__ Df,
                                                                    double *__restrict__ partials, SearchShape sh) {
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    int pidx, alpha, tm, tn;
    map_tile(sh, pidx, alpha, tm, tn);

    // four distinct LDS objects (4 x 32 KiB), so the compiler can tell the
    // copies into one buffer from the reads of another
    __shared__ half8 As0[32 * 64];
    __shared__ half8 As1[32 * 64];
    __shared__ half8 As2[32 * 64];
    __shared__ half8 As3[32 * 64];
    const int64_t xstride = sh.MB32 * 4 * 64;          // half8 per 64-k stage of X
    const int64_t dstride = sh.NB32c * 4 * 64;         // half8 per 64-k stage of D
    const half8 *xsrc = Xf + (static_cast<int64_t>(tm) * 8 + wave * 2) * 4 * 64 + lane;  // this wave's 8 chunks
    const half8 *dsrc = Df + (static_cast<int64_t>(alpha) * sh.KB64 * sh.NB32c + tn * 8 + wave * 2) * 4 * 64 + lane;

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
            if constexpr (BF) {
                const bf16x8 am = __builtin_bit_cast(bf16x8, a[m]);
                acc[m][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(am, __builtin_bit_cast(bf16x8, b[kq]), acc[m][0], 0, 0, 0);
                acc[m][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(am, __builtin_bit_cast(bf16x8, b[4 + kq]), acc[m][1], 0,
                                                                    0, 0);
            } else {
                acc[m][0] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[m], b[kq], acc[m][0], 0, 0, 0);
                acc[m][1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[m], b[4 + kq], acc[m][1], 0, 0, 0);
            }
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
    if (tid == 0) partials[pidx] = ((wred[0] + wred[1]) + wred[2]) + wred[3];
}

// fp32 path (small layers, fp32 inputs): v_mfma_f32_16x16x4_f32, wave w owns
// columns [64w, 64w+64) and all 256 rows of the tile; X staged through LDS.
__global__ __launch_bounds__(kThreads, 1) void loss_gemm_f32_kernel(const float *__restrict__ Xf,
                                                                    const float *__restrict__ Df,
                                                                    double *__restrict__ partials, SearchShape sh) {
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    int pidx, alpha, tm, tn;
    map_tile(sh, pidx, alpha, tm, tn);

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
                b[nt] = Df[(((static_cast<int64_t>(alpha) * sh.KB + kb) * sh.NBc + tn * 16 + wave * 4 + nt) * 8 + ks) * 64 + lane];
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
    if (tid == 0) partials[pidx] = ((wred[0] + wred[1]) + wred[2]) + wred[3];
}

// L(alpha_k) = 2^-2(kx+kd_k) · sum of the tile partials of alpha k: one wave
// per alpha, lanes stride over the tiles, then a fixed butterfly, so the
// result does not depend on scheduling.  alpha* = first minimum; a
// non-finite input or loss gives best = -1.
__global__ __launch_bounds__(1024) void reduce_argmin_kernel(const double *__restrict__ partials, int64_t tiles,
                                                             int n_alpha, const SearchState *__restrict__ st,
                                                             const float *__restrict__ s_tab, int64_t D_in,
                                                             double *__restrict__ losses, int32_t *__restrict__ best,
                                                             float *__restrict__ s_best) {
    __shared__ double L[64];
    __shared__ int bsel;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    for (int k = wave; k < n_alpha; k += 16) {
        const double *p = partials + k * tiles;
        double s0 = 0.0, s1 = 0.0, s2 = 0.0, s3 = 0.0;
        int64_t i = lane;
        for (; i + 192 < tiles; i += 256) {
            s0 += p[i];
            s1 += p[i + 64];
            s2 += p[i + 128];
            s3 += p[i + 192];
        }
        for (; i < tiles; i += 64) s0 += p[i];
        const double v = wave_sum((s0 + s1) + (s2 + s3));
        if (lane == 0) {
            const double Lk = ldexp(v, -2 * (st->kx + st->kd[k]));
            L[k] = Lk;
            losses[k] = Lk;
        }
    }
    __syncthreads();
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
        for (int64_t j = tid; j < D_in; j += 1024) s_best[j] = s_tab[b * D_in + j];
}

// Quantiser at alpha*: codes (int8, row-major [D_in x D_out]) and steps.
// One thread per (group, column); lanes are consecutive columns.
// GC, P: as for quant_all_kernel (P = 4: the workgroup's waves split the
// group's rows of the same 64 columns; columns past D_out compute on w = 0
// and store nothing).
template <int GC, bool WB, bool ASYM, int P>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void quant_select_kernel(
    const void *__restrict__ W, SearchShape sh, const float *__restrict__ s_tab, const int32_t *__restrict__ best,
    int8_t *__restrict__ codes, float *__restrict__ scales, uint8_t *__restrict__ zeros) {
    static_assert(P == 1 || ((P == 2 || P == 4) && GC > 0), "waves per group");
    const int k = best[0];
    if (k < 0) return;   // uniform over the grid
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int part = wave % P;
    const int64_t o = static_cast<int64_t>(blockIdx.x) * (256 / P) + (wave / P) * 64 + lane;
    const int64_t g = blockIdx.y;
    const bool live = o < sh.D_out;
    if (P == 1 && !live) return;
    const int group = GC > 0 ? GC * P : sh.group;
    const int64_t j0 = g * group + part * GC;   // this lane's first row
    const float *s = s_tab + static_cast<int64_t>(k) * sh.D_in + j0;
    const float qmax = ASYM ? static_cast<float>((1 << sh.bits) - 1) : static_cast<float>((1 << (sh.bits - 1)) - 1);
    const float qlo = ASYM ? 0.0f : -qmax;
    const float thr = quant_margin(qmax);
    const int oi = static_cast<int>(live ? o : sh.D_out - 1);   // in-bounds loads
    const uint32_t keep = live ? 0xFFFFFFFFu : 0u;
    auto wp_at = [&](int r) {
        const unsigned char *row = static_cast<const unsigned char *>(W) + (j0 + r) * sh.D_out * (WB ? 2 : 4);
        return s[r] * ld_w_masked<WB>(row, oi, keep);
    };
    auto store8 = [&](int r0, const float *q) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            // symmetric: the clamp only matters for non-finite inputs (which
            // yield best = -1); zero point: quant8z has clamped already
            const float qc = fminf(fmaxf(q[i], qlo), qmax);
            if (!live) continue;
            if constexpr (ASYM)
                reinterpret_cast<uint8_t *>(codes + (j0 + r0 + i) * sh.D_out)[oi] = static_cast<uint8_t>(qc);
            else
                (codes + (j0 + r0 + i) * sh.D_out)[oi] = static_cast<int8_t>(qc);
        }
    };
    // steps stored as float32, or as FP16 bits with FP16 step storage
    auto store_step = [&](float step) {
        if (part != 0 || !live) return;
        if (sh.f16_steps)
            reinterpret_cast<uint16_t *>(scales)[g * sh.D_out + o] =
                __builtin_bit_cast(uint16_t, static_cast<_Float16>(step));
        else
            scales[g * sh.D_out + o] = step;
    };
    auto q8 = [&](const float *wp, float step, float rstep, float zf, float *q) {
        if constexpr (ASYM)
            quant8z(wp, step, rstep, thr, zf, qmax, q);
        else
            quant8(wp, step, rstep, thr, q);
    };
    if constexpr (GC > 0) {
        float wp[GC];
#pragma unroll
        for (int r = 0; r < GC; ++r) wp[r] = wp_at(r);
        float step, zf = 0.0f;
        if constexpr (ASYM) {
            float wlo = 0.0f, whi = 0.0f;
#pragma unroll
            for (int r = 0; r < GC; ++r) {
                wlo = fminf(wlo, wp[r]);
                whi = fmaxf(whi, wp[r]);
            }
            if constexpr (P > 1) {
                __shared__ GroupXchg<P> xchg;
                xchg.combine(0, wave, lane, whi, wlo);
            }
            zp_step(wlo, whi, qmax, sh.f16_steps, step, zf);
            if (part == 0 && live) zeros[g * sh.D_out + o] = static_cast<uint8_t>(zf);
        } else {
            float m = 0.0f;
#pragma unroll
            for (int r = 0; r < GC; ++r) m = fmaxf(m, fabsf(wp[r]));
            if constexpr (P > 1) {
                __shared__ GroupXchg<P> xchg;
                float unused = 0.0f;
                xchg.combine(0, wave, lane, m, unused);
            }
            step = m / qmax;
            if (sh.f16_steps) step = f16_step(step);
        }
        store_step(step);
        if (codes) {
            const float rstep = recip_step(step);
#pragma unroll
            for (int r0 = 0; r0 < GC; r0 += 8) {
                float q[8];
                q8(wp + r0, step, rstep, zf, q);
                store8(r0, q);
            }
        }
    } else {
        float step, zf = 0.0f;
        if constexpr (ASYM) {
            float wlo = 0.0f, whi = 0.0f;
            for (int r = 0; r < group; ++r) {
                const float p = wp_at(r);
                wlo = fminf(wlo, p);
                whi = fmaxf(whi, p);
            }
            zp_step(wlo, whi, qmax, sh.f16_steps, step, zf);
            zeros[g * sh.D_out + o] = static_cast<uint8_t>(zf);
        } else {
            float m = 0.0f;
            for (int r = 0; r < group; ++r) m = fmaxf(m, fabsf(wp_at(r)));
            step = m / qmax;
            if (sh.f16_steps) step = f16_step(step);
        }
        store_step(step);
        if (codes) {
            const float rstep = recip_step(step);
            for (int r0 = 0; r0 < group; r0 += 8) {
                float wp[8], q[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) wp[i] = wp_at(r0 + i);
                q8(wp, step, rstep, zf, q);
                store8(r0, q);
            }
        }
    }
}

// ------------------------------------------------------------- launcher ----

// Waves that share one group's rows in the quantisers: 4 for groups of 256,
// else 1 (splitting groups of 128 over 2 or 4 waves measured no faster).
static int quant_waves_per_group(int group) { return group == 256 ? 4 : 1; }
// The all-alpha quantiser on the bf16 path splits groups of 128 over 2 waves
// as well: one wave holding a column's 128 rows together with the residual
// code of the correction rows needs more than the 168 registers of three
// waves per SIMD and spilled (8.0 ms against 2.4 ms at 8192 x 28672).
static int quant_all_waves_per_group(const SearchShape &sh) {
    return (sh.bf16 && sh.group == 128) ? 2 : quant_waves_per_group(sh.group);
}

SearchWorkspace search_workspace_layout(const SearchShape &sh, int64_t chunk_cols) {
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
    w.off_sel = off;
    off += sh.bf16 ? al(static_cast<size_t>(sh.D_in + kCorrRows) * 4) : 0;
    w.off_x = off;
    off += al(static_cast<size_t>(sh.Mp) * sh.Kp * elt);
    w.off_d = off;
    off += al(static_cast<size_t>(sh.n_alpha) * sh.Kp * static_cast<size_t>(chunk_cols) * elt);
    w.off_part = off;
    off += al(static_cast<size_t>(sh.n_alpha) * sh.tiles_m * sh.tiles_n * 8);
    w.total = off;
    return w;
}

void set_search_chunk(SearchShape &sh, int64_t col0, int64_t cols) {
    sh.col0 = col0;
    sh.Nc = cols;
    sh.NB32c = cols / 32;
    sh.NBc = cols / 16;
    sh.tiles_nc = cols / kTileN;
}

#define AWQ_LAUNCH_CHECK()                          \
    do {                                            \
        hipError_t e__ = hipGetLastError();         \
        if (e__ != hipSuccess) return e__;          \
    } while (0)

static unsigned grid_for_bytes(int64_t bytes, unsigned cap) {
    const int64_t per = 256 * 16 * 4;   // one iteration of four 16-byte loads per thread
    int64_t b = (bytes + per - 1) / per;
    b = b < 1 ? 1 : b;
    return static_cast<unsigned>(b > cap ? cap : b);
}

hipError_t launch_search(const void *X, int xt, const void *W, int wt, const float *a, const float *b,
                         uint8_t *zeros, const AlphaGrid &alphas,
                         const SearchShape &sh, double *losses, int32_t *best, float *s_best, float *scales,
                         int8_t *codes, unsigned char *ws, int64_t chunk_cols, hipStream_t st,
                         hipEvent_t *events) {
    const SearchWorkspace L = search_workspace_layout(sh, chunk_cols);
    SearchState *state = reinterpret_cast<SearchState *>(ws + L.off_state);
    float *s_tab = reinterpret_cast<float *>(ws + L.off_s);
    float *invp_tab = reinterpret_cast<float *>(ws + L.off_invp);
    void *Xf = ws + L.off_x;
    void *Df = ws + L.off_d;
    double *partials = reinterpret_cast<double *>(ws + L.off_part);
    int *sel_pos = sh.bf16 ? reinterpret_cast<int *>(ws + L.off_sel) : nullptr;
    int *sel_idx = sh.bf16 ? sel_pos + sh.D_in : nullptr;
    const int64_t G = sh.D_in / sh.group;
    auto mark = [&](int i) -> hipError_t { return events ? hipEventRecord(events[i], st) : hipSuccess; };
#define AWQ_MARK(i)                              \
    do {                                         \
        hipError_t e__ = mark(i);                \
        if (e__ != hipSuccess) return e__;       \
    } while (0)

    AWQ_MARK(0);
    const int64_t nx = sh.N * sh.D_in, nw = sh.D_in * sh.D_out;
    const unsigned bx = grid_for_bytes(nx * (xt == 1 ? 2 : 4), kAbsmaxXBlocks);
    const unsigned bw = grid_for_bytes(nw * (wt == 1 ? 2 : 4), kAbsmaxWBlocks);
    hipLaunchKernelGGL(absmax_kernel, dim3(bx + bw), dim3(256), 0, st, X, xt, nx, W, wt, nw, static_cast<int>(bx),
                       state);
    AWQ_LAUNCH_CHECK();
    {
        const int gpw = sh.group <= 256 ? 256 / sh.group : 1;
        const int64_t G_ = sh.D_in / sh.group;
        const dim3 grid(static_cast<unsigned>((G_ + gpw - 1) / gpw), static_cast<unsigned>(sh.n_alpha));
        hipLaunchKernelGGL(scale_table_kernel, grid, dim3(256), 0, st, a, b, alphas, sh.D_in, sh.group, gpw, s_tab,
                           state, static_cast<int>(bx), static_cast<int>(bw));
    }
    AWQ_LAUNCH_CHECK();
    if (sh.bf16) {
        hipLaunchKernelGGL(select_rows_kernel, dim3(1), dim3(kSelThreads), 0, st, a, sh.D_in, sel_pos, sel_idx);
        AWQ_LAUNCH_CHECK();
    }
    {
        const int64_t nfin = static_cast<int64_t>(sh.n_alpha) * ((sh.D_in + 255) / 256);
        if (sh.f16) {
            const int64_t nprep = sh.MB32 * ((sh.KB64 + kPrepKB - 1) / kPrepKB);
            if (sh.bf16)
                hipLaunchKernelGGL(prep_x_f16_kernel<true>, dim3(static_cast<unsigned>(nprep + nfin)), dim3(256), 0, st,
                                   static_cast<const uint16_t *>(X), sh, state, static_cast<half8 *>(Xf), nprep, s_tab,
                                   invp_tab, sel_idx);
            else
                hipLaunchKernelGGL(prep_x_f16_kernel<false>, dim3(static_cast<unsigned>(nprep + nfin)), dim3(256), 0,
                                   st, static_cast<const uint16_t *>(X), sh, state, static_cast<half8 *>(Xf), nprep,
                                   s_tab, invp_tab, sel_idx);
        } else {
            const int64_t n = sh.Mp * sh.Kp, nprep = (n + 255) / 256;
            hipLaunchKernelGGL(prep_x_f32_kernel, dim3(static_cast<unsigned>(nprep + nfin)), dim3(256), 0, st, X, xt,
                               sh, static_cast<float *>(Xf), state, nprep, s_tab, invp_tab);
        }
    }
    AWQ_LAUNCH_CHECK();
    AWQ_MARK(1);
    // Error weights and loss contraction, one output-column chunk at a time
    // (one chunk unless the workspace holds fewer columns' error weights).
    for (int64_t col0 = 0; col0 < sh.Np; col0 += chunk_cols) {
        SearchShape shc = sh;
        set_search_chunk(shc, col0, sh.Np - col0 < chunk_cols ? sh.Np - col0 : chunk_cols);
        {
            // 256 / P columns per workgroup (P waves split a group's rows)
            const int64_t cols = 256 / quant_all_waves_per_group(sh);
            const int64_t per_slice = ((shc.Nc + cols - 1) / cols) * G;
            const int aslice = quant_alpha_slice(per_slice, sh.n_alpha, sh.D_in * shc.Nc * (wt == 1 ? 2 : 4));
            const dim3 grid(static_cast<unsigned>((shc.Nc + cols - 1) / cols), static_cast<unsigned>(G),
                            static_cast<unsigned>((sh.n_alpha + aslice - 1) / aslice));
#define AWQ_QALL3(F16, GC, AS, P, BF)                                                                             \
    do {                                                                                                          \
        if (wt == 1)                                                                                              \
            hipLaunchKernelGGL((quant_all_kernel<F16, GC, true, AS, P, BF>), grid, dim3(256), 0, st, W, shc,      \
                               s_tab, invp_tab, Df, aslice, sel_pos);                                             \
        else                                                                                                      \
            hipLaunchKernelGGL((quant_all_kernel<F16, GC, false, AS, P, BF>), grid, dim3(256), 0, st, W, shc,     \
                               s_tab, invp_tab, Df, aslice, sel_pos);                                             \
    } while (0)
#define AWQ_QALL2(F16, GC, AS, P)                                 \
    do {                                                          \
        /* the bf16 path never runs one wave over 128 rows */    \
        if constexpr (F16 && GC != 128) {                         \
            if (sh.bf16)                                          \
                AWQ_QALL3(F16, GC, AS, P, true);                  \
            else                                                  \
                AWQ_QALL3(F16, GC, AS, P, false);                 \
        } else {                                                  \
            AWQ_QALL3(F16, GC, AS, P, false);                     \
        }                                                         \
    } while (0)
#define AWQ_QALL1(F16, GC, P)                \
    do {                                     \
        if (sh.asym)                         \
            AWQ_QALL2(F16, GC, true, P);     \
        else                                 \
            AWQ_QALL2(F16, GC, false, P);    \
    } while (0)
#define AWQ_QALL(F16)                        \
    do {                                     \
        switch (sh.group) {                  \
        case 32: AWQ_QALL1(F16, 32, 1); break;   \
        case 64: AWQ_QALL1(F16, 64, 1); break;   \
        case 128:                                \
            if (F16 && sh.bf16)                  \
                AWQ_QALL1(F16, 64, 2);           \
            else                                 \
                AWQ_QALL1(F16, 128, 1);          \
            break;                               \
        case 256: AWQ_QALL1(F16, 64, 4); break;  \
        default: AWQ_QALL1(F16, 0, 1); break;    \
        }                                    \
    } while (0)
            if (sh.f16)
                AWQ_QALL(true);
            else
                AWQ_QALL(false);
#undef AWQ_QALL
#undef AWQ_QALL1
#undef AWQ_QALL2
#undef AWQ_QALL3
        }
        AWQ_LAUNCH_CHECK();
        if (col0 == 0) AWQ_MARK(2);
        {
            const int64_t blocks = shc.tiles_m * shc.tiles_nc * sh.n_alpha;
            if (sh.bf16)
                hipLaunchKernelGGL(loss_gemm_f16_kernel<true>, dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0,
                                   st, static_cast<const half8 *>(Xf), static_cast<const half8 *>(Df), partials, shc);
            else if (sh.f16)
                hipLaunchKernelGGL(loss_gemm_f16_kernel<false>, dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0,
                                   st, static_cast<const half8 *>(Xf), static_cast<const half8 *>(Df), partials, shc);
            else
                hipLaunchKernelGGL(loss_gemm_f32_kernel, dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0, st,
                                   static_cast<const float *>(Xf), static_cast<const float *>(Df), partials, shc);
        }
        AWQ_LAUNCH_CHECK();
    }
    AWQ_MARK(3);
    hipLaunchKernelGGL(reduce_argmin_kernel, dim3(1), dim3(1024), 0, st, partials, sh.tiles_m * sh.tiles_n,
                       sh.n_alpha, state, s_tab, sh.D_in, losses, best, s_best);
    AWQ_LAUNCH_CHECK();
    {
        const int64_t cols = 256 / quant_waves_per_group(sh.group);   // as for quant_all
        const dim3 grid(static_cast<unsigned>((sh.D_out + cols - 1) / cols), static_cast<unsigned>(G));
#define AWQ_QSEL2(GC, AS, P)                                                                                  \
    do {                                                                                                      \
        if (wt == 1)                                                                                          \
            hipLaunchKernelGGL((quant_select_kernel<GC, true, AS, P>), grid, dim3(256), 0, st, W, sh, s_tab,  \
                               best, codes, scales, zeros);                                                   \
        else                                                                                                  \
            hipLaunchKernelGGL((quant_select_kernel<GC, false, AS, P>), grid, dim3(256), 0, st, W, sh, s_tab, \
                               best, codes, scales, zeros);                                                   \
    } while (0)
#define AWQ_QSEL(GC, P)                  \
    do {                                 \
        if (sh.asym)                     \
            AWQ_QSEL2(GC, true, P);      \
        else                             \
            AWQ_QSEL2(GC, false, P);     \
    } while (0)
        switch (sh.group) {
        case 32: AWQ_QSEL(32, 1); break;
        case 64: AWQ_QSEL(64, 1); break;
        case 128: AWQ_QSEL(128, 1); break;
        case 256: AWQ_QSEL(64, 4); break;
        default: AWQ_QSEL(0, 1); break;
        }
#undef AWQ_QSEL
#undef AWQ_QSEL2
    }
    AWQ_LAUNCH_CHECK();
    AWQ_MARK(4);
#undef AWQ_MARK
    return hipSuccess;
}

}  // namespace awq
