// W4A16 product at prefill batch sizes (M >= 192 rows):
// Y = bf16(X·diag(inv_s)) · Dequant(W_q) on the matrix cores.
//
// [CA] "推論時的等效實現": Y = (X·diag(1/s*))·Dequant(W_quantized), the
// activation scaling folded into the kernel's activation tiles.  [MR]
// "即时权重反量化": the INT4 weights are dequantised to FP16 inside the main
// loop ("为什么 AWQ 能加速本地设备上的 LLM": in the context stage the product
// is compute-bound, unlike decoding).
//
// Design for CDNA4:
//  * A pre-pass finds max|X·inv_s| and, per output column, the largest group
//    step; both become exact power-of-two factors kx and kw[o] that put the
//    activations and the dequantised weights in FP16's range (they are
//    divided out again in the epilogue, exactly).
//  * A second pass writes kx·bf16(X·inv_s) as FP16 (exact: 8 significant bits
//    fit in 11) in v_mfma_f32_32x32x16_f16 A-fragment order, rows padded to
//    256 and k to 64 with zeros.
//  * One workgroup = 4 waves computes a 256x256 tile of Y; wave w owns
//    columns [64w, 64w+64) and all 256 rows (8 x 2 blocks of 32x32 = 256
//    accumulation registers).  Per 64-k stage the workgroup copies the
//    32 KiB activation block straight into LDS (global_load_lds; a ring of
//    four buffers) and each wave loads its packed words (8 per lane per
//    stage: one word = 8 k of one column, exactly one B fragment), both four
//    stages ahead.  The stage barrier sits before the last k-step of a
//    stage, whose fragments are already in registers: the buffer is refilled
//    right after it, and the next stage's first fragments are read while
//    that k-step's MFMAs run.
//  * Dequantisation in registers, two weights per instruction: the nibble
//    order of a word puts rows 2d and 2d+1 at nibbles d and d+4, so one
//    shift and one and-or make the FP16 pair (1024 + n, 1024 + n'), exactly;
//    a packed subtract of 1032 leaves q = n - 8 exactly, and a packed
//    multiply by the column's FP16 step kw·step gives the FP16 weight with
//    one rounding of the product (the step itself is rounded to FP16 once).
//  * The per-stage traffic is 32 KiB of activations and 8 KiB of packed
//    weights for 8.4 MFLOP (about 210 FLOP per byte).
#include "awq_internal.h"

#include <algorithm>

namespace awq {

namespace {

constexpr int kPfTile = 256;
constexpr int kPfParts = 1024;  // most pre-pass blocks over X (one partial maximum each)

typedef _Float16 half2v __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t bf16_bits_rne(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
}

// 2^(top - E) for m in [2^(E-1), 2^E): m·factor lands in [2^(top-1), 2^top).
// 1 for a zero or non-finite m; the exponent is kept well inside float32.
__device__ __forceinline__ float pow2_factor(float m, int top) {
    if (!(m > 0.0f) || !(m <= 3.0e38f)) return 1.0f;
    int E;
    (void)frexpf(m, &E);
    int e = top - E;
    e = e < -100 ? -100 : (e > 100 ? 100 : e);
    return ldexpf(1.0f, e);
}

__device__ __forceinline__ float block_max256(float v, float *red) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    const int wave = threadIdx.x >> 6;
    __syncthreads();
    if ((threadIdx.x & 63) == 0) red[wave] = v;
    __syncthreads();
    return fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

// Pre-pass.  Blocks [0, nbx): partial maxima of |X·inv_s| (float32 product)
// into part[b].  They form a grid of nrb blocks of 256 sixteen-byte column
// runs x nbx / nrb row slabs: a thread keeps one run (so its 8 factors of
// inv_s are loaded once) and reads its rows 8 at a time, a wave one 1 KiB
// row segment per load.  Blocks [nbx, ...): 64 output
// columns each, four group slices per column; kw[o] = power of two with
// max_g |step[g, o]|·kw[o] in [2^11, 2^12), so |q|·step·kw < 2^15 in FP16.
__global__ __launch_bounds__(256) void pf_prep_kernel(const uint16_t *__restrict__ X,
                                                      const float *__restrict__ inv_s, int64_t M, int64_t D_in,
                                                      int nbx, const float *__restrict__ scales, int64_t G,
                                                      int64_t D_out, float *__restrict__ part,
                                                      float *__restrict__ kw) {
    __shared__ float red[256];
    if (static_cast<int>(blockIdx.x) < nbx) {
        const int64_t runs = D_in / 8;
        const int64_t nrb = (runs + 255) / 256;
        const int64_t nrb_grid = nrb < nbx ? nrb : nbx;       // run blocks in the grid (nbx is a multiple)
        const int64_t nslab = nbx / nrb_grid;
        const int64_t slab = blockIdx.x / nrb_grid;
        const uint4 *X4 = reinterpret_cast<const uint4 *>(X);
        float m = 0.0f;
        for (int64_t rb = blockIdx.x % nrb_grid; rb < nrb; rb += nrb_grid) {
            const int64_t run = rb * 256 + threadIdx.x;
            if (run >= runs) continue;
            float iv[8] = {1.0f, 1.0f, 1.0f, 1.0f, 1.0f, 1.0f, 1.0f, 1.0f};
            if (inv_s) {
                const float4 i0v = *reinterpret_cast<const float4 *>(inv_s + run * 8);
                const float4 i1v = *reinterpret_cast<const float4 *>(inv_s + run * 8 + 4);
                iv[0] = i0v.x; iv[1] = i0v.y; iv[2] = i0v.z; iv[3] = i0v.w;
                iv[4] = i1v.x; iv[5] = i1v.y; iv[6] = i1v.z; iv[7] = i1v.w;
            }
            for (int64_t r0 = slab; r0 < M; r0 += 8 * nslab) {
                uint4 xv[8];
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const int64_t row = r0 + u * nslab;
                    xv[u] = row < M ? X4[row * runs + run] : make_uint4(0u, 0u, 0u, 0u);
                }
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const uint32_t xw[4] = {xv[u].x, xv[u].y, xv[u].z, xv[u].w};
#pragma unroll
                    for (int p = 0; p < 4; ++p) {
                        m = fmaxf(m, fabsf(__uint_as_float(xw[p] << 16) * iv[2 * p]));
                        m = fmaxf(m, fabsf(__uint_as_float(xw[p] & 0xFFFF0000u) * iv[2 * p + 1]));
                    }
                }
            }
        }
        m = block_max256(m, red);
        if (threadIdx.x == 0) part[blockIdx.x] = m;
        return;
    }
    const int c = threadIdx.x & 63, slice = threadIdx.x >> 6;
    const int64_t o = static_cast<int64_t>(blockIdx.x - nbx) * 64 + c;
    float m = 0.0f;
    if (o < D_out)
        for (int64_t g = slice; g < G; g += 4) m = fmaxf(m, fabsf(scales[g * D_out + o]));
    red[threadIdx.x] = m;
    __syncthreads();
    if (slice == 0 && o < D_out)
        kw[o] = pow2_factor(fmaxf(fmaxf(red[c], red[c + 64]), fmaxf(red[c + 128], red[c + 192])), 12);
}

// Activation fragments: element (row, k) of kx·bf16(X·inv_s), as FP16, goes
// to half-word slot (((k/64)·MB32 + row/32)·4 + (k%64)/16)·512 +
// ((k%16)/8)·256 + (row%32)·8 + k%8, i.e. lane (k%16)/8·32 + row%32 of chunk
// ((kb·MB32 + mb)·4 + kq).  kx is a power of two with max|X·inv_s|·kx in
// [2^14, 2^15).  One workgroup per 32-row block and kpb 64-k blocks: each
// block is read row-contiguously (8 lanes per 128-byte row run), transposed
// through LDS and written as one contiguous 4 KiB run of fragments.  Zero
// rows >= M and k >= D_in.  Block 0 also stores 1/kx for the epilogue.
__global__ __launch_bounds__(256) void pf_xfrag_kernel(const uint16_t *__restrict__ X,
                                                       const float *__restrict__ inv_s, int64_t M, int64_t D_in,
                                                       int64_t MB32, int64_t KB64, int kpb,
                                                       const float *__restrict__ part, int nbx,
                                                       uint4 *__restrict__ Xf, float *__restrict__ kxinv) {
    __shared__ float red[4];
    __shared__ uint4 tile[256];
    float pm = 0.0f;
    for (int i = threadIdx.x; i < nbx; i += 256) pm = fmaxf(pm, part[i]);
    const float kx = pow2_factor(block_max256(pm, red), 15);
    if (blockIdx.x == 0 && threadIdx.x == 0) kxinv[0] = 1.0f / kx;

    const int64_t mb = blockIdx.x % MB32, kb0 = (blockIdx.x / MB32) * kpb;
    const int r = threadIdx.x >> 3, run = threadIdx.x & 7;
    const int64_t row = mb * 32 + r;
    for (int64_t kb = kb0; kb < kb0 + kpb && kb < KB64; ++kb) {
        const int64_t k0 = kb * 64 + run * 8;
        uint32_t hw[4] = {0u, 0u, 0u, 0u};
        if (row < M && k0 < D_in) {
            const uint4 xv = *reinterpret_cast<const uint4 *>(X + row * D_in + k0);
            const uint32_t xw[4] = {xv.x, xv.y, xv.z, xv.w};
            float iv[8] = {1.0f, 1.0f, 1.0f, 1.0f, 1.0f, 1.0f, 1.0f, 1.0f};
            if (inv_s) {
                const float4 i0 = *reinterpret_cast<const float4 *>(inv_s + k0);
                const float4 i1 = *reinterpret_cast<const float4 *>(inv_s + k0 + 4);
                iv[0] = i0.x; iv[1] = i0.y; iv[2] = i0.z; iv[3] = i0.w;
                iv[4] = i1.x; iv[5] = i1.y; iv[6] = i1.z; iv[7] = i1.w;
            }
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                float lo = __uint_as_float(xw[p] << 16), hi = __uint_as_float(xw[p] & 0xFFFF0000u);
                if (inv_s) {
                    lo = __uint_as_float(bf16_bits_rne(lo * iv[2 * p]) << 16);
                    hi = __uint_as_float(bf16_bits_rne(hi * iv[2 * p + 1]) << 16);
                }
                const half2v h = {static_cast<_Float16>(lo * kx), static_cast<_Float16>(hi * kx)};
                hw[p] = __builtin_bit_cast(uint32_t, h);
            }
        }
        __syncthreads();   // the previous block's tile has been read
        tile[(run >> 1) * 64 + (run & 1) * 32 + r] = make_uint4(hw[0], hw[1], hw[2], hw[3]);
        __syncthreads();
        Xf[(kb * MB32 + mb) * 256 + threadIdx.x] = tile[threadIdx.x];
    }
}

// (mask & a) | (~mask & b) in one instruction (the compiler otherwise emits
// an and and an or, gfx9 VOP3 taking no literal operands)
__device__ __forceinline__ uint32_t bit_insert(uint32_t mask, uint32_t a, uint32_t b) {
    uint32_t r;
    asm("v_bfi_b32 %0, %1, %2, %3" : "=v"(r) : "s"(mask), "v"(a), "v"(b));
    return r;
}

// off1 / off16 are 1024 + 8 and 1024 + 16·8 for signed codes (nibble q + 8),
// 1024 + z and 1024 + 16z for zero-point codes (all exact in FP16).
__device__ __forceinline__ half8 dequant_word(uint32_t w, half2v step16, half2v step16_16, half2v off1,
                                              half2v off16) {
    const uint32_t w8 = w >> 8;
    const uint32_t p0 = bit_insert(0x000F000Fu, w, 0x64006400u);
    const uint32_t p1 = bit_insert(0x00F000F0u, w, 0x64006400u);
    const uint32_t p2 = bit_insert(0x000F000Fu, w8, 0x64006400u);
    const uint32_t p3 = bit_insert(0x00F000F0u, w8, 0x64006400u);
    const half2v h0 = (__builtin_bit_cast(half2v, p0) - off1) * step16;
    const half2v h1 = (__builtin_bit_cast(half2v, p1) - off16) * step16_16;
    const half2v h2 = (__builtin_bit_cast(half2v, p2) - off1) * step16;
    const half2v h3 = (__builtin_bit_cast(half2v, p3) - off16) * step16_16;
    half8 v;
    v[0] = h0[0]; v[1] = h0[1];
    v[2] = h1[0]; v[3] = h1[1];
    v[4] = h2[0]; v[5] = h2[1];
    v[6] = h3[0]; v[7] = h3[1];
    return v;
}

// XCD-contiguous tile order (workgroups are dispatched round-robin over the
// 8 XCDs), walked in groups of 8 row tiles x all column tiles.
__device__ __forceinline__ void pf_map_tile(int64_t tiles_m, int64_t tiles_n, int &tm, int &tn) {
    const unsigned total = static_cast<unsigned>(tiles_m * tiles_n);
    const unsigned bid = blockIdx.x;
    const unsigned xcd = bid % 8u, local = bid / 8u, q = total / 8u, r = total % 8u;
    const unsigned t = xcd * q + (xcd < r ? xcd : r) + local;
    constexpr unsigned GM = 8;
    const unsigned tm_all = static_cast<unsigned>(tiles_m);
    const unsigned per_group = GM * static_cast<unsigned>(tiles_n);
    const unsigned first_m = (t / per_group) * GM;
    const unsigned gm = (tm_all - first_m) < GM ? (tm_all - first_m) : GM;
    const unsigned in_group = t % per_group;
    tm = static_cast<int>(first_m + in_group % gm);
    tn = static_cast<int>(in_group / gm);
}

struct PfShape {
    int64_t M, D_in, D_out, Mp, KB64, MB32, tiles_m, tiles_n;
    int64_t ld;          // row stride of packed, scales, zeros and Y (the layer's columns; D_out: this launch's)
    int group, gshift;   // group = 2^gshift
    int kb_per;          // 64-k stages per k split (gridDim.y splits; KB64 when 1)
};

// GPS: group steps per 64-k stage (1 when group >= 64, 2 when group == 32).
// ZP: zero-point codes, weight (n − z)·step with z from zeros[g][o].
template <int GPS, bool OUT_BF16, bool ZP>
__global__ __launch_bounds__(256, 1) void w4a16_prefill_kernel(const uint4 *__restrict__ Xf,
                                                               const uint32_t *__restrict__ packed,
                                                               const float *__restrict__ scales,
                                                               const uint8_t *__restrict__ zeros,
                                                               const float *__restrict__ kw,
                                                               const float *__restrict__ kxinv, PfShape sh,
                                                               void *__restrict__ Y, float *__restrict__ ypart) {
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform, kept in a scalar register
    int tm, tn;
    pf_map_tile(sh.tiles_m, sh.tiles_n, tm, tn);

    __shared__ uint4 As0[32 * 64];
    __shared__ uint4 As1[32 * 64];
    __shared__ uint4 As2[32 * 64];
    __shared__ uint4 As3[32 * 64];
    // this workgroup's k split: stages [kbase, kbase + KB) of the 64-k stages
    const int kbase = static_cast<int>(blockIdx.y) * sh.kb_per;
    // Every stage address is a wave-uniform base plus a 32-bit lane offset.
    const int64_t xstage = sh.MB32 * 4 * 64 * 16;                                       // bytes per 64-k stage
    const char *xbase = reinterpret_cast<const char *>(Xf) + (static_cast<int64_t>(tm) * 8 + wave * 2) * 4 * 1024;
    const uint32_t xlane = static_cast<uint32_t>(lane) * 16u;

    // this lane's two columns (one per 32-column block) and k half of the fragment
    const int hi = lane >> 5;
    const int64_t col0 = static_cast<int64_t>(tn) * kPfTile + wave * 64 + (lane & 31);
    const uint32_t colA = static_cast<uint32_t>(col0 < sh.D_out ? col0 : sh.D_out - 1);        // clamped loads
    const uint32_t colB = static_cast<uint32_t>(col0 + 32 < sh.D_out ? col0 + 32 : sh.D_out - 1);
    const float kwA = kw[colA], kwB = kw[colB];
    const uint32_t sA = colA * 4u, sB = colB * 4u;                                        // step offsets
    const uint32_t wA = (static_cast<uint32_t>(hi) * static_cast<uint32_t>(sh.ld) + colA) * 4u;
    const uint32_t wB = (static_cast<uint32_t>(hi) * static_cast<uint32_t>(sh.ld) + colB) * 4u;
    const int glast = static_cast<int>((sh.D_in >> sh.gshift) - 1);
    const int KR2 = static_cast<int>(sh.D_in / 8 - 2);                          // last even row block
    const int64_t rowbytes = sh.ld * 4;

    floatx16 acc[8][2];
#pragma unroll
    for (int m = 0; m < 8; ++m)
#pragma unroll
        for (int n = 0; n < 2; ++n)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[m][n][i] = 0.0f;

    struct Stage {
        uint32_t w[4][2];           // [k step][column block]
        float sc[GPS][2];           // group steps
        uint32_t zp[ZP ? GPS : 1][2];   // zero points (zero-point codes only), converted at use
    };
    Stage s0, s1, s2, s3;

    // 8 copies of 1 KiB per wave and stage; the immediate offset advances the
    // global and the LDS address together
    auto load_a = [&](int kb, int buf) {
        const char *src = xbase + static_cast<int64_t>(kbase + kb) * xstage + xlane;
        uint4 *dst = (buf == 0 ? As0 : (buf == 1 ? As1 : (buf == 2 ? As2 : As3))) + wave * 512;
        const auto *g0 = (const __attribute__((address_space(1))) void *)src;
        const auto *g1 = (const __attribute__((address_space(1))) void *)(src + 4096);
        auto *l0 = (__attribute__((address_space(3))) void *)dst;
        auto *l1 = (__attribute__((address_space(3))) void *)(dst + 256);
        __builtin_amdgcn_global_load_lds(g0, l0, 16, 0, 0);
        __builtin_amdgcn_global_load_lds(g0, l0, 16, 1024, 0);
        __builtin_amdgcn_global_load_lds(g0, l0, 16, 2048, 0);
        __builtin_amdgcn_global_load_lds(g0, l0, 16, 3072, 0);
        __builtin_amdgcn_global_load_lds(g1, l1, 16, 0, 0);
        __builtin_amdgcn_global_load_lds(g1, l1, 16, 1024, 0);
        __builtin_amdgcn_global_load_lds(g1, l1, 16, 2048, 0);
        __builtin_amdgcn_global_load_lds(g1, l1, 16, 3072, 0);
    };
    auto load_b = [&](int kb, Stage &S) {
#pragma unroll
        for (int kq = 0; kq < 4; ++kq) {
            int rb = (kbase + kb) * 8 + kq * 2;  // row block of lanes 0-31; lanes 32-63 take the next
            rb = rb < KR2 ? rb : KR2;            // k padding: any finite weight (the activations there are 0)
            const char *row = reinterpret_cast<const char *>(packed) + static_cast<int64_t>(rb) * rowbytes;
            S.w[kq][0] = *reinterpret_cast<const uint32_t *>(row + wA);
            S.w[kq][1] = *reinterpret_cast<const uint32_t *>(row + wB);
        }
#pragma unroll
        for (int j = 0; j < GPS; ++j) {
            int g = ((kbase + kb) * 64 + j * 32) >> sh.gshift;
            g = g < glast ? g : glast;
            const char *srow = reinterpret_cast<const char *>(scales) + static_cast<int64_t>(g) * rowbytes;
            S.sc[j][0] = *reinterpret_cast<const float *>(srow + sA);
            S.sc[j][1] = *reinterpret_cast<const float *>(srow + sB);
            if constexpr (ZP) {
                const uint8_t *zrow = zeros + static_cast<int64_t>(g) * sh.ld;
                S.zp[j][0] = zrow[colA];
                S.zp[j][1] = zrow[colB];
            }
        }
    };
    auto read_a = [&](int buf, int kq, half8 *a) {
        const uint4 *base = (buf == 0 ? As0 : (buf == 1 ? As1 : (buf == 2 ? As2 : As3))) + kq * 64 + lane;
#pragma unroll
        for (int m = 0; m < 8; ++m) {
            const uint4 v = base[m * 4 * 64];
            a[m] = __builtin_bit_cast(half8, v);
        }
    };
    // per stage and wave: 8 LDS copies + 8 word loads + 2·GPS step loads
    // (+ 2·GPS zero-point loads)
    constexpr int kVm = 16 + 2 * GPS * (ZP ? 2 : 1);
    static_assert(2 * kVm <= 63, "stage loads must fit the wait count");
    // s_waitcnt encoding of vmcnt(2·kVm) lgkmcnt(0): vmcnt[3:0] in bits 3:0,
    // vmcnt[5:4] in bits 15:14, expcnt 7 (no wait) in bits 6:4
    constexpr int kWaitStage = (((2 * kVm) >> 4) << 14) | ((2 * kVm) & 15) | 0x70;
    // the prologue's first wait: vmcnt(3·kVm) lgkmcnt(0)
    static_assert(3 * kVm <= 63, "three stages of loads must fit the wait count");
    constexpr int kWaitFirst = (((3 * kVm) >> 4) << 14) | ((3 * kVm) & 15) | 0x70;
    // One stage = 4 k-steps of 16.  The 8 A fragments of k-step kq+1 are read
    // from LDS while the 16 MFMAs of k-step kq run (two register sets), and
    // the B fragments of the next k-step are dequantised meanwhile; the last
    // k-step dequantises k-step 0 of the next stage, carried in bq.
    // FP16 steps kw·step of this lane's two columns, and the same / 16
    // and the FP16 offsets of the nibble pairs (see dequant_word)
    auto steps16 = [&](const Stage &S, half2v (&st)[GPS][2][4]) {
#pragma unroll
        for (int j = 0; j < GPS; ++j) {
            const float fa = S.sc[j][0] * kwA, fb = S.sc[j][1] * kwB;
            const _Float16 sa = static_cast<_Float16>(fa), sb = static_cast<_Float16>(fb);
            const _Float16 sa16 = static_cast<_Float16>(static_cast<float>(sa) * 0.0625f);
            const _Float16 sb16 = static_cast<_Float16>(static_cast<float>(sb) * 0.0625f);
            st[j][0][0] = half2v{sa, sa};
            st[j][0][1] = half2v{sa16, sa16};
            st[j][1][0] = half2v{sb, sb};
            st[j][1][1] = half2v{sb16, sb16};
#pragma unroll
            for (int n = 0; n < 2; ++n) {
                const float z = ZP ? static_cast<float>(S.zp[ZP ? j : 0][n]) : 8.0f;
                const _Float16 o1 = static_cast<_Float16>(1024.0f + z), o16 = static_cast<_Float16>(1024.0f + 16.0f * z);
                st[j][n][2] = half2v{o1, o1};
                st[j][n][3] = half2v{o16, o16};
            }
        }
    };
    half8 bq[2];
    auto lds_buf = [&](int buf) { return buf == 0 ? As0 : (buf == 1 ? As1 : (buf == 2 ? As2 : As3)); };
    // 16 MFMAs of one k-step; with a_next, the 8 A fragments of k-step rkq of
    // buffer rbuf are read meanwhile (one read per two MFMAs)
    auto mma_step = [&](const half8 *a, const half8 *b, int rbuf, int rkq, half8 *a_next) {
#pragma unroll
        for (int m = 0; m < 8; ++m) {
            acc[m][0] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[m], b[0], acc[m][0], 0, 0, 0);
            acc[m][1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[m], b[1], acc[m][1], 0, 0, 0);
            if (a_next) a_next[m] = __builtin_bit_cast(half8, lds_buf(rbuf)[(m * 4 + rkq) * 64 + lane]);
        }
    };
    // stage s+1 has landed when at most 2·kVm later loads are outstanding (the
    // groups of stages s+2 and s+3); then all waves meet (no memory fence:
    // each wave waited for its own copies and its own LDS reads)
    auto wait_stage = [&]() {
        __builtin_amdgcn_s_waitcnt(kWaitStage);
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
    };
    // Scheduling of the two regions of a stage.  A (k-steps 0..2, before the
    // stage barrier): 12 units of "2 MFMA, 1 LDS read, 2 MFMA, 1 LDS read".
    // B (k-step 3, after it): 4 units of "2 MFMA, 1 LDS read, 2 MFMA, 1 LDS
    // read, global loads" (the next stage's k-step 0 fragments, then this
    // stage's refill: 8 activation copies and kVm - 8 word and step loads).
    // The dequantisation VALU is left to the scheduler, which spreads it
    // between the MFMAs.
    auto pin_a = [&]() {
#pragma unroll
        for (int u = 0; u < 12; ++u) {
            __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
    };
    auto pin_b = [&]() {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            if (u < kVm % 4)
                __builtin_amdgcn_sched_group_barrier(0x010, kVm / 4 + 1, 0);
            else
                __builtin_amdgcn_sched_group_barrier(0x010, kVm / 4, 0);
        }
    };

    const int KB = static_cast<int>(sh.KB64 - kbase < sh.kb_per ? sh.KB64 - kbase : sh.kb_per);   // >= 1
    const int last = KB - 1;
    auto clampk = [&](int k) { return k < last ? k : last; };
    // One stage s in LDS buffer buf = s % 4 with words S (stage s) and Sn
    // (stage s+1); a0 holds its k-step 0 fragments on entry and the next
    // stage's on exit.  The stage barrier sits between k-steps 2 and 3: the
    // fragments of k-step 3 are already in registers, so buffer buf is free
    // for the activations of stage s+4, and the reads of the next stage's
    // k-step 0 and the barrier's skew hide behind the 16 MFMAs of k-step 3.
    half8 a0[8];
    auto stage = [&](int s, int buf, Stage &S, const Stage &Sn) {
        half2v st[GPS][2][4];
        steps16(S, st);
        half8 b0[2], b1[2], a1[8];
#pragma unroll
        for (int n = 0; n < 2; ++n) b1[n] = dequant_word(S.w[1][n], st[0][n][0], st[0][n][1], st[0][n][2], st[0][n][3]);
        mma_step(a0, bq, buf, 1, a1);
#pragma unroll
        for (int n = 0; n < 2; ++n) b0[n] = dequant_word(S.w[2][n], st[GPS - 1][n][0], st[GPS - 1][n][1], st[GPS - 1][n][2],
                                                       st[GPS - 1][n][3]);
        mma_step(a1, b1, buf, 2, a0);
#pragma unroll
        for (int n = 0; n < 2; ++n) b1[n] = dequant_word(S.w[3][n], st[GPS - 1][n][0], st[GPS - 1][n][1], st[GPS - 1][n][2],
                                                       st[GPS - 1][n][3]);
        mma_step(a0, b0, buf, 3, a1);
        pin_a();
        __builtin_amdgcn_sched_barrier(0);
        wait_stage();
        __builtin_amdgcn_sched_barrier(0);
        mma_step(a1, b1, (buf + 1) & 3, 0, a0);
        {
            // the next stage's first B fragments: its words landed with the
            // stage wait above
            half2v stn[GPS][2][4];
            steps16(Sn, stn);
#pragma unroll
            for (int n = 0; n < 2; ++n) bq[n] = dequant_word(Sn.w[0][n], stn[0][n][0], stn[0][n][1], stn[0][n][2], stn[0][n][3]);
        }
        load_a(clampk(s + 4), buf);
        load_b(clampk(s + 4), S);
        pin_b();
        __builtin_amdgcn_sched_barrier(0);
    };

    // Load groups, one per stage: group t = the activations of stage t+4 (into
    // buffer t % 4, free after the barrier of stage t) and the words of stage
    // t+4.  The prologue issues groups -4..-1 (stages 0..3) in order; the
    // first wait lets groups -3..-1 stay in flight.
    load_a(0, 0);
    load_b(0, s0);
    __builtin_amdgcn_sched_barrier(0);
    load_a(clampk(1), 1);
    load_b(clampk(1), s1);
    __builtin_amdgcn_sched_barrier(0);
    load_a(clampk(2), 2);
    load_b(clampk(2), s2);
    __builtin_amdgcn_sched_barrier(0);
    load_a(clampk(3), 3);
    load_b(clampk(3), s3);
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(kWaitFirst);
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    {
        half8 *dst = a0;
#pragma unroll
        for (int m = 0; m < 8; ++m) dst[m] = __builtin_bit_cast(half8, As0[(m * 4) * 64 + lane]);
        half2v st0[GPS][2][4];
        steps16(s0, st0);
#pragma unroll
        for (int n = 0; n < 2; ++n) bq[n] = dequant_word(s0.w[0][n], st0[0][n][0], st0[0][n][1], st0[0][n][2], st0[0][n][3]);
    }
    // four stages per iteration (the register sets rotate with the buffers),
    // then the last KB mod 4 stages (wave-uniform conditions; exits between
    // the stages of the loop body make the compiler spill)
    int kb = 0;
    for (; kb + 4 <= KB; kb += 4) {
        stage(kb, 0, s0, s1);
        stage(kb + 1, 1, s1, s2);
        stage(kb + 2, 2, s2, s3);
        stage(kb + 3, 3, s3, s0);
    }
    if (kb < KB) {
        stage(kb, 0, s0, s1);
        if (kb + 1 < KB) {
            stage(kb + 1, 1, s1, s2);
            if (kb + 2 < KB) stage(kb + 2, 2, s2, s3);
        }
    }
    // the refills past the last stage (clamped, never read) land before exit
    __builtin_amdgcn_s_waitcnt(0x0070);   // vmcnt(0) lgkmcnt(0)

    // undo the power-of-two factors (exact); 32x32 C layout: register r of
    // block (m, n) holds row 8·(r/4) + 4·(lane/32) + r%4, column lane%32
    const float kxi = kxinv[0];
    const float un[2] = {kxi * (1.0f / kwA), kxi * (1.0f / kwB)};
#pragma unroll
    for (int m = 0; m < 8; ++m)
#pragma unroll
        for (int n = 0; n < 2; ++n) {
            const int64_t col = static_cast<int64_t>(tn) * kPfTile + wave * 64 + n * 32 + (lane & 31);
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int64_t row = static_cast<int64_t>(tm) * kPfTile + m * 32 + 8 * (r / 4) + 4 * hi + r % 4;
                if (row < sh.M && col < sh.D_out) {
                    const float v = acc[m][n][r] * un[n];
                    if (gridDim.y > 1)   // a k split: float32 partial, summed in split order afterwards
                        ypart[(static_cast<int64_t>(blockIdx.y) * sh.M + row) * sh.D_out + col] = v;
                    else if (OUT_BF16)
                        static_cast<uint16_t *>(Y)[row * sh.ld + col] = static_cast<uint16_t>(bf16_bits_rne(v));
                    else
                        static_cast<float *>(Y)[row * sh.ld + col] = v;
                }
            }
        }
}

// k splits of the product: grids of fewer than 256 tiles (one workgroup per
// CU) split k so that about 256 workgroups run, each split at least 8 stages.
static int pf_ksplit(int64_t M, int64_t D_in, int64_t D_out) {
    const int64_t tiles = ((M + kPfTile - 1) / kPfTile) * ((D_out + kPfTile - 1) / kPfTile);
    const int64_t KB = (D_in + 63) / 64;
    int z = 1;
    while (z < 4 && tiles * z * 2 <= 256 && KB >= static_cast<int64_t>(z) * 2 * 8) z *= 2;
    return z;
}

// Tail split: with one 256 x 256 tile per CU, a last round of R < 256 tiles
// leaves CUs idle.  When at least one full round precedes it and the last
// ceil(R / tiles_m) column tiles hold at most half as many tiles as there
// are CUs, those column tiles run in a second launch split 2 ways along k
// (each half at least 8 stages), summed in split order by
// pf_tail_reduce_kernel.  A lightly loaded last round already runs faster
// per tile than a full one, so the gain is smaller than half a round:
// 8192 x 28672 (HIP events per call), M = 1280 698 -> 639 µs, M = 1792
// 934 -> 863 µs, M = 2048 938 -> 908 µs.
constexpr int64_t kPfCUs = 256;
static int64_t pf_tail_cols(int64_t M, int64_t D_in, int64_t D_out) {
    if (pf_ksplit(M, D_in, D_out) > 1) return 0;
    const int64_t tm = (M + kPfTile - 1) / kPfTile, tn = (D_out + kPfTile - 1) / kPfTile;
    const int64_t T = tm * tn, R = T % kPfCUs;
    if (T < kPfCUs || R == 0 || (D_in + 63) / 64 < 16) return 0;
    const int64_t tc = (R + tm - 1) / tm;
    return (tc < tn && 2 * tc * tm <= kPfCUs) ? tc : 0;
}

// Y[row, col] (row stride ld) = part[0][row][col] + part[1][row][col] over
// M x nc contiguous partials, in split order.
template <bool OUT_BF16>
__global__ __launch_bounds__(256) void pf_tail_reduce_kernel(const float *__restrict__ part, int64_t M, int64_t nc,
                                                             int64_t ld, void *__restrict__ Y) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    if (i >= M * nc) return;
    const int64_t row = i / nc, col = i % nc;
    float v = 0.0f;
    v += part[i];
    v += part[M * nc + i];
    if (OUT_BF16)
        static_cast<uint16_t *>(Y)[row * ld + col] = static_cast<uint16_t>(bf16_bits_rne(v));
    else
        static_cast<float *>(Y)[row * ld + col] = v;
}

struct PfLayout {
    size_t off_kw, off_part, off_kx, off_ypart, total;
};

PfLayout pf_layout(int64_t M, int64_t D_in, int64_t D_out) {
    auto up = [](size_t b) { return (b + 255) / 256 * 256; };
    const int64_t Mp = (M + kPfTile - 1) / kPfTile * kPfTile, Kp = (D_in + 63) / 64 * 64;
    PfLayout L{};
    L.off_kw = up(static_cast<size_t>(Mp) * static_cast<size_t>(Kp) * 2);
    L.off_part = L.off_kw + up(static_cast<size_t>(D_out) * 4);
    L.off_kx = L.off_part + up(kPfParts * 4);
    L.off_ypart = L.off_kx + 256;
    const int z = pf_ksplit(M, D_in, D_out);
    const int64_t tail = pf_tail_cols(M, D_in, D_out);
    const int64_t tail_nc = tail > 0 ? D_out - ((D_out + kPfTile - 1) / kPfTile - tail) * kPfTile : 0;
    size_t part_bytes = z > 1 ? static_cast<size_t>(z) * M * D_out * 4 : 0;
    part_bytes = std::max(part_bytes, static_cast<size_t>(2) * M * tail_nc * 4);
    L.total = L.off_ypart + up(part_bytes);
    return L;
}

}  // namespace

bool w4a16_prefill_applies(int64_t M, int64_t D_in, int64_t D_out) {
    const int64_t tiles = ((M + kPfTile - 1) / kPfTile) * ((D_out + kPfTile - 1) / kPfTile);
    // from 192 rows: at 128-160 rows the decode passes still win (8192 x 28672, M = 128:
    // 133-141 against 189-202 µs; M = 192: equal; M = 256: 248 against 194 µs)
    return M >= 192 && tiles >= 64 && D_in >= 64;
}

size_t w4a16_prefill_workspace_bytes(int64_t M, int64_t D_in, int64_t D_out) {
    return pf_layout(M, D_in, D_out).total;
}

hipError_t launch_w4a16_prefill(const void *X, int64_t M, int64_t D_in, int64_t D_out, const uint32_t *packed,
                                const float *scales, const uint8_t *zeros, int group, const float *inv_s, void *Y,
                                int yt, void *ws, hipStream_t st) {
    PfShape sh{};
    sh.M = M;
    sh.D_in = D_in;
    sh.D_out = D_out;
    sh.Mp = (M + kPfTile - 1) / kPfTile * kPfTile;
    sh.KB64 = (D_in + 63) / 64;
    sh.MB32 = sh.Mp / 32;
    sh.tiles_m = sh.Mp / kPfTile;
    sh.tiles_n = (D_out + kPfTile - 1) / kPfTile;
    sh.ld = D_out;
    sh.group = group;
    sh.gshift = 0;
    while ((1 << sh.gshift) < group) ++sh.gshift;   // group is 32·2^k
    const int z = pf_ksplit(M, D_in, D_out);
    sh.kb_per = static_cast<int>((sh.KB64 + z - 1) / z);
    const PfLayout L = pf_layout(M, D_in, D_out);
    unsigned char *base = static_cast<unsigned char *>(ws);
    uint4 *Xf = reinterpret_cast<uint4 *>(base);
    float *kw = reinterpret_cast<float *>(base + L.off_kw);
    float *part = reinterpret_cast<float *>(base + L.off_part);
    float *kxinv = reinterpret_cast<float *>(base + L.off_kx);
    float *ypart = reinterpret_cast<float *>(base + L.off_ypart);
    const int64_t n8 = M * (D_in / 8);
    // about 2048 sixteen-byte loads per block, at most kPfParts blocks, as a
    // whole number of row slabs over the run blocks
    const int64_t nrb = std::min<int64_t>((D_in / 8 + 255) / 256, kPfParts);
    const int64_t want = std::min<int64_t>(kPfParts, std::max<int64_t>(1, (n8 + 2047) / 2048));
    const int64_t nslab = std::max<int64_t>(1, std::min<int64_t>(M, want / nrb));
    const int nbx = static_cast<int>(nrb * nslab);
    const int ncb = static_cast<int>((D_out + 63) / 64);
    hipLaunchKernelGGL(pf_prep_kernel, dim3(static_cast<unsigned>(nbx + ncb)), dim3(256), 0, st,
                       static_cast<const uint16_t *>(X), inv_s, M, D_in, nbx, scales, D_in / group, D_out, part, kw);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    {
        const int64_t blocks = sh.MB32 * sh.KB64;
        const int kpb = static_cast<int>(std::min<int64_t>(8, std::max<int64_t>(1, blocks / 1024)));
        const int64_t grid = sh.MB32 * ((sh.KB64 + kpb - 1) / kpb);
        hipLaunchKernelGGL(pf_xfrag_kernel, dim3(static_cast<unsigned>(grid)), dim3(256), 0, st,
                           static_cast<const uint16_t *>(X), inv_s, M, D_in, sh.MB32, sh.KB64, kpb, part, nbx, Xf,
                           kxinv);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    // one launch of the product over columns [c0, c0 + shape.D_out) with
    // gridDim.y = zs k splits
    auto launch = [&](const PfShape &shape, int64_t c0, int zs) {
        const dim3 grid(static_cast<unsigned>(shape.tiles_m * shape.tiles_n), static_cast<unsigned>(zs));
        const uint32_t *pk = packed + c0;
        const float *sc = scales + c0;
        const uint8_t *zr = zeros ? zeros + c0 : nullptr;
        const float *kwc = kw + c0;
        void *Yc = static_cast<unsigned char *>(Y) + c0 * (yt == 1 ? 2 : 4);
#define AWQ_PF(GPS, OB, ZP) \
    hipLaunchKernelGGL((w4a16_prefill_kernel<GPS, OB, ZP>), grid, dim3(256), 0, st, Xf, pk, sc, zr, kwc, kxinv, \
                       shape, Yc, ypart)
#define AWQ_PF2(GPS, OB)            \
    do {                            \
        if (zr)                     \
            AWQ_PF(GPS, OB, true);  \
        else                        \
            AWQ_PF(GPS, OB, false); \
    } while (0)
        if (group >= 64) {
            if (yt == 1)
                AWQ_PF2(1, true);
            else
                AWQ_PF2(1, false);
        } else {
            // group 32: signed codes only (zero-point codes take the decode path)
            if (yt == 1)
                AWQ_PF(2, true, false);
            else
                AWQ_PF(2, false, false);
        }
#undef AWQ_PF2
#undef AWQ_PF
        return hipGetLastError();
    };
    const int64_t tail = pf_tail_cols(M, D_in, D_out);
    if (tail == 0) {
        e = launch(sh, 0, z);
        if (e != hipSuccess || z == 1) return e;
        return launch_w4a16_reduce(ypart, z, M * D_out, Y, yt, st);
    }
    // full rounds over the leading column tiles, then the tail's column tiles
    // split 2 ways along k and summed in split order
    const int64_t c0 = (sh.tiles_n - tail) * kPfTile;
    PfShape head = sh, rest = sh;
    head.D_out = c0;
    head.tiles_n = sh.tiles_n - tail;
    rest.D_out = D_out - c0;
    rest.tiles_n = tail;
    rest.kb_per = static_cast<int>((sh.KB64 + 1) / 2);
    e = launch(head, 0, 1);
    if (e != hipSuccess) return e;
    e = launch(rest, c0, 2);
    if (e != hipSuccess) return e;
    const int64_t count = M * rest.D_out;
    void *Yc = static_cast<unsigned char *>(Y) + c0 * (yt == 1 ? 2 : 4);
    if (yt == 1)
        hipLaunchKernelGGL(pf_tail_reduce_kernel<true>, dim3(static_cast<unsigned>((count + 255) / 256)), dim3(256), 0,
                           st, ypart, M, rest.D_out, D_out, Yc);
    else
        hipLaunchKernelGGL(pf_tail_reduce_kernel<false>, dim3(static_cast<unsigned>((count + 255) / 256)), dim3(256),
                           0, st, ypart, M, rest.D_out, D_out, Yc);
    return hipGetLastError();
}

}  // namespace awq
