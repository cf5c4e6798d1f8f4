// W4A16 inference product Y = (X·diag(inv_s))·Dequant(W_q).
//
// [CA] "推論時的等效實現": online, Y = (X·diag(1/s*))·Dequant(W_quantized), the
// activation scaling may be fused into the kernel.  [MR] "即时权重反量化": INT4
// weights are dequantised on the fly inside the main loop, and "为什么 AWQ 能加
// 速本地设备上的 LLM": at decode batch sizes the product is bound by weight
// traffic, which 4-bit storage cuts to a quarter.
//
// Design for CDNA4 (decode, M <= 32 rows per launch):
//  * One workgroup of 8 waves (4 without the two-batch pipeline below) owns
//    64 output columns; the waves split the k axis and meet in LDS at the end
//    (fixed order, deterministic).  D_out/64 workgroups, times a k split
//    across workgroups when that leaves too few of them.
//  * Per 32-row k step, lane (c, n) = (lane/16, lane%16) holds the packed
//    words of rows 8c..8c+7 for columns 4n..4n+3 in one 16-byte load: a wave
//    reads 1 KiB as four 256-byte runs.  Each wave issues the loads of 4 k
//    steps (words, activation fragments, steps) as one batch.  Up to 16 rows
//    with groups of 128 or more, each wave keeps two batches in flight (the
//    next batch's loads are issued before the current one is consumed), so
//    about one 8-wave workgroup per CU already has enough bytes in flight and
//    most layers need no k split, hence no reduction launch; otherwise one
//    batch is in flight per wave and many small workgroups per CU hide each
//    other's latency.
//  * Word t becomes the B operand of a 16x16x32 bf16 MFMA with two ALU ops
//    per register pair, ((w >> 4d) & 0x000F000F) | 0x43004300 = bf16(136 + q);
//    the constant offset is removed by one extra MFMA against bf16(136)
//    (136·sum X per row), and the per-group step scales the float32 partial of
//    each group, so no per-weight multiply is needed.
//  * The activations bf16(X·inv_s) (X itself without inv_s, rounded once)
//    reach the waves in one of four ways: up to 8 rows (4 with one strip),
//    each workgroup stages its whole k range in LDS; 9..16 rows on wide
//    layers, w4a16_ring_kernel stages 1024-k chunks in an LDS ring; up to 16
//    rows on layers of at most 2^26 weights, the waves convert the caller's
//    rows in registers; otherwise a small pre-pass writes them once per call
//    into the caller's workspace, k-step-major per 32-row pass ([k step][row]
//    [32 k]), so that the activation fragment of one k step is one
//    contiguous M x 64-byte block (full cache lines) instead of M row
//    segments 2·D_in bytes apart.
#include "awq_internal.h"


namespace awq {

// (lo, hi) -> the bf16 pair lo | hi << 16, each rounded to nearest even
// (one v_cvt_pk_bf16_f32 on gfx950; NaN stays NaN)
__device__ __forceinline__ uint32_t bf16_pair_rne(float lo, float hi) {
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
    const f32x2 f = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2v));
}
__device__ __forceinline__ uint16_t bf16_rne(float f) { return static_cast<uint16_t>(bf16_pair_rne(f, 0.0f)); }

// Xk = activations of one call, 8 elements per thread: for row m in the
// 32-row pass p = m / 32 (mc rows), element k goes to
// p·32·D_in + ((k / 32)·mc + m % 32)·32 + k % 32.  With inv_s the value is
// bf16(float32(X[m, k]) · inv_s[k]), else X[m, k] unchanged.
__global__ __launch_bounds__(256) void xk_kernel(const uint16_t *__restrict__ X, const float *__restrict__ inv_s,
                                                 int64_t M, int64_t D_in, uint16_t *__restrict__ Xk) {
    const int64_t runs = D_in / 8;
    const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (idx >= M * runs) return;
    const int64_t row = idx / runs, k0 = (idx % runs) * 8;
    const uint4 xv = *reinterpret_cast<const uint4 *>(X + row * D_in + k0);
    uint32_t xw[4] = {xv.x, xv.y, xv.z, xv.w};
    if (inv_s) {
        const float4 i0 = *reinterpret_cast<const float4 *>(inv_s + k0);
        const float4 i1 = *reinterpret_cast<const float4 *>(inv_s + k0 + 4);
        const float iv[8] = {i0.x, i0.y, i0.z, i0.w, i1.x, i1.y, i1.z, i1.w};
#pragma unroll
        for (int p = 0; p < 4; ++p)
            xw[p] = bf16_pair_rne(__uint_as_float(xw[p] << 16) * iv[2 * p],
                                  __uint_as_float(xw[p] & 0xFFFF0000u) * iv[2 * p + 1]);
    }
    const int64_t pass = row / 32, r = row % 32;
    const int64_t mc = (M - pass * 32) < 32 ? (M - pass * 32) : 32;
    const int64_t dst = pass * 32 * D_in + ((k0 / 32) * mc + r) * 32 + k0 % 32;
    *reinterpret_cast<uint4 *>(Xk + dst) = make_uint4(xw[0], xw[1], xw[2], xw[3]);
}

// Packed weights are read once per call: streaming (nontemporal) loads.  On
// 8192 x 28672 and 28672 x 8192, whose weights stream from HBM, they took
// 2.5-3.2 us off every decode call (8192 x 28672, M = 1 / 8 / 16: 29.2 / 34.2
// / 37.1 -> 26.7 / 31.7 / 34.7 us).  Layers small enough to stay in the
// Infinity Cache between calls lose up to 3% with them at M <= 4, and 2-10%
// on the in-kernel conversion path (DX), which therefore keeps cached loads.
__device__ __forceinline__ uint4 load_stream(const uint32_t *p) {
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

// One packed word (rows 0..7 of an 8-row block at nibble slots 0,2,4,6,1,3,
// 5,7 as value q+8) -> the four bf16 register pairs (rows 2d, 2d+1) of an
// MFMA B fragment, each value 128 + (q + 8).  Split the nibbles into bytes
// (t1: slots 0,2,4,6 = rows 0,4,1,5; t2: slots 1,3,5,7 = rows 2,6,3,7) and
// let v_perm_b32 place one row byte under each 0x43 high byte: 7 ALU ops.
__device__ __forceinline__ void unpack_word(uint32_t w, uint32_t magic, uint32_t *bw) {
    const uint32_t t1 = w & 0x0F0F0F0Fu;
    const uint32_t t2 = (w >> 4) & 0x0F0F0F0Fu;
    // selector bytes: 0..3 pick from the row bytes, 4 picks 0x43
    bw[0] = __builtin_amdgcn_perm(magic, t1, 0x04020400u);  // rows 0, 1
    bw[1] = __builtin_amdgcn_perm(magic, t2, 0x04020400u);  // rows 2, 3
    bw[2] = __builtin_amdgcn_perm(magic, t1, 0x04030401u);  // rows 4, 5
    bw[3] = __builtin_amdgcn_perm(magic, t2, 0x04030401u);  // rows 6, 7
}

// FP16 bits (low 16 bits of v) -> float32, exact
__device__ __forceinline__ float half_bits_to_float(uint32_t v) {
    return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(v)));
}

constexpr int kDecBatch = 4;   // k steps whose loads are issued together (when they divide D_in/32)
// LDS of a workgroup that stages its activations with two column strips (one
// such workgroup per CU: the two-strip grids have at most about one per CU)
constexpr int kDecStageBytes = 132 * 1024;

// Whether a kernel keeps two batches in registers (the loads of batch b+1 in
// flight while batch b feeds the matrix cores): one row tile of one column
// strip per wave, full batches with one step application per batch (groups
// of 128 or more), and neither the in-kernel conversion (DX) nor zero points
// with activation fragments in registers.  Otherwise a second batch's
// registers cost more occupancy than the overlap gains, or spill.
template <int MT, int NB, int GS, bool FX, bool ZP, bool DX, int CW = 1>
constexpr bool dec_pipe() { return MT == 1 && CW == 1 && NB == kDecBatch && GS == NB && !DX && (FX || !ZP); }
// Whether a kernel without the two-batch pipeline rolls its batch registers
// (the loads of k step i of the next batch are issued as soon as k step i of
// the current one is consumed): pre-pass activations, or activations staged
// in LDS with two column strips; full batches with one step application per
// batch.  Not with zero points on two row tiles of two column strips, which
// then spill.
template <int MT, int NB, int GS, bool FX, bool ZP, bool DX, int CW>
constexpr bool dec_roll() {
    return !dec_pipe<MT, NB, GS, FX, ZP, DX, CW>() && NB == kDecBatch && GS == NB && (!FX || CW == 2) && !DX &&
           !(ZP && MT == 2 && CW == 2);
}
// Waves per workgroup (each takes a slice of the workgroup's k range): 8,
// or 4 for one row tile of one column strip without the two-batch pipeline
// (many small workgroups then hide each other's latency).  The workgroups
// may also split k (decode_ksplit, decode_ksplit_two_tiles).
constexpr int dec_waves(int MT, bool pipe, int CW = 1) { return MT == 1 && CW == 1 && !pipe ? 4 : 8; }
template <int MT, int NB, int GS, bool FX, bool ZP, bool DX, int CW = 1>
constexpr int dec_block() { return 64 * dec_waves(MT, dec_pipe<MT, NB, GS, FX, ZP, DX, CW>(), CW); }

// Registers of one batch of k steps: packed words, activation fragments and
// the steps of the groups the batch covers.
template <int MT, int NB, int NSC, bool FX, bool SH, int CW>
struct DecBatch {
    uint4 w[NB][CW];
    uint4 x[NB][FX ? 1 : MT];   // unused when the activations come from LDS
    // steps of the lane's 4 columns: float32, or FP16 bits (widened at use, so
    // that no wait for the load lands at the issue point)
    std::conditional_t<SH, uint2, float4> sc[NSC][CW];
    uint32_t zp[NSC][CW];       // zero points of the lane's 4 columns (zero-point codes only)
};

// One workgroup: 64·CW output columns x one of gridDim.y k ranges; its waves
// (dec_block / 64) split that range again.  GS = min(group/32, kDecBatch): k steps between two
// applications of a group step.  With gridDim.y > 1 the workgroup writes a
// float32 partial to part[blockIdx.y] (reduced by w4a16_reduce_kernel), else
// it writes Y directly.
//
// CW (column strips per wave, 1 or 2; not with DX): each wave covers CW
// strips of 64 columns, so every activation fragment it loads feeds CW times
// as many weights.  Each strip keeps its own accumulators and the
// k ranges of the waves do not change, so every output is summed in the same
// order as with one strip.
//
// FX (at most 4 rows, or 8 with two column strips; one pass): X is the
// caller's row-major activations.
// Each workgroup forms X·inv_s (rounded once to bf16; X itself when inv_s is
// NULL) for its own k range in LDS, in the space the reduction uses later;
// the waves then read their activation fragments from LDS.  No pre-pass
// launch.
//
// ZP (zero-point codes): the nibble n is q itself and the weight is
// (n − z)·step with z per group and column.  The extra MFMA then runs
// against bf16(1), giving sum X per row, and each group flush subtracts
// (128 + z_o)·sum X per column.
//
// SH: the steps are FP16 (uint16 bits), read as such and widened exactly.
//
// DX (one pass of at most 16 rows, not FX): the waves read their activation
// fragments straight from the caller's row-major X (16 rows x 64 bytes per k
// step) and form bf16(X·inv_s) in registers, with the workgroup's slice of
// inv_s (ones without it) staged in LDS (in the space the reduction uses
// later).  No pre-pass launch.
template <int MT, int NB, int GS, bool OUT_BF16, bool FX, bool ZP, bool SH, bool DX = false, int CW = 1>
__global__ __launch_bounds__((dec_block<MT, NB, GS, FX, ZP, DX, CW>())) __attribute__((amdgpu_waves_per_eu(MT == 1 && CW == 1 ? 4 : 2))) void
w4a16_kernel(const uint16_t *__restrict__ X, int64_t M, int64_t D_in, int64_t D_out,
             const uint32_t *__restrict__ packed, const void *__restrict__ scales, int group,
             void *__restrict__ Y, float *__restrict__ part, const float *__restrict__ inv_s,
             const uint8_t *__restrict__ zeros) {
    constexpr int NSC = NB / GS;
    constexpr int kDecWaves = dec_block<MT, NB, GS, FX, ZP, DX, CW>() / 64;
    const int tid = threadIdx.x, lane = tid & 63;
    // wave index in a scalar register: every k-dependent quantity below is
    // wave-uniform and is computed by the scalar unit
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int c = lane >> 4, n = lane & 15;
    const int64_t o0 = static_cast<int64_t>(blockIdx.x) * 64 * CW;
    // strip j: this lane's four columns o0 + 64j + 4n .. +3, clamped so that
    // loads stay in bounds without branches
    uint32_t woff[CW], soff[CW];
#pragma unroll
    for (int j = 0; j < CW; ++j) {
        const int64_t oc = o0 + 64 * j + 4 * n;
        const int64_t occ = oc < D_out ? oc : D_out - 4;
        woff[j] = static_cast<uint32_t>(c * D_out + occ);
        soff[j] = static_cast<uint32_t>(occ);
    }
    static_assert(CW == 1 || !DX, "the in-kernel conversion serves one column strip per wave");
    const int KS = static_cast<int>(D_in / 32);        // 32-row k steps
    const int gsteps = group / 32;
    const int NBt = (KS + NB - 1) / NB;
    const int nsplit = static_cast<int>(gridDim.y) * kDecWaves;
    const int split = static_cast<int>(blockIdx.y) * kDecWaves + wave;
    const int b0 = NBt * split / nsplit, b1 = NBt * (split + 1) / nsplit;
    // per-lane 32-bit element offsets (constant over k); the k-dependent part of
    // every address is wave-uniform and lives in scalar registers
    uint32_t xoff[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) {
        const int64_t rowc = (m * 16 + n) < M ? (m * 16 + n) : M - 1;
        // k-step-major activations, or (DX) the caller's rows
        xoff[m] = static_cast<uint32_t>(DX ? rowc * D_in + 8 * c : rowc * 32 + 8 * c);
    }

    floatx4 ytot[MT][4 * CW], acc[MT][4 * CW], acc1[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) {
        acc1[m] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int t = 0; t < 4 * CW; ++t) {
            ytot[m][t] = floatx4{0.f, 0.f, 0.f, 0.f};
            acc[m][t] = floatx4{0.f, 0.f, 0.f, 0.f};
        }
    }
    const uint32_t kMagic = 0x43434343u;  // bf16 high byte of 128 + n, four times
    bf16x8 ones;
    {
        const uint32_t kc = ZP ? 0x3F803F80u : 0x43084308u;  // bf16(1) or bf16(136), twice
        uint32_t tmp[4] = {kc, kc, kc, kc};
        ones = *reinterpret_cast<bf16x8 *>(tmp);
    }

    // LDS: the reduction buffer; with FX it first holds this workgroup's
    // activations, [row][k - 32·ks0] in bf16, staged before the first batch
    // (with two strips in a larger buffer, rows padded by 16 bytes so that the
    // fragment reads of different rows fall in different banks)
    constexpr int kRedFloats = kDecWaves * MT * 16 * CW * 64;
    constexpr int kLdsFloats = (FX && CW == 2) ? (kDecStageBytes / 4 > kRedFloats ? kDecStageBytes / 4 : kRedFloats)
                                               : kRedFloats;
    __shared__ __align__(16) float lds[kLdsFloats];
    auto red = reinterpret_cast<float (*)[MT * 16 * CW][64]>(lds);
    uint16_t *xs = reinterpret_cast<uint16_t *>(lds);
    float *ivs = lds;   // DX: inv_s[32·ks0 ..]
    int ks0 = 0, kr = 0;
    if constexpr (FX || DX) {
        const int wb0 = NBt * (static_cast<int>(blockIdx.y) * kDecWaves) / nsplit;
        const int wb1 = NBt * (static_cast<int>(blockIdx.y) * kDecWaves + kDecWaves) / nsplit;
        ks0 = wb0 * NB;
        kr = (wb1 - wb0) * NB * 32;
    }
    const int xstr = (FX && CW == 2) ? kr + 8 : kr;   // row stride of the staged activations

    // packed words and activation fragments of k step i of batch b
    auto load_step = [&](int b, int i, DecBatch<MT, NB, NSC, FX, SH, CW> &B) {
        int ks = b * NB + i;
        ks = ks < KS ? ks : KS - 1;
        const uint32_t *wrow = packed + static_cast<int64_t>(ks) * 4 * D_out;   // uniform
#pragma unroll
        for (int j = 0; j < CW; ++j)
            B.w[i][j] = DX ? *reinterpret_cast<const uint4 *>(wrow + woff[j]) : load_stream(wrow + woff[j]);
        if constexpr (!FX) {
            const uint16_t *xcol = X + static_cast<int64_t>(ks) * (DX ? 32 : M * 32);   // uniform
#pragma unroll
            for (int m = 0; m < MT; ++m) B.x[i][m] = *reinterpret_cast<const uint4 *>(xcol + xoff[m]);
        }
    };
    // steps (and zero points) of the groups batch b covers
    auto load_scales = [&](int b, DecBatch<MT, NB, NSC, FX, SH, CW> &B) {
        // group of the first k step of each GS-run (GS divides gsteps or equals it)
        const int g0 = (b * NB) / gsteps;
#pragma unroll
        for (int j = 0; j < NSC; ++j) {
            int g = (GS == NB || gsteps > NB) ? g0 : g0 + j;
            const int glast = KS / gsteps - 1;
            g = g < glast ? g : glast;
#pragma unroll
            for (int s = 0; s < CW; ++s) {
                if constexpr (SH) {
                    const uint16_t *srow = static_cast<const uint16_t *>(scales) + static_cast<int64_t>(g) * D_out;
                    B.sc[j][s] = *reinterpret_cast<const uint2 *>(srow + soff[s]);
                } else {
                    const float *srow = static_cast<const float *>(scales) + static_cast<int64_t>(g) * D_out;
                    B.sc[j][s] = *reinterpret_cast<const float4 *>(srow + soff[s]);
                }
                if constexpr (ZP)
                    B.zp[j][s] = *reinterpret_cast<const uint32_t *>(zeros + static_cast<int64_t>(g) * D_out + soff[s]);
            }
        }
    };
    auto load_batch = [&](int b, DecBatch<MT, NB, NSC, FX, SH, CW> &B) {
#pragma unroll
        for (int i = 0; i < NB; ++i) load_step(b, i, B);
        load_scales(b, B);
    };
    // after_step(i) runs once the matrix instructions of k step i are issued
    // (its packed words and activation fragments are then dead)
    auto compute_batch = [&](int b, DecBatch<MT, NB, NSC, FX, SH, CW> &B, auto &&after_step) {
#pragma unroll
        for (int i = 0; i < NB; ++i) {
            // NB divides the number of k steps, so every batch is full.  Rows
            // >= M read a clamped, valid row: their outputs are never stored,
            // so they need no masking.
            bf16x8 av[MT];
            if constexpr (FX) {
                const int rowc = n < M ? n : static_cast<int>(M) - 1;
                const int ks = b * NB + i;
                av[0] = *reinterpret_cast<const bf16x8 *>(xs + rowc * xstr + (ks - ks0) * 32 + 8 * c);
            } else if constexpr (DX) {
                {
                    // bf16(float32(X)·inv_s), rounded once, as the pre-pass does
                    // (without inv_s the staged factors are 1: X unchanged, exactly)
                    const int ks = b * NB + i;
                    const float4 i0 = *reinterpret_cast<const float4 *>(ivs + (ks - ks0) * 32 + 8 * c);
                    const float4 i1 = *reinterpret_cast<const float4 *>(ivs + (ks - ks0) * 32 + 8 * c + 4);
                    const float iv[8] = {i0.x, i0.y, i0.z, i0.w, i1.x, i1.y, i1.z, i1.w};
#pragma unroll
                    for (int m = 0; m < MT; ++m) {
                        const uint32_t xw[4] = {B.x[i][m].x, B.x[i][m].y, B.x[i][m].z, B.x[i][m].w};
                        uint32_t yw[4];
#pragma unroll
                        for (int p = 0; p < 4; ++p)
                            yw[p] = bf16_pair_rne(__uint_as_float(xw[p] << 16) * iv[2 * p],
                                                  __uint_as_float(xw[p] & 0xFFFF0000u) * iv[2 * p + 1]);
                        av[m] = *reinterpret_cast<const bf16x8 *>(yw);
                    }
                }
            } else {
#pragma unroll
                for (int m = 0; m < MT; ++m) av[m] = *reinterpret_cast<const bf16x8 *>(&B.x[i][m]);
            }
#pragma unroll
            for (int j = 0; j < CW; ++j) {
                const uint32_t words[4] = {B.w[i][j].x, B.w[i][j].y, B.w[i][j].z, B.w[i][j].w};
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    uint32_t bw[4];
                    unpack_word(words[t], kMagic, bw);
                    const bf16x8 bv = *reinterpret_cast<bf16x8 *>(bw);
#pragma unroll
                    for (int m = 0; m < MT; ++m)
                        acc[m][4 * j + t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[m], bv, acc[m][4 * j + t], 0, 0, 0);
                }
            }
#pragma unroll
            for (int m = 0; m < MT; ++m)
                acc1[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[m], ones, acc1[m], 0, 0, 0);
            after_step(i);
            if ((i + 1) % GS == 0) {
                // end of a group (or of a batch inside a larger group): apply its step
#pragma unroll
                for (int j = 0; j < CW; ++j) {
                    float4 sc;
                    if constexpr (SH) {
                        const uint2 h = B.sc[i / GS][j];
                        sc = float4{half_bits_to_float(h.x & 0xFFFFu), half_bits_to_float(h.x >> 16),
                                    half_bits_to_float(h.y & 0xFFFFu), half_bits_to_float(h.y >> 16)};
                    } else {
                        sc = B.sc[i / GS][j];
                    }
                    // columns past D_out computed on clamped, valid words and steps: their sums are
                    // never stored, so the steps need no mask (a select on the loaded value would
                    // also make the compiler wait for the load where it is issued)
                    const float scv[4] = {sc.x, sc.y, sc.z, sc.w};
                    float off[4] = {1.0f, 1.0f, 1.0f, 1.0f};
                    if constexpr (ZP) {
                        const uint32_t zw = B.zp[i / GS][j];
#pragma unroll
                        for (int t = 0; t < 4; ++t) off[t] = 128.0f + static_cast<float>((zw >> (8 * t)) & 0xFFu);
                    }
#pragma unroll
                    for (int m = 0; m < MT; ++m) {
#pragma unroll
                        for (int t = 0; t < 4; ++t) {
#pragma unroll
                            for (int e = 0; e < 4; ++e) {
                                if constexpr (ZP)
                                    ytot[m][4 * j + t][e] += scv[t] * fmaf(-off[t], acc1[m][e], acc[m][4 * j + t][e]);
                                else
                                    ytot[m][4 * j + t][e] += scv[t] * (acc[m][4 * j + t][e] - acc1[m][e]);
                            }
                            acc[m][4 * j + t] = floatx4{0.f, 0.f, 0.f, 0.f};
                        }
                    }
                }
#pragma unroll
                for (int m = 0; m < MT; ++m) acc1[m] = floatx4{0.f, 0.f, 0.f, 0.f};
            }
        }
    };

    auto no_step = [](int) {};
    using Batch = DecBatch<MT, NB, NSC, FX, SH, CW>;
    // B0 holds the first batch of this wave's range: loaded by run_batches, or
    // (FX) already in flight while the activations were being staged.
    Batch B0;
    auto run_batches = [&]() {
        if (b0 >= b1) return;
        if constexpr (!FX) load_batch(b0, B0);
        if constexpr (dec_pipe<MT, NB, GS, FX, ZP, DX, CW>()) {
            Batch B1;
            int b = b0;
            for (; b + 1 < b1; b += 2) {
                load_batch(b + 1, B1);
                compute_batch(b, B0, no_step);
                if (b + 2 < b1) load_batch(b + 2, B0);
                compute_batch(b + 1, B1, no_step);
            }
            if (b < b1) compute_batch(b, B0, no_step);
        } else if constexpr (dec_roll<MT, NB, GS, FX, ZP, DX, CW>()) {
            // Rolling ring: the loads of k step i of batch b+1 go out as soon as
            // the matrix instructions of k step i of batch b are issued, into
            // the registers that step has just released, so the next batch is
            // in flight while this one is consumed without a second register
            // set (which spills with two row tiles or two column strips).  The steps of batch
            // b+1 follow the group flush of batch b.  The last batch is peeled
            // off, so that every load in the loop is unconditional.
            for (int b = b0; b + 1 < b1; ++b) {
                compute_batch(b, B0, [&](int i) { load_step(b + 1, i, B0); });
                load_scales(b + 1, B0);
            }
            compute_batch(b1 - 1, B0, no_step);
        } else {
            // One batch in registers at a time; many small workgroups per CU
            // hide the latency of each other's batches.
            compute_batch(b0, B0, no_step);
            for (int b = b0 + 1; b < b1; ++b) {
                Batch B;
                load_batch(b, B);
                compute_batch(b, B, no_step);
            }
        }
    };
    if constexpr (FX) {
        // Stage the workgroup's activations: thread t converts the 8-element
        // chunks at k offsets 8q, q = t and t + T (T threads), of every row,
        // loading both (and their inv_s) before converting either.  The first
        // batch's packed words are issued right behind those loads (clamped:
        // in bounds even for a wave without batches), so the conversion runs
        // under their HBM latency.
        constexpr int kThreads = 64 * kDecWaves;
        constexpr int kFxRows = CW == 2 ? 8 : 4;   // the most rows a staging plan admits (dec_plan)
        struct StageRegs {
            uint4 x[2][kFxRows];
            float4 iv[2][2];
        };
        const int nq = kr / 8;
        const uint16_t *xb = X + static_cast<int64_t>(ks0) * 32;
        const float *isb = inv_s ? inv_s + static_cast<int64_t>(ks0) * 32 : nullptr;
        auto stage_issue = [&](int q0, StageRegs &R) {
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                int q = q0 + u * kThreads + tid;
                q = q < nq ? q : nq - 1;
#pragma unroll
                for (int r = 0; r < kFxRows; ++r)
                    if (r < M) R.x[u][r] = *reinterpret_cast<const uint4 *>(xb + r * D_in + q * 8);
                if (inv_s) {
                    R.iv[u][0] = *reinterpret_cast<const float4 *>(isb + q * 8);
                    R.iv[u][1] = *reinterpret_cast<const float4 *>(isb + q * 8 + 4);
                }
            }
        };
        auto stage_write = [&](int q0, StageRegs &R) {
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int q = q0 + u * kThreads + tid;
                if (q >= nq) continue;
                const float iv[8] = {R.iv[u][0].x, R.iv[u][0].y, R.iv[u][0].z, R.iv[u][0].w,
                                     R.iv[u][1].x, R.iv[u][1].y, R.iv[u][1].z, R.iv[u][1].w};
#pragma unroll
                for (int r = 0; r < kFxRows; ++r) {
                    if (r >= M) continue;
                    uint32_t xw[4] = {R.x[u][r].x, R.x[u][r].y, R.x[u][r].z, R.x[u][r].w};
                    if (inv_s) {
#pragma unroll
                        for (int p2 = 0; p2 < 4; ++p2)
                            xw[p2] = bf16_pair_rne(__uint_as_float(xw[p2] << 16) * iv[2 * p2],
                                                   __uint_as_float(xw[p2] & 0xFFFF0000u) * iv[2 * p2 + 1]);
                    }
                    *reinterpret_cast<uint4 *>(xs + r * xstr + q * 8) = make_uint4(xw[0], xw[1], xw[2], xw[3]);
                }
            }
        };
        StageRegs R;
        if (nq > 0) stage_issue(0, R);
        load_batch(b0, B0);
        if (nq > 0) stage_write(0, R);
        for (int q0 = 2 * kThreads; q0 < nq; q0 += 2 * kThreads) {
            stage_issue(q0, R);
            stage_write(q0, R);
        }
        __syncthreads();
        run_batches();
        __syncthreads();   // every wave is done with the activations before the buffer is reused
    } else if constexpr (DX) {
        // the workgroup's slice of inv_s (ones without it), four 16-byte loads
        // in flight per thread
        typedef float f32x4 __attribute__((ext_vector_type(4)));
        constexpr int kThreads = 64 * kDecWaves;
        const f32x4 *src = inv_s ? reinterpret_cast<const f32x4 *>(inv_s + static_cast<int64_t>(ks0) * 32) : nullptr;
        f32x4 *dst = reinterpret_cast<f32x4 *>(ivs);
        const int n4 = kr / 4;
        const f32x4 one4 = {1.0f, 1.0f, 1.0f, 1.0f};
        for (int e0 = 0; e0 < n4; e0 += 4 * kThreads) {
            const int e = e0 + tid;
            f32x4 v0 = one4, v1 = one4, v2 = one4, v3 = one4;
            if (inv_s) {   // clamped loads, masked stores
                v0 = src[e < n4 ? e : n4 - 1];
                v1 = src[e + kThreads < n4 ? e + kThreads : n4 - 1];
                v2 = src[e + 2 * kThreads < n4 ? e + 2 * kThreads : n4 - 1];
                v3 = src[e + 3 * kThreads < n4 ? e + 3 * kThreads : n4 - 1];
            }
            if (e < n4) dst[e] = v0;
            if (e + kThreads < n4) dst[e + kThreads] = v1;
            if (e + 2 * kThreads < n4) dst[e + 2 * kThreads] = v2;
            if (e + 3 * kThreads < n4) dst[e + 3 * kThreads] = v3;
        }
        __syncthreads();
        run_batches();
        __syncthreads();   // every wave is done with the factors before the buffer is reused
    } else {
        run_batches();
    }

    // combine the waves' k ranges through LDS (fixed order)
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int t = 0; t < 4 * CW; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i) red[wave][(m * 4 * CW + t) * 4 + i][lane] = ytot[m][t][i];
    __syncthreads();
    for (int item = tid; item < MT * 16 * CW * 64; item += 64 * kDecWaves) {
        const int slot = item / 64, l = item % 64;
        const int m = slot / (16 * CW), tt = (slot / 4) % (4 * CW), i = slot % 4;
        const int j = tt / 4, t = tt % 4;
        float v = 0.0f;
#pragma unroll
        for (int w = 0; w < kDecWaves; ++w) v += red[w][slot][l];
        // MFMA C layout: lane l holds rows 4*(l/16)+i, column l%16 of the tile
        const int64_t row = m * 16 + 4 * (l >> 4) + i;
        const int64_t col = o0 + 64 * j + 4 * (l & 15) + t;
        if (row < M && col < D_out) {
            if (gridDim.y > 1)
                part[(static_cast<int64_t>(blockIdx.y) * M + row) * D_out + col] = v;
            else if (OUT_BF16)
                static_cast<uint16_t *>(Y)[row * D_out + col] = bf16_rne(v);
            else
                static_cast<float *>(Y)[row * D_out + col] = v;
        }
    }
}

// Ring-staged activations (one pass of 9..16 rows: one row tile, two column
// strips, groups of 128 or more, no k split): the 8 waves of a workgroup take
// the batches of the k axis in turn (wave w: batches w, w + 8, ...), so at
// any time they all work inside one 1024-k chunk.  The workgroup stages each
// chunk of bf16(X·inv_s) (X itself without inv_s) from the caller's row-major
// X into a two-slot LDS ring, one chunk ahead, with one barrier per chunk: no
// pre-pass launch and no activation loads in the waves' batches.  Thread t
// converts the 8-element k slice t % 128 of rows t / 128, t / 128 + 4, ...,
// loading all of them (and their inv_s once) before converting any, and
// writes them after the current chunk's batch.  Each wave rolls its batch
// registers as in w4a16_kernel (the next batch's packed words go out as the
// current one is consumed) and keeps its own sums; the waves meet in LDS at
// the end in a fixed order.
constexpr int kRingWaves = 8;
constexpr int kRingChunk = kRingWaves * kDecBatch * 32;   // k per chunk: one batch per wave

template <bool OUT_BF16, bool ZP, bool SH>
__global__ __launch_bounds__(64 * kRingWaves) __attribute__((amdgpu_waves_per_eu(2))) void
w4a16_ring_kernel(const uint16_t *__restrict__ X, int64_t M, int64_t D_in, int64_t D_out,
                  const uint32_t *__restrict__ packed, const void *__restrict__ scales, int group,
                  void *__restrict__ Y, const float *__restrict__ inv_s, const uint8_t *__restrict__ zeros) {
    constexpr int MT = 1, CW = 2, NB = kDecBatch;
    constexpr int kThreads = 64 * kRingWaves;
    constexpr int kXstr = kRingChunk + 8;                // staged row stride (bf16): rows 16 bytes apart in banks
    constexpr int kBuf = MT * 16 * kXstr;                // bf16 per ring slot
    constexpr int kStageRows = MT * 16 / 4;              // rows per thread (4 row phases x 128 k slices)
    constexpr int kRedFloats = kRingWaves * 16 * CW * 64;   // the waves' sums
    constexpr int kSlot0Floats = kBuf / 2 > kRedFloats ? kBuf / 2 : kRedFloats;
    using Batch = DecBatch<MT, NB, 1, true, SH, CW>;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int c = lane >> 4, n = lane & 15;
    const int64_t o0 = static_cast<int64_t>(blockIdx.x) * 64 * CW;
    uint32_t woff[CW], soff[CW];
#pragma unroll
    for (int j = 0; j < CW; ++j) {
        const int64_t oc = o0 + 64 * j + 4 * n;
        const int64_t occ = oc < D_out ? oc : D_out - 4;
        woff[j] = static_cast<uint32_t>(c * D_out + occ);
        soff[j] = static_cast<uint32_t>(occ);
    }
    const int KS = static_cast<int>(D_in / 32);
    const int gsteps = group / 32;   // >= NB
    const int NBt = KS / NB;         // batches (NB divides KS)
    const int nchunk = (NBt + kRingWaves - 1) / kRingWaves;

    __shared__ __align__(16) float slot0[kSlot0Floats];   // ring slot 0, then the reduction
    __shared__ __align__(16) uint16_t slot1[kBuf];
    uint16_t *xs0 = reinterpret_cast<uint16_t *>(slot0);
    auto red = reinterpret_cast<float (*)[16 * CW][64]>(slot0);

    floatx4 ytot[MT][4 * CW], acc[MT][4 * CW], acc1[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) {
        acc1[m] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int t = 0; t < 4 * CW; ++t) {
            ytot[m][t] = floatx4{0.f, 0.f, 0.f, 0.f};
            acc[m][t] = floatx4{0.f, 0.f, 0.f, 0.f};
        }
    }
    const uint32_t kMagic = 0x43434343u;
    bf16x8 ones;
    {
        const uint32_t kc = ZP ? 0x3F803F80u : 0x43084308u;  // bf16(1) or bf16(136), twice
        uint32_t tmp[4] = {kc, kc, kc, kc};
        ones = *reinterpret_cast<bf16x8 *>(tmp);
    }

    // packed words of k step i of batch b (b < NBt)
    auto load_step = [&](int b, int i, Batch &B) {
        const uint32_t *wrow = packed + static_cast<int64_t>(b * NB + i) * 4 * D_out;
#pragma unroll
        for (int j = 0; j < CW; ++j) B.w[i][j] = load_stream(wrow + woff[j]);
    };
    auto load_scales = [&](int b, Batch &B) {
        const int g = (b * NB) / gsteps;
#pragma unroll
        for (int s = 0; s < CW; ++s) {
            if constexpr (SH) {
                const uint16_t *srow = static_cast<const uint16_t *>(scales) + static_cast<int64_t>(g) * D_out;
                B.sc[0][s] = *reinterpret_cast<const uint2 *>(srow + soff[s]);
            } else {
                const float *srow = static_cast<const float *>(scales) + static_cast<int64_t>(g) * D_out;
                B.sc[0][s] = *reinterpret_cast<const float4 *>(srow + soff[s]);
            }
            if constexpr (ZP)
                B.zp[0][s] = *reinterpret_cast<const uint32_t *>(zeros + static_cast<int64_t>(g) * D_out + soff[s]);
        }
    };
    auto load_batch = [&](int b, Batch &B) {
#pragma unroll
        for (int i = 0; i < NB; ++i) load_step(b, i, B);
        load_scales(b, B);
    };
    // batch b of this wave from a ring slot; one step application at its end
    auto compute_batch = [&](int b, const uint16_t *xsl, Batch &B, auto &&after_step) {
        const uint16_t *xb = xsl + (b % kRingWaves) * (NB * 32);
#pragma unroll
        for (int i = 0; i < NB; ++i) {
            bf16x8 av[MT];
#pragma unroll
            for (int m = 0; m < MT; ++m) {
                const int rowc = m * 16 + n < M ? m * 16 + n : static_cast<int>(M) - 1;   // rows >= M: never stored
                av[m] = *reinterpret_cast<const bf16x8 *>(xb + rowc * kXstr + i * 32 + 8 * c);
            }
#pragma unroll
            for (int j = 0; j < CW; ++j) {
                const uint32_t words[4] = {B.w[i][j].x, B.w[i][j].y, B.w[i][j].z, B.w[i][j].w};
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    uint32_t bw[4];
                    unpack_word(words[t], kMagic, bw);
                    const bf16x8 bv = *reinterpret_cast<bf16x8 *>(bw);
#pragma unroll
                    for (int m = 0; m < MT; ++m)
                        acc[m][4 * j + t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[m], bv, acc[m][4 * j + t], 0, 0, 0);
                }
            }
#pragma unroll
            for (int m = 0; m < MT; ++m) acc1[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[m], ones, acc1[m], 0, 0, 0);
            after_step(i);
        }
#pragma unroll
        for (int j = 0; j < CW; ++j) {
            float4 sc;
            if constexpr (SH) {
                const uint2 h = B.sc[0][j];
                sc = float4{half_bits_to_float(h.x & 0xFFFFu), half_bits_to_float(h.x >> 16),
                            half_bits_to_float(h.y & 0xFFFFu), half_bits_to_float(h.y >> 16)};
            } else {
                sc = B.sc[0][j];
            }
            const float scv[4] = {sc.x, sc.y, sc.z, sc.w};   // columns past D_out: never stored
            float off[4] = {1.0f, 1.0f, 1.0f, 1.0f};
            if constexpr (ZP) {
                const uint32_t zw = B.zp[0][j];
#pragma unroll
                for (int t = 0; t < 4; ++t) off[t] = 128.0f + static_cast<float>((zw >> (8 * t)) & 0xFFu);
            }
#pragma unroll
            for (int m = 0; m < MT; ++m)
#pragma unroll
                for (int t = 0; t < 4; ++t) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        if constexpr (ZP)
                            ytot[m][4 * j + t][e] += scv[t] * fmaf(-off[t], acc1[m][e], acc[m][4 * j + t][e]);
                        else
                            ytot[m][4 * j + t][e] += scv[t] * (acc[m][4 * j + t][e] - acc1[m][e]);
                    }
                    acc[m][4 * j + t] = floatx4{0.f, 0.f, 0.f, 0.f};
                }
        }
#pragma unroll
        for (int m = 0; m < MT; ++m) acc1[m] = floatx4{0.f, 0.f, 0.f, 0.f};
    };

    Batch B;
    auto no_step = [](int) {};
    {
        // register staging of chunk ch: this thread's k slice q and rows rp, rp + 4, ...
        const int q = tid % (kRingChunk / 8), rp = tid / (kRingChunk / 8);
        struct StageRegs {
            uint4 x[kStageRows];
            float4 iv[2];
        };
        auto stage_issue = [&](int ch, StageRegs &R) {
            int64_t k = static_cast<int64_t>(ch) * kRingChunk + q * 8;
            k = k < D_in ? k : D_in - 8;   // clamped: slices past the end are not stored
#pragma unroll
            for (int r = 0; r < kStageRows; ++r) {
                const int row = rp + 4 * r;
                if (row < M) R.x[r] = *reinterpret_cast<const uint4 *>(X + row * D_in + k);
            }
            if (inv_s) {
                R.iv[0] = *reinterpret_cast<const float4 *>(inv_s + k);
                R.iv[1] = *reinterpret_cast<const float4 *>(inv_s + k + 4);
            }
        };
        auto stage_write = [&](int ch, StageRegs &R) {
            if (static_cast<int64_t>(ch) * kRingChunk + q * 8 >= D_in) return;
            const float iv[8] = {R.iv[0].x, R.iv[0].y, R.iv[0].z, R.iv[0].w,
                                 R.iv[1].x, R.iv[1].y, R.iv[1].z, R.iv[1].w};
            uint16_t *dst = ((ch & 1) ? slot1 : xs0) + q * 8;
#pragma unroll
            for (int r = 0; r < kStageRows; ++r) {
                const int row = rp + 4 * r;
                if (row >= M) continue;
                uint32_t xw[4] = {R.x[r].x, R.x[r].y, R.x[r].z, R.x[r].w};
                if (inv_s) {
#pragma unroll
                    for (int p = 0; p < 4; ++p)
                        xw[p] = bf16_pair_rne(__uint_as_float(xw[p] << 16) * iv[2 * p],
                                              __uint_as_float(xw[p] & 0xFFFF0000u) * iv[2 * p + 1]);
                }
                *reinterpret_cast<uint4 *>(dst + row * kXstr) = make_uint4(xw[0], xw[1], xw[2], xw[3]);
            }
        };
        StageRegs R;
        stage_issue(0, R);
        load_batch(wave < NBt ? wave : NBt - 1, B);   // clamped for a wave without a batch
        stage_write(0, R);
        __syncthreads();
        // every chunk but the last: the wave's batch, the next batch's loads
        // rolled in behind it (clamped in the last chunk's range), the next
        // chunk staged
        for (int ch = 0; ch + 1 < nchunk; ++ch) {
            stage_issue(ch + 1, R);
            const int b = ch * kRingWaves + wave;   // < NBt
            int bn = b + kRingWaves;
            bn = bn < NBt ? bn : NBt - 1;
            compute_batch(b, (ch & 1) ? slot1 : xs0, B, [&](int i) { load_step(bn, i, B); });
            load_scales(bn, B);
            stage_write(ch + 1, R);
            __syncthreads();
        }
        const int b = (nchunk - 1) * kRingWaves + wave;
        if (b < NBt) compute_batch(b, ((nchunk - 1) & 1) ? slot1 : xs0, B, no_step);
    }

    // combine the waves' k ranges through LDS (fixed order)
#pragma unroll
    for (int m = 0; m < MT; ++m) {
        __syncthreads();   // the ring is no longer read
#pragma unroll
        for (int t = 0; t < 4 * CW; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i) red[wave][t * 4 + i][lane] = ytot[m][t][i];
        __syncthreads();
        for (int item = tid; item < 16 * CW * 64; item += kThreads) {
            const int slot = item / 64, l = item % 64;
            const int tt = slot / 4, i = slot % 4;
            const int j = tt / 4, t = tt % 4;
            float v = 0.0f;
#pragma unroll
            for (int w = 0; w < kRingWaves; ++w) v += red[w][slot][l];
            // MFMA C layout: lane l holds rows 4*(l/16)+i, column l%16 of the tile
            const int64_t row = m * 16 + 4 * (l >> 4) + i;
            const int64_t col = o0 + 64 * j + 4 * (l & 15) + t;
            if (row < M && col < D_out) {
                if (OUT_BF16)
                    static_cast<uint16_t *>(Y)[row * D_out + col] = bf16_rne(v);
                else
                    static_cast<float *>(Y)[row * D_out + col] = v;
            }
        }
    }
}

// Y = sum over the k-range partials in split order.
template <bool OUT_BF16>
__global__ __launch_bounds__(256) void w4a16_reduce_kernel(const float *__restrict__ part, int nz, int64_t count,
                                                           void *__restrict__ Y) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i >= count) return;
    float v = 0.0f;
    for (int z = 0; z < nz; ++z) v += part[z * count + i];
    if (OUT_BF16)
        static_cast<uint16_t *>(Y)[i] = bf16_rne(v);
    else
        static_cast<float *>(Y)[i] = v;
}

hipError_t launch_w4a16_reduce(const float *part, int nz, int64_t count, void *Y, int yt, hipStream_t st) {
    const dim3 grid(static_cast<unsigned>((count + 255) / 256));
    if (yt == 1)
        hipLaunchKernelGGL(w4a16_reduce_kernel<true>, grid, dim3(256), 0, st, part, nz, count, Y);
    else
        hipLaunchKernelGGL(w4a16_reduce_kernel<false>, grid, dim3(256), 0, st, part, nz, count, Y);
    return hipGetLastError();
}

// k-range splits across workgroups (passes of at most 16 rows).  A split
// costs a reduction launch.  With the two-batch pipeline (8 waves), a layer
// whose k range gives each wave of an unsplit grid at most 4 batches is not
// split, and otherwise the splits double until there are about one
// workgroup per CU; without it (4 waves), until there are about four.  Each
// wave keeps at least two batches.
static int decode_ksplit(int64_t D_in, int64_t D_out, bool pipe) {
    const int waves = dec_waves(1, pipe);
    const int64_t strips = (D_out + 63) / 64;
    const int64_t batches = (D_in / 32 + kDecBatch - 1) / kDecBatch;
    if (pipe && batches <= 4 * waves) return 1;
    const int64_t target = pipe ? 256 : 1024;
    int z = 1;
    while (strips * z < target && batches >= static_cast<int64_t>(z) * 2 * waves) z *= 2;
    return z;
}

// k-range splits of a pass of 17..32 rows (two row tiles, 8 waves, about one
// workgroup per CU): only where the 64-column strips leave a quarter of the
// CUs or more idle, doubling while there are fewer than 192 workgroups.  Cold
// weights, M = 32: 28672 x 8192 (128 strips, split 2 ways) 61.7 -> 44.5 us,
// 14336 x 4096 (64 strips, 4 ways) 34.3 -> 21.1 us, 8192 x 8192 24.1 -> 20.8
// us; 4096 x 14336 (224 strips) is 30% slower split, so it is not.
static int decode_ksplit_two_tiles(int64_t D_in, int64_t D_out) {
    const int64_t strips = (D_out + 63) / 64;
    const int64_t batches = (D_in / 32 + kDecBatch - 1) / kDecBatch;
    int z = 1;
    while (strips * z < 192 && batches >= static_cast<int64_t>(z) * 2 * 8) z *= 2;
    return z;
}

// Launch plan of one pass of mc rows of a call of M rows: the ring kernel
// (9..16 rows, one pass, wide layers), FX (at most 4 rows, or 8 with two
// column strips, one pass: each workgroup's activations, M x its k range in
// bf16, fit in its LDS buffer), else DX (at most 16 rows, one pass, layers of
// up to 2^26 weights: each workgroup's slice of inv_s fits in that buffer),
// else the pre-pass; whether the kernel pipelines two batches (dec_pipe:
// gfull = full batches with groups of 128 or more); and the k splits.  DX on
// layers up to 2^26 weights only: there the pre-pass launch costs more than
// the in-kernel conversion (8192² at M = 8: 17 against 20 µs); on 8192 x
// 28672 the in-kernel conversion's registers cost occupancy (42 against 39
// µs at M = 16).
struct DecPlan {
    bool fx = false, dx = false, pipe = false;
    bool ring = false;   // w4a16_ring_kernel (one pass, two strips, no split)
    int z = 1;
    int cw = 1;   // column strips per wave
};
constexpr int64_t kDirectMaxWeights = int64_t(1) << 26;
constexpr int64_t kRingMinRows = 9;   // fewer rows stage the whole k range (FX)
constexpr int64_t kDecTwoStripMinCols = 192 * 128;
// LDS bytes of the reduction buffer of a one-tile workgroup
static int64_t dec_red_bytes(bool pipe) { return static_cast<int64_t>(dec_waves(1, pipe)) * 16 * 64 * 4; }
// upper bound of the k range (elements) of one workgroup with z splits
static int64_t dec_kr_max(int64_t D_in, int z) {
    const int64_t nbt = D_in / 32 / kDecBatch;
    return ((nbt + z - 1) / z + 1) * kDecBatch * 32;
}
static DecPlan dec_plan(int64_t M, int64_t mc, int64_t D_in, int64_t D_out, bool gfull, bool zp) {
    DecPlan p;
    const bool uniform = (D_in / 32) % kDecBatch == 0;
    // Ring-staged activations: a one-pass call of 9..16 rows on a layer wide
    // enough for about 192 or more workgroups of 128 columns, with one step
    // application per batch (groups of 128 or more).  8192 x 28672 (cold
    // weights, per call): M = 9 / 12 / 16 30.1 / 30.5 / 31.1 -> 26.3 / 26.5 /
    // 26.8 us, zero points M = 12 37.2 -> 27.8 us (the pre-pass and a 4-way k
    // split before).  With two row tiles (17..32 rows) the staging registers
    // spill; copying the chunks straight into LDS and converting at the
    // fragment reads was slower than the pre-pass (M = 32 38.0 against 37.3
    // us), as was converting row-major fragments in registers (DX) with two
    // strips (also spilling with two row tiles; at one tile the ring is 2 us
    // faster).
    if (gfull && uniform && M == mc && M >= kRingMinRows && M <= 16 && D_out >= kDecTwoStripMinCols) {
        p.ring = true;
        p.cw = 2;
        return p;
    }
    if (mc <= 16) {
        if (uniform && M <= 8) {
            const bool pipe = gfull;
            const int z = decode_ksplit(D_in, D_out, pipe);
            // Two column strips (rolled, 8 waves, one workgroup per CU) on wide
            // layers: the activations stage in a kDecStageBytes buffer with
            // padded rows (up to 8 rows of 8192), for either code kind.  With
            // the first batch in flight during the staging, 8192 x 28672 (cold
            // weights, per call): M = 1 / 4 / 6 / 8 25.7 / 25.8 / 26.1 / 27.1 us
            // against 25.8 / 27.6 / 29.2 / 29.6 us for staging each chunk in
            // turn (up to 5 rows) and the pre-pass beyond; zero points M = 8
            // 31.1 -> 27.3 us.  k range of one workgroup: at most ceil(batches /
            // z) full batches.
            const bool two = gfull && z == 1 && D_out >= kDecTwoStripMinCols && M <= 8;
            const int64_t kr2 = (D_in / 32 / kDecBatch + z - 1) / z * kDecBatch * 32;
            const bool fits = two ? M * (kr2 + 8) * 2 <= kDecStageBytes
                                  : M <= 4 && M * dec_kr_max(D_in, z) * 2 <= dec_red_bytes(pipe);
            if (fits) {
                p.fx = true;
                p.pipe = pipe && !two;
                p.z = z;
                p.cw = two ? 2 : 1;
                return p;
            }
        }
        if (uniform && M <= 16 && D_in * D_out <= kDirectMaxWeights) {
            const int z = decode_ksplit(D_in, D_out, false);
            if (dec_kr_max(D_in, z) * 4 <= dec_red_bytes(false)) {
                p.dx = true;
                p.z = z;
                return p;
            }
        }
        p.pipe = gfull && uniform && !zp;
        p.z = decode_ksplit(D_in, D_out, p.pipe);
    } else {
        p.z = decode_ksplit_two_tiles(D_in, D_out);
    }
    // Two column strips per wave (rolled) on layers that still give about 192
    // or more workgroups of 128 columns, with one step application per batch
    // (groups of 128 or more: with two per batch, two row tiles spill); with
    // zero points from 12 rows on.  8192 x 28672 (cold weights): M = 8 32.2
    // -> 29.8 us, M = 16 35.1 -> 31.3 us, M = 32 44.1 -> 37.5 us; zero points
    // at M <= 8 are 3% slower with two strips.  8192 x 16384 (128
    // workgroups): 20-30% slower.
    if (gfull && uniform && p.z == 1 && mc >= (zp ? 12 : 2) && D_out >= kDecTwoStripMinCols) p.cw = 2;
    return p;
}

// Rows of the pass that needs the largest partial buffer (z x rows), or 0,
// over every pass size, group size and code kind.  The passes of one call
// run in stream order and share the buffer.
static int64_t partial_rows(int64_t M, int64_t D_in, int64_t D_out) {
    const int64_t tail = M % 32 != 0 ? M % 32 : 32;   // rows of the last pass; all others have 32
    int64_t rows = 0;
    for (int pass = 0; pass < 2; ++pass) {
        const int64_t mc = pass == 0 ? tail : 32;
        if (pass == 1 && M <= 32) break;
        for (int v = 0; v < 4; ++v) {
            const int z = dec_plan(M, mc, D_in, D_out, (v & 1) != 0, (v & 2) != 0).z;
            if (z > 1 && z * mc > rows) rows = z * mc;
        }
    }
    return rows;
}

// FP16 steps -> float32 (exact), for the product's float32 step loads.
__global__ __launch_bounds__(256) void widen_f16_kernel(const uint16_t *__restrict__ src, int64_t n,
                                                        float *__restrict__ dst) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    if (i < n) dst[i] = static_cast<float>(__builtin_bit_cast(_Float16, src[i]));
}

hipError_t launch_widen_f16(const uint16_t *src, int64_t n, float *dst, hipStream_t st) {
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(widen_f16_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, st, src, n, dst);
    return hipGetLastError();
}

// Workspace: [activations, k-step-major, M x D_in bf16, 256-byte aligned]
// [float32 partials z x rows x D_out for a split pass].  Where the prefill
// regime applies, the larger of both regimes' needs: zero-point codes with
// group 32 take the decode path at any M.
size_t w4a16_workspace_bytes(int64_t M, int64_t D_in, int64_t D_out, bool /*has_inv*/) {
    size_t bytes = (static_cast<size_t>(M) * static_cast<size_t>(D_in) * 2 + 255) / 256 * 256;
    bytes += static_cast<size_t>(partial_rows(M, D_in, D_out)) * static_cast<size_t>(D_out) * 4;
    if (w4a16_prefill_applies(M, D_in, D_out)) {
        const size_t pf = w4a16_prefill_workspace_bytes(M, D_in, D_out);
        bytes = pf > bytes ? pf : bytes;
    }
    return bytes;
}

// With FP16 steps: the prefill regime reads a float32 copy of the steps,
// kept 256-aligned after the regime's own workspace.
size_t w4a16_step_copy_offset(int64_t M, int64_t D_in, int64_t D_out) {
    return (w4a16_workspace_bytes(M, D_in, D_out, true) + 255) / 256 * 256;
}

size_t w4a16_workspace_bytes_ex(int64_t M, int64_t D_in, int64_t D_out, int group, bool steps_f16) {
    if (steps_f16 && w4a16_prefill_applies(M, D_in, D_out))
        return w4a16_step_copy_offset(M, D_in, D_out) + static_cast<size_t>(D_in / group) * D_out * 4;
    return w4a16_workspace_bytes(M, D_in, D_out, true);
}

hipError_t launch_w4a16_gemm(const void *X, int64_t M, int64_t D_in, int64_t D_out, const uint32_t *packed,
                             const void *scales, bool steps_f16, const uint8_t *zeros, int group, const float *inv_s,
                             void *Y, int yt, void *ws, hipStream_t st) {
    if (w4a16_prefill_applies(M, D_in, D_out) && !(zeros && group < 64)) {
        const float *sc32 = static_cast<const float *>(scales);
        if (steps_f16) {
            // the prefill regime converts float32 steps itself: widen the FP16
            // steps first (exact), into the workspace tail
            float *wide = reinterpret_cast<float *>(static_cast<unsigned char *>(ws) +
                                                    w4a16_step_copy_offset(M, D_in, D_out));
            const hipError_t e = launch_widen_f16(static_cast<const uint16_t *>(scales), (D_in / group) * D_out,
                                                  wide, st);
            if (e != hipSuccess) return e;
            sc32 = wide;
        }
        return launch_w4a16_prefill(X, M, D_in, D_out, packed, sc32, zeros, group, inv_s, Y, yt, ws, st);
    }
    unsigned char *wsp = static_cast<unsigned char *>(ws);
    // batch of kDecBatch k steps when it divides D_in/32 (all common shapes), else 1
    const bool bfull = (D_in / 32) % kDecBatch == 0;
    const int gs = bfull ? (group / 32 >= kDecBatch ? kDecBatch : group / 32) : 1;
    const bool gfull = bfull && gs == kDecBatch;
    const DecPlan call = dec_plan(M, M, D_in, D_out, gfull, zeros != nullptr);   // FX and DX: one-pass calls only
    const bool fx = call.fx, dx = call.dx;
    if (call.ring) {
        const dim3 grid(static_cast<unsigned>((D_out + 127) / 128));
#define AWQ_RING2(ZPV, SHV)                                                                                      \
    do {                                                                                                          \
        if (yt == 1)                                                                                              \
            hipLaunchKernelGGL((w4a16_ring_kernel<true, ZPV, SHV>), grid, dim3(64 * kRingWaves), 0, st,             \
                               static_cast<const uint16_t *>(X), M, D_in, D_out, packed, scales, group, Y, inv_s,  \
                               zeros);                                                                            \
        else                                                                                                      \
            hipLaunchKernelGGL((w4a16_ring_kernel<false, ZPV, SHV>), grid, dim3(64 * kRingWaves), 0, st,            \
                               static_cast<const uint16_t *>(X), M, D_in, D_out, packed, scales, group, Y, inv_s,  \
                               zeros);                                                                            \
    } while (0)
        if (zeros) {
            if (steps_f16)
                AWQ_RING2(true, true);
            else
                AWQ_RING2(true, false);
        } else {
            if (steps_f16)
                AWQ_RING2(false, true);
            else
                AWQ_RING2(false, false);
        }
#undef AWQ_RING2
        return hipGetLastError();
    }
    if (!fx && !dx) {
        const int64_t n = M * (D_in / 8);
        hipLaunchKernelGGL(xk_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, st,
                           static_cast<const uint16_t *>(X), inv_s, M, D_in, reinterpret_cast<uint16_t *>(wsp));
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    const uint16_t *Xa = (fx || dx) ? static_cast<const uint16_t *>(X) : reinterpret_cast<const uint16_t *>(wsp);
    wsp += (static_cast<size_t>(M) * static_cast<size_t>(D_in) * 2 + 255) / 256 * 256;
    float *part = reinterpret_cast<float *>(wsp);
    const size_t ybytes = yt == 1 ? 2 : 4;
    for (int64_t m0 = 0; m0 < M; m0 += 32) {
        const int64_t mc = (M - m0) < 32 ? (M - m0) : 32;
        const DecPlan pass = dec_plan(M, mc, D_in, D_out, gfull, zeros != nullptr);
        const int z = pass.z;
        const bool cw2 = pass.cw == 2;
        const int64_t wg_cols = cw2 ? 128 : 64;
        const dim3 grid(static_cast<unsigned>((D_out + wg_cols - 1) / wg_cols), static_cast<unsigned>(z));
        const uint16_t *Xc = Xa + m0 * D_in;
        void *Yc = static_cast<unsigned char *>(Y) + static_cast<size_t>(m0 * D_out) * ybytes;
#define AWQ_DEC_LAUNCH4(MT, NB, GS, FX, ZP, SH, DXV, CWV)                                                        \
    do {                                                                                                          \
        if (yt == 1)                                                                                              \
            hipLaunchKernelGGL((w4a16_kernel<MT, NB, GS, true, FX, ZP, SH, DXV, CWV>), grid,                       \
                               dim3(dec_block<MT, NB, GS, FX, ZP, DXV, CWV>()), 0, st, Xc, mc, D_in, D_out, packed, scales, \
                               group, Yc, part, inv_s, zeros);                                                    \
        else                                                                                                      \
            hipLaunchKernelGGL((w4a16_kernel<MT, NB, GS, false, FX, ZP, SH, DXV, CWV>), grid,                      \
                               dim3(dec_block<MT, NB, GS, FX, ZP, DXV, CWV>()), 0, st, Xc, mc, D_in, D_out, packed, scales, \
                               group, Yc, part, inv_s, zeros);                                                    \
    } while (0)
// two column strips: not with DX, one step application per batch
#define AWQ_DEC_LAUNCH3(MT, NB, GS, FX, ZP, SH, DXV)                     \
    do {                                                                 \
        if constexpr (!(DXV) && (NB) == kDecBatch && (GS) == (NB)) {     \
            if (cw2) {                                                   \
                AWQ_DEC_LAUNCH4(MT, NB, GS, FX, ZP, SH, DXV, 2);         \
                break;                                                   \
            }                                                            \
        }                                                                \
        AWQ_DEC_LAUNCH4(MT, NB, GS, FX, ZP, SH, DXV, 1);                 \
    } while (0)
#define AWQ_DEC_LAUNCH2(MT, NB, GS, FX, ZP, DXV)               \
    do {                                                       \
        if (steps_f16)                                         \
            AWQ_DEC_LAUNCH3(MT, NB, GS, FX, ZP, true, DXV);    \
        else                                                   \
            AWQ_DEC_LAUNCH3(MT, NB, GS, FX, ZP, false, DXV);   \
    } while (0)
#define AWQ_DEC_LAUNCH(MT, NB, GS, FX, DXV)               \
    do {                                                  \
        if (zeros)                                        \
            AWQ_DEC_LAUNCH2(MT, NB, GS, FX, true, DXV);   \
        else                                              \
            AWQ_DEC_LAUNCH2(MT, NB, GS, FX, false, DXV);  \
    } while (0)
#define AWQ_DEC_GS(MT)                                  \
    do {                                                \
        if (!bfull)                                     \
            AWQ_DEC_LAUNCH(MT, 1, 1, false, false);     \
        else if (gs == 1)                               \
            AWQ_DEC_LAUNCH(MT, kDecBatch, 1, false, false);     \
        else if (gs == 2)                               \
            AWQ_DEC_LAUNCH(MT, kDecBatch, 2, false, false);     \
        else                                            \
            AWQ_DEC_LAUNCH(MT, kDecBatch, 4, false, false);     \
    } while (0)
        if (fx) {
            if (gs == 1)
                AWQ_DEC_LAUNCH(1, kDecBatch, 1, true, false);
            else if (gs == 2)
                AWQ_DEC_LAUNCH(1, kDecBatch, 2, true, false);
            else
                AWQ_DEC_LAUNCH(1, kDecBatch, 4, true, false);
        } else if (dx) {
            if (gs == 1)
                AWQ_DEC_LAUNCH(1, kDecBatch, 1, false, true);
            else if (gs == 2)
                AWQ_DEC_LAUNCH(1, kDecBatch, 2, false, true);
            else
                AWQ_DEC_LAUNCH(1, kDecBatch, 4, false, true);
        } else if (mc <= 16) {
            AWQ_DEC_GS(1);
        } else {
            AWQ_DEC_GS(2);
        }
#undef AWQ_DEC_GS
#undef AWQ_DEC_LAUNCH
#undef AWQ_DEC_LAUNCH2
#undef AWQ_DEC_LAUNCH3
#undef AWQ_DEC_LAUNCH4
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        if (z > 1) {
            const int64_t count = mc * D_out;
            if (yt == 1)
                hipLaunchKernelGGL(w4a16_reduce_kernel<true>, dim3(static_cast<unsigned>((count + 255) / 256)),
                                   dim3(256), 0, st, part, z, count, Yc);
            else
                hipLaunchKernelGGL(w4a16_reduce_kernel<false>, dim3(static_cast<unsigned>((count + 255) / 256)),
                                   dim3(256), 0, st, part, z, count, Yc);
            e = hipGetLastError();
            if (e != hipSuccess) return e;
        }
    }
    return hipSuccess;
}

}  // namespace awq
