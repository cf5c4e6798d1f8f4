// Pack signed codes into 4-bit words.
//
// [MR] "SIMD 感知权重打包": on GPUs every 8 weights share one 32-bit word in
// the order w0, w2, w4, w6, w1, w3, w5, w7.  Nibble slot i (bits 4i..4i+3,
// least significant first) holds row P[i] of the 8-row block as q + 8 (q
// itself for the unsigned codes of the zero-point quantiser).
//
// Why this order suits CDNA: (word >> 4d) & 0x000F000F puts rows 2d and 2d+1
// into the low and high 16-bit halves of one register, i.e. one k-consecutive
// pair of a 16x16x32 bf16 MFMA B operand, and OR-ing 0x43004300 turns both
// nibbles n into the bf16 values 128 + n without any conversion instruction.
//
// One thread per (8-row block, 4 adjacent columns): four 4-byte code loads
// per row (coalesced along D_out), one 16-byte word store.  HBM bound:
// 1 byte read + 0.5 byte written per weight.
#include "awq_internal.h"

namespace awq {

// `offset` is added to every code: 8 for signed codes, 0 for the unsigned
// codes of the zero-point quantiser.
__global__ __launch_bounds__(256) void pack_kernel(const int8_t *__restrict__ codes, int64_t D_in, int64_t D_out,
                                                   int offset, uint32_t *__restrict__ packed) {
    const int64_t quads = (D_out + 3) / 4;
    const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (idx >= (D_in / 8) * quads) return;
    const int64_t kw = idx / quads;
    const int64_t o0 = (idx % quads) * 4;
    // slot -> row of the 8-row block
    constexpr int kRowOfSlot[8] = {0, 2, 4, 6, 1, 3, 5, 7};
    uint32_t word[4] = {0u, 0u, 0u, 0u};
    const bool full = (o0 + 4 <= D_out) && (D_out % 4 == 0);
#pragma unroll
    for (int slot = 0; slot < 8; ++slot) {
        const int64_t row = kw * 8 + kRowOfSlot[slot];
        const int8_t *src = codes + row * D_out + o0;
        int8_t c[4];
        if (full) {
            const uint32_t v = *reinterpret_cast<const uint32_t *>(src);
            c[0] = static_cast<int8_t>(v & 0xFF);
            c[1] = static_cast<int8_t>((v >> 8) & 0xFF);
            c[2] = static_cast<int8_t>((v >> 16) & 0xFF);
            c[3] = static_cast<int8_t>(v >> 24);
        } else {
#pragma unroll
            for (int t = 0; t < 4; ++t) c[t] = (o0 + t < D_out) ? src[t] : 0;
        }
#pragma unroll
        for (int t = 0; t < 4; ++t)
            word[t] |= (static_cast<uint32_t>(c[t] + offset) & 0xFu) << (4 * slot);
    }
    uint32_t *dst = packed + kw * D_out + o0;
    if (full) {
        *reinterpret_cast<uint4 *>(dst) = make_uint4(word[0], word[1], word[2], word[3]);
    } else {
        for (int t = 0; t < 4; ++t)
            if (o0 + t < D_out) dst[t] = word[t];
    }
}

hipError_t launch_pack(const int8_t *codes, int64_t D_in, int64_t D_out, int offset, uint32_t *packed,
                       hipStream_t st) {
    const int64_t n = (D_in / 8) * ((D_out + 3) / 4);
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(pack_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, st, codes, D_in,
                       D_out, offset, packed);
    return hipGetLastError();
}

}  // namespace awq
