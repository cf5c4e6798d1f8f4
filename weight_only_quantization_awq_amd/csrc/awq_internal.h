// Internal declarations shared by the HIP sources of the AWQ library.
//
// Data layout in HBM (all device buffers are caller-owned):
//
//  * Search operands are stored in "fragment order": the exact register image
//    one 64-lane wavefront feeds to an MFMA, so that every global load, every
//    direct-to-LDS copy and every LDS read in the loss contraction is a
//    contiguous, conflict-free 16-byte (or 4-byte) vector access.
//      fp16 path (v_mfma_f32_32x32x16_f16): a chunk is 32 rows/cols x 16 k;
//        lane l = c*32 + r holds 8 consecutive k (k = 64*kb + 16*kq + 8*c + i)
//        of row/column r -> 64 lanes x 16 B = 1 KiB per chunk.  X chunks are
//        ordered [kb][mb32][kq], error-weight chunks [alpha][kb][nb32][kq], so
//        one workgroup's 256-row x 64-k A tile is a contiguous 32 KiB block.
//      fp32 path (v_mfma_f32_16x16x4_f32): a 32-k block holds 8 sub-chunks of
//        4 k; lane l = c*16 + r holds k = 32*kb + 4*ks + c -> 8 x 256 B,
//        ordered [kb][mb16][ks] and [alpha][kb][nb16][ks].
//    Rows, columns and k are zero-padded to multiples of 256, 256 and 64.
//  * Per-group steps, codes, packed words and outputs use plain row-major
//    layouts documented in include/awq.h.
#pragma once

#include <hip/hip_runtime.h>
#include <type_traits>
#include <stdint.h>

namespace awq {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

// Search-contraction tile (one workgroup = 4 waves = 256 x 256 outputs).
constexpr int kTileM = 256;
constexpr int kTileN = 256;
constexpr int kTileK = 64;   // k per LDS stage (k padding unit)
constexpr int kThreads = 256;

inline int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

struct AlphaGrid {
    float v[64];
};

// Per-search scalar state kept in the workspace (device side).
constexpr int kAbsmaxXBlocks = 512;    // workgroups that scan X for max|X| (at most)
constexpr int kAbsmaxWBlocks = 1024;   // workgroups that scan W for max|W| (at most)
struct SearchState {
    unsigned int max_abs_x_bits;   // bits of max|X| as a float (> 0x7F800000 for NaN)
    unsigned int max_abs_w_bits;   // bits of max|W|
    int kx;                        // X prescale exponent (fp16 path), 0 for fp32
    int pad0;
    int kd[64];                    // error-weight prescale exponent per alpha
    unsigned int sminbits[64];     // float bits of the smallest scale s_j, per alpha
    unsigned int part_x[kAbsmaxXBlocks];   // per-workgroup max|X| bits, reduced into max_abs_x_bits
    unsigned int part_w[kAbsmaxWBlocks];   // per-workgroup max|W| bits
};

// Shape bundle for the search.
struct SearchShape {
    int64_t N, D_in, D_out;
    int64_t Mp, Kp, Np;       // padded extents
    int64_t MB, KB, NB;       // fp32-path chunk counts: Mp/16, Kp/32, Np/16
    int64_t MB32, KB64, NB32; // fp16-path chunk counts: Mp/32, Kp/64, Np/32
    int64_t tiles_m, tiles_n; // Mp/256, Np/256
    // Output-column chunk of the error-weight pass and the loss contraction:
    // columns [col0, col0 + Nc) of the padded Np (col0 and Nc multiples of
    // 256).  The whole layer in one chunk unless the caller's workspace only
    // holds the error weights of fewer columns.
    int64_t col0, Nc;
    int64_t NB32c, NBc, tiles_nc;   // Nc/32, Nc/16, Nc/256
    // Rows of D and X the quantiser covers (D_in rounded up to 64), and the
    // correction rows after them (kCorrRows on the bf16 path, else 0):
    // Kp = Kq + Kc.
    int64_t Kq;
    int Kc;
    int group, bits, n_alpha;
    bool f16;                 // true: 16-bit MFMA path (bf16 inputs); false: fp32
    bool bf16;                // 16-bit path on bf16 matrix cores with correction rows (else fp16)
    bool asym;                // zero-point codes in [0, 2^bits - 1]
    bool f16_steps;           // steps rounded to and stored in FP16
};

// Workspace carve-up (byte offsets, each 256-aligned).
struct SearchWorkspace {
    size_t off_state, off_s, off_invp, off_sel, off_x, off_d, off_part, total;
};

// bf16 path of the loss contraction: input channels with the largest
// activation statistic whose error weights also carry their bf16 rounding
// residual, as extra contraction rows (one 64-k stage), and the layers that
// take this path (D_in range, least N·D_in·D_out).
constexpr int kCorrRows = 64;
constexpr int64_t kMinBf16Rows = 2048;
constexpr int64_t kMaxBf16Rows = 16384;
constexpr double kMinBf16Macs = 549755813888.0;   // 2^39 multiply-adds per alpha (N·D_in·D_out)

// Layout with an error-weight region for `chunk_cols` output columns (a
// multiple of 256, at most Np).
SearchWorkspace search_workspace_layout(const SearchShape &sh, int64_t chunk_cols);
// Sets the chunk fields of `sh` for columns [col0, col0 + cols).
void set_search_chunk(SearchShape &sh, int64_t col0, int64_t cols);

// Sets the calling thread's awq_last_error() text and returns `code` (an
// awq_status value), for entry points defined outside awq_api.hip.
int report_error(int code, const char *msg);

// ---- launchers (each returns hipError_t of the launch) ----------------------
hipError_t launch_act_stats(const void *X, int xt, int64_t N, int64_t D_in, int stat, float *a,
                            hipStream_t st);
hipError_t launch_weight_stats(const void *W, int wt, int64_t D_in, int64_t D_out, float *b,
                               hipStream_t st);
hipError_t launch_search(const void *X, int xt, const void *W, int wt, const float *a,
                         const float *b, uint8_t *zeros, const AlphaGrid &alphas, const SearchShape &sh, double *losses,
                         int32_t *best, float *s_best, float *scales, int8_t *codes,
                         unsigned char *ws, int64_t chunk_cols, hipStream_t st, hipEvent_t *events);
hipError_t launch_pack(const int8_t *codes, int64_t D_in, int64_t D_out, int offset, uint32_t *packed,
                       hipStream_t st);
size_t w4a16_workspace_bytes(int64_t M, int64_t D_in, int64_t D_out, bool has_inv);
bool clip_group_supported(int group);
size_t clip_workspace_bytes(int64_t N, int64_t D_in, int group);
hipError_t launch_clip(const void *X, int xt, int64_t N, int64_t D_in, const void *W, int wt,
                       int64_t D_out, const float *s, const AlphaGrid &ratios, int n_ratio, int bits,
                       int group, int32_t *ratio_idx, float *scales, int8_t *codes, float *errors,
                       void *ws, hipStream_t st);
bool w4a16_prefill_applies(int64_t M, int64_t D_in, int64_t D_out);
size_t w4a16_prefill_workspace_bytes(int64_t M, int64_t D_in, int64_t D_out);
hipError_t launch_w4a16_prefill(const void *X, int64_t M, int64_t D_in, int64_t D_out,
                                const uint32_t *packed, const float *scales, const uint8_t *zeros,
                                int group, const float *inv_s, void *Y, int yt, void *ws, hipStream_t st);
// Y = sum of nz float32 partials part[z][count] in split order (bf16 or float32 Y)
hipError_t launch_w4a16_reduce(const float *part, int nz, int64_t count, void *Y, int yt, hipStream_t st);
// FP16 step bits -> float32 (exact), n elements
hipError_t launch_widen_f16(const uint16_t *src, int64_t n, float *dst, hipStream_t st);
// Workspace with FP16 steps (steps_f16): the prefill regime's float32 copy of
// the steps sits at w4a16_step_copy_offset; otherwise w4a16_workspace_bytes.
size_t w4a16_step_copy_offset(int64_t M, int64_t D_in, int64_t D_out);
size_t w4a16_workspace_bytes_ex(int64_t M, int64_t D_in, int64_t D_out, int group, bool steps_f16);
// zeros: NULL for signed codes (nibble = q + 8), else zero points [D_in/group x D_out];
// scales: float32, or FP16 bits when steps_f16
hipError_t launch_w4a16_gemm(const void *X, int64_t M, int64_t D_in, int64_t D_out,
                             const uint32_t *packed, const void *scales, bool steps_f16, const uint8_t *zeros,
                             int group, const float *inv_s, void *Y, int yt, void *ws, hipStream_t st);

}  // namespace awq
