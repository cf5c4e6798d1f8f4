// awq_w4a16_gemm_noalloc: the W4A16 product for callers that cannot allocate
// (code under HIP graph capture, tight serving loops, harnesses that forbid
// hipMalloc).  It runs exactly the kernels of awq_w4a16_gemm; their scratch
// memory (the scaled, k-step-major activations, split-k float32 partials, or
// the prefill regime's fragments) lives in a file-scope device array instead
// of a caller workspace.
//
// The array is one per GPU: each device that loads the library holds its own
// copy until the process ends.  Host code never passes the array's name to a
// kernel (on the host that name is only a stand-in, not a device address):
// the device address is looked up once per device with hipGetSymbolAddress,
// with that device current, and only that pointer is used afterwards.
//
// No kernel on this path needs zeroed scratch (every byte read was written
// earlier in the same call), so nothing is cleared.  Every call on a GPU
// shares that GPU's array: calls that overlap on one GPU (two streams, or two
// host threads) race on it and must be serialised by the caller.
#include "awq.h"  // include/awq.h (on the -I path)

#include <mutex>
#include <stdio.h>

#include "awq_internal.h"

namespace {

constexpr size_t kScratchBytes = size_t(32) << 20;   // 32 MiB per GPU
constexpr int kMaxDevices = 64;

__device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_lock;
void *g_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device (looked up once per device).
hipError_t scratch_ptr(void **out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> g(g_lock);
    if (!g_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_ptr[dev] = p;
    }
    *out = g_ptr[dev];
    return hipSuccess;
}

}  // namespace

extern "C" {

size_t awq_w4a16_noalloc_scratch_bytes(void) { return kScratchBytes; }

awq_status awq_w4a16_gemm_noalloc(const void *X, int64_t M, int64_t D_in, int64_t D_out, const uint32_t *packed,
                                  const float *scales, int group, const float *inv_s, void *Y, awq_dtype yt,
                                  hipStream_t stream) {
    // the requirement of this shape (0 and an error text for a bad shape,
    // which the full validation below reports again)
    const size_t need = awq_w4a16_workspace_size(M, D_in, D_out, inv_s != nullptr);
    if (need > kScratchBytes) {
        char msg[256];
        snprintf(msg, sizeof(msg),
                 "awq_w4a16_gemm_noalloc: this shape needs %zu bytes of scratch; the library's static scratch "
                 "holds %zu (use awq_w4a16_gemm with a caller workspace)",
                 need, kScratchBytes);
        return static_cast<awq_status>(awq::report_error(AWQ_ERR_WORKSPACE, msg));
    }
    void *ws = nullptr;
    const hipError_t e = scratch_ptr(&ws);
    if (e != hipSuccess) {
        char msg[256];
        snprintf(msg, sizeof(msg), "awq_w4a16_gemm_noalloc: scratch lookup: %s", hipGetErrorString(e));
        return static_cast<awq_status>(awq::report_error(AWQ_ERR_HIP, msg));
    }
    return awq_w4a16_gemm(X, M, D_in, D_out, packed, scales, group, inv_s, Y, yt, ws, kScratchBytes, stream);
}

}  // extern "C"
