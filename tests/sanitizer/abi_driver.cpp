// Host-side driver for the sanitizer test: calls every entry point of the C
// ABI with arguments that validation must reject (no device memory is ever
// touched), checks the status codes and the thread-local messages, and
// exercises the workspace-size functions.  Built together with the library's
// host code under AddressSanitizer and UndefinedBehaviorSanitizer.
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <thread>
#include <vector>

#include "awq.h"

static int failures = 0;

#define EXPECT(call, code)                                                                         \
    do {                                                                                           \
        const int got__ = static_cast<int>(call);                                                  \
        if (got__ != (code)) {                                                                     \
            std::printf("FAIL %s:%d %s -> %d, want %d (%s)\n", __FILE__, __LINE__, #call, got__,   \
                        static_cast<int>(code), awq_last_error());                                  \
            ++failures;                                                                            \
        } else if ((code) != 0 && std::strlen(awq_last_error()) == 0) {                            \
            std::printf("FAIL %s:%d %s: empty message\n", __FILE__, __LINE__, #call);              \
            ++failures;                                                                            \
        }                                                                                          \
    } while (0)

// a plausible but never dereferenced device address (validation fails first)
static void *fake(uintptr_t off = 0) { return reinterpret_cast<void *>(uintptr_t(0x10000) + off); }

static void run_all() {
    float al[21];
    for (int k = 0; k < 21; ++k) al[k] = k / 20.0f;
    hipStream_t st = nullptr;
    const size_t big = size_t(1) << 40;
    float *ff = static_cast<float *>(fake());
    double *fd = static_cast<double *>(fake());
    int32_t *fi = static_cast<int32_t *>(fake());

    // statistics
    EXPECT(awq_act_stats(nullptr, AWQ_BF16, 16, 256, ff, st), AWQ_ERR_ARG);
    EXPECT(awq_act_stats(fake(), AWQ_BF16, 0, 256, ff, st), AWQ_ERR_SHAPE);
    EXPECT(awq_act_stats(fake(), static_cast<awq_dtype>(9), 16, 256, ff, st), AWQ_ERR_DTYPE);
    EXPECT(awq_act_stats_ex(fake(), AWQ_BF16, 16, 256, static_cast<awq_statistic>(7), ff, st), AWQ_ERR_ARG);
    EXPECT(awq_weight_stats(nullptr, AWQ_BF16, 256, 256, ff, st), AWQ_ERR_ARG);

    // search workspace sizes: valid, and invalid (0)
    if (awq_search_workspace_size(2048, 4096, 4096, AWQ_BF16, 4, 128, 21) == 0) {
        std::printf("FAIL valid search workspace size is 0\n");
        ++failures;
    }
    if (awq_search_workspace_size(128, 250, 256, AWQ_F32, 4, 128, 21) != 0) {
        std::printf("FAIL invalid search workspace size is not 0\n");
        ++failures;
    }

    // searches: NULL outputs, bad alpha, bad group, too small a workspace
    EXPECT(awq_search_layer(fake(), AWQ_BF16, 256, 256, fake(), AWQ_BF16, 256, ff, al, 21, 4, 128, fd, fi, ff,
                            nullptr, nullptr, fake(0x100000), big, st),
           AWQ_ERR_ARG);
    float bad_al[2] = {0.5f, 1.5f};
    EXPECT(awq_search_layer(fake(), AWQ_BF16, 256, 256, fake(), AWQ_BF16, 256, ff, bad_al, 2, 4, 128, fd, fi, ff,
                            ff, nullptr, fake(0x100000), big, st),
           AWQ_ERR_ARG);
    EXPECT(awq_search_layer(fake(), AWQ_BF16, 256, 256, fake(), AWQ_BF16, 256, ff, al, 21, 4, 12, fd, fi, ff, ff,
                            nullptr, fake(0x100000), big, st),
           AWQ_ERR_ARG);
    EXPECT(awq_search_layer(fake(), AWQ_BF16, 256, 256, fake(), AWQ_BF16, 256, ff, al, 21, 4, 128, fd, fi, ff, ff,
                            nullptr, fake(0x100000), 1024, st),
           AWQ_ERR_WORKSPACE);
    EXPECT(awq_search_layer_ex(fake(), AWQ_BF16, 256, 256, fake(), AWQ_BF16, 256, ff, al, 21, 9, 128, fd, fi, ff,
                               ff, nullptr, fake(0x100000), big, st, nullptr, 0),
           AWQ_ERR_ARG);
    EXPECT(awq_search_layer_wscale(fake(), AWQ_BF16, 256, 256, fake(), AWQ_BF16, 256, ff, static_cast<float *>(fake(2)),
                                   al, 21, 4, 128, fd, fi, ff, ff, nullptr, fake(0x100000), big, st),
           AWQ_ERR_ARG);
    EXPECT(awq_search_layer_zp(fake(), AWQ_BF16, 256, 256, fake(), AWQ_BF16, 256, ff, nullptr, al, 21, 4, 128, fd,
                               fi, ff, ff, nullptr, nullptr, fake(0x100000), big, st),
           AWQ_ERR_ARG);
    EXPECT(awq_search_layer_flags(fake(), AWQ_BF16, 256, 256, fake(), AWQ_BF16, 256, ff, nullptr, al, 21, 4, 128,
                                  16u, fd, fi, ff, fake(), nullptr, nullptr, fake(0x100000), big, st),
           AWQ_ERR_ARG);

    // clip
    if (awq_clip_workspace_size(2048, 4096, 128) == 0) {
        std::printf("FAIL valid clip workspace size is 0\n");
        ++failures;
    }
    EXPECT(awq_clip_search(fake(), AWQ_BF16, 256, 256, fake(), AWQ_BF16, 256, ff, al, 21, 4, 256, fi, ff, nullptr,
                           nullptr, fake(0x100000), big, st),
           AWQ_ERR_ARG);

    // pack
    EXPECT(awq_pack(nullptr, 8, 8, 4, static_cast<uint32_t *>(fake()), st), AWQ_ERR_ARG);
    EXPECT(awq_pack_ex(static_cast<int8_t *>(fake()), 12, 8, 4, 1, static_cast<uint32_t *>(fake()), st),
           AWQ_ERR_SHAPE);

    // products
    const uint32_t *fw = static_cast<const uint32_t *>(fake());
    EXPECT(awq_w4a16_gemm(fake(), 1, 256, 254, fw, ff, 128, nullptr, fake(), AWQ_F32, nullptr, 0, st),
           AWQ_ERR_SHAPE);
    EXPECT(awq_w4a16_gemm(fake(), 1, 256, 64, fw, ff, 128, ff, fake(), AWQ_F32, nullptr, 0, st), AWQ_ERR_WORKSPACE);
    EXPECT(awq_w4a16_gemm_zp(fake(), 1, 256, 64, fw, ff, nullptr, 128, nullptr, fake(), AWQ_F32, fake(), big, st),
           AWQ_ERR_ARG);
    EXPECT(awq_w4a16_gemm_ex(fake(), 1, 256, 64, fw, fake(), AWQ_BF16, nullptr, 128, nullptr, fake(), AWQ_F32, fake(),
                             big, st),
           AWQ_ERR_DTYPE);
    const size_t need = awq_w4a16_workspace_size_ex(512, 8192, 28672, 128, AWQ_F16);
    EXPECT(awq_w4a16_gemm_ex(fake(), 512, 8192, 28672, fw, fake(), AWQ_F16, nullptr, 128, nullptr, fake(), AWQ_F32,
                             fake(), need - 4, st),
           AWQ_ERR_WORKSPACE);
    if (std::strstr(awq_version(), "gfx950") == nullptr) {
        std::printf("FAIL version string\n");
        ++failures;
    }
}

int main() {
    run_all();
    // the error string is thread-local: the same checks from several threads at once
    std::vector<std::thread> th;
    for (int t = 0; t < 4; ++t) th.emplace_back(run_all);
    for (auto &t : th) t.join();
    if (failures) {
        std::printf("%d failures\n", failures);
        return 1;
    }
    std::printf("sanitized ABI checks passed\n");
    return 0;
}
