// Host-side checks of libqoq's C ABI, built with AddressSanitizer and
// UndefinedBehaviorSanitizer over the library's host code (device code is
// not compiled in). Every entry point is called with invalid arguments
// (each must return its documented status before anything is launched) and
// the size queries are swept over many shapes, including extreme ones, so
// the planners' integer arithmetic runs under UBSan. On a host without a
// GPU, calls with valid arguments then run the whole host path up to the
// launch, which fails with QOQ_ERR_HIP: nothing is ever dereferenced.
// Refuses to run when a GPU is visible (the fake pointers below would then
// reach a kernel).
#include <hip/hip_runtime.h>
#include <cstdint>
#include <cstdio>
#include <vector>

#include "qoq.h"
#include "qoq_kv4.h"
#include "qoq_measure.h"
#include "qoq_variants.h"

static int failures = 0;

#define EXPECT(call, want)                                                              \
    do {                                                                                \
        const int got_ = int(call);                                                     \
        if (got_ != int(want)) {                                                        \
            std::printf("FAIL %s:%d: %s -> %d, want %d\n", __FILE__, __LINE__, #call,   \
                        got_, int(want));                                               \
            ++failures;                                                                 \
        }                                                                               \
    } while (0)

int main() {
    int n = 0;
    if (hipGetDeviceCount(&n) == hipSuccess && n > 0) {
        std::printf("a GPU is visible: refusing to run host-only checks\n");
        return 2;
    }
    void* P = reinterpret_cast<void*>(uintptr_t(1) << 20);   // aligned, never dereferenced
    auto* p8 = static_cast<int8_t*>(P);
    auto* pf = static_cast<float*>(P);
    auto* p16 = static_cast<uint16_t*>(P);
    auto* p32 = static_cast<int32_t*>(P);
    auto* pu8 = static_cast<uint8_t*>(P);
    void* Pm = reinterpret_cast<void*>((uintptr_t(1) << 20) + 4);   // misaligned

    // ---- invalid arguments: each returns its status, nothing launched
    EXPECT(qoq_pack_weights(pf, 4096, 4096, 64, P, p16, nullptr, 0, nullptr), QOQ_ERR_GROUP);
    EXPECT(qoq_pack_weights(pf, 4090, 4096, 128, P, p16, nullptr, 0, nullptr), QOQ_ERR_SHAPE);
    EXPECT(qoq_pack_weights(nullptr, 16, 128, 128, P, p16, nullptr, 0, nullptr), QOQ_ERR_NULL);
    EXPECT(qoq_pack_weights(pf, 16, 128, 128, Pm, p16, nullptr, 0, nullptr), QOQ_ERR_ALIGN);
    EXPECT(qoq_pack_weights(pf, 16, 128, 128, P, p16, nullptr, 2, nullptr), QOQ_ERR_FLAGS);
    EXPECT(qoq_quantize_act(p16, -1, 128, p8, pf, nullptr), QOQ_ERR_SHAPE);
    EXPECT(qoq_quantize_act(p16, 4, 100, p8, pf, nullptr), QOQ_ERR_SHAPE);
    EXPECT(qoq_quantize_act(nullptr, 4, 128, p8, pf, nullptr), QOQ_ERR_NULL);
    EXPECT(qoq_quantize_act(static_cast<uint16_t*>(Pm), 4, 128, p8, pf, nullptr), QOQ_ERR_ALIGN);
    EXPECT(qoq_quantize_act(nullptr, 0, 128, nullptr, nullptr, nullptr), QOQ_OK);
    EXPECT(qoq_w4a8_gemm(p8, pf, 4, 128, P, p16, 20, 128, p16, nullptr, nullptr, 0, nullptr),
           QOQ_ERR_SHAPE);
    EXPECT(qoq_w4a8_gemm(p8, pf, 4, QOQ_MAX_GEMM_K + 128, P, p16, 16, 128, p16, nullptr, nullptr,
                         0, nullptr), QOQ_ERR_SHAPE);
    EXPECT(qoq_w4a8_gemm(nullptr, pf, 4, 128, P, p16, 16, 128, p16, nullptr, nullptr, 0, nullptr),
           QOQ_ERR_NULL);
    EXPECT(qoq_w4a8_gemm(p8, pf, 64, 16384, P, p16, 4096, 128, p16, nullptr, nullptr, 0, nullptr),
           QOQ_ERR_WORKSPACE);
    EXPECT(qoq_w4a8_gemm_noalloc(p8, pf, 1280, 24576, P, p16, 8192, 128, p16, nullptr, nullptr),
           QOQ_ERR_WORKSPACE);
    EXPECT(qoq_w4a8_linear(p16, 64, 4096, P, p16, 4096, 128, p16, nullptr, nullptr, 0, nullptr),
           QOQ_ERR_WORKSPACE);
    EXPECT(qoq_w4a8_linear(p16, -3, 4096, P, p16, 4096, 128, p16, nullptr, nullptr, 0, nullptr),
           QOQ_ERR_SHAPE);
    EXPECT(qoq_w8a8_gemm(p8, pf, 4, 133120 + 128, P, p16, 16, p16, nullptr, nullptr), QOQ_ERR_SHAPE);
    EXPECT(qoq_w4a4_gemm(nullptr, 4, 128, P, 16, p16, nullptr), QOQ_ERR_NULL);
    EXPECT(qoq_w4a16_gemm(p16, 4, 100, P, 16, p16, nullptr), QOQ_ERR_SHAPE);
    EXPECT(qoq_kv4_decode_attention(p16, 4, 32, 7, 128, p16, P, 64, p32, 64, p16, nullptr, 0,
                                    nullptr), QOQ_ERR_SHAPE);
    EXPECT(qoq_kv4_append(p16, p16, 2, 3, 8, 64, p16, p32, P, 64, nullptr), QOQ_ERR_SHAPE);
    EXPECT(qoq_stream_read(P, 1000, 0, reinterpret_cast<uint32_t*>(P), nullptr), QOQ_ERR_SHAPE);

    // ---- size queries over many shapes (planner arithmetic under UBSan)
    const std::vector<int64_t> ms = {0, 1, 2, 7, 8, 9, 15, 16, 17, 31, 32, 33, 63, 64, 65, 100, 127,
                                     128, 129, 200, 255, 256, 257, 511, 512, 513, 1000, 1024, 2048,
                                     4096, 8192, 65535, 65536, int64_t(1) << 20, int64_t(1) << 30,
                                     (int64_t(1) << 30) + 1, int64_t(1) << 40, -1,
                                     INT64_MAX};
    const std::vector<int64_t> ns = {16, 32, 48, 208, 528, 1040, 4096, 6144, 8192, 14336, 24576,
                                     28672, 49152, 131072, int64_t(1) << 30, 15, -16, INT64_MAX};
    const std::vector<int64_t> ks = {128, 256, 384, 640, 1152, 2560, 4096, 8192, 14336, 16384, 24576,
                                     131072, QOQ_MAX_GEMM_K, QOQ_MAX_GEMM_K + 128, int64_t(1) << 30,
                                     100, 0, -128, INT64_MAX};
    size_t sink = 0;
    for (int64_t M : ms)
        for (int64_t N : ns)
            for (int64_t K : ks) {
                sink += qoq_gemm_workspace_bytes(M, N, K);
                sink += qoq_linear_workspace_bytes(M, N, K);
                sink += size_t(qoq_linear_path(M, N, K) + 1);
                sink += qoq_packed_weight_bytes(N, K, 128);
                sink += qoq_act_bytes(M, K);
                sink += qoq_w8a8_weight_bytes(N, K) + qoq_w4a4_weight_bytes(N, K);
                sink += qoq_w4a16_weight_bytes(N, K) + qoq_w4a4_act_bytes(M, K);
            }
    for (int64_t B : {int64_t(0), int64_t(1), int64_t(4), int64_t(64), int64_t(1) << 20, int64_t(-1)})
        for (int64_t H : {int64_t(8), int64_t(32), int64_t(64), int64_t(7)})
            for (int64_t L : {int64_t(0), int64_t(1), int64_t(31), int64_t(2048), int64_t(16384),
                              int64_t(1) << 30, int64_t(-5)}) {
                sink += qoq_kv4_cache_bytes(B, H, 32 * ((L + 31) / 32 + 1), 128);
                sink += qoq_kv16_cache_bytes(B, H, 32 * ((L + 31) / 32 + 1), 128);
                for (int64_t G : {int64_t(1), int64_t(4), int64_t(16)})
                    sink += qoq_kv4_attention_workspace_bytes(B, H * G, H, 128, L);
            }

    // ---- valid arguments: the host path runs up to the launch, which fails
    // without a GPU (QOQ_ERR_HIP); every planner branch is reached
    const std::vector<int64_t> run_m = {1, 8, 17, 32, 64, 100, 200, 256, 300, 1024, 4096};
    const std::vector<std::pair<int64_t, int64_t>> run_kn = {
        {4096, 4096}, {4096, 6144}, {4096, 28672}, {14336, 4096}, {8192, 49152},
        {24576, 8192}, {8192, 24576}, {512, 512}, {1152, 528}, {131072, 32768}};
    std::vector<uint8_t> ws_dummy;   // host bytes: only the size is ever looked at
    for (int64_t M : run_m)
        for (auto [K, N] : run_kn) {
            const size_t wsb = qoq_gemm_workspace_bytes(M, N, K);
            void* ws = wsb ? P : nullptr;
            EXPECT(qoq_w4a8_gemm(p8, pf, M, K, P, p16, N, 128, p16, p32, ws, wsb, nullptr),
                   QOQ_ERR_HIP);
            const size_t lwb = qoq_linear_workspace_bytes(M, N, K);
            EXPECT(qoq_w4a8_linear(p16, M, K, P, p16, N, 128, p16, nullptr, lwb ? P : nullptr, lwb,
                                   nullptr), QOQ_ERR_HIP);
        }
    EXPECT(qoq_quantize_act(p16, 64, 4096, p8, pf, nullptr), QOQ_ERR_HIP);
    EXPECT(qoq_pack_weights(pf, 4096, 4096, 128, P, p16, nullptr, 0, nullptr), QOQ_ERR_HIP);
    EXPECT(qoq_w4a8_gemm_noalloc(p8, pf, 64, 16384, P, p16, 4096, 128, p16, nullptr, nullptr),
           QOQ_ERR_HIP);
    (void)pu8;
    std::printf("%s (%d failures, sink %zu)\n", failures ? "FAILED" : "ok", failures, sink & 1);
    return failures ? 1 : 0;
}
