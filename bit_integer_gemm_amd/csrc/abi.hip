// The C ABI of libqoq: host-side validation, then one or two kernel
// launches on the caller's stream. Nothing here allocates, frees,
// synchronizes or prints.
#include "qoq.h"
#include "qoq_variants.h"
#include "qoq_kv4.h"
#include "qoq_internal.hpp"

#include <cstring>
#include <mutex>
#include <string>

namespace {

// Plan overrides set by qoq_set_tuning (measurement and test aid; the only
// mutable state of the library besides the no-alloc entry point's scratch
// address cache).
std::mutex tune_mu;
std::string tune_val[qoq::kTuneCount];
const char* const tune_key[qoq::kTuneCount] = {"gemm", "variant", "kv4_splits", "kv4_paired"};


bool misaligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) != 0; }

// Largest K and N the 32-bit index arithmetic of the kernels supports.
constexpr int64_t kMaxDim = int64_t(1) << 30;

// Largest K (a multiple of 128) whose INT32 accumulators stay exact:
// |acc| <= K * 127 * 121 < 2^31 (activation codes within 127, dequantized
// weights within 121 by the protective range).
constexpr int64_t kMaxAccK = 139648;
// The same bound for the W8A8 comparison GEMM (weights within 127).
constexpr int64_t kMaxAccKW8A8 = 133120;
static_assert(kMaxAccK * 127 * 121 < (int64_t(1) << 31) && (kMaxAccK + 128) * 127 * 121 >= (int64_t(1) << 31),
              "accumulator bound");
static_assert(kMaxAccKW8A8 * 127 * 127 < (int64_t(1) << 31) &&
              (kMaxAccKW8A8 + 128) * 127 * 127 >= (int64_t(1) << 31), "accumulator bound");

qoq_status check_gemm_k(int64_t K) { return K > kMaxAccK ? QOQ_ERR_SHAPE : QOQ_OK; }

qoq_status check_weight_shape(int64_t N, int64_t K, int32_t group) {
    if (group != qoq::kGroup) return QOQ_ERR_GROUP;
    if (N <= 0 || K <= 0 || N > kMaxDim || K > kMaxDim) return QOQ_ERR_SHAPE;
    if (N % qoq::kBlockCols != 0 || K % group != 0) return QOQ_ERR_SHAPE;
    return QOQ_OK;
}

}  // namespace

std::string qoq::tuning(TuningKey key) {
    std::lock_guard<std::mutex> lock(tune_mu);
    return tune_val[key];
}

extern "C" {

qoq_status qoq_set_tuning(const char* key, const char* value) {
    if (key == nullptr) return QOQ_ERR_NULL;
    for (int k = 0; k < qoq::kTuneCount; ++k) {
        if (std::strcmp(key, tune_key[k]) == 0) {
            std::lock_guard<std::mutex> lock(tune_mu);
            tune_val[k] = value ? value : "";
            return QOQ_OK;
        }
    }
    return QOQ_ERR_CONFIG;
}


size_t qoq_packed_weight_bytes(int64_t N, int64_t K, int32_t group) {
    if (check_weight_shape(N, K, group) != QOQ_OK) return 0;
    return size_t(qoq::packed_layout(N, K).total);
}

size_t qoq_act_bytes(int64_t M, int64_t K) {
    if (M <= 0 || K <= 0 || K % qoq::kGroup != 0 || M > kMaxDim || K > kMaxDim) return 0;
    return size_t(qoq::act_bytes(M, K));
}

size_t qoq_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K) {
    if (M <= 0 || check_weight_shape(N, K, qoq::kGroup) != QOQ_OK || M > kMaxDim ||
        check_gemm_k(K) != QOQ_OK)
        return 0;
    const qoq::GemmPlan plan = qoq::plan_gemm(M, N, K);
    return plan.kind < 0 ? 0 : size_t(plan.ws_bytes);
}

qoq_status qoq_pack_weights(const float* W, int64_t N, int64_t K, int32_t group, void* packed,
                            uint16_t* s1, const qoq_canonical* canon, uint32_t flags,
                            void* stream) {
    if (flags & ~QOQ_PACK_FROM_CANONICAL) return QOQ_ERR_FLAGS;
    const bool from_canonical = (flags & QOQ_PACK_FROM_CANONICAL) != 0;
    const qoq_status st = check_weight_shape(N, K, group);
    if (st != QOQ_OK) return st;
    if (packed == nullptr) return QOQ_ERR_NULL;
    uint8_t* cq4 = nullptr;
    int8_t* cs2 = nullptr;
    uint8_t* cz = nullptr;
    if (canon != nullptr) {
        if (canon->q4 == nullptr || canon->s2 == nullptr || canon->z == nullptr)
            return QOQ_ERR_NULL;
        cq4 = canon->q4;
        cs2 = canon->s2;
        cz = canon->z;
    }
    if (from_canonical) {
        if (canon == nullptr) return QOQ_ERR_NULL;
    } else {
        if (W == nullptr || s1 == nullptr) return QOQ_ERR_NULL;
        if (misaligned(W)) return QOQ_ERR_ALIGN;
    }
    if (misaligned(packed)) return QOQ_ERR_ALIGN;
    const hipError_t e = qoq::launch_pack(W, N, K, static_cast<uint8_t*>(packed), s1, cq4, cs2, cz,
                                          from_canonical, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? QOQ_OK : QOQ_ERR_HIP;
}

qoq_status qoq_quantize_act(const uint16_t* x, int64_t M, int64_t K, int8_t* x8, float* s_x,
                            void* stream) {
    if (M < 0 || K <= 0 || K % qoq::kGroup != 0 || M > kMaxDim || K > kMaxDim)
        return QOQ_ERR_SHAPE;
    if (M == 0) return QOQ_OK;
    if (x == nullptr || x8 == nullptr || s_x == nullptr) return QOQ_ERR_NULL;
    if (misaligned(x) || misaligned(x8)) return QOQ_ERR_ALIGN;
    const hipError_t e =
        qoq::launch_quantize_act(x, M, K, x8, s_x, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? QOQ_OK : QOQ_ERR_HIP;
}

qoq_status qoq_w4a8_gemm(const int8_t* x8, const float* s_x, int64_t M, int64_t K,
                         const void* packed, const uint16_t* s1, int64_t N, int32_t group,
                         uint16_t* y, int32_t* acc_debug, void* workspace,
                         size_t workspace_bytes, void* stream) {
    const qoq_status st = check_weight_shape(N, K, group);
    if (st != QOQ_OK) return st;
    if (M < 0 || M > kMaxDim || check_gemm_k(K) != QOQ_OK) return QOQ_ERR_SHAPE;
    if (M == 0) return QOQ_OK;
    if (x8 == nullptr || s_x == nullptr || packed == nullptr || s1 == nullptr || y == nullptr)
        return QOQ_ERR_NULL;
    if (misaligned(x8) || misaligned(packed) || misaligned(y)) return QOQ_ERR_ALIGN;
    const qoq::GemmPlan plan = qoq::plan_gemm(M, N, K);
    if (plan.kind < 0) return QOQ_ERR_CONFIG;
    if (plan.ws_bytes > 0) {
        if (workspace == nullptr || workspace_bytes < size_t(plan.ws_bytes))
            return QOQ_ERR_WORKSPACE;
        if (misaligned(workspace)) return QOQ_ERR_ALIGN;
    }
    const hipError_t e = qoq::launch_gemm(plan, x8, s_x, M, K, static_cast<const uint8_t*>(packed),
                                          s1, N, y, acc_debug, workspace,
                                          static_cast<hipStream_t>(stream));
    return e == hipSuccess ? QOQ_OK : QOQ_ERR_HIP;
}

qoq_status qoq_w4a8_gemm_noalloc(const int8_t* x8, const float* s_x, int64_t M, int64_t K,
                                 const void* packed, const uint16_t* s1, int64_t N,
                                 int32_t group, uint16_t* y, int32_t* acc_debug, void* stream) {
    static_assert(QOQ_NOALLOC_SCRATCH_BYTES == qoq::kStaticScratchBytes, "scratch size");
    const qoq_status st = check_weight_shape(N, K, group);
    if (st != QOQ_OK) return st;
    if (M < 0 || M > kMaxDim || check_gemm_k(K) != QOQ_OK) return QOQ_ERR_SHAPE;
    if (M == 0) return QOQ_OK;
    if (x8 == nullptr || s_x == nullptr || packed == nullptr || s1 == nullptr || y == nullptr)
        return QOQ_ERR_NULL;
    if (misaligned(x8) || misaligned(packed) || misaligned(y)) return QOQ_ERR_ALIGN;
    const qoq::GemmPlan plan = qoq::plan_gemm(M, N, K);
    if (plan.kind < 0) return QOQ_ERR_CONFIG;
    if (plan.ws_bytes > qoq::kStaticScratchBytes) return QOQ_ERR_WORKSPACE;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    void* scratch = nullptr;
    if (plan.ws_bytes > 0 && qoq::static_scratch(s, &scratch) != hipSuccess) return QOQ_ERR_HIP;
    const hipError_t e = qoq::launch_gemm(plan, x8, s_x, M, K, static_cast<const uint8_t*>(packed),
                                          s1, N, y, acc_debug, scratch, s);
    return e == hipSuccess ? QOQ_OK : QOQ_ERR_HIP;
}

size_t qoq_linear_workspace_bytes(int64_t M, int64_t N, int64_t K) {
    if (M <= 0 || check_weight_shape(N, K, qoq::kGroup) != QOQ_OK || M > kMaxDim ||
        check_gemm_k(K) != QOQ_OK)
        return 0;
    const qoq::LinearPlan plan = qoq::plan_linear(M, N, K);
    return plan.valid ? size_t(plan.ws_bytes) : 0;
}

int qoq_linear_path(int64_t M, int64_t N, int64_t K) {
    if (M <= 0 || check_weight_shape(N, K, qoq::kGroup) != QOQ_OK || M > kMaxDim ||
        check_gemm_k(K) != QOQ_OK)
        return -1;
    const qoq::LinearPlan plan = qoq::plan_linear(M, N, K);
    if (!plan.valid) return -1;
    return plan.fused ? 1 : 0;
}

qoq_status qoq_w4a8_linear(const uint16_t* x, int64_t M, int64_t K, const void* packed,
                           const uint16_t* s1, int64_t N, int32_t group, uint16_t* y,
                           int32_t* acc_debug, void* workspace, size_t workspace_bytes,
                           void* stream) {
    const qoq_status st = check_weight_shape(N, K, group);
    if (st != QOQ_OK) return st;
    if (M < 0 || M > kMaxDim || check_gemm_k(K) != QOQ_OK) return QOQ_ERR_SHAPE;
    if (M == 0) return QOQ_OK;
    if (x == nullptr || packed == nullptr || s1 == nullptr || y == nullptr) return QOQ_ERR_NULL;
    if (misaligned(x) || misaligned(packed) || misaligned(y)) return QOQ_ERR_ALIGN;
    const qoq::LinearPlan plan = qoq::plan_linear(M, N, K);
    if (!plan.valid) return QOQ_ERR_CONFIG;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    const uint8_t* pk = static_cast<const uint8_t*>(packed);
    if (plan.fused) {
        const hipError_t e = qoq::launch_linear_fused(plan, x, M, K, pk, s1, N, y, acc_debug, s);
        return e == hipSuccess ? QOQ_OK : QOQ_ERR_HIP;
    }
    if (workspace == nullptr || workspace_bytes < size_t(plan.ws_bytes)) return QOQ_ERR_WORKSPACE;
    if (misaligned(workspace)) return QOQ_ERR_ALIGN;
    uint8_t* ws = static_cast<uint8_t*>(workspace);
    int8_t* x8 = reinterpret_cast<int8_t*>(ws + plan.x8_offset);
    float* s_x = reinterpret_cast<float*>(ws + plan.sx_offset);
    hipError_t e = qoq::launch_quantize_act(x, M, K, x8, s_x, s);
    if (e != hipSuccess) return QOQ_ERR_HIP;
    e = qoq::launch_gemm(plan.gemm, x8, s_x, M, K, pk, s1, N, y, acc_debug,
                         plan.gemm.ws_bytes > 0 ? ws + plan.gemm_ws_offset : nullptr, s);
    return e == hipSuccess ? QOQ_OK : QOQ_ERR_HIP;
}

size_t qoq_w8a8_weight_bytes(int64_t N, int64_t K) {
    if (check_weight_shape(N, K, qoq::kGroup) != QOQ_OK) return 0;
    return size_t(N * K);
}

qoq_status qoq_w8a8_pack_weights(const float* W, int64_t N, int64_t K, void* packed, uint16_t* s,
                                 void* stream) {
    const qoq_status st = check_weight_shape(N, K, qoq::kGroup);
    if (st != QOQ_OK) return st;
    if (W == nullptr || packed == nullptr || s == nullptr) return QOQ_ERR_NULL;
    if (misaligned(W) || misaligned(packed)) return QOQ_ERR_ALIGN;
    const hipError_t e = qoq::launch_w8a8_pack(W, N, K, static_cast<uint8_t*>(packed), s,
                                               static_cast<hipStream_t>(stream));
    return e == hipSuccess ? QOQ_OK : QOQ_ERR_HIP;
}

qoq_status qoq_w8a8_gemm(const int8_t* x8, const float* s_x, int64_t M, int64_t K,
                         const void* packed, const uint16_t* s, int64_t N, uint16_t* y,
                         int32_t* acc_debug, void* stream) {
    const qoq_status st = check_weight_shape(N, K, qoq::kGroup);
    if (st != QOQ_OK) return st;
    if (M < 0 || M > kMaxDim || K > kMaxAccKW8A8) return QOQ_ERR_SHAPE;
    if (M == 0) return QOQ_OK;
    if (x8 == nullptr || s_x == nullptr || packed == nullptr || s == nullptr || y == nullptr)
        return QOQ_ERR_NULL;
    if (misaligned(x8) || misaligned(packed) || misaligned(y)) return QOQ_ERR_ALIGN;
    if (N * K >= (int64_t(1) << 31) || qoq::act_bytes(M, K) >= (int64_t(1) << 31))
        return QOQ_ERR_SHAPE;
    const qoq::VariantPlan plan = qoq::plan_variant(qoq::kVariantW8A8, M, N, K);
    if (!plan.valid) return QOQ_ERR_CONFIG;
    const hipError_t e = qoq::launch_w8a8_gemm(plan, x8, s_x, M, K,
                                               static_cast<const uint8_t*>(packed), s, N, y,
                                               acc_debug, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? QOQ_OK : QOQ_ERR_HIP;
}

size_t qoq_w4a4_weight_bytes(int64_t N, int64_t K) { return qoq_packed_weight_bytes(N, K, qoq::kGroup); }

size_t qoq_w4a4_act_bytes(int64_t M, int64_t K) {
    if (M <= 0 || K <= 0 || K % qoq::kGroup != 0 || M > kMaxDim || K > kMaxDim) return 0;
    return size_t(qoq::w4a4_act_bytes(M, K));
}

qoq_status qoq_w4a4_pack_weights(const float* W, int64_t N, int64_t K, void* packed,
                                 void* stream) {
    const qoq_status st = check_weight_shape(N, K, qoq::kGroup);
    if (st != QOQ_OK) return st;
    if (W == nullptr || packed == nullptr) return QOQ_ERR_NULL;
    if (misaligned(W) || misaligned(packed)) return QOQ_ERR_ALIGN;
    const hipError_t e = qoq::launch_w4a4_pack(W, N, K, static_cast<uint8_t*>(packed),
                                               static_cast<hipStream_t>(stream));
    return e == hipSuccess ? QOQ_OK : QOQ_ERR_HIP;
}

qoq_status qoq_w4a4_quantize_act(const uint16_t* x, int64_t M, int64_t K, void* act,
                                 void* stream) {
    if (M < 0 || K <= 0 || K % qoq::kGroup != 0 || M > kMaxDim || K > kMaxDim)
        return QOQ_ERR_SHAPE;
    if (M == 0) return QOQ_OK;
    if (x == nullptr || act == nullptr) return QOQ_ERR_NULL;
    if (misaligned(x) || misaligned(act)) return QOQ_ERR_ALIGN;
    if (qoq::w4a4_act_bytes(M, K) >= (int64_t(1) << 31)) return QOQ_ERR_SHAPE;
    const hipError_t e = qoq::launch_w4a4_quantize_act(x, M, K, static_cast<uint8_t*>(act),
                                                       static_cast<hipStream_t>(stream));
    return e == hipSuccess ? QOQ_OK : QOQ_ERR_HIP;
}

qoq_status qoq_w4a4_gemm(const void* act, int64_t M, int64_t K, const void* packed, int64_t N,
                         uint16_t* y, void* stream) {
    const qoq_status st = check_weight_shape(N, K, qoq::kGroup);
    if (st != QOQ_OK) return st;
    if (M < 0 || M > kMaxDim) return QOQ_ERR_SHAPE;
    if (M == 0) return QOQ_OK;
    if (act == nullptr || packed == nullptr || y == nullptr) return QOQ_ERR_NULL;
    if (misaligned(act) || misaligned(packed) || misaligned(y)) return QOQ_ERR_ALIGN;
    if (N * K / 2 >= (int64_t(1) << 31) || qoq::w4a4_act_bytes(M, K) >= (int64_t(1) << 31))
        return QOQ_ERR_SHAPE;
    const qoq::VariantPlan plan = qoq::plan_variant(qoq::kVariantW4A4, M, N, K);
    if (!plan.valid) return QOQ_ERR_CONFIG;
    const hipError_t e = qoq::launch_w4a4_gemm(plan, static_cast<const uint8_t*>(act), M, K,
                                               static_cast<const uint8_t*>(packed), N, y,
                                               static_cast<hipStream_t>(stream));
    return e == hipSuccess ? QOQ_OK : QOQ_ERR_HIP;
}

size_t qoq_w4a16_weight_bytes(int64_t N, int64_t K) {
    if (check_weight_shape(N, K, qoq::kGroup) != QOQ_OK) return 0;
    const qoq::PackedLayout L = qoq::packed_layout(N, K);
    return size_t(L.total + L.rec_bytes);
}

qoq_status qoq_w4a16_pack_weights(const float* W, int64_t N, int64_t K, void* packed,
                                  void* stream) {
    const qoq_status st = check_weight_shape(N, K, qoq::kGroup);
    if (st != QOQ_OK) return st;
    if (W == nullptr || packed == nullptr) return QOQ_ERR_NULL;
    if (misaligned(W) || misaligned(packed)) return QOQ_ERR_ALIGN;
    const hipError_t e = qoq::launch_w4a16_pack(W, N, K, static_cast<uint8_t*>(packed),
                                                static_cast<hipStream_t>(stream));
    return e == hipSuccess ? QOQ_OK : QOQ_ERR_HIP;
}

qoq_status qoq_w4a16_gemm(const uint16_t* x, int64_t M, int64_t K, const void* packed, int64_t N,
                          uint16_t* y, void* stream) {
    const qoq_status st = check_weight_shape(N, K, qoq::kGroup);
    if (st != QOQ_OK) return st;
    if (M < 0 || M > kMaxDim) return QOQ_ERR_SHAPE;
    if (M == 0) return QOQ_OK;
    if (x == nullptr || packed == nullptr || y == nullptr) return QOQ_ERR_NULL;
    if (misaligned(x) || misaligned(packed) || misaligned(y)) return QOQ_ERR_ALIGN;
    if (N * K / 2 >= (int64_t(1) << 31) || M * K * 2 >= (int64_t(1) << 31)) return QOQ_ERR_SHAPE;
    const qoq::VariantPlan plan = qoq::plan_variant(qoq::kVariantW4A16, M, N, K);
    if (!plan.valid) return QOQ_ERR_CONFIG;
    const hipError_t e = qoq::launch_w4a16_gemm(plan, x, M, K, static_cast<const uint8_t*>(packed),
                                                N, y, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? QOQ_OK : QOQ_ERR_HIP;
}

// ---------------------------------------------------------------------------
// KV4 decode attention
// ---------------------------------------------------------------------------
namespace {
using qoq::kKv4MaxCapacity;

qoq_status check_kv4_heads(int64_t B, int64_t H, int64_t Hkv, int64_t D) {
    if (D != 128 || B < 0 || B > kMaxDim || Hkv <= 0 || Hkv > 4096 || H <= 0 || H % Hkv != 0 ||
        H / Hkv > 16)
        return QOQ_ERR_SHAPE;
    return QOQ_OK;
}

// A dispatch counts its work-items in 32 bits: the attention grid, and the
// merge of split contexts (64 work-items per (sequence, query head)).
bool kv_launch_fits(const qoq::Kv4Plan& p, int64_t B, int64_t H) {
    const int64_t lim = int64_t(1) << 32;
    return p.grid < lim / (64 * p.waves) && B * H < lim / 64;
}

// caches of B x H_kv regions of C tokens (512 bytes per token at most) must
// have byte offsets far inside int64
bool kv_cache_fits(int64_t B, int64_t Hkv, int64_t C) {
    return double(B) * double(Hkv) * double(C) * 512.0 < 4.0e18;
}
}  // namespace

size_t qoq_kv4_cache_bytes(int64_t B, int64_t H_kv, int64_t capacity, int64_t D) {
    if (check_kv4_heads(B, H_kv, H_kv, D) != QOQ_OK || B == 0) return 0;
    if (capacity <= 0 || capacity % 32 != 0 || capacity > kKv4MaxCapacity) return 0;
    if (!kv_cache_fits(B, H_kv, capacity)) return 0;
    return size_t(qoq::kv4_cache_bytes(B, H_kv, capacity));
}

qoq_status qoq_kv4_smooth_factors(const uint16_t* k_calib, int64_t T, int64_t H_kv, int64_t D,
                                  uint16_t* lambda, void* stream) {
    if (check_kv4_heads(1, H_kv, H_kv, D) != QOQ_OK || T <= 0 || T > kMaxDim) return QOQ_ERR_SHAPE;
    if (k_calib == nullptr || lambda == nullptr) return QOQ_ERR_NULL;
    if (misaligned(k_calib) || misaligned(lambda)) return QOQ_ERR_ALIGN;
    const hipError_t e = qoq::launch_kv4_smooth(k_calib, T, H_kv, lambda,
                                                static_cast<hipStream_t>(stream));
    return e == hipSuccess ? QOQ_OK : QOQ_ERR_HIP;
}

qoq_status qoq_kv4_append(const uint16_t* k, const uint16_t* v, int64_t B, int64_t T_new,
                          int64_t H_kv, int64_t D, const uint16_t* lambda, const int32_t* start,
                          void* cache, int64_t capacity, void* stream) {
    if (check_kv4_heads(B, H_kv, H_kv, D) != QOQ_OK || T_new < 0 || T_new > kKv4MaxCapacity)
        return QOQ_ERR_SHAPE;
    if (capacity <= 0 || capacity % 32 != 0 || capacity > kKv4MaxCapacity ||
        !kv_cache_fits(B, H_kv, capacity))
        return QOQ_ERR_SHAPE;
    if (B == 0 || T_new == 0) return QOQ_OK;
    if (B * T_new * H_kv > (int64_t(1) << 31) ||
        B * H_kv * ((T_new + 31) / 32 + 1) * 512 > (int64_t(1) << 31))
        return QOQ_ERR_SHAPE;
    if (k == nullptr || v == nullptr || lambda == nullptr || start == nullptr || cache == nullptr)
        return QOQ_ERR_NULL;
    if (misaligned(k) || misaligned(v) || misaligned(lambda) || misaligned(cache))
        return QOQ_ERR_ALIGN;
    const hipError_t e = qoq::launch_kv4_append(k, v, B, T_new, H_kv, lambda, start,
                                                static_cast<uint8_t*>(cache), capacity,
                                                static_cast<hipStream_t>(stream));
    return e == hipSuccess ? QOQ_OK : QOQ_ERR_HIP;
}

size_t qoq_kv4_attention_workspace_bytes(int64_t B, int64_t H, int64_t H_kv, int64_t D,
                                         int64_t max_len) {
    if (check_kv4_heads(B, H, H_kv, D) != QOQ_OK || max_len < 0 || max_len > kKv4MaxCapacity)
        return 0;
    if (B == 0) return 0;
    const qoq::Kv4Plan p = qoq::plan_kv4(B, H_kv, max_len);
    if (!kv_launch_fits(p, B, H)) return 0;   // the call itself refuses these
    return size_t(qoq::kv4_workspace_bytes(p, B, H));
}

qoq_status qoq_kv4_decode_attention(const uint16_t* q, int64_t B, int64_t H, int64_t H_kv,
                                    int64_t D, const uint16_t* lambda, const void* cache,
                                    int64_t capacity, const int32_t* lens, int64_t max_len,
                                    uint16_t* out, void* workspace, size_t workspace_bytes,
                                    void* stream) {
    const qoq_status st = check_kv4_heads(B, H, H_kv, D);
    if (st != QOQ_OK) return st;
    if (capacity <= 0 || capacity % 32 != 0 || capacity > kKv4MaxCapacity ||
        !kv_cache_fits(B, H_kv, capacity))
        return QOQ_ERR_SHAPE;
    if (max_len < 0 || max_len > capacity) return QOQ_ERR_SHAPE;
    if (B == 0) return QOQ_OK;
    if (q == nullptr || lambda == nullptr || cache == nullptr || lens == nullptr || out == nullptr)
        return QOQ_ERR_NULL;
    if (misaligned(q) || misaligned(lambda) || misaligned(cache) || misaligned(out))
        return QOQ_ERR_ALIGN;
    const qoq::Kv4Plan p = qoq::plan_kv4(B, H_kv, max_len);
    if (!kv_launch_fits(p, B, H)) return QOQ_ERR_SHAPE;
    const int64_t need = qoq::kv4_workspace_bytes(p, B, H);
    if (need > 0) {
        if (workspace == nullptr || workspace_bytes < size_t(need)) return QOQ_ERR_WORKSPACE;
        if (misaligned(workspace)) return QOQ_ERR_ALIGN;
    }
    const hipError_t e = qoq::launch_kv4_attention(
        p, q, B, H, H_kv, lambda, static_cast<const uint8_t*>(cache), capacity, lens, max_len, out,
        static_cast<float*>(need > 0 ? workspace : nullptr), static_cast<hipStream_t>(stream));
    return e == hipSuccess ? QOQ_OK : QOQ_ERR_HIP;
}

size_t qoq_kv16_cache_bytes(int64_t B, int64_t H_kv, int64_t capacity, int64_t D) {
    if (check_kv4_heads(B, H_kv, H_kv, D) != QOQ_OK || B == 0) return 0;
    if (capacity <= 0 || capacity % 32 != 0 || capacity > kKv4MaxCapacity) return 0;
    if (!kv_cache_fits(B, H_kv, capacity)) return 0;
    return size_t(qoq::kv16_cache_bytes(B, H_kv, capacity));
}

qoq_status qoq_kv16_append(const uint16_t* k, const uint16_t* v, int64_t B, int64_t T_new,
                           int64_t H_kv, int64_t D, const int32_t* start, void* cache,
                           int64_t capacity, void* stream) {
    if (check_kv4_heads(B, H_kv, H_kv, D) != QOQ_OK || T_new < 0 || T_new > kKv4MaxCapacity)
        return QOQ_ERR_SHAPE;
    if (capacity <= 0 || capacity % 32 != 0 || capacity > kKv4MaxCapacity ||
        !kv_cache_fits(B, H_kv, capacity))
        return QOQ_ERR_SHAPE;
    if (B == 0 || T_new == 0) return QOQ_OK;
    if (B * T_new * H_kv > (int64_t(1) << 31)) return QOQ_ERR_SHAPE;
    if (k == nullptr || v == nullptr || start == nullptr || cache == nullptr) return QOQ_ERR_NULL;
    if (misaligned(k) || misaligned(v) || misaligned(cache)) return QOQ_ERR_ALIGN;
    const hipError_t e = qoq::launch_kv16_append(k, v, B, T_new, H_kv, start,
                                                 static_cast<uint8_t*>(cache), capacity,
                                                 static_cast<hipStream_t>(stream));
    return e == hipSuccess ? QOQ_OK : QOQ_ERR_HIP;
}

qoq_status qoq_kv16_decode_attention(const uint16_t* q, int64_t B, int64_t H, int64_t H_kv,
                                     int64_t D, const void* cache, int64_t capacity,
                                     const int32_t* lens, int64_t max_len, uint16_t* out,
                                     void* workspace, size_t workspace_bytes, void* stream) {
    const qoq_status st = check_kv4_heads(B, H, H_kv, D);
    if (st != QOQ_OK) return st;
    if (capacity <= 0 || capacity % 32 != 0 || capacity > kKv4MaxCapacity ||
        !kv_cache_fits(B, H_kv, capacity))
        return QOQ_ERR_SHAPE;
    if (max_len < 0 || max_len > capacity) return QOQ_ERR_SHAPE;
    if (B == 0) return QOQ_OK;
    if (q == nullptr || cache == nullptr || lens == nullptr || out == nullptr) return QOQ_ERR_NULL;
    if (misaligned(q) || misaligned(cache) || misaligned(out)) return QOQ_ERR_ALIGN;
    const qoq::Kv4Plan p = qoq::plan_kv4(B, H_kv, max_len);
    if (!kv_launch_fits(p, B, H)) return QOQ_ERR_SHAPE;
    const int64_t need = qoq::kv4_workspace_bytes(p, B, H);
    if (need > 0) {
        if (workspace == nullptr || workspace_bytes < size_t(need)) return QOQ_ERR_WORKSPACE;
        if (misaligned(workspace)) return QOQ_ERR_ALIGN;
    }
    const hipError_t e = qoq::launch_kv16_attention(
        p, q, B, H, H_kv, static_cast<const uint8_t*>(cache), capacity, lens, max_len, out,
        static_cast<float*>(need > 0 ? workspace : nullptr), static_cast<hipStream_t>(stream));
    return e == hipSuccess ? QOQ_OK : QOQ_ERR_HIP;
}

const char* qoq_status_string(int status) {
    switch (status) {
        case QOQ_OK: return "ok";
        case QOQ_ERR_NULL: return "a required pointer is NULL";
        case QOQ_ERR_SHAPE: return "invalid shape (sizes must be non-negative, N % 16 == 0, K % 128 == 0)";
        case QOQ_ERR_ALIGN: return "a pointer is not 16-byte aligned";
        case QOQ_ERR_GROUP: return "unsupported group size (only 128)";
        case QOQ_ERR_WORKSPACE: return "workspace missing or too small";
        case QOQ_ERR_HIP: return "HIP kernel launch failed";
        case QOQ_ERR_FLAGS: return "unknown flag bits";
        case QOQ_ERR_CONFIG: return "a tuning override names no compiled kernel configuration for this shape, or an unknown tuning key";
        default: return "unknown status";
    }
}

}  // extern "C"
