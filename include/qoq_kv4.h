/* Decode attention over a 4-bit KV cache with SmoothAttention scaling
 * (C ABI, gfx950).
 *
 * Pages: "QServe: W4A8KV4 Quantization and System Co-design for Efficient LLM
 * Serving" (velog notes), sections "Insight" and "Methods / 1) Algorithm:
 * QoQ" (4-bit KV cache; SmoothAttention moves the key quantization
 * difficulty onto the queries, which stay unquantized); the QServe abstract
 * (memory-bound fused attention over the KV4 cache); "Part5 LLM部署技术"
 * sections 1.1 (the SmoothQuant migration the factor follows) and 3.
 *
 * Arithmetic (readings of the pages, which give no formulas):
 *   lambda[h, d] = fp16(sqrt(fp32(max_t |k[t, h, d]|))), 1 for an all-zero
 *   channel; each cached vector (one token, one KV head, D = 128 values;
 *   keys first divided by lambda in fp32) is one group of the W4A16 weight
 *   format: lo = min(0, min x), hi = max(0, max x), s = fp16((hi - lo) / 15),
 *   z = clamp(rne(-lo / s), 0, 15), code = clamp(rne(x / s) + z, 0, 15),
 *   standing for (code - z) * s (an all-zero vector: s = 0, codes 0);
 *   q~ = fp16(fp32(q) * fp32(lambda)); query head h reads KV head
 *   h / (H / H_kv); out = softmax(q~ . k^ / sqrt(D)) v^ over the first
 *   lens[b] cached tokens (0 for an empty context), fp16.
 *
 * Cache: caller-owned device memory of qoq_kv4_cache_bytes(B, H_kv, C, D)
 * bytes; region (b, h) of 133 C bytes holds the key codes, the value codes
 * (32-token blocks of 2 KiB each, in MFMA lane order) and 160-byte metadata
 * blocks (per 32 tokens: 32 fp16 s_k, 32 fp16 s_v and 32 bytes z_k | z_v << 4,
 * in the same lane order) -- the 4.16 bits per cached value the format
 * needs. The layout is versioned by
 * QOQ_KV4_LAYOUT_VERSION; tokens never appended hold whatever the memory held
 * (they are never read as values).
 *
 * All pointers are device pointers, 16-byte aligned; fp16 is passed as
 * uint16_t bits; work is enqueued on `stream` (a hipStream_t, NULL for the
 * default stream); nothing allocates, frees or synchronizes. Errors return
 * before any launch. D must be 128.
 */
#ifndef QOQ_KV4_H
#define QOQ_KV4_H

#include <stddef.h>
#include <stdint.h>

#include "qoq.h"

#ifdef __cplusplus
extern "C" {
#endif

#define QOQ_KV4_LAYOUT_VERSION 1

/* Bytes of a KV4 cache for B sequences, H_kv heads and capacity C tokens
 * per sequence (C > 0, C % 32 == 0, D == 128); 0 if invalid. Host-only. */
size_t qoq_kv4_cache_bytes(int64_t B, int64_t H_kv, int64_t capacity, int64_t D);

/* Smoothing factors from calibration keys k_calib [T, H_kv, D] fp16 into
 * lambda [H_kv, D] fp16. T >= 1.
 * Errors: QOQ_ERR_NULL, QOQ_ERR_SHAPE, QOQ_ERR_ALIGN, QOQ_ERR_HIP. */
qoq_status qoq_kv4_smooth_factors(const uint16_t* k_calib, int64_t T, int64_t H_kv, int64_t D,
                                  uint16_t* lambda, void* stream);

/* Append T_new tokens per sequence: k, v [B, T_new, H_kv, D] fp16 go to
 * positions start[b] .. start[b] + T_new - 1 (start: device int32 [B],
 * negative read as 0); keys are smoothed by lambda [H_kv, D]. Positions at
 * or past the capacity are not written. Calls on one cache run in stream
 * order; two concurrent appends to one cache race.
 * Errors: QOQ_ERR_NULL, QOQ_ERR_SHAPE, QOQ_ERR_ALIGN, QOQ_ERR_HIP. */
qoq_status qoq_kv4_append(const uint16_t* k, const uint16_t* v, int64_t B, int64_t T_new,
                          int64_t H_kv, int64_t D, const uint16_t* lambda, const int32_t* start,
                          void* cache, int64_t capacity, void* stream);

/* Workspace bytes of qoq_kv4_decode_attention (partial results when the
 * contexts are split over several workgroups; 0 otherwise). Host-only. */
size_t qoq_kv4_attention_workspace_bytes(int64_t B, int64_t H, int64_t H_kv, int64_t D,
                                         int64_t max_len);

/* Decode attention: q [B, H, D] fp16 (one new token per sequence), lambda
 * [H_kv, D], cache as above, lens device int32 [B] (context lengths; values
 * are clamped to [0, min(max_len, capacity)]), max_len host-side bound of
 * the lengths (sets how contexts are split), out [B, H, D] fp16.
 * H % H_kv == 0 and H / H_kv <= 16. The "kv4_splits" key of
 * qoq_set_tuning forces n splits (at most 65536), "kv4_paired" = "0" turns
 * the paired schedule off, "1" forces it where the batch allows it.
 * QOQ_ERR_SHAPE also when a launch would count 2^32
 * work-items or more (B * H >= 2^26, or a forced split count that large).
 * Errors: QOQ_ERR_NULL, QOQ_ERR_SHAPE, QOQ_ERR_ALIGN, QOQ_ERR_WORKSPACE,
 * QOQ_ERR_HIP. */
qoq_status qoq_kv4_decode_attention(const uint16_t* q, int64_t B, int64_t H, int64_t H_kv,
                                    int64_t D, const uint16_t* lambda, const void* cache,
                                    int64_t capacity, const int32_t* lens, int64_t max_len,
                                    uint16_t* out, void* workspace, size_t workspace_bytes,
                                    void* stream);

/* The comparison point: the same decode attention on an fp16 cache (what the
 * pages set the 4-bit cache against), 512 bytes per token and KV head
 * (keys and values as stored, in the same MFMA lane order), queries
 * unsmoothed: out = softmax(q . k / sqrt(D)) v. Same shapes, errors,
 * workspace (qoq_kv4_attention_workspace_bytes) and tuning keys as the
 * KV4 calls. */
size_t qoq_kv16_cache_bytes(int64_t B, int64_t H_kv, int64_t capacity, int64_t D);
qoq_status qoq_kv16_append(const uint16_t* k, const uint16_t* v, int64_t B, int64_t T_new,
                           int64_t H_kv, int64_t D, const int32_t* start, void* cache,
                           int64_t capacity, void* stream);
qoq_status qoq_kv16_decode_attention(const uint16_t* q, int64_t B, int64_t H, int64_t H_kv,
                                     int64_t D, const void* cache, int64_t capacity,
                                     const int32_t* lens, int64_t max_len, uint16_t* out,
                                     void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* QOQ_KV4_H */
