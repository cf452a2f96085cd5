/*
 * qoq_variants.h -- C ABI of the comparison GEMMs in libqoq: the low-bit GEMM
 * families the QServe pages set QoQ's W4A8 against, built on the same
 * 32x32x32 tile kernel skeleton as the W4A8 GEMM so that a measured
 * difference is the format and its dequantization, not the tiling.
 *
 * Pages: "QServe: W4A8KV4 Quantization and System Co-design for Efficient LLM
 * Serving" (velog notes), sections "문제 정의" (existing INT4 systems lose
 * 20-90 % of their time to dequantization on general-purpose cores) and
 * "Background" (W8A8 = per-channel weights, per-token activations, no
 * dequantization in the main loop; per-group W4A4 must convert and scale
 * every group's INT32 partial sums inside the main loop); the QServe
 * abstract.
 *
 *   W8A8   weights: per-channel symmetric INT8 over [-127, 127], fp16 scale
 *          s[n] = fp16(fp32(absmax / 127)); activations: qoq_quantize_act
 *          (per-token INT8, tile layout); y = fp16(acc * s_x[m] * s[n]) with
 *          the exact INT32 accumulator over all of K.
 *   W4A16  weights: per (channel, group of 128) asymmetric UINT4 with an fp16
 *          scale and a UINT4 zero, dequantized in the main loop to fp16;
 *          activations fp16; fp16 MFMA, fp32 accumulation, fp16 y.
 *   W4A4   weights: per (channel, group of 128) symmetric INT4 in [-7, 7],
 *          fp16 scale fp16(fp32(absmax / 7)); activations: per (token,
 *          group) symmetric INT4, inv = fp32(7 / absmax), codes
 *          clamp(rne(fp32(x * inv)), -7, 7), fp32 scale absmax / 7;
 *          y = fp16(sum over groups of fp32(P_g) * (s_a * s_w)), P_g the
 *          exact INT32 partial sum of group g, accumulated in fp32.
 *
 * Conventions as in qoq.h: device pointers owned by the caller, 16-byte
 * alignment of every buffer (checked), shapes checked before any launch,
 * N % 16 == 0, K % 128 == 0, nothing allocated, freed or synchronized, all
 * work enqueued on `stream`. The "variant" key of qoq_set_tuning
 * ("MT,CB,PB,WGPERCU,NW") forces one compiled tile configuration of the
 * GEMMs (QOQ_ERR_CONFIG otherwise).
 */
#ifndef QOQ_VARIANTS_H
#define QOQ_VARIANTS_H

#include <stddef.h>
#include <stdint.h>

#include "qoq.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Bytes of the W8A8 packed weights: N*K, int8 codes in MFMA operand order
 * [N/16][K/128][2][64][16] (block (nb, g), half s, lane c + 16h holds the
 * codes of channel 16nb + c, inputs 128g + 64s + 16h .. +15). 0 if invalid. */
size_t qoq_w8a8_weight_bytes(int64_t N, int64_t K);

/* W8A8 weight quantization and packing.
 *   W [N,K] fp32 (Linear layout); packed out (qoq_w8a8_weight_bytes);
 *   s out [N] fp16 bits. Errors: QOQ_ERR_NULL, QOQ_ERR_SHAPE, QOQ_ERR_ALIGN,
 *   QOQ_ERR_HIP. */
qoq_status qoq_w8a8_pack_weights(const float* W, int64_t N, int64_t K, void* packed,
                                 uint16_t* s, void* stream);

/* W8A8 GEMM: x8/s_x from qoq_quantize_act, y out [M,N] fp16, acc_debug NULL
 * or out [M,N] int32 (exact accumulators). Requires N*K and the x8 buffer
 * below 2^31 bytes and K <= 133120 (K * 127 * 127 < 2^31: the INT32
 * accumulators stay exact). Errors: QOQ_ERR_NULL, QOQ_ERR_SHAPE, QOQ_ERR_ALIGN,
 * QOQ_ERR_CONFIG, QOQ_ERR_HIP. */
qoq_status qoq_w8a8_gemm(const int8_t* x8, const float* s_x, int64_t M, int64_t K,
                         const void* packed, const uint16_t* s, int64_t N, uint16_t* y,
                         int32_t* acc_debug, void* stream);

/* Bytes of the W4A16 packed weights: the W4A8 nibble layout holding the
 * UINT4 codes q, then two regions of the W4A8 record shape holding, per
 * (channel, group), the fp16 scale and the zero (uint16). 0 if invalid. */
size_t qoq_w4a16_weight_bytes(int64_t N, int64_t K);

/* W4A16 weight quantization and packing (W [N,K] fp32 -> packed): per
 * (channel, group of 128) lo = min(0, min w), hi = max(0, max w),
 * s = fp16(fp32(fp32(hi - lo) / 15)), z = clamp(rne(fp32(-lo / s)), 0, 15),
 * q = clamp(rne(fp32(w / s)) + z, 0, 15). */
qoq_status qoq_w4a16_pack_weights(const float* W, int64_t N, int64_t K, void* packed,
                                  void* stream);

/* W4A16 GEMM: x [M,K] fp16 row-major, weights dequantized to
 * fp16((q - z) * s) in the main loop, fp16 MFMA with fp32 accumulation,
 * y out [M,N] fp16. Requires N*K/2 and 2*M*K below 2^31 bytes. */
qoq_status qoq_w4a16_gemm(const uint16_t* x, int64_t M, int64_t K, const void* packed, int64_t N,
                          uint16_t* y, void* stream);

/* Bytes of the W4A4 packed weights: the W4A8 packed layout's size; nibbles
 * hold u = code + 8 and each group's record slot holds its fp16 scale. */
size_t qoq_w4a4_weight_bytes(int64_t N, int64_t K);

/* W4A4 weight quantization and packing (W [N,K] fp32 -> packed). */
qoq_status qoq_w4a4_pack_weights(const float* W, int64_t N, int64_t K, void* packed,
                                 void* stream);

/* Bytes of a W4A4 activation buffer for M tokens of K inputs: the x4 codes
 * (M rounded up to 16 rows, K/2 bytes per row; row m, inputs 16j .. 16j+15
 * are 8 bytes at ((m/16)*(K/16) + j)*128 + (m%16)*8, byte b holding
 * u(16j+b) | u(16j+8+b) << 4 with u = code + 8), then, 256-byte aligned, the
 * fp32 group scales [K/128][Mp], Mp = M rounded up to 128 (rows past M 0).
 * 0 for invalid shapes. */
size_t qoq_w4a4_act_bytes(int64_t M, int64_t K);

/* Per-(token, group) INT4 activation quantization: x [M,K] fp16 -> act. */
qoq_status qoq_w4a4_quantize_act(const uint16_t* x, int64_t M, int64_t K, void* act,
                                 void* stream);

/* W4A4 GEMM with per-group partial-sum scaling: act from
 * qoq_w4a4_quantize_act, packed from qoq_w4a4_pack_weights, y out [M,N]
 * fp16. Errors: QOQ_ERR_NULL, QOQ_ERR_SHAPE, QOQ_ERR_ALIGN, QOQ_ERR_CONFIG,
 * QOQ_ERR_HIP. */
qoq_status qoq_w4a4_gemm(const void* act, int64_t M, int64_t K, const void* packed, int64_t N,
                         uint16_t* y, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* QOQ_VARIANTS_H */
