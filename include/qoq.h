/*
 * qoq.h -- C ABI of libqoq: the W4A8 GEMM of QoQ with progressive group
 * quantization, for AMD Instinct MI355X (gfx950).
 *
 * What is computed (pages: "QServe: W4A8KV4 Quantization and System
 * Co-design for Efficient LLM Serving", sections "Methods / 1) Algorithm:
 * QoQ" and "Methods / 2) System: QServe"; the QServe abstract; "Part5
 * LLM部署技术", section 3 on QServe):
 *
 *   weights, offline   W[N,K] fp32 -> level 1: per-output-channel symmetric
 *                      INT8 codes q8 in the protective range [-119, 119]
 *                      with an FP16 scale s1[n];
 *                      -> level 2: per group of 128 inputs of one channel,
 *                      UINT4 codes q4 with an integer scale s2 in [1, 16]
 *                      and a UINT4 zero z (dequantized w8 = q4*s2 - z*s2,
 *                      always inside INT8);
 *   activations        x[M,K] fp16 -> per-token symmetric INT8 x8 with an
 *                      fp32 scale s_x[m];
 *   GEMM               acc[m,n] = sum_k x8[m,k] * w8[n,k] in INT32 over the
 *                      whole of K (no partial sum is ever scaled), then
 *                      y[m,n] = fp16(acc * s_x[m] * s1[n]).
 *
 * Conventions for every entry point:
 *   - All data pointers are device pointers (hipMalloc'd or equivalent),
 *     owned by the caller; W, packed, x, x8, y and the workspace must be
 *     16-byte aligned (checked), the others naturally aligned. The library never allocates,
 *     frees or synchronizes; all work is enqueued on `stream` (a
 *     hipStream_t; NULL = the null stream) and completes asynchronously.
 *   - Shapes are checked on the host before anything is launched; on any
 *     error nothing is launched and nothing is written.
 *   - Integer results (codes, scales, accumulators) are deterministic and
 *     independent of the launch configuration.
 *   - Inputs must be finite; results for NaN or Inf inputs are unspecified
 *     (but every memory access stays in bounds: indices depend on shapes
 *     only).
 *   - The library keeps no mutable global state except the tuning
 *     overrides of qoq_set_tuning (a measurement and test aid, unset by
 *     default) and the scratch addresses of qoq_w4a8_gemm_noalloc; calls on
 *     different streams are independent unless they share an output, a
 *     workspace or (no-alloc calls) a GPU's scratch array.
 */
#ifndef QOQ_H
#define QOQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum qoq_status {
    QOQ_OK = 0,
    QOQ_ERR_NULL = 1,      /* a required pointer is NULL                      */
    QOQ_ERR_SHAPE = 2,     /* negative size, N % 16 != 0, K % group != 0 ...  */
    QOQ_ERR_ALIGN = 3,     /* a pointer is not 16-byte aligned                */
    QOQ_ERR_GROUP = 4,     /* group size other than 128                       */
    QOQ_ERR_WORKSPACE = 5, /* workspace NULL or smaller than required         */
    QOQ_ERR_HIP = 6,       /* a kernel launch failed (hipGetLastError)        */
    QOQ_ERR_FLAGS = 7,     /* unknown flag bits                               */
    QOQ_ERR_CONFIG = 8     /* a tuning override names no compiled configuration,
                              or qoq_set_tuning got an unknown key          */
} qoq_status;

/* Group size of level 2 (inputs of one output channel per group). */
#define QOQ_GROUP 128

/* Largest K of the GEMM entry points: the INT32 accumulators stay exact
 * while K * 127 * 121 < 2^31 (activation codes within 127, dequantized
 * weights within 121); larger K is refused with QOQ_ERR_SHAPE (the packer
 * accepts any K). */
#define QOQ_MAX_GEMM_K 139648

/* Version of the packed-weight layout produced by qoq_pack_weights. */
#define QOQ_PACKED_LAYOUT_VERSION 1

/* Flag for qoq_pack_weights: skip quantization and pack the caller's
 * canonical (q4, s2, z) as they are. */
#define QOQ_PACK_FROM_CANONICAL 0x1u

/* Activation tile layout (version 1) of the INT8 activations x8 that
 * qoq_quantize_act writes and qoq_w4a8_gemm reads. Rows are grouped in tiles
 * of 16 and each row in 16-byte chunks; code (m, k) is at byte
 *     ((m / 16) * (K / 16) + k / 16) * 256 + (m % 16) * 16 + k % 16,
 * so one 256-byte unit holds a 16-row x 16-input block, row-major. Four
 * consecutive units are one v_mfma_i32_16x16x64_i8 A operand (lane l reads
 * bytes 16 l .. 16 l + 15) and a v_mfma_i32_32x32x32_i8 A operand is two
 * 512-byte runs: every activation load reads whole cache lines. The buffer
 * holds qoq_act_bytes(M, K) bytes; the bytes of rows M .. 16*ceil(M/16) - 1
 * are never written and never read. */
#define QOQ_ACT_LAYOUT_VERSION 1

/* Canonical level-2 output / input, all device pointers, row-major:
 *   q4 [N*K]        one UINT4 code per byte (0..15), element (n, k) at n*K + k
 *   s2 [N*K/128]    group scale, int8 in 1..16, group (n, g) at n*(K/128) + g
 *   z  [N*K/128]    group zero, uint8 in 0..15
 * When packing from canonical data the caller must keep every group inside
 * the unpack's byte lanes: 0 <= q4*s2 + (128 - z*s2) <= 255 for all codes
 * (true for anything level 2 produces, and for s2 = 1 with z in 0..15);
 * otherwise the GEMM result is unspecified (still in bounds). */
typedef struct qoq_canonical {
    uint8_t* q4;
    int8_t* s2;
    uint8_t* z;
} qoq_canonical;

/* Bytes of the packed-weight buffer for an N x K weight (layout version 1):
 * N*K/2 bytes of nibbles in MFMA operand order, then the per-group
 * (s2, 128 - z*s2) byte pairs. Returns 0 for invalid shapes (N <= 0,
 * K <= 0, N % 16 != 0, K % group != 0, group != 128). Host-only. */
size_t qoq_packed_weight_bytes(int64_t N, int64_t K, int32_t group);

/* Bytes of the x8 buffer for M tokens of K inputs in the activation tile
 * layout: 16 * ceil(M / 16) * K. Returns 0 for M <= 0 and for invalid K
 * (K <= 0, K % 128 != 0). Host-only. */
size_t qoq_act_bytes(int64_t M, int64_t K);

/* Progressive group quantization and compute-aware packing (offline).
 * Pages: velog notes "Methods / 1) Algorithm: QoQ" (8-bit with per-channel
 * FP16 scales, then 4-bit) and "Methods / 2) System: QServe" (protective
 * range; compute-aware weight reordering).
 *   W       [N,K] fp32, Linear layout (row n = output channel n). Ignored
 *           (may be NULL) with QOQ_PACK_FROM_CANONICAL.
 *   N, K    N % 16 == 0, K % group == 0, both > 0.
 *   group   must be 128.
 *   packed  out, qoq_packed_weight_bytes(N, K, group) bytes, opaque.
 *   s1      out [N] fp16 bits (per-channel scale). Not written (may be
 *           NULL) with QOQ_PACK_FROM_CANONICAL: the caller then owns s1.
 *   canon   without the flag: NULL, or all three pointers non-NULL to also
 *           receive the canonical codes; with the flag: required input.
 *   flags   0 or QOQ_PACK_FROM_CANONICAL.
 * Errors: QOQ_ERR_NULL, QOQ_ERR_SHAPE, QOQ_ERR_GROUP, QOQ_ERR_ALIGN,
 * QOQ_ERR_FLAGS, QOQ_ERR_HIP. */
qoq_status qoq_pack_weights(const float* W, int64_t N, int64_t K, int32_t group,
                            void* packed, uint16_t* s1, const qoq_canonical* canon,
                            uint32_t flags, void* stream);

/* Per-token symmetric INT8 activation quantization (run time).
 * Pages: QServe abstract (8-bit activations); velog notes "Background"
 * (per-token activation scale next to per-channel weight scale).
 *   x    [M,K] fp16 bits, row-major.   M >= 0, K > 0, K % 128 == 0.
 *   x8   out, qoq_act_bytes(M, K) bytes: the int8 codes in the activation
 *        tile layout (above).           s_x  out [M] fp32.
 * Row m: a = max|x[m,:]|; s_x = fp32(a/127); x8 = clamp(rne(x * fp32(127/a)),
 * -127, 127); a zero row gives s_x = 0 and zero codes. M == 0 launches
 * nothing. Errors: QOQ_ERR_NULL, QOQ_ERR_SHAPE, QOQ_ERR_ALIGN, QOQ_ERR_HIP. */
qoq_status qoq_quantize_act(const uint16_t* x, int64_t M, int64_t K,
                            int8_t* x8, float* s_x, void* stream);

/* Workspace bytes qoq_w4a8_gemm needs for this shape (0 if none). For
 * shapes whose K is split over workgroups (long K over few output tiles) the
 * workspace holds the exact INT32 partial sums, splits x M x N x 4 bytes;
 * a second kernel adds them in split order and applies the epilogue. Every
 * element is written before it is read, so no clearing is needed, and the
 * workspace can be reused by later calls on the same stream. Calls that
 * overlap in time must not share a workspace. Host-only. */
size_t qoq_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K);

/* W4A8 GEMM (run time, the hot path).
 * Pages: velog notes "Methods / 1) Algorithm: QoQ" (every GEMM operation on
 * INT8 matrix units), "Methods / 2) System: QServe" (register-level
 * parallel INT4->INT8 dequantization, subtraction after multiplication) and
 * "Background" (partial-sum dequantization in the main loop is the cost to
 * avoid); "Part5 LLM部署技术" section 3 (no partial-sum dequantization).
 *   x8, s_x      from qoq_quantize_act: int8 codes in the activation tile
 *                layout (qoq_act_bytes(M, K) bytes), [M] fp32.
 *   M >= 0, K > 0, K % 128 == 0, K <= QOQ_MAX_GEMM_K, N > 0, N % 16 == 0,
 *   group == 128.
 *   packed, s1   from qoq_pack_weights for the same N, K.
 *   y            out [M,N] fp16 bits, row-major: fp16(acc * s_x[m] * s1[n]).
 *   acc_debug    NULL, or out [M,N] int32: the exact accumulators.
 *   workspace    qoq_gemm_workspace_bytes(M, N, K) bytes, 16-byte aligned
 *                (may be NULL when that is 0).
 * M == 0 launches nothing.
 * Kernel choice: the library picks a kernel family and tile from (M, N, K);
 * the "gemm" key of qoq_set_tuning forces one compiled configuration for
 * measurements and tests (see there); every configuration computes the same
 * INT32 accumulators.
 * Errors: QOQ_ERR_NULL, QOQ_ERR_SHAPE, QOQ_ERR_GROUP, QOQ_ERR_ALIGN,
 * QOQ_ERR_WORKSPACE, QOQ_ERR_CONFIG, QOQ_ERR_HIP. */
qoq_status qoq_w4a8_gemm(const int8_t* x8, const float* s_x, int64_t M, int64_t K,
                         const void* packed, const uint16_t* s1, int64_t N, int32_t group,
                         uint16_t* y, int32_t* acc_debug,
                         void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of the scratch array behind qoq_w4a8_gemm_noalloc (one per GPU). */
#define QOQ_NOALLOC_SCRATCH_BYTES (64ll << 20)

/* qoq_w4a8_gemm without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc). Same arguments, kernels and
 * results as qoq_w4a8_gemm, bit for bit; where that call would use the
 * workspace (K split over workgroups), this one uses a fixed scratch array
 * of QOQ_NOALLOC_SCRATCH_BYTES inside the library, one copy per GPU, held
 * until the process ends. Its address is looked up on the first call on a
 * device (the stream's device, or the current device for the null stream);
 * nothing is ever allocated or freed by this call. Shapes whose workspace
 * (qoq_gemm_workspace_bytes) exceeds QOQ_NOALLOC_SCRATCH_BYTES are refused
 * with QOQ_ERR_WORKSPACE before anything is launched. Every call on one GPU
 * shares that GPU's array and leaves its partial sums there: calls that
 * overlap in time on one GPU (two streams, two threads) race and give
 * unspecified results; calls in one stream are ordered and safe. Every
 * element of the scratch is written before it is read, so nothing needs
 * clearing between calls.
 * Errors: as qoq_w4a8_gemm (QOQ_ERR_WORKSPACE for a too large split;
 * QOQ_ERR_HIP also when the scratch address cannot be looked up). */
qoq_status qoq_w4a8_gemm_noalloc(const int8_t* x8, const float* s_x, int64_t M, int64_t K,
                                 const void* packed, const uint16_t* s1, int64_t N,
                                 int32_t group, uint16_t* y, int32_t* acc_debug,
                                 void* stream);

/* Workspace bytes qoq_w4a8_linear needs for this shape: 0 when it runs as
 * one fused launch (see qoq_w4a8_linear), otherwise room for the x8 codes,
 * the token scales and the GEMM's own workspace. No zero-fill is needed.
 * Host-only. */
size_t qoq_linear_workspace_bytes(int64_t M, int64_t N, int64_t K);

/* How qoq_w4a8_linear runs this shape: 1 one fused launch (tokens
 * quantized by every workgroup, no workspace), 0 the quantizer then the
 * GEMM, -1 invalid shape or "gemm" tuning override. Host-only. */
int qoq_linear_path(int64_t M, int64_t N, int64_t K);

/* Per-token activation quantization and W4A8 GEMM in one call (run time).
 * Same result as qoq_quantize_act followed by qoq_w4a8_gemm, bit for bit
 * (codes, accumulators and y). For up to 12 tokens (9-12 only when
 * K >= 4096) with K <= 8192 and M * K * ceil(N / 16) <= 64e6 (the values the
 * workgroups quantize in all) a single kernel does both: every workgroup
 * quantizes the few tokens itself, which removes a launch of almost no work
 * from the decode step (pages: velog notes on
 * QServe, "Methods / 2) System: QServe", and "Part5 LLM部署技术" section 3,
 * on fusing the CUDA-core work into the GEMM). Other shapes run the
 * quantizer into `workspace`, then the GEMM.
 *   x            [M,K] fp16 bits, row-major, 16-byte aligned.
 *   M >= 0, K > 0, K % 128 == 0, K <= QOQ_MAX_GEMM_K, N > 0, N % 16 == 0,
 *   group == 128.
 *   packed, s1   from qoq_pack_weights for the same N, K.
 *   y            out [M,N] fp16 bits.   acc_debug  NULL or out [M,N] int32.
 *   workspace    qoq_linear_workspace_bytes(M, N, K) bytes, 16-byte aligned
 *                (may be NULL when that is 0); overlapping calls must not
 *                share it.
 * The "gemm" tuning value "fused,KW" (KW in 4, 8, 16) forces the fused kernel
 * (M <= 16, K <= 512 KW);
 * any other family forces the two-call path with that GEMM configuration.
 * Errors: QOQ_ERR_NULL, QOQ_ERR_SHAPE, QOQ_ERR_GROUP, QOQ_ERR_ALIGN,
 * QOQ_ERR_WORKSPACE, QOQ_ERR_CONFIG, QOQ_ERR_HIP. */
qoq_status qoq_w4a8_linear(const uint16_t* x, int64_t M, int64_t K,
                           const void* packed, const uint16_t* s1, int64_t N, int32_t group,
                           uint16_t* y, int32_t* acc_debug,
                           void* workspace, size_t workspace_bytes, void* stream);

/* Plan overrides for measurements and tests (not for production use): the
 * library reads no environment variables; these process-wide settings
 * force a launch configuration instead. value NULL or "" clears a key.
 *   "gemm"        GEMM plan: "decode,MT,CB,KW,PD", "lds,MT,CB,NW,PD[,SPLITS]",
 *                 "tile32,MT,CB,PB,WGPERCU[,NW[,SPLITS]]",
 *                 "ksplit,MT,CB,KW,PD", "wide,MT,CB,NW,R,WGPERCU[,SPLITS]",
 *                 "stream,MT,CB,NW,PD,CH[,SPLITS]", "generic,MT,2", or (for
 *                 qoq_w4a8_linear) "fused,KW". SPLITS: K ranges over
 *                 workgroups, 1..64, rounded to whole chunks of 8 groups.
 *                 A value naming no compiled configuration valid for the
 *                 shape makes the GEMM calls fail with QOQ_ERR_CONFIG
 *                 (nothing launched).
 *   "variant"     comparison GEMMs (qoq_variants.h): "MT,CB,PB,WGPERCU,NW".
 *   "kv4_splits"  decode attention (qoq_kv4.h): split count n > 0 (<= 65536).
 *   "kv4_paired"  decode attention: "0" turns the paired schedule off, "1"
 *                 takes it whenever the batch allows it (by default only for
 *                 contexts of 1024 tokens or more).
 * Settings apply to calls made after this one returns; setting a key while
 * another thread enqueues work races with that thread's plan.
 * Errors: QOQ_ERR_NULL (key NULL), QOQ_ERR_CONFIG (unknown key). */
qoq_status qoq_set_tuning(const char* key, const char* value);

/* Static description of a status code (never NULL). */
const char* qoq_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* QOQ_H */
