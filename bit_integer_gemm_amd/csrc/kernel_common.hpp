// Device helpers shared by the GEMM kernel families (W4A8 QoQ and the
// comparison formats) and the activation quantizer: operand vector types,
// the register-parallel UINT4 dequantization, the per-token activation
// codes, the fp16 epilogue, group-record access and the XCD-aware tile
// order.
#pragma once

#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qoq {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef unsigned short us2 __attribute__((ext_vector_type(2)));

// Four UINT4 codes (one per byte) -> four INT8 weights, register-parallel.
__device__ __forceinline__ int dequant4(uint32_t codes, uint32_t mul2, uint32_t add2) {
    const us2 r = __builtin_bit_cast(us2, codes) * __builtin_bit_cast(us2, mul2) +
                  __builtin_bit_cast(us2, add2);
    return int(__builtin_bit_cast(uint32_t, r) ^ 0x80808080u);
}

__device__ __forceinline__ float h2f(uint16_t b) { return __half2float(__ushort_as_half(b)); }

// Per-token activation codes of two fp16 values (one 32-bit word) with the
// row's fp32 inverse scale: clamp(rne(x * inv), -127, 127), two bytes.
__device__ __forceinline__ uint32_t quant_pair(uint32_t two_halves, float inv) {
    const float a = rintf(h2f(uint16_t(two_halves & 0xffffu)) * inv);
    const float b = rintf(h2f(uint16_t(two_halves >> 16)) * inv);
    const int qa = int(fminf(fmaxf(a, -127.0f), 127.0f));
    const int qb = int(fminf(fmaxf(b, -127.0f), 127.0f));
    return (uint32_t(qa) & 0xffu) | ((uint32_t(qb) & 0xffu) << 8);
}

__device__ __forceinline__ uint16_t epilogue_value(int32_t acc, float sx, float sw) {
    const float v = float(acc) * (sx * sw);
    return __half_as_ushort(__float2half_rn(v));
}

// One lane's 16 packed bytes (32 codes of one channel) -> the B operands of
// the two MFMA steps of the group: low nibbles -> step 0, high -> step 1.
// `rec` holds s2 in bits 0-7 and 128 - z*s2 in bits 8-15.
__device__ __forceinline__ void dequant_block(const uint4 q, uint32_t rec, v4i& b0, v4i& b1) {
    // byte permutes: s2 into both 16-bit halves, the bias into all four bytes
    const uint32_t mul2 = __builtin_amdgcn_perm(0u, rec, 0x0c000c00u);
    const uint32_t add2 = __builtin_amdgcn_perm(0u, rec, 0x01010101u);
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        b0[i] = dequant4(w[i] & 0x0F0F0F0Fu, mul2, add2);
        b1[i] = dequant4((w[i] >> 4) & 0x0F0F0F0Fu, mul2, add2);
    }
}

// Record of group (8j + u) from the 16-byte chunk of groups 8j..8j+7 (u static).
__device__ __forceinline__ uint32_t record_of(const uint4 chunk, int u) {
    const uint32_t w[4] = {chunk.x, chunk.y, chunk.z, chunk.w};
    return (w[u >> 1] >> (16 * (u & 1))) & 0xffffu;
}

// Tiles are assigned XCD-aware: the workgroups that land on one XCD (ids
// congruent mod 8, the hardware's round-robin dispatch) take a contiguous run
// of tiles in grouped order (8 tile rows at a time), so each XCD's L2 sees a
// compact block of activation rows and weight columns.
__device__ __forceinline__ void tile_of(int L, int tiles_m, int tiles_n, int& tm, int& tn) {
    const int T = tiles_m * tiles_n;
    const int xcd = L & 7;
    const int j = L >> 3;
    const int per = T >> 3, extra = T & 7;
    const int t = xcd * per + min(xcd, extra) + j;
    constexpr int GM = 8;
    const int group = t / (GM * tiles_n);
    const int first_m = group * GM;
    const int gm = min(GM, tiles_m - first_m);
    const int in = t - group * GM * tiles_n;
    tm = first_m + in % gm;
    tn = in / gm;
}

}  // namespace qoq
