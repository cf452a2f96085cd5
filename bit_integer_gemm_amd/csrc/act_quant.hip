// Per-token symmetric INT8 quantization of the activations.
//
// The QServe abstract names 8-bit activations; the velog notes on QServe,
// section "Background", pair per-channel weight scales with per-token
// activation scales (that page's granularity labels are shifted by one item;
// the per-token reading is the one the rest of the pages support).
//
// One workgroup per token. Pass 1 takes the row absmax (exact in any
// reduction order: a max of exactly converted fp16 values); pass 2 writes the
// codes from the values still held in registers (rows up to 8192 values) or
// re-reads the row (longer rows; it is still in the caches). 16-byte loads,
// 8 fp16 values per lane; the codes go out in the activation tile layout
// (16-byte chunks of a row 256 bytes apart), 8 bytes per lane.
#include "qoq_internal.hpp"
#include "kernel_common.hpp"

#include <hip/hip_fp16.h>

namespace qoq {
namespace {

// Rows up to kRegK values are held in registers between the two passes (one
// memory round trip); longer rows are re-read for the second pass.
constexpr int kRegChunks = 4;                       // 16-byte chunks per thread
constexpr int kRegK = 256 * 8 * kRegChunks;         // 8192 values

template <bool kInRegs>
__global__ void __launch_bounds__(256) act_quant_kernel(const uint16_t* __restrict__ x,
                                                        int64_t K, int8_t* __restrict__ x8,
                                                        float* __restrict__ s_x) {
    const int64_t m = blockIdx.x;
    const uint16_t* row = x + m * K;
    int8_t* out = x8 + act_row_offset(m, K);
    // pass 1: absmax. For finite fp16, |x| ordering equals the ordering of the
    // magnitude bits, so the max is taken on (bits & 0x7fff).
    uint4 v[kRegChunks];
    uint32_t mbits = 0;
    if (kInRegs) {
#pragma unroll
        for (int u = 0; u < kRegChunks; ++u) {
            const int64_t k = (int64_t(u) * 256 + threadIdx.x) * 8;
            v[u] = k < K ? *reinterpret_cast<const uint4*>(row + k) : uint4{0, 0, 0, 0};
        }
#pragma unroll
        for (int u = 0; u < kRegChunks; ++u) {
            const uint32_t w[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
            for (int i = 0; i < 4; ++i)
                mbits = max(mbits, max(w[i] & 0x7fffu, (w[i] >> 16) & 0x7fffu));
        }
    } else {
        for (int64_t k = int64_t(threadIdx.x) * 8; k < K; k += 256 * 8) {
            const uint4 t = *reinterpret_cast<const uint4*>(row + k);
            const uint32_t w[4] = {t.x, t.y, t.z, t.w};
#pragma unroll
            for (int i = 0; i < 4; ++i)
                mbits = max(mbits, max(w[i] & 0x7fffu, (w[i] >> 16) & 0x7fffu));
        }
    }
    for (int off = 32; off > 0; off >>= 1) mbits = max(mbits, uint32_t(__shfl_xor(int(mbits), off, 64)));
    __shared__ uint32_t part[4];
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = mbits;
    __syncthreads();
    mbits = max(max(part[0], part[1]), max(part[2], part[3]));
    const float a = h2f(uint16_t(mbits));
    const float inv = a > 0.0f ? float(kActMax) / a : 0.0f;   // correctly rounded fp32
    if (threadIdx.x == 0) s_x[m] = a > 0.0f ? a / float(kActMax) : 0.0f;
    // pass 2: codes
    auto emit = [&](const uint4 t, int64_t k) {
        uint2 o;
        o.x = quant_pair(t.x, inv) | (quant_pair(t.y, inv) << 16);
        o.y = quant_pair(t.z, inv) | (quant_pair(t.w, inv) << 16);
        *reinterpret_cast<uint2*>(out + (k >> 4) * kActUnit + (k & 15)) = o;
    };
    if (kInRegs) {
#pragma unroll
        for (int u = 0; u < kRegChunks; ++u) {
            const int64_t k = (int64_t(u) * 256 + threadIdx.x) * 8;
            if (k < K) emit(v[u], k);
        }
    } else {
        for (int64_t k = int64_t(threadIdx.x) * 8; k < K; k += 256 * 8)
            emit(*reinterpret_cast<const uint4*>(row + k), k);
    }
}

}  // namespace

hipError_t launch_quantize_act(const uint16_t* x, int64_t M, int64_t K, int8_t* x8, float* s_x,
                               hipStream_t stream) {
    if (K <= kRegK)
        return launch_kernel(act_quant_kernel<true>, dim3(unsigned(M)), dim3(256), 0, stream, x, K,
                             x8, s_x);
    return launch_kernel(act_quant_kernel<false>, dim3(unsigned(M)), dim3(256), 0, stream, x, K,
                         x8, s_x);
}

}  // namespace qoq
