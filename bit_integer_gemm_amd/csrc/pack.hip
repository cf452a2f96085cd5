// Progressive group quantization of the weights and compute-aware packing.
//
// Level 1 (per output channel, symmetric INT8 inside the protective range,
// FP16 scale) and level 2 (per group of 128 inputs, UINT4 codes with an
// integer scale and a UINT4 zero) follow "QServe: W4A8KV4 Quantization and
// System Co-design for Efficient LLM Serving" (velog notes), section
// "Methods / 1) Algorithm: QoQ", with the protective range of "Methods / 2)
// System: QServe". The reordering into MFMA operand order is that section's
// compute-aware weight reordering, derived here for gfx950's
// v_mfma_i32_16x16x64_i8 (layout in qoq_internal.hpp).
#include "qoq_internal.hpp"

#include <hip/hip_fp16.h>

namespace qoq {
namespace {

__device__ __forceinline__ float half_bits_to_float(uint16_t b) {
    return __half2float(__ushort_as_half(b));
}

// Round-half-to-even of the exact rational num/den, den > 0.
__device__ __forceinline__ int rne_div(int num, int den) {
    int q = num / den;
    int r = num - q * den;
    if (r < 0) { q -= 1; r += den; }      // floor division
    int twice = 2 * r;
    if (twice > den || (twice == den && (q & 1))) q += 1;
    return q;
}

// Level 1, scale: one workgroup per output channel; absmax is exact in any
// reduction order.
__global__ void __launch_bounds__(256) level1_scale_kernel(const float* __restrict__ W,
                                                           int64_t K, uint16_t* __restrict__ s1) {
    const int64_t n = blockIdx.x;
    const float* row = W + n * K;
    float m = 0.0f;
    for (int64_t k = int64_t(threadIdx.x) * 4; k < K; k += 256 * 4) {
        const float4 v = *reinterpret_cast<const float4*>(row + k);
        m = fmaxf(m, fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
    }
    for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
    __shared__ float part[4];
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = m;
    __syncthreads();
    if (threadIdx.x == 0) {
        m = fmaxf(fmaxf(part[0], part[1]), fmaxf(part[2], part[3]));
        const float s = m / float(kProtect);           // correctly rounded fp32
        s1[n] = __half_as_ushort(__float2half_rn(s));   // round to nearest even
    }
}

// Level 2 + packing: one wave per (channel, group). Lane i handles inputs
// 128g + i and 128g + 64 + i, which are exactly the two nibbles of byte
// (i & 15) of GEMM lane (c + 16 * (i >> 4)) in the packed block.
template <bool kFromCanonical>
__global__ void __launch_bounds__(256) level2_pack_kernel(
    const float* __restrict__ W, const uint16_t* __restrict__ s1, int64_t N, int64_t K,
    uint8_t* __restrict__ nib, uint8_t* __restrict__ rec, int64_t ng8,
    uint8_t* __restrict__ cq4, int8_t* __restrict__ cs2, uint8_t* __restrict__ cz) {
    const int lane = threadIdx.x & 63;
    const int64_t wave = int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6);
    const int64_t ng = K / kGroup;
    if (wave >= N * ng) return;
    const int c = int(wave & 15);
    const int64_t rest = wave >> 4;
    const int64_t g = rest % ng;
    const int64_t nb = rest / ng;
    const int64_t n = nb * kBlockCols + c;
    const int64_t k0 = n * K + g * kGroup + lane;

    int q0, q1, s2, z;
    if (!kFromCanonical) {
        const float sc = half_bits_to_float(s1[n]);
        int c0 = 0, c1 = 0;
        if (sc != 0.0f) {
            const float r0 = rintf(W[k0] / sc);
            const float r1 = rintf(W[k0 + 64] / sc);
            c0 = int(fminf(fmaxf(r0, -float(kProtect)), float(kProtect)));
            c1 = int(fminf(fmaxf(r1, -float(kProtect)), float(kProtect)));
        }
        int lo = min(0, min(c0, c1));
        int hi = max(0, max(c0, c1));
        for (int off = 32; off > 0; off >>= 1) {
            lo = min(lo, __shfl_xor(lo, off, 64));
            hi = max(hi, __shfl_xor(hi, off, 64));
        }
        s2 = max(1, (hi - lo + 14) / 15);       // ceil((hi - lo) / 15), hi - lo >= 0
        z = rne_div(-lo, s2);
        q0 = min(15, max(0, rne_div(c0, s2) + z));
        q1 = min(15, max(0, rne_div(c1, s2) + z));
        if (cq4 != nullptr) {
            cq4[k0] = uint8_t(q0);
            cq4[k0 + 64] = uint8_t(q1);
            if (lane == 0) {
                cs2[n * ng + g] = int8_t(s2);
                cz[n * ng + g] = uint8_t(z);
            }
        }
    } else {
        q0 = cq4[k0] & 15;
        q1 = cq4[k0 + 64] & 15;
        s2 = int(cs2[n * ng + g]) & 0xff;
        z = cz[n * ng + g] & 15;
    }
    const int64_t block = nb * ng + g;
    nib[block * kBlockBytes + 16 * (c + 16 * (lane >> 4)) + (lane & 15)] =
        uint8_t(q0 | (q1 << 4));
    if (lane < kRecChunk) {
        // lane 0 writes this group's record; on the last group, lanes 1..7
        // zero the padding entries of the last chunk.
        const int64_t gi = g + lane;
        const bool mine = lane == 0;
        const bool pad = (g == ng - 1) && lane > 0 && gi < ng8 * kRecChunk;
        if (mine || pad) {
            const int64_t off = ((nb * ng8 + gi / kRecChunk) * kBlockCols + c) * (kRecChunk * 2) +
                                (gi % kRecChunk) * 2;
            rec[off] = mine ? uint8_t(s2) : uint8_t(0);
            rec[off + 1] = mine ? uint8_t(128 - z * s2) : uint8_t(0);
        }
    }
}

}  // namespace

hipError_t launch_pack(const float* W, int64_t N, int64_t K, uint8_t* packed, uint16_t* s1,
                       uint8_t* cq4, int8_t* cs2, uint8_t* cz, bool from_canonical,
                       hipStream_t stream) {
    const PackedLayout L = packed_layout(N, K);
    uint8_t* nib = packed;
    uint8_t* rec = packed + L.rec_offset;
    const int64_t waves = N * L.ng;
    const dim3 grid(unsigned((waves + 3) / 4));
    if (!from_canonical) {
        hipError_t e = launch_kernel(level1_scale_kernel, dim3(unsigned(N)), dim3(256), 0, stream,
                                     W, K, s1);
        if (e != hipSuccess) return e;
        return launch_kernel(level2_pack_kernel<false>, grid, dim3(256), 0, stream, W,
                             (const uint16_t*)s1, N, K, nib, rec, L.ng8, cq4, cs2, cz);
    }
    return launch_kernel(level2_pack_kernel<true>, grid, dim3(256), 0, stream, W,
                         (const uint16_t*)s1, N, K, nib, rec, L.ng8, cq4, cs2, cz);
}

}  // namespace qoq
