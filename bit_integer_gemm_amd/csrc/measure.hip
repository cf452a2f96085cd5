// Streaming-read reference kernel (measurement only; not part of the GEMM).
#include "qoq_measure.h"
#include "qoq_internal.hpp"

namespace {

// Thread t of a grid of G threads reads the 16-byte words t, t + G, ...;
// four independent loads per iteration keep 64 bytes in flight per thread.
__global__ void __launch_bounds__(256) stream_read_kernel(const uint4* __restrict__ p, int64_t n,
                                                          uint32_t* __restrict__ sink) {
    const int64_t stride = int64_t(gridDim.x) * 256;
    int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
    uint4 a{0, 0, 0, 0}, b{0, 0, 0, 0}, c{0, 0, 0, 0}, d{0, 0, 0, 0};
    for (; i + 3 * stride < n; i += 4 * stride) {
        const uint4 u0 = p[i], u1 = p[i + stride], u2 = p[i + 2 * stride], u3 = p[i + 3 * stride];
        a.x ^= u0.x; a.y ^= u0.y; a.z ^= u0.z; a.w ^= u0.w;
        b.x ^= u1.x; b.y ^= u1.y; b.z ^= u1.z; b.w ^= u1.w;
        c.x ^= u2.x; c.y ^= u2.y; c.z ^= u2.z; c.w ^= u2.w;
        d.x ^= u3.x; d.y ^= u3.y; d.z ^= u3.z; d.w ^= u3.w;
    }
    for (; i < n; i += stride) {
        const uint4 u = p[i];
        a.x ^= u.x; a.y ^= u.y; a.z ^= u.z; a.w ^= u.w;
    }
    const uint32_t v = a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w ^ c.x ^ c.y ^ c.z ^ c.w ^
                       d.x ^ d.y ^ d.z ^ d.w;
    if (v == 0x9E3779B9u) *sink = v;
}

}  // namespace

extern "C" qoq_status qoq_stream_read(const void* buf, size_t bytes, int32_t workgroups,
                                      uint32_t* sink, void* stream) {
    if (buf == nullptr || sink == nullptr) return QOQ_ERR_NULL;
    if (bytes == 0 || bytes % 16 != 0 || bytes > (size_t(1) << 40) || workgroups < 0 ||
        workgroups > 65536)
        return QOQ_ERR_SHAPE;
    if ((reinterpret_cast<uintptr_t>(buf) & 15u) != 0) return QOQ_ERR_ALIGN;
    const unsigned grid = workgroups == 0 ? 1024u : unsigned(workgroups);
    const hipError_t e = qoq::launch_kernel(stream_read_kernel, dim3(grid), dim3(256), 0,
                                            static_cast<hipStream_t>(stream),
                                            static_cast<const uint4*>(buf), int64_t(bytes / 16), sink);
    return e == hipSuccess ? QOQ_OK : QOQ_ERR_HIP;
}
