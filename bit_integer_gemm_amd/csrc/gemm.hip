// W4A8 GEMM main loop and epilogue for gfx950.
//
// Main loop (pages: velog notes on QServe, "Methods / 1) Algorithm: QoQ"
// and "Methods / 2) System: QServe"; "Part5 LLM部署技术" section 3):
//   - the packed UINT4 codes of a 16-channel x 128-input block arrive with
//     one 16-byte load per lane, already in MFMA operand order;
//   - each 32-bit word holds 8 codes; `& 0x0F0F0F0F` and `>> 4 & 0x0F0F0F0F`
//     give two words of 4 byte-lanes, and one packed 16-bit multiply-add per
//     word computes q4*s2 + (128 - z*s2) for 4 weights at once: the product
//     q4*s2 <= 225 and the sum w8 + 128 in [7, 249] never carry out of a
//     byte, which is what the protective range guarantees ("subtraction
//     after multiplication": the zero enters pre-multiplied by the scale);
//   - XOR 0x80 per byte turns w8 + 128 into the two's-complement INT8 w8;
//   - v_mfma_i32_16x16x64_i8 accumulates INT32 over the whole K range:
//     no partial sum is ever converted or scaled, so the accumulator is exact
//     and independent of tiling and of the split of K.
// Epilogue: y = fp16(acc * (s_x[m] * s1[n])), once per output.
#include "qoq_internal.hpp"

#include <hip/hip_fp16.h>

namespace qoq {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef unsigned short us2 __attribute__((ext_vector_type(2)));

// Four UINT4 codes (one per byte) -> four INT8 weights, register-parallel.
__device__ __forceinline__ int dequant4(uint32_t codes, uint32_t mul2, uint32_t add2) {
    const us2 r = __builtin_bit_cast(us2, codes) * __builtin_bit_cast(us2, mul2) +
                  __builtin_bit_cast(us2, add2);
    return int(__builtin_bit_cast(uint32_t, r) ^ 0x80808080u);
}

__device__ __forceinline__ float h2f(uint16_t b) { return __half2float(__ushort_as_half(b)); }

__device__ __forceinline__ uint16_t epilogue_value(int32_t acc, float sx, float sw) {
    const float v = float(acc) * (sx * sw);
    return __half_as_ushort(__float2half_rn(v));
}

// Streaming tile family: a workgroup of 4 waves; wave w owns CB column
// blocks (16 channels each) and MT row tiles (16 tokens each), over the
// groups [g0, g1) of its split of K.
template <int MT, int CB>
__global__ void __launch_bounds__(256) gemm_stream_kernel(
    const int8_t* __restrict__ x8, const float* __restrict__ s_x, int M, int K,
    const uint8_t* __restrict__ nib, const uint8_t* __restrict__ rec, int ng8,
    const uint16_t* __restrict__ s1, int N, uint16_t* __restrict__ y,
    int32_t* __restrict__ acc_debug, int32_t* __restrict__ ws_acc,
    uint32_t* __restrict__ ws_cnt, int gps) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int c = lane & 15;
    const int h = lane >> 4;
    const int ng = K >> 7;
    const int nbt = N >> 4;
    const int nb_first = (blockIdx.x * 4 + wave) * CB;
    const int m0 = blockIdx.y * 16 * MT;
    const int g0 = blockIdx.z * gps;
    const int g1 = min(ng, g0 + gps);

    int nbc[CB];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) nbc[cb] = min(nb_first + cb, nbt - 1);

    const int8_t* arow[MT];
    bool aval[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        const int r = m0 + 16 * mt + c;
        aval[mt] = r < M;
        arow[mt] = x8 + int64_t(aval[mt] ? r : 0) * K + 16 * h;
    }

    v4i acc[MT][CB];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) acc[mt][cb] = v4i{0, 0, 0, 0};

    for (int g = g0; g < g1; ++g) {
        uint4 q[CB];
        uint32_t sb[CB];
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) {
            q[cb] = *reinterpret_cast<const uint4*>(
                nib + (int64_t(nbc[cb]) * ng + g) * kBlockBytes + lane * 16);
            sb[cb] = *reinterpret_cast<const uint16_t*>(
                rec + ((int64_t(nbc[cb]) * ng8 + (g >> 3)) * kBlockCols + c) * (kRecChunk * 2) +
                (g & 7) * 2);
        }
        v4i a[MT][2];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int s = 0; s < 2; ++s)
                a[mt][s] = aval[mt] ? *reinterpret_cast<const v4i*>(arow[mt] + g * kGroup + 64 * s)
                                    : v4i{0, 0, 0, 0};
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) {
            const uint32_t s2 = sb[cb] & 0xffu;
            const uint32_t bias = sb[cb] >> 8;
            const uint32_t mul2 = s2 | (s2 << 16);
            const uint32_t add2 = bias * 0x01010101u;
            const uint32_t w[4] = {q[cb].x, q[cb].y, q[cb].z, q[cb].w};
            v4i b0, b1;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                b0[i] = dequant4(w[i] & 0x0F0F0F0Fu, mul2, add2);
                b1[i] = dequant4((w[i] >> 4) & 0x0F0F0F0Fu, mul2, add2);
            }
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                acc[mt][cb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[mt][0], b0, acc[mt][cb], 0, 0, 0);
                acc[mt][cb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[mt][1], b1, acc[mt][cb], 0, 0, 0);
            }
        }
    }

    // Output element of acc[mt][cb][r]: token m0 + 16mt + 4h + r, channel
    // 16(nb_first + cb) + c (the 16x16 MFMA result layout).
    if (gridDim.z == 1) {
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) {
            if (nb_first + cb >= nbt) continue;
            const int n = 16 * (nb_first + cb) + c;
            const float sw = h2f(s1[n]);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int m = m0 + 16 * mt + 4 * h + r;
                    if (m >= M) continue;
                    const int32_t v = acc[mt][cb][r];
                    if (acc_debug) acc_debug[int64_t(m) * N + n] = v;
                    y[int64_t(m) * N + n] = epilogue_value(v, s_x[m], sw);
                }
        }
        return;
    }

    // Split K: integer partial sums are combined with atomics (exact, order
    // independent); the last workgroup of the tile to arrive runs the
    // epilogue and returns the workspace to zero for the next call.
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
        if (nb_first + cb >= nbt) continue;
        const int n = 16 * (nb_first + cb) + c;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int m = m0 + 16 * mt + 4 * h + r;
                if (m < M) atomicAdd(ws_acc + int64_t(m) * N + n, acc[mt][cb][r]);
            }
    }
    __threadfence();
    __syncthreads();
    __shared__ int is_last;
    const int tile = blockIdx.y * gridDim.x + blockIdx.x;
    if (threadIdx.x == 0) is_last = atomicAdd(ws_cnt + tile, 1u) == gridDim.z - 1;
    __syncthreads();
    if (!is_last) return;
    __threadfence();
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
        if (nb_first + cb >= nbt) continue;
        const int n = 16 * (nb_first + cb) + c;
        const float sw = h2f(s1[n]);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int m = m0 + 16 * mt + 4 * h + r;
                if (m >= M) continue;
                int32_t* p = ws_acc + int64_t(m) * N + n;
                const int32_t v = __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                if (acc_debug) acc_debug[int64_t(m) * N + n] = v;
                y[int64_t(m) * N + n] = epilogue_value(v, s_x[m], sw);
                *p = 0;
            }
    }
    if (threadIdx.x == 0) ws_cnt[tile] = 0;
}

template <int MT, int CB>
hipError_t launch_stream(const GemmPlan& p, const int8_t* x8, const float* s_x, int M, int K,
                         const uint8_t* nib, const uint8_t* rec, int ng8, const uint16_t* s1,
                         int N, uint16_t* y, int32_t* acc_debug, int32_t* ws_acc,
                         uint32_t* ws_cnt, hipStream_t stream) {
    return launch_kernel(gemm_stream_kernel<MT, CB>, dim3(p.grid_x, p.grid_y, p.splits),
                         dim3(256), 0, stream, x8, s_x, M, K, nib, rec, ng8, s1, N, y, acc_debug,
                         ws_acc, ws_cnt, p.groups_per_split);
}

int64_t round_up(int64_t v, int64_t a) { return (v + a - 1) / a * a; }

}  // namespace

GemmPlan plan_gemm(int64_t M, int64_t N, int64_t K) {
    GemmPlan p{};
    p.kind = 0;
    p.mt = M <= 16 ? 1 : (M <= 32 ? 2 : 4);
    p.cb = 2;
    const int64_t nbt = N / kBlockCols;
    const int64_t ng = K / kGroup;
    p.grid_x = int((nbt + 4 * p.cb - 1) / (4 * p.cb));
    p.grid_y = int((M + 16 * p.mt - 1) / (16 * p.mt));
    const int64_t base = int64_t(p.grid_x) * p.grid_y;
    int64_t splits = 1;
    if (base < 512) splits = std::min<int64_t>(ng, (1024 + base - 1) / base);
    if (splits < 1) splits = 1;
    const int64_t gps = (ng + splits - 1) / splits;
    p.groups_per_split = int(gps);
    p.splits = int((ng + gps - 1) / gps);
    if (p.splits > 1) {
        p.ws_acc_bytes = round_up(M * N * 4, 256);
        p.ws_cnt_bytes = round_up(base * 4, 256);
        p.ws_bytes = p.ws_acc_bytes + p.ws_cnt_bytes;
    }
    return p;
}

hipError_t launch_gemm(const GemmPlan& p, const int8_t* x8, const float* s_x, int64_t M, int64_t K,
                       const uint8_t* packed, const uint16_t* s1, int64_t N, uint16_t* y,
                       int32_t* acc_debug, void* workspace, hipStream_t stream) {
    const PackedLayout L = packed_layout(N, K);
    const uint8_t* nib = packed;
    const uint8_t* rec = packed + L.rec_offset;
    int32_t* ws_acc = nullptr;
    uint32_t* ws_cnt = nullptr;
    if (p.splits > 1) {
        ws_acc = static_cast<int32_t*>(workspace);
        ws_cnt = reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(workspace) + p.ws_acc_bytes);
    }
    const int m = int(M), k = int(K), n = int(N), g8 = int(L.ng8);
    switch (p.mt) {
        case 1:
            return launch_stream<1, 2>(p, x8, s_x, m, k, nib, rec, g8, s1, n, y, acc_debug, ws_acc,
                                       ws_cnt, stream);
        case 2:
            return launch_stream<2, 2>(p, x8, s_x, m, k, nib, rec, g8, s1, n, y, acc_debug, ws_acc,
                                       ws_cnt, stream);
        default:
            return launch_stream<4, 2>(p, x8, s_x, m, k, nib, rec, g8, s1, n, y, acc_debug, ws_acc,
                                       ws_cnt, stream);
    }
}

}  // namespace qoq
