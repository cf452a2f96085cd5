// Comparison GEMMs for the dequantization-overhead argument of the pages:
// W8A8 with per-channel INT8 weights (no dequantization in the main loop)
// and per-group W4A4 (both operands INT4 with a scale per group; each
// group's INT32 partial sum is converted and scaled inside the main loop).
// Pages: "QServe: W4A8KV4 Quantization and System Co-design for Efficient LLM
// Serving" (velog notes), sections "문제 정의" and "Background"; the QServe
// abstract.
//
// Both run on the skeleton of the W4A8 32x32x32 tile kernel (same tile
// order, LDS staging of activations, register rings, epilogue), so that
// measured differences come from the weight format and where it is
// dequantized, not from the tiling. Layouts:
//   W8A8 weights   [N/16][K/128][2 halves][64 lanes][16 bytes]: the 2 KiB
//                  block (nb, g) holds, for lane l = c + 16h and half s,
//                  the int8 codes of channel 16nb + c, inputs
//                  128g + 64s + 16h .. +15 (the v_mfma_i32_16x16x64_i8 B
//                  operand order; a 32x32x32 step st of lane (j, q) is the
//                  16 bytes at (c + 16q) * 16 + 512 st).
//   W8A8 act       QoQ's x8 tile layout and s_x (qoq_quantize_act).
//   W4A4 weights   QoQ's nibble layout with u = code + 8 in each nibble and
//                  the fp16 group scale in each group's 2-byte record slot.
//   W4A16 weights  QoQ's nibble layout with u = q (UINT4 code), then two
//                  record regions of QoQ's record shape: the fp16 group
//                  scales, then the group zeros (uint16).
//   W4A16 act      fp16 x, row-major [M, K] (no quantization).
//   W4A4 act       x4 tile layout: row m, inputs 16j .. 16j + 15 are 8 bytes
//                  at ((m / 16) * (K / 16) + j) * 128 + (m % 16) * 8, byte b
//                  holding u(16j + b) | u(16j + 8 + b) << 4 with u = code + 8;
//                  then, 256-byte aligned, the fp32 group scales s_a[g][Mp]
//                  (Mp = M rounded up to 128, so every tile's rows exist;
//                  rows past M are 0).
#include "qoq_internal.hpp"
#include "kernel_common.hpp"

#include <cstdio>
#include <cstdlib>
#include <string>

namespace qoq {
namespace {

constexpr int kW8Max = 127;
constexpr int kInt4Max = 7;
constexpr int kW8BlockBytes = 2048;
constexpr int kFmtW8 = 1;
constexpr int kFmtW4A4 = 2;
constexpr int kFmtW4A16 = 3;

// ---------------------------------------------------------------------------
// weight and activation quantizers
// ---------------------------------------------------------------------------

// W8A8 channel scale: one workgroup per output channel, s = fp16(absmax/127).
__global__ void __launch_bounds__(256) w8_scale_kernel(const float* __restrict__ W, int64_t K,
                                                       uint16_t* __restrict__ s) {
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
        s[n] = __half_as_ushort(__float2half_rn(m / float(kW8Max)));
    }
}

// W8A8 codes and packing: one thread per 16-byte lane chunk of the layout.
__global__ void __launch_bounds__(256) w8_pack_kernel(const float* __restrict__ W,
                                                      const uint16_t* __restrict__ s, int64_t N,
                                                      int64_t K, uint8_t* __restrict__ packed) {
    const int64_t t = int64_t(blockIdx.x) * 256 + threadIdx.x;
    if (t >= N * K / 16) return;
    const int64_t ng = K / kGroup;
    const int lane = int(t & 63);
    const int half = int((t >> 6) & 1);
    const int64_t blk = t >> 7;
    const int64_t g = blk % ng;
    const int64_t nb = blk / ng;
    const int c = lane & 15;
    const int h = lane >> 4;
    const int64_t n = nb * kBlockCols + c;
    const float sc = h2f(s[n]);
    const float* src = W + n * K + g * kGroup + 64 * half + 16 * h;
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float4 v = *reinterpret_cast<const float4*>(src + 4 * i);
        const float f[4] = {v.x, v.y, v.z, v.w};
        uint32_t word = 0;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            int code = 0;
            if (sc != 0.0f)
                code = int(fminf(fmaxf(rintf(f[b] / sc), -float(kW8Max)), float(kW8Max)));
            word |= (uint32_t(code) & 0xffu) << (8 * b);
        }
        w[i] = word;
    }
    *reinterpret_cast<uint4*>(packed + t * 16) = uint4{w[0], w[1], w[2], w[3]};
}

// W4A4 weights: one wave per (channel, group); lane i handles inputs
// 128g + i and 128g + 64 + i (the two nibbles of one byte of the layout).
__global__ void __launch_bounds__(256) w4_pack_kernel(const float* __restrict__ W, int64_t N,
                                                      int64_t K, uint8_t* __restrict__ nib,
                                                      uint8_t* __restrict__ rec, int64_t ng8) {
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
    const float w0 = W[k0], w1 = W[k0 + 64];
    float a = fmaxf(fabsf(w0), fabsf(w1));
    for (int off = 32; off > 0; off >>= 1) a = fmaxf(a, __shfl_xor(a, off, 64));
    const uint16_t sbits = __half_as_ushort(__float2half_rn(a / float(kInt4Max)));
    const float sc = h2f(sbits);
    int c0 = 0, c1 = 0;
    if (sc != 0.0f) {
        c0 = int(fminf(fmaxf(rintf(w0 / sc), -float(kInt4Max)), float(kInt4Max)));
        c1 = int(fminf(fmaxf(rintf(w1 / sc), -float(kInt4Max)), float(kInt4Max)));
    }
    const int64_t block = nb * ng + g;
    nib[block * kBlockBytes + 16 * (c + 16 * (lane >> 4)) + (lane & 15)] =
        uint8_t((c0 + 8) | ((c1 + 8) << 4));
    if (lane < kRecChunk) {
        const int64_t gi = g + lane;
        const bool mine = lane == 0;
        const bool pad = (g == ng - 1) && lane > 0 && gi < ng8 * kRecChunk;
        if (mine || pad) {
            const int64_t off = ((nb * ng8 + gi / kRecChunk) * kBlockCols + c) * (kRecChunk * 2) +
                                (gi % kRecChunk) * 2;
            rec[off] = mine ? uint8_t(sbits & 0xff) : uint8_t(0);
            rec[off + 1] = mine ? uint8_t(sbits >> 8) : uint8_t(0);
        }
    }
}

// W4A4 activations: one workgroup per token row (rows past M write zero
// scales); eight consecutive threads share a group of 128 inputs, 16 each.
__global__ void __launch_bounds__(256) a4_quant_kernel(const uint16_t* __restrict__ x, int M,
                                                       int64_t K, int Mp, uint8_t* __restrict__ x4,
                                                       float* __restrict__ s_a) {
    const int m = blockIdx.x;
    const int64_t ng = K / kGroup;
    if (m >= M) {
        for (int64_t g = threadIdx.x; g < ng; g += 256) s_a[g * Mp + m] = 0.0f;
        return;
    }
    const uint16_t* row = x + int64_t(m) * K;
    uint8_t* out = x4 + int64_t(m >> 4) * (K >> 4) * 128 + (m & 15) * 8;
    for (int64_t k0 = int64_t(threadIdx.x) * 16; k0 < K; k0 += 256 * 16) {
        // all eight threads of a group take this branch together (K % 128 == 0)
        const uint4 v0 = *reinterpret_cast<const uint4*>(row + k0);
        const uint4 v1 = *reinterpret_cast<const uint4*>(row + k0 + 8);
        const uint32_t w[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
        uint32_t mb = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) mb = max(mb, max(w[i] & 0x7fffu, (w[i] >> 16) & 0x7fffu));
#pragma unroll
        for (int off = 4; off > 0; off >>= 1) mb = max(mb, uint32_t(__shfl_xor(int(mb), off, 8)));
        const float a = h2f(uint16_t(mb));
        const float inv = a > 0.0f ? float(kInt4Max) / a : 0.0f;
        uint32_t u[16];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
                const float p = rintf(h2f(uint16_t(hf ? w[i] >> 16 : w[i] & 0xffffu)) * inv);
                u[2 * i + hf] = uint32_t(int(fminf(fmaxf(p, -float(kInt4Max)), float(kInt4Max))) + 8);
            }
        }
        uint32_t lo = 0, hi = 0;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            lo |= (u[b] | (u[8 + b] << 4)) << (8 * b);
            hi |= (u[4 + b] | (u[12 + b] << 4)) << (8 * b);
        }
        *reinterpret_cast<uint2*>(out + (k0 >> 4) * 128) = uint2{lo, hi};
        if ((threadIdx.x & 7) == 0) s_a[(k0 >> 7) * Mp + m] = a > 0.0f ? a / float(kInt4Max) : 0.0f;
    }
}

// W4A16 weights: one wave per (channel, group); lane i handles inputs
// 128g + i and 128g + 64 + i. Range including 0, fp16 scale, UINT4 zero.
__global__ void __launch_bounds__(256) w4a16_pack_kernel(const float* __restrict__ W, int64_t N,
                                                         int64_t K, uint8_t* __restrict__ nib,
                                                         uint8_t* __restrict__ srec,
                                                         uint8_t* __restrict__ zrec, int64_t ng8) {
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
    const float w0 = W[k0], w1 = W[k0 + 64];
    float lo = fminf(0.0f, fminf(w0, w1)), hi = fmaxf(0.0f, fmaxf(w0, w1));
    for (int off = 32; off > 0; off >>= 1) {
        lo = fminf(lo, __shfl_xor(lo, off, 64));
        hi = fmaxf(hi, __shfl_xor(hi, off, 64));
    }
    const uint16_t sbits = __half_as_ushort(__float2half_rn((hi - lo) / 15.0f));
    const float sc = h2f(sbits);
    int q0 = 0, q1 = 0, z = 0;
    if (sc != 0.0f) {
        z = int(fminf(fmaxf(rintf(-lo / sc), 0.0f), 15.0f));
        q0 = min(15, max(0, int(rintf(w0 / sc)) + z));
        q1 = min(15, max(0, int(rintf(w1 / sc)) + z));
    }
    const int64_t block = nb * ng + g;
    nib[block * kBlockBytes + 16 * (c + 16 * (lane >> 4)) + (lane & 15)] = uint8_t(q0 | (q1 << 4));
    if (lane < kRecChunk) {
        const int64_t gi = g + lane;
        const bool mine = lane == 0;
        const bool pad = (g == ng - 1) && lane > 0 && gi < ng8 * kRecChunk;
        if (mine || pad) {
            const int64_t off = ((nb * ng8 + gi / kRecChunk) * kBlockCols + c) * (kRecChunk * 2) +
                                (gi % kRecChunk) * 2;
            *reinterpret_cast<uint16_t*>(srec + off) = mine ? sbits : uint16_t(0);
            *reinterpret_cast<uint16_t*>(zrec + off) = mine ? uint16_t(z) : uint16_t(0);
        }
    }
}

// Eight offset-coded nibbles u = code + 8 (one word) -> two words of four
// INT8 codes: low nibbles and high nibbles. u + 120 stays inside a byte
// (<= 135), and xor 0x80 subtracts the 128: byte = u - 8 = code.
__device__ __forceinline__ void unpack_s4(uint32_t w, int& lo, int& hi) {
    lo = int(((w & 0x0F0F0F0Fu) + 0x78787878u) ^ 0x80808080u);
    hi = int((((w >> 4) & 0x0F0F0F0Fu) + 0x78787878u) ^ 0x80808080u);
}

// ---------------------------------------------------------------------------
// the GEMM: 32x32x32 tiles, NW waves side by side along N
// ---------------------------------------------------------------------------
template <int FMT, int MT, int CB, int PB, int MINB, int NW>
__global__ void __launch_bounds__(64 * NW, MINB) gemm_variant_kernel(
    const uint8_t* __restrict__ act, const float* __restrict__ ascale, int M, int Mp, int K,
    const uint8_t* __restrict__ wts, const uint8_t* __restrict__ rec, int ng8,
    const uint16_t* __restrict__ s1, int N, uint16_t* __restrict__ y,
    int32_t* __restrict__ acc_debug) {
    constexpr bool W8 = FMT == kFmtW8;
    constexpr int AF = 4 * MT;
    constexpr int AFW = (AF + NW - 1) / NW;
    constexpr int BQ = W8 ? 4 : 2;                // 16-byte weight loads per tile per group
    static_assert(AF * 2 <= 64, "LDS slots above 64 KiB");
    static_assert(PB == 1 || PB == 2 || PB == 4 || PB == 8, "weight ring depth divides 8");
    constexpr int kSlotsBytes = 2 * AF * 64 * 16;
    constexpr int kStageBytes = NW * 32 * 32 * CB * 2;
    __shared__ v4i lds_raw[(kSlotsBytes > kStageBytes ? kSlotsBytes : kStageBytes) / 16];
    v4i (*As)[AF][64] = reinterpret_cast<v4i (*)[AF][64]>(lds_raw);
    constexpr int BM = 32 * MT, BNB = 2 * CB * NW;
    // W4A4: the tile's token scales of the staged groups (two slots, like A)
    __shared__ __attribute__((aligned(16))) float sa_lds[2][W8 ? 4 : BM];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int j = lane & 31;
    const int q = lane >> 5;
    const int c = lane & 15;
    const int ng = K >> 7;
    const int nbt = N >> 4;
    const int tiles_m = (M + BM - 1) / BM;
    const int tiles_n = (nbt + BNB - 1) / BNB;
    int tm, tn;
    tile_of(blockIdx.x, tiles_m, tiles_n, tm, tn);
    const int m0 = tm * BM;
    const int nbw = tn * BNB + wave * 2 * CB;

    const int act_size = W8 ? int(act_bytes(M, K)) : int(act_bytes(M, K) / 2);
    const __amdgpu_buffer_rsrc_t ra =
        __builtin_amdgcn_make_buffer_rsrc((void*)act, (short)0, act_size, 0x00020000);
    const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
        (void*)wts, (short)0, nbt * ng * (W8 ? kW8BlockBytes : kBlockBytes), 0x00020000);
    const __amdgpu_buffer_rsrc_t rr = __builtin_amdgcn_make_buffer_rsrc(
        (void*)rec, (short)0, W8 ? 0 : nbt * ng8 * (kBlockCols * kRecChunk * 2), 0x00020000);
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)ascale, (short)0, W8 ? 0 : ng * Mp * 4, 0x00020000);

    // A fragment f = (32-row tile f / 4, step f % 4); wave w stages
    // fragments w, w + NW, ...; rows past M read the last row.
    int a_lane[AFW], a_soff[AFW];
#pragma unroll
    for (int u = 0; u < AFW; ++u) {
        const int f = min(wave + NW * u, AF - 1);
        const int r = min(m0 + 32 * (f >> 2) + j, M - 1);
        if constexpr (W8) {
            a_lane[u] = int(act_row_offset(r, K)) + kActUnit * q;
            a_soff[u] = 2 * kActUnit * (f & 3);
        } else {
            a_lane[u] = (r >> 4) * 8 * K + (r & 15) * 8 + 128 * q;
            a_soff[u] = 256 * (f & 3);
        }
    }
    auto owns = [&](int u) { return wave + NW * u < AF; };
    int b_lane[CB], r_lane[CB];
#pragma unroll
    for (int t = 0; t < CB; ++t) {
        const int blk = min(nbw + 2 * t + (j >> 4), nbt - 1);
        b_lane[t] = blk * ng * (W8 ? kW8BlockBytes : kBlockBytes) + (c + 16 * q) * 16;
        r_lane[t] = (blk * ng8 * kBlockCols + c) * (kRecChunk * 2);
    }

    v16i acc[MT][CB];      // W8A8: the INT32 result; W4A4: the current group's partial sum
    float accf[W8 ? 1 : MT][W8 ? 1 : CB][16];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int t = 0; t < CB; ++t)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[mt][t][r] = 0;
    if constexpr (!W8) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int t = 0; t < CB; ++t)
#pragma unroll
                for (int r = 0; r < 16; ++r) accf[mt][t][r] = 0.0f;
    }

    v4i ar[AFW];
    uint4 qn[PB][CB][BQ];
    uint32_t wsc[PB][CB];                   // W4A4: fp16 group scale, ring like the weights
    float sa_ld = 0.0f;                     // W4A4, wave 0: one token scale per lane
    // W4A4 token scales of group g (rows m0 .. m0 + BM - 1 < Mp): wave 0
    // fetches one per lane and stages them in LDS with the activations
    auto load_sa = [&](int g) {
        if (wave == 0)
            sa_ld = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                rs, (m0 + min(lane, BM - 1)) * 4, min(g, ng - 1) * Mp * 4, 0));
    };
    auto stage_sa = [&](int slot) {
        if (wave == 0 && lane < BM) sa_lds[slot][lane] = sa_ld;
    };
    auto load_a = [&](int g) {
        g = min(g, ng - 1);
#pragma unroll
        for (int u = 0; u < AFW; ++u) {
            if constexpr (W8) {
                ar[u] = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(
                    ra, a_lane[u], g * kActGroupBytes + a_soff[u], 0));
            } else {
                const auto v = __builtin_amdgcn_raw_buffer_load_b64(ra, a_lane[u], g * 1024 + a_soff[u], 0);
                const uint2 w = __builtin_bit_cast(uint2, v);
                // the held 16 codes, kept packed until staging
                ar[u] = v4i{int(w.x), int(w.y), 0, 0};
            }
        }
    };
    auto stage_a = [&](int slot) {
#pragma unroll
        for (int u = 0; u < AFW; ++u) {
            if (!owns(u)) continue;
            if constexpr (W8) {
                As[slot][wave + NW * u][lane] = ar[u];
            } else {
                int l0, h0, l1, h1;
                unpack_s4(uint32_t(ar[u][0]), l0, h0);
                unpack_s4(uint32_t(ar[u][1]), l1, h1);
                As[slot][wave + NW * u][lane] = v4i{l0, l1, h0, h1};
            }
        }
    };
    auto load_b = [&](int p, int g) {
        g = min(g, ng - 1);
#pragma unroll
        for (int t = 0; t < CB; ++t) {
#pragma unroll
            for (int e = 0; e < BQ; ++e)
                qn[p][t][e] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                    rb, b_lane[t], g * (W8 ? kW8BlockBytes : kBlockBytes) + 512 * e, 0));
            if constexpr (!W8)
                wsc[p][t] = uint32_t(__builtin_amdgcn_raw_buffer_load_b16(
                    rr, r_lane[t], (g >> 3) * (kBlockCols * kRecChunk * 2) + (g & 7) * 2, 0));
        }
    };
    auto step = [&](int i, int u, bool full) {
        if (i + 1 < ng) {
            stage_a((u + 1) & 1);
            if constexpr (!W8) stage_sa((u + 1) & 1);
        }
        load_a(i + 2);
        if constexpr (!W8) load_sa(i + 2);
        v4i bq[CB][4];
        float sw[CB];
#pragma unroll
        for (int t = 0; t < CB; ++t) {
            if constexpr (W8) {
#pragma unroll
                for (int st = 0; st < 4; ++st) bq[t][st] = __builtin_bit_cast(v4i, qn[u % PB][t][st]);
            } else {
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    const uint4 w = qn[u % PB][t][e];
                    const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
                    for (int k = 0; k < 4; ++k) {
                        int lo, hi;
                        unpack_s4(ww[k], lo, hi);
                        bq[t][e][k] = lo;
                        bq[t][e + 2][k] = hi;
                    }
                }
                sw[t] = h2f(uint16_t(wsc[u % PB][t]));
            }
        }
        load_b(u % PB, i + PB);
        if (full || i < ng) {
#pragma unroll
            for (int st = 0; st < 4; ++st)
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    const v4i a = As[u & 1][4 * mt + st][lane];
#pragma unroll
                    for (int t = 0; t < CB; ++t) {
                        if constexpr (W8) {
                            acc[mt][t] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, bq[t][st], acc[mt][t], 0, 0, 0);
                        } else {
                            const v16i zero = {0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};
                            acc[mt][t] = __builtin_amdgcn_mfma_i32_32x32x32_i8(
                                a, bq[t][st], st == 0 ? zero : acc[mt][t], 0, 0, 0);
                        }
                    }
                }
            if constexpr (!W8) {
                // the partial-sum dequantization: every group's INT32 sums are
                // converted and scaled by s_a[m, g] * s_w[n, g] in fp32
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    float4 sa[4];
#pragma unroll
                    for (int k = 0; k < 4; ++k)
                        sa[k] = *reinterpret_cast<const float4*>(&sa_lds[u & 1][32 * mt + 8 * k + 4 * q]);
#pragma unroll
                    for (int t = 0; t < CB; ++t)
#pragma unroll
                        for (int r = 0; r < 16; ++r) {
                            const float4 s4 = sa[r >> 2];
                            const float s = (r & 3) == 0 ? s4.x : (r & 3) == 1 ? s4.y : (r & 3) == 2 ? s4.z : s4.w;
                            accf[mt][t][r] = __builtin_fmaf(float(acc[mt][t][r]), s * sw[t], accf[mt][t][r]);
                        }
                }
            }
        }
        __syncthreads();
    };

    if constexpr (!W8) load_sa(0);
    load_a(0);
#pragma unroll
    for (int p = 0; p < PB; ++p) load_b(p, p);
    stage_a(0);
    if constexpr (!W8) {
        stage_sa(0);
        load_sa(1);
    }
    load_a(1);
    __syncthreads();
    // W8A8 unrolls by 8 like the W4A8 kernel; W4A4 by 2 only: unrolled
    // further, the compiler overlaps the per-group conversions of several
    // groups and runs out of registers
    constexpr int U = W8 ? 8 : 2;
    static_assert(U % PB == 0, "ring depth must divide the unroll");
    int i0 = 0;
    for (; i0 + U <= ng; i0 += U) {
#pragma unroll
        for (int u = 0; u < U; ++u) step(i0 + u, u, true);
    }
    if (i0 < ng) {
#pragma unroll
        for (int u = 0; u < U; ++u) step(i0 + u, u, false);
    }

    // epilogue through LDS (lane (j, q), register r of tile (mt, t) is row
    // 32mt + 8(r/4) + 4q + r%4, column 32t + j of the wave's columns)
    __syncthreads();
    uint16_t* stage = reinterpret_cast<uint16_t*>(lds_raw) + wave * (32 * 32 * CB);
    const int n0w = 16 * nbw;
    float swe[CB];
#pragma unroll
    for (int t = 0; t < CB; ++t) swe[t] = W8 ? h2f(s1[min(n0w + 32 * t + j, N - 1)]) : 0.0f;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        float sxr[16];
#pragma unroll
        for (int r = 0; r < 16; ++r)
            sxr[r] = W8 ? ascale[min(m0 + 32 * mt + 8 * (r >> 2) + 4 * q + (r & 3), M - 1)] : 0.0f;
#pragma unroll
        for (int t = 0; t < CB; ++t)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = 8 * (r >> 2) + 4 * q + (r & 3);
                uint16_t v;
                if constexpr (W8) v = epilogue_value(acc[mt][t][r], sxr[r], swe[t]);
                else v = __half_as_ushort(__float2half_rn(accf[mt][t][r]));
                stage[row * (32 * CB) + 32 * t + j] = v;
            }
        if (W8 && acc_debug) {
#pragma unroll
            for (int t = 0; t < CB; ++t)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int m = m0 + 32 * mt + 8 * (r >> 2) + 4 * q + (r & 3);
                    const int n = n0w + 32 * t + j;
                    if (m < M && n < N) acc_debug[int64_t(m) * N + n] = acc[mt][t][r];
                }
        }
        __syncthreads();
#pragma unroll
        for (int u = 0; u < 2 * CB; ++u) {
            const int kk = lane + 64 * u;
            const int row = kk / (4 * CB);
            const int ch = kk % (4 * CB);
            const int m = m0 + 32 * mt + row;
            const int n = n0w + 8 * ch;
            const uint4 v = *reinterpret_cast<const uint4*>(stage + row * (32 * CB) + 8 * ch);
            if (m < M && n < N) *reinterpret_cast<uint4*>(y + int64_t(m) * N + n) = v;
        }
        __syncthreads();
    }
}

typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

// Eight UINT4 codes, one per byte of the pair (w0, w1), low or high nibble ->
// the eight fp16 weights fp16((q - z) * s) in byte order. 0x6400 | q is the
// fp16 value 1024 + q, so (1024 + q) - (1024 + z) = q - z exactly, and one
// fp16 multiply rounds the product once.
template <bool kHigh>
__device__ __forceinline__ v8h dequant_f16x8(uint32_t w0, uint32_t w1, h2 zz, h2 ss) {
    const uint32_t w[2] = {w0, w1};
    v8h r;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            // bytes 2p, 2p + 1 of w[i] into the two 16-bit halves
            const uint32_t t = __builtin_amdgcn_perm(0u, w[i], p ? 0x0c030c02u : 0x0c010c00u);
            const uint32_t bits = ((kHigh ? t >> 4 : t) & 0x000F000Fu) | 0x64006400u;
            const h2 v = (__builtin_bit_cast(h2, bits) - zz) * ss;
            r[4 * i + 2 * p] = v[0];
            r[4 * i + 2 * p + 1] = v[1];
        }
    }
    return r;
}

// W4A16 GEMM: fp16 activations staged in LDS in v_mfma_f32_32x32x16_f16
// fragment order (lane l: row l % 32, inputs 8 (l / 32) .. +7 of a 16-input
// step), UINT4 weights dequantized to fp16 per step, fp32 accumulation, fp16
// output. Same tile order, rings and epilogue as the integer kernels.
template <int MT, int CB, int PB, int MINB, int NW>
__global__ void __launch_bounds__(64 * NW, MINB) gemm_w4a16_kernel(
    const uint16_t* __restrict__ x, int M, int K, const uint8_t* __restrict__ nib,
    const uint8_t* __restrict__ srec, const uint8_t* __restrict__ zrec, int ng8, int N,
    uint16_t* __restrict__ y) {
    constexpr int AF = 8 * MT;                    // fragments per group (8 steps of 16)
    constexpr int BM = 32 * MT, BNB = 2 * CB * NW;
    constexpr int AL = BM / (4 * NW);             // 1 KiB row loads per wave per group
    static_assert(AL >= 1 && BM % (4 * NW) == 0, "rows per wave");
    static_assert(PB == 1 || PB == 2, "ring depth divides the unroll");
    constexpr int kSlotsBytes = 2 * AF * 64 * 16;
    constexpr int kStageBytes = NW * 32 * 32 * CB * 2;
    __shared__ v4i lds_raw[(kSlotsBytes > kStageBytes ? kSlotsBytes : kStageBytes) / 16];
    v4i (*As)[AF][64] = reinterpret_cast<v4i (*)[AF][64]>(lds_raw);
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int j = lane & 31;
    const int q = lane >> 5;
    const int c = lane & 15;
    const int ng = K >> 7;
    const int nbt = N >> 4;
    const int tiles_m = (M + BM - 1) / BM;
    const int tiles_n = (nbt + BNB - 1) / BNB;
    int tm, tn;
    tile_of(blockIdx.x, tiles_m, tiles_n, tm, tn);
    const int m0 = tm * BM;
    const int nbw = tn * BNB + wave * 2 * CB;

    const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
        (void*)x, (short)0, M * K * 2, 0x00020000);
    const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
        (void*)nib, (short)0, nbt * ng * kBlockBytes, 0x00020000);
    const int rec_bytes = nbt * ng8 * (kBlockCols * kRecChunk * 2);
    const __amdgpu_buffer_rsrc_t rsr = __builtin_amdgcn_make_buffer_rsrc(
        (void*)srec, (short)0, rec_bytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t rzr = __builtin_amdgcn_make_buffer_rsrc(
        (void*)zrec, (short)0, rec_bytes, 0x00020000);

    // A staging: load u of this wave covers tile rows 4 (wave + NW u) + l / 16,
    // bytes 16 (l % 16) of the row's 256-byte group chunk (inputs 8 (l % 16)
    // ..), which is lane (row % 32) + 32 (l % 2) of fragment
    // (row / 32, (l % 16) / 2). Rows past M read the last row.
    int a_lane[AL], a_dst[AL];
#pragma unroll
    for (int u = 0; u < AL; ++u) {
        const int row = 4 * (wave + NW * u) + (lane >> 4);
        a_lane[u] = min(m0 + row, M - 1) * K * 2 + 16 * (lane & 15);
        a_dst[u] = ((row >> 5) * 8 + ((lane & 15) >> 1)) * 64 + (row & 31) + 32 * (lane & 1);
    }
    int b_lane[CB], r_lane[CB];
#pragma unroll
    for (int t = 0; t < CB; ++t) {
        const int blk = min(nbw + 2 * t + (j >> 4), nbt - 1);
        b_lane[t] = blk * ng * kBlockBytes + c * 16 + 8 * q;
        r_lane[t] = (blk * ng8 * kBlockCols + c) * (kRecChunk * 2);
    }

    v16f acc[MT][CB];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int t = 0; t < CB; ++t)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[mt][t][r] = 0.0f;

    v4i ar[AL];
    uint2 qn[PB][CB][4];        // per 32-column tile: block lanes c + 16h, 8 bytes each
    uint32_t sz[PB][CB][2];     // fp16 scale bits, zero
    auto load_a = [&](int g) {
        g = min(g, ng - 1);
#pragma unroll
        for (int u = 0; u < AL; ++u)
            ar[u] = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(ra, a_lane[u], g * 256, 0));
    };
    auto stage_a = [&](int slot) {
        v4i* base = &As[slot][0][0];
#pragma unroll
        for (int u = 0; u < AL; ++u) base[a_dst[u]] = ar[u];
    };
    auto load_b = [&](int p, int g) {
        g = min(g, ng - 1);
#pragma unroll
        for (int t = 0; t < CB; ++t) {
#pragma unroll
            for (int h = 0; h < 4; ++h)
                qn[p][t][h] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(
                    rb, b_lane[t], g * kBlockBytes + 256 * h, 0));
            const int roff = (g >> 3) * (kBlockCols * kRecChunk * 2) + (g & 7) * 2;
            sz[p][t][0] = uint32_t(__builtin_amdgcn_raw_buffer_load_b16(rsr, r_lane[t], roff, 0));
            sz[p][t][1] = uint32_t(__builtin_amdgcn_raw_buffer_load_b16(rzr, r_lane[t], roff, 0));
        }
    };
    auto step = [&](int i, int u, bool full) {
        if (i + 1 < ng) stage_a((u + 1) & 1);
        load_a(i + 2);
        uint2 bw[CB][4];
        h2 zz[CB], ss[CB];
#pragma unroll
        for (int t = 0; t < CB; ++t) {
#pragma unroll
            for (int h = 0; h < 4; ++h) bw[t][h] = qn[u % PB][t][h];
            const _Float16 s16 = __builtin_bit_cast(_Float16, uint16_t(sz[u % PB][t][0]));
            const _Float16 z16 = __builtin_bit_cast(_Float16, uint16_t(0x6400u | sz[u % PB][t][1]));
            ss[t] = h2{s16, s16};
            zz[t] = h2{z16, z16};
        }
        load_b(u % PB, i + PB);
        if (full || i < ng) {
#pragma unroll
            for (int st = 0; st < 8; ++st) {
                v8h b[CB];
#pragma unroll
                for (int t = 0; t < CB; ++t)
                    b[t] = st < 4 ? dequant_f16x8<false>(bw[t][st & 3].x, bw[t][st & 3].y, zz[t], ss[t])
                                  : dequant_f16x8<true>(bw[t][st & 3].x, bw[t][st & 3].y, zz[t], ss[t]);
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    const v8h a = __builtin_bit_cast(v8h, As[u & 1][8 * mt + st][lane]);
#pragma unroll
                    for (int t = 0; t < CB; ++t)
                        acc[mt][t] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b[t], acc[mt][t], 0, 0, 0);
                }
            }
        }
        __syncthreads();
    };

    load_a(0);
#pragma unroll
    for (int p = 0; p < PB; ++p) load_b(p, p);
    stage_a(0);
    load_a(1);
    __syncthreads();
    constexpr int U = 2;
    int i0 = 0;
    for (; i0 + U <= ng; i0 += U) {
#pragma unroll
        for (int u = 0; u < U; ++u) step(i0 + u, u, true);
    }
    if (i0 < ng) {
#pragma unroll
        for (int u = 0; u < U; ++u) step(i0 + u, u, false);
    }

    __syncthreads();
    uint16_t* stage = reinterpret_cast<uint16_t*>(lds_raw) + wave * (32 * 32 * CB);
    const int n0w = 16 * nbw;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
        for (int t = 0; t < CB; ++t)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = 8 * (r >> 2) + 4 * q + (r & 3);
                stage[row * (32 * CB) + 32 * t + j] = __half_as_ushort(__float2half_rn(acc[mt][t][r]));
            }
        __syncthreads();
#pragma unroll
        for (int u = 0; u < 2 * CB; ++u) {
            const int kk = lane + 64 * u;
            const int row = kk / (4 * CB);
            const int ch = kk % (4 * CB);
            const int m = m0 + 32 * mt + row;
            const int n = n0w + 8 * ch;
            const uint4 v = *reinterpret_cast<const uint4*>(stage + row * (32 * CB) + 8 * ch);
            if (m < M && n < N) *reinterpret_cast<uint4*>(y + int64_t(m) * N + n) = v;
        }
        __syncthreads();
    }
}

// Compiled configurations: (MT, CB, PB, workgroups per CU, waves).
#define QOQ_W8_CONFIGS(X)                                                                 \
    X(4, 2, 2, 2, 4) X(4, 2, 2, 1, 8) X(4, 1, 2, 1, 8) X(2, 2, 2, 2, 4) X(2, 1, 4, 2, 4)    \
    X(1, 1, 4, 3, 4) X(2, 1, 2, 2, 4)
#define QOQ_W4A4_CONFIGS(X)                                                               \
    X(2, 1, 2, 2, 4) X(2, 1, 2, 1, 8) X(1, 1, 2, 3, 4) X(2, 2, 2, 2, 4)
#define QOQ_W4A16_CONFIGS(X)                                                              \
    X(2, 1, 2, 2, 4) X(2, 2, 2, 2, 4) X(4, 1, 2, 1, 8) X(1, 1, 2, 3, 4) X(4, 2, 2, 1, 8)

template <int FMT>
bool variant_config_exists(int mt, int cb, int pb, int minb, int nw) {
    if (FMT == kFmtW4A16) {
#define X(a, b, c, d, e) if (mt == a && cb == b && pb == c && minb == d && nw == e) return true;
        QOQ_W4A16_CONFIGS(X)
#undef X
    } else if (FMT == kFmtW8) {
#define X(a, b, c, d, e) if (mt == a && cb == b && pb == c && minb == d && nw == e) return true;
        QOQ_W8_CONFIGS(X)
#undef X
    } else {
#define X(a, b, c, d, e) if (mt == a && cb == b && pb == c && minb == d && nw == e) return true;
        QOQ_W4A4_CONFIGS(X)
#undef X
    }
    return false;
}

}  // namespace

// Launch plan of the comparison GEMMs: W8A8 takes the W4A8 plan's 32x32
// tile when it is compiled for it; W4A4 (twice the accumulators) uses
// 64-row tiles. The "variant" tuning key "MT,CB,PB,WGPERCU,NW" forces one
// compiled configuration; anything else is an error.
VariantPlan plan_variant(int fmt, int64_t M, int64_t N, int64_t K) {
    VariantPlan p{};
    p.valid = true;
    p.fmt = fmt;
    const bool w8 = fmt == kFmtW8;
    auto exists = [&](int a, int b, int c, int d, int e) {
        return w8 ? variant_config_exists<kFmtW8>(a, b, c, d, e)
                  : fmt == kFmtW4A16 ? variant_config_exists<kFmtW4A16>(a, b, c, d, e)
                                     : variant_config_exists<kFmtW4A4>(a, b, c, d, e);
    };
    const GemmPlan g = plan_gemm(M, N, K);
    if (M <= 32) {
        p.mt = 1; p.cb = 1; p.pb = w8 ? 4 : 2; p.pa = 3; p.nw = 4;
    } else if (w8 && g.kind == 4 && exists(g.mt, g.cb, g.pd, g.pa, g.nw)) {
        p.mt = g.mt; p.cb = g.cb; p.pb = g.pd; p.pa = g.pa; p.nw = g.nw;
    } else if (fmt == kFmtW4A16 && M > 256) {
        p.mt = 4; p.cb = 1; p.pb = 2; p.pa = 1; p.nw = 8;
    } else if (!w8 && M > 256) {
        p.mt = 2; p.cb = 1; p.pb = 2; p.pa = 1; p.nw = 8;
    } else {
        p.mt = 2; p.cb = 1; p.pb = w8 ? 4 : 2; p.pa = 2; p.nw = 4;
    }
    const std::string tune = tuning(kTuneVariant);
    if (!tune.empty()) {
        const char* env = tune.c_str();
        {
            int a = 0, b = 0, c = 0, d = 0, e = 0;
            const int nf = std::sscanf(env, "%d,%d,%d,%d,%d", &a, &b, &c, &d, &e);
            if (nf != 5 || !exists(a, b, c, d, e)) {
                p.valid = false;
                return p;
            }
            p.mt = a; p.cb = b; p.pb = c; p.pa = d; p.nw = e;
        }
    }
    const int64_t nbt = N / kBlockCols;
    const int64_t tm = (M + 32 * p.mt - 1) / (32 * p.mt);
    const int64_t tn = (nbt + 2 * p.cb * p.nw - 1) / (2 * p.cb * p.nw);
    p.grid_x = int(tm * tn);
    return p;
}

int64_t w4a4_rows_padded(int64_t M) { return (M + 127) / 128 * 128; }

int64_t w4a4_act_bytes(int64_t M, int64_t K) {
    const int64_t x4 = act_bytes(M, K) / 2;
    const int64_t Mp = w4a4_rows_padded(M);
    return (x4 + 255) / 256 * 256 + (K / kGroup) * Mp * 4;
}

hipError_t launch_w8a8_pack(const float* W, int64_t N, int64_t K, uint8_t* packed, uint16_t* s,
                            hipStream_t stream) {
    hipError_t e = launch_kernel(w8_scale_kernel, dim3(unsigned(N)), dim3(256), 0, stream, W, K, s);
    if (e != hipSuccess) return e;
    const int64_t threads = N * K / 16;
    return launch_kernel(w8_pack_kernel, dim3(unsigned((threads + 255) / 256)), dim3(256), 0,
                         stream, W, (const uint16_t*)s, N, K, packed);
}

hipError_t launch_w4a16_pack(const float* W, int64_t N, int64_t K, uint8_t* packed,
                             hipStream_t stream) {
    const PackedLayout L = packed_layout(N, K);
    const int64_t waves = N * L.ng;
    return launch_kernel(w4a16_pack_kernel, dim3(unsigned((waves + 3) / 4)), dim3(256), 0, stream,
                         W, N, K, packed, packed + L.rec_offset, packed + L.rec_offset + L.rec_bytes,
                         L.ng8);
}

hipError_t launch_w4a16_gemm(const VariantPlan& p, const uint16_t* x, int64_t M, int64_t K,
                             const uint8_t* packed, int64_t N, uint16_t* y, hipStream_t stream) {
    const PackedLayout L = packed_layout(N, K);
    const uint8_t* srec = packed + L.rec_offset;
    const uint8_t* zrec = srec + L.rec_bytes;
#define X(A, B, C, D, E)                                                                        \
    if (p.mt == A && p.cb == B && p.pb == C && p.pa == D && p.nw == E)                              \
        return launch_kernel(gemm_w4a16_kernel<A, B, C, D, E>, dim3(p.grid_x), dim3(64 * E), 0,     \
                             stream, x, int(M), int(K), packed, srec, zrec, int(L.ng8), int(N), y);
    QOQ_W4A16_CONFIGS(X)
#undef X
    return hipErrorInvalidConfiguration;
}

hipError_t launch_w4a4_pack(const float* W, int64_t N, int64_t K, uint8_t* packed,
                            hipStream_t stream) {
    const PackedLayout L = packed_layout(N, K);
    const int64_t waves = N * L.ng;
    return launch_kernel(w4_pack_kernel, dim3(unsigned((waves + 3) / 4)), dim3(256), 0, stream, W,
                         N, K, packed, packed + L.rec_offset, L.ng8);
}

hipError_t launch_w4a4_quantize_act(const uint16_t* x, int64_t M, int64_t K, uint8_t* act,
                                    hipStream_t stream) {
    const int64_t Mp = w4a4_rows_padded(M);
    const int64_t x4 = act_bytes(M, K) / 2;
    float* s_a = reinterpret_cast<float*>(act + (x4 + 255) / 256 * 256);
    return launch_kernel(a4_quant_kernel, dim3(unsigned(Mp)), dim3(256), 0, stream, x, int(M), K,
                         int(Mp), act, s_a);
}

template <int FMT, int MT, int CB, int PB, int MINB, int NW>
hipError_t launch_variant_t(const VariantPlan& p, const uint8_t* act, const float* ascale, int M,
                            int Mp, int K, const uint8_t* wts, const uint8_t* rec, int ng8,
                            const uint16_t* s1, int N, uint16_t* y, int32_t* acc_debug,
                            hipStream_t stream) {
    return launch_kernel(gemm_variant_kernel<FMT, MT, CB, PB, MINB, NW>, dim3(p.grid_x),
                         dim3(64 * NW), 0, stream, act, ascale, M, Mp, K, wts, rec, ng8, s1, N, y,
                         acc_debug);
}

hipError_t launch_w8a8_gemm(const VariantPlan& p, const int8_t* x8, const float* s_x, int64_t M,
                            int64_t K, const uint8_t* packed, const uint16_t* s, int64_t N,
                            uint16_t* y, int32_t* acc_debug, hipStream_t stream) {
    const uint8_t* a = reinterpret_cast<const uint8_t*>(x8);
#define X(A, B, C, D, E)                                                                  \
    if (p.mt == A && p.cb == B && p.pb == C && p.pa == D && p.nw == E)                        \
        return launch_variant_t<kFmtW8, A, B, C, D, E>(p, a, s_x, int(M), int(M), int(K), packed, \
                                                       nullptr, 0, s, int(N), y, acc_debug,    \
                                                       stream);
    QOQ_W8_CONFIGS(X)
#undef X
    return hipErrorInvalidConfiguration;
}

hipError_t launch_w4a4_gemm(const VariantPlan& p, const uint8_t* act, int64_t M, int64_t K,
                            const uint8_t* packed, int64_t N, uint16_t* y, hipStream_t stream) {
    const PackedLayout L = packed_layout(N, K);
    const int64_t Mp = w4a4_rows_padded(M);
    const int64_t x4 = act_bytes(M, K) / 2;
    const float* s_a = reinterpret_cast<const float*>(act + (x4 + 255) / 256 * 256);
#define X(A, B, C, D, E)                                                                    \
    if (p.mt == A && p.cb == B && p.pb == C && p.pa == D && p.nw == E)                          \
        return launch_variant_t<kFmtW4A4, A, B, C, D, E>(p, act, s_a, int(M), int(Mp), int(K),   \
                                                         packed, packed + L.rec_offset,         \
                                                         int(L.ng8), nullptr, int(N), y,        \
                                                         nullptr, stream);
    QOQ_W4A4_CONFIGS(X)
#undef X
    return hipErrorInvalidConfiguration;
}

}  // namespace qoq
