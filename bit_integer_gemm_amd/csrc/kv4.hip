// Decode attention over a 4-bit KV cache with SmoothAttention scaling.
//
// Pages: "QServe: W4A8KV4 Quantization and System Co-design for Efficient LLM
// Serving" (velog notes), sections "Insight" and "Methods / 1) Algorithm:
// QoQ": the KV cache is held in 4 bits and SmoothAttention moves the
// quantization difficulty of the keys onto the (unquantized) queries; the
// QServe abstract: the fused attention is made memory-bound so the 4-bit
// cache turns into throughput; "Part5 LLM部署技术" section 1.1 (the
// SmoothQuant migration the smoothing factor follows) and section 3.
//
// Arithmetic (the readings the library and its oracle share):
//   lambda[h, d] = fp16(sqrt(max_t |k[t, h, d]|)), 1 for an all-zero channel;
//   a cached vector x (one token, one KV head, D = 128 values; keys are
//   first divided by lambda in fp32) -> lo = min(0, min x), hi = max(0, max x),
//   s = fp16((hi - lo) / 15), z = clamp(rne(-lo / s), 0, 15),
//   code = clamp(rne(x / s) + z, 0, 15); it stands for (code - z) * s;
//   q~ = fp16(q * lambda), scores q~ . k^ / sqrt(D), softmax, sum of p v^.
//
// Cache layout, per (sequence b, KV head h) region of C tokens (C a multiple
// of 32), 133 C bytes: C/32 key blocks of 2 KiB, C/32 value blocks of 2 KiB,
// then C/32 metadata blocks of 160 bytes. Everything is laid out in the lane
// order of v_mfma_f32_16x16x32_f16, so every lane fetches its operands and
// their scales with 16-byte loads and no address arithmetic in the loop:
//   key block (32 tokens): 16 bytes at ((tile * 4 + g) * 16 + t) * 16 hold
//     token 16 tile + t, dims 32 st + 8 g + e (word st, e = 0..7); element e
//     of a word sits at bit 4 (e / 2) + 16 (e % 2), so (w >> 4p) & 0x000F000F
//     is the pair e = 2p, 2p + 1 in the two 16-bit halves;
//   value block (32 tokens): 4 bytes at ((g * 16 + d) * 8 + c) * 4 hold dim
//     16 c + d of tokens pi(8 g + e), e = 0..7, same nibble order, where
//     pi(8 g + e) = 4 g + e (e < 4), 16 + 4 g + e - 4 (e >= 4);
//   metadata block (32 tokens): 32 fp16 s_k, 32 fp16 s_v and 32 bytes
//     z_k | z_v << 4, each indexed by k = 8 g + e for token pi(k).
// pi is the order in which the score MFMA leaves the tokens in the lanes
// (lane (j, g) holds query j, tokens 4 g .. 4 g + 3 of each 16-token tile),
// so the probabilities are already the B operand of the value MFMA.
#include "qoq_internal.hpp"
#include "kernel_common.hpp"

#include <hip/hip_fp16.h>

#include <algorithm>
#include <cstdlib>
#include <type_traits>

namespace qoq {
namespace {

typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kD = 128;
constexpr int kBlk = 32;                 // tokens per block
constexpr int kBlkBytes = 2048;          // 32 tokens x 128 dims x 4 bits
constexpr int kMetaBlkBytes = 160;       // per 32 tokens: 2 x 32 fp16 + 32 bytes
constexpr int kRegionPerToken = kD + kMetaBlkBytes / kBlk;   // 133
// the attention addresses a region's key and value codes with 32-bit
// buffer offsets
static_assert(kKv4MaxCapacity / kBlk * kBlkBytes <= INT32_MAX, "32-bit offsets");

__device__ __forceinline__ int64_t region_offset(int64_t region, int64_t C) {
    return region * C * kRegionPerToken;
}

// Per-vector UINT4 parameters of 64 lanes x 2 values (fp32); returns the
// fp16 scale bits and the zero, identical in every lane.
__device__ __forceinline__ void vec_params(float x0, float x1, uint16_t& sbits, int& z) {
    float lo = fminf(0.0f, fminf(x0, x1)), hi = fmaxf(0.0f, fmaxf(x0, x1));
    for (int off = 32; off > 0; off >>= 1) {
        lo = fminf(lo, __shfl_xor(lo, off, 64));
        hi = fmaxf(hi, __shfl_xor(hi, off, 64));
    }
    sbits = __half_as_ushort(__float2half_rn((hi - lo) / 15.0f));
    const float sc = h2f(sbits);
    z = sc != 0.0f ? int(fminf(fmaxf(rintf(-lo / sc), 0.0f), 15.0f)) : 0;
}

__device__ __forceinline__ int vec_code(float x, float sc, int z) {
    return sc != 0.0f ? min(15, max(0, int(rintf(x / sc)) + z)) : 0;
}

// ---------------------------------------------------------------------------
// smoothing factors: one workgroup per 64 channels, 4 row phases
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256) kv4_smooth_kernel(const uint16_t* __restrict__ k, int64_t T,
                                                         int cols, uint16_t* __restrict__ lam) {
    const int col = blockIdx.x * 64 + (threadIdx.x & 63);
    const int ph = threadIdx.x >> 6;
    uint32_t m = 0;
    if (col < cols)
        for (int64_t t = ph; t < T; t += 4) m = max(m, uint32_t(k[t * cols + col]) & 0x7fffu);
    __shared__ uint32_t part[4][64];
    part[ph][threadIdx.x & 63] = m;
    __syncthreads();
    if (ph == 0 && col < cols) {
        m = max(max(part[0][threadIdx.x], part[1][threadIdx.x]),
                max(part[2][threadIdx.x], part[3][threadIdx.x]));
        const float a = h2f(uint16_t(m));
        lam[col] = a > 0.0f ? __half_as_ushort(__float2half_rn(sqrtf(a))) : uint16_t(0x3c00);
    }
}

// ---------------------------------------------------------------------------
// append: keys (smoothed) and metadata; one wave per (sequence, new token,
// KV head), lane l holds dims 2l, 2l + 1
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256) kv4_append_keys_kernel(
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ v, int B, int Tn, int Hkv,
    const uint16_t* __restrict__ lam, const int32_t* __restrict__ start, uint8_t* __restrict__ cache,
    int64_t C) {
    const int lane = threadIdx.x & 63;
    const int64_t w = int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6);
    if (w >= int64_t(B) * Tn * Hkv) return;
    const int h = int(w % Hkv);
    const int i = int((w / Hkv) % Tn);
    const int b = int(w / (int64_t(Hkv) * Tn));
    const int64_t pos = int64_t(max(start[b], 0)) + i;
    if (pos >= C) return;
    const int64_t src = ((int64_t(b) * Tn + i) * Hkv + h) * kD + 2 * lane;
    const uint32_t kk = *reinterpret_cast<const uint32_t*>(k + src);
    const uint32_t vv = *reinterpret_cast<const uint32_t*>(v + src);
    const uint32_t ll = *reinterpret_cast<const uint32_t*>(lam + h * kD + 2 * lane);
    const float k0 = h2f(uint16_t(kk & 0xffffu)) / h2f(uint16_t(ll & 0xffffu));
    const float k1 = h2f(uint16_t(kk >> 16)) / h2f(uint16_t(ll >> 16));
    const float v0 = h2f(uint16_t(vv & 0xffffu)), v1 = h2f(uint16_t(vv >> 16));
    uint16_t sk, sv;
    int zk, zv;
    vec_params(k0, k1, sk, zk);
    vec_params(v0, v1, sv, zv);
    const float fk = h2f(sk);
    const int c0 = vec_code(k0, fk, zk), c1 = vec_code(k1, fk, zk);
    // word wi = lane / 4 holds dims 8 wi + e; lane 4wi + r holds e = 2r and
    // 2r + 1, which sit at bits 4r and 16 + 4r of the word
    const int r4 = 4 * (lane & 3);
    uint32_t word = (uint32_t(c0) << r4) | (uint32_t(c1) << (16 + r4));
    word |= __shfl_xor(word, 1, 64);
    word |= __shfl_xor(word, 2, 64);
    uint8_t* region = cache + region_offset(int64_t(b) * Hkv + h, C);
    const int64_t blk = pos / kBlk;
    const int tt = int(pos % kBlk);
    if ((lane & 3) == 0) {
        const int wi = lane >> 2;
        const int st = wi >> 2, g = wi & 3;
        const int64_t off = blk * kBlkBytes + ((tt >> 4) * 4 + g) * 256 + (tt & 15) * 16 + 4 * st;
        *reinterpret_cast<uint32_t*>(region + off) = word;
    }
    if (lane < 3) {
        // k-index of the token in its block: lane group g = (tt % 16) / 4,
        // e = tt % 4 + 4 (tt / 16)
        const int kk = 8 * ((tt & 15) >> 2) + (tt & 3) + 4 * (tt >> 4);
        uint8_t* meta = region + (C / kBlk) * 2 * kBlkBytes + blk * kMetaBlkBytes;
        if (lane < 2) reinterpret_cast<uint16_t*>(meta)[lane * 32 + kk] = lane == 0 ? sk : sv;
        else meta[128 + kk] = uint8_t(zk | (zv << 4));
    }
}

// append: value codes. One thread per 4-byte word (g, d, c) of every block
// the new tokens touch; it rewrites the nibbles of the new tokens and keeps
// the others (tokens of one word may arrive in different calls).
__global__ void __launch_bounds__(256) kv4_append_values_kernel(
    const uint16_t* __restrict__ v, int B, int Tn, int Hkv, const int32_t* __restrict__ start,
    uint8_t* __restrict__ cache, int64_t C, int nblk_touch) {
    const int64_t gid = int64_t(blockIdx.x) * 256 + threadIdx.x;
    const int64_t per_region = int64_t(nblk_touch) * 512;
    if (gid >= int64_t(B) * Hkv * per_region) return;
    const int64_t region = gid / per_region;
    const int b = int(region / Hkv), h = int(region % Hkv);
    const int rem = int(gid % per_region);
    const int64_t s0 = max(start[b], 0);
    const int64_t blk = s0 / kBlk + rem / 512;
    const int word = rem % 512;
    const int g = word >> 7, d = (word >> 3) & 15, c = word & 7;
    if (blk >= C / kBlk) return;
    uint8_t* rg = cache + region_offset(region, C);
    uint32_t* wp = reinterpret_cast<uint32_t*>(rg + (C / kBlk) * kBlkBytes + blk * kBlkBytes + word * 4);
    const uint8_t* meta = rg + (C / kBlk) * 2 * kBlkBytes + blk * kMetaBlkBytes;
    uint32_t wv = *wp;
    bool any = false;
    for (int e = 0; e < 8; ++e) {
        const int tok = e < 4 ? 4 * g + e : 16 + 4 * g + (e - 4);
        const int64_t pos = blk * kBlk + tok;
        const int64_t i = pos - s0;
        if (i < 0 || i >= Tn || pos >= C) continue;
        const float sc = h2f(reinterpret_cast<const uint16_t*>(meta)[32 + 8 * g + e]);
        const int z = int(meta[128 + 8 * g + e] >> 4);
        const float x = h2f(v[((int64_t(b) * Tn + i) * Hkv + h) * kD + 16 * c + d]);
        const uint32_t code = uint32_t(vec_code(x, sc, z));
        const int sh = 4 * (e >> 1) + 16 * (e & 1);
        wv = (wv & ~(0xfu << sh)) | (code << sh);
        any = true;
    }
    if (any) *wp = wv;
}

// fp16 cache append (the comparison point): one wave per (sequence, new
// token, KV head), lane l stores dims 2l, 2l + 1 of the key and the value
// at their places in the fp16 MFMA-ordered layout.
__global__ void __launch_bounds__(256) kv16_append_kernel(
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ v, int B, int Tn, int Hkv,
    const int32_t* __restrict__ start, uint8_t* __restrict__ cache, int64_t C) {
    const int lane = threadIdx.x & 63;
    const int64_t w = int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6);
    if (w >= int64_t(B) * Tn * Hkv) return;
    const int h = int(w % Hkv);
    const int i = int((w / Hkv) % Tn);
    const int b = int(w / (int64_t(Hkv) * Tn));
    const int64_t pos = int64_t(max(start[b], 0)) + i;
    if (pos >= C) return;
    const int64_t src = ((int64_t(b) * Tn + i) * Hkv + h) * kD + 2 * lane;
    const uint32_t kk = *reinterpret_cast<const uint32_t*>(k + src);
    const uint32_t vv = *reinterpret_cast<const uint32_t*>(v + src);
    uint8_t* rg = cache + (int64_t(b) * Hkv + h) * C * (4 * kD);
    const int64_t blk = pos / kBlk;
    const int tt = int(pos % kBlk);
    const int d = 2 * lane;
    const int st = d >> 5, g = (d & 31) >> 3, e = d & 7;
    *reinterpret_cast<uint32_t*>(rg + blk * 4 * kBlkBytes + (((tt >> 4) * 4 + g) * 16 + (tt & 15)) * 64 +
                                 16 * st + 2 * e) = kk;
    const int gt = (tt & 15) >> 2, et = (tt & 3) + 4 * (tt >> 4);
    uint8_t* vb = rg + (C / kBlk) * 4 * kBlkBytes + blk * 4 * kBlkBytes;
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        const int dd = d + r;
        *reinterpret_cast<uint16_t*>(vb + ((gt * 16 + (dd & 15)) * 8 + (dd >> 4)) * 16 + 2 * et) =
            uint16_t(vv >> (16 * r));
    }
}

// ---------------------------------------------------------------------------
// attention
// ---------------------------------------------------------------------------
// Eight codes of a word (element e at bit 4 (e / 2) + 16 (e % 2)) -> four
// fp16 pairs in e order.
//   unpack_tiny: the fp16 bit patterns of code * 2^-24 (subnormals, exact);
//   unpack_1024: 1024 + code (exponent bits 0x64 or-ed in).
__device__ __forceinline__ void unpack_tiny(uint32_t w, uint32_t m, h2 (&r)[4]) {
#pragma unroll
    for (int p = 0; p < 4; ++p) r[p] = __builtin_bit_cast(h2, (w >> (4 * p)) & m);
}
__device__ __forceinline__ void unpack_1024(uint32_t w, uint32_t m, uint32_t e64, h2 (&r)[4]) {
#pragma unroll
    for (int p = 0; p < 4; ++p) r[p] = __builtin_bit_cast(h2, ((w >> (4 * p)) & m) | e64);
}

__device__ __forceinline__ v8h join(const h2 (&r)[4]) {
    v8h o;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        o[2 * i] = r[i][0];
        o[2 * i + 1] = r[i][1];
    }
    return o;
}

// fp32 x times the fp16 in the low (HI = false) or high half of w, one
// rounding: an FMA with a +0 addend on the converted half, which the
// compiler issues as one mixed-precision FMA (no conversion instruction)
template <bool HI>
__device__ __forceinline__ float mul_f16(float x, uint32_t w) {
    const h2 v = __builtin_bit_cast(h2, w);
    return __builtin_fmaf(x, float(v[HI ? 1 : 0]), 0.0f);
}

// Max over the four lanes l, l ^ 16, l ^ 32, l ^ 48 (the four lane groups
// that hold one query's scores) with gfx950's row swaps: swapping the upper
// 32 lanes of one copy with the lower 32 of another leaves x[l] and
// x[l ^ 32] in the two results of every lane, and the 16-lane row swap does
// the same for l ^ 16; no LDS round trip.
__device__ __forceinline__ float group_max(float x) {
    const uint32_t u = __float_as_uint(x);
    const auto s32 = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    const float y = fmaxf(__uint_as_float(s32[0]), __uint_as_float(s32[1]));
    const uint32_t v = __float_as_uint(y);
    const auto s16 = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    return fmaxf(__uint_as_float(s16[0]), __uint_as_float(s16[1]));
}

struct AttnArgs {
    const uint16_t* q;         // [B, H, D]
    const uint16_t* lam;       // [Hkv, D]
    const uint8_t* cache;
    const int32_t* lens;       // [B]
    uint16_t* out;             // [B, H, D]
    float* part;               // [B, H, splits, D + 2] when splits > 1
    int64_t C;
    int B, H, Hkv, G, splits, bps, max_len;
    int paired;                // 1: workgroup p takes the KV head's contexts of length
                               // ranks p and B - 1 - p (splits == 1, B <= kPairMaxB)
};

// Largest batch the paired schedule ranks in LDS.
constexpr int kPairMaxB = 256;

// One workgroup (NW = 4 or 8 waves) per (sequence, KV head, split), or, in
// the paired schedule, per (pair of sequences, KV head): the sequences are
// ranked by context length in the workgroup (ties by index) and workgroup p
// takes ranks p and B - 1 - p one after the other, so every workgroup holds
// about the same number of tokens and none waits for the longest context
// alone. Wave w takes the blocks w, w + NW, ...; per block: 2 score MFMAs
// tiles x 4 steps (tokens x queries), online softmax per query, 8 value
// MFMAs (dims x queries). The waves' states are merged in LDS at the end of
// each context.
// kF16: the same kernel on an fp16 cache (the comparison point for what the
// 4-bit cache buys): keys and values are the MFMA operands as stored, the
// query is used unsmoothed, nothing is dequantized. Per 32-token block the
// fp16 layout holds keys [tile 2][g 4][t 16][st 4][8 halves] and values
// [g 4][d 16][c 8][8 halves] (tokens pi(8 g + e)), 8 KiB each.
template <bool kF16, int NW>
__global__ void __launch_bounds__(64 * NW)
__attribute__((amdgpu_waves_per_eu(kF16 ? 1 : (NW == 8 ? 2 : 3))))
kv4_attention_kernel(AttnArgs a) {
    // blocks a wave holds in registers: the next block's loads are in flight
    // while one is computed (deeper rings, 3-5 blocks, measured slower on
    // every benchmarked batch: more registers, no latency left to hide)
    constexpr int R = 2;
    // the 8-wave 4-bit workgroups run the paired schedule with both contexts
    // in one stream of blocks: one merge slot per context
    constexpr bool kPairStream = !kF16 && NW == 8;
    constexpr int kSlots = kPairStream ? 2 : 1;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int j = lane & 15;          // query of the group (MFMA column)
    const int g = lane >> 4;          // lane group
    const int64_t C = a.C;
    __shared__ float sm[kSlots][NW][16], sl[kSlots][NW][16];
    __shared__ float so[kSlots][NW][16][kD + 4];
    __shared__ int rank_len[kPairMaxB], by_rank[kPairMaxB];
    auto clamped_len = [&](int b) { return int(min(int64_t(max(min(a.lens[b], a.max_len), 0)), C)); };
    // scores in the log2 domain: log2(e) / sqrt(D)
    const float kScale = 1.4426950408889634f * 0.08838834764831845f;
    const bool qvalid = j < a.G;

    // state of the context being processed: its length, the smoothed query
    // operand (lane (j, g), step st holds dims 32 st + 8 g + e) and the sum
    // of its elements, the running maximum and sum, the output accumulators
    int len = 0;
    v8h qop[4];
    float qsum = 0.0f;
    v8h qz;                           // query side of the zero-point MFMA
    float m = -INFINITY, l = 0.0f;
    v4f o[8];

    auto set_query = [&](int b, int h, v8h (&qo)[4], float& qs) {
        const int qh = h * a.G + min(j, a.G - 1);
        qs = 0.0f;
#pragma unroll
        for (int st = 0; st < 4; ++st) {
            const int d0 = 32 * st + 8 * g;
            const uint4 qq = *reinterpret_cast<const uint4*>(a.q + (int64_t(b) * a.H + qh) * kD + d0);
            const uint4 ll = kF16 ? uint4{0x3c003c00u, 0x3c003c00u, 0x3c003c00u, 0x3c003c00u}
                                  : *reinterpret_cast<const uint4*>(a.lam + h * kD + d0);
            const uint32_t qw[4] = {qq.x, qq.y, qq.z, qq.w}, lw[4] = {ll.x, ll.y, ll.z, ll.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
#pragma unroll
                for (int hf = 0; hf < 2; ++hf) {
                    const float x = h2f(uint16_t(qw[i] >> (16 * hf))) * h2f(uint16_t(lw[i] >> (16 * hf)));
                    const _Float16 xs = qvalid ? static_cast<_Float16>(x) : _Float16(0.0f);
                    qo[st][2 * i + hf] = xs;
                    qs += float(xs);
                }
            }
        }
        qs += __shfl_xor(qs, 16, 64);
        qs += __shfl_xor(qs, 32, 64);
    };
    // The key zero point enters the scores through a fifth MFMA per tile:
    // its key side holds z_k 2^-17 in the lanes of the first k group
    // (k = 0, 1, 2): the fp16 bit pattern z_k << 7 (patterns up to 0x7ff are
    // linear in value, 2^-24 apart, so this is exact for z_k <= 15); its
    // query side holds -sum(q~) 2^-7 there as three fp16 parts (their sum
    // is the fp32 value but for the parts' 2^-24 resolution; 128 values of
    // at most 65504 keep the largest part finite), so the MFMA adds
    // -z_k sum(q~) 2^-24 to the 2^-24-scaled score.
    auto make_qz = [&](float qs) {
        const float x = qs * 0.0078125f;
        const _Float16 p0 = static_cast<_Float16>(x);
        const float r1 = x - float(p0);
        const _Float16 p1 = static_cast<_Float16>(r1);
        const _Float16 p2 = static_cast<_Float16>(r1 - float(p1));
        v8h v;
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = _Float16(0.0f);
        if (g == 0) {
            v[0] = -p0;
            v[1] = -p1;
            v[2] = -p2;
        }
        return v;
    };
    auto reset = [&]() {
        m = -INFINITY;
        l = 0.0f;
#pragma unroll
        for (int c = 0; c < 8; ++c) o[c] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
    };

    auto region_base = [&](int b, int h) {
        const int region = b * a.Hkv + h;
        return kF16 ? a.cache + int64_t(region) * C * (4 * kD) : a.cache + region_offset(region, C);
    };
    // 4-bit cache sections of a region as buffers (key and value codes at
    // most 2^24 / 32 blocks x 2 KiB = 1 GiB each: 32-bit offsets)
    struct Rs {
        __amdgpu_buffer_rsrc_t k, v, m;
    };
    const int64_t nblk = C / kBlk;
    auto region_rsrc = [&](int b, int h) {
        const uint8_t* rg = region_base(b, h);
        Rs rs;
        rs.k = __builtin_amdgcn_make_buffer_rsrc((void*)rg, (short)0, int(nblk * kBlkBytes), 0x00020000);
        rs.v = __builtin_amdgcn_make_buffer_rsrc((void*)(rg + nblk * kBlkBytes), (short)0,
                                                 int(nblk * kBlkBytes), 0x00020000);
        rs.m = __builtin_amdgcn_make_buffer_rsrc((void*)(rg + nblk * 2 * kBlkBytes), (short)0,
                                                 int(nblk * kMetaBlkBytes), 0x00020000);
        return rs;
    };

    auto kofs = [&](int tile) { return (tile * 4 + g) * 256 + j * 16; };
    const int vofs = (g * 16 + j) * 32;
    // per block: key codes (2 tiles), value codes, and the lane's 8 entries
    // of each metadata array (s_k, s_v, zero bytes); or the fp16 operands
    struct Blk4 {
        uint4 k0, k1, v0, v1, sk, sv;
        uint2 z;      // zero bytes of the lane's output tokens
        uint2 zr;     // zero bytes of the lane's key row tokens (j, 16 + j)
    };
    struct Blk16 {
        uint4 k[8], v[8];
    };
    auto load16 = [&](Blk16& r, const uint8_t* rg, int blk) {
        const uint8_t* kb = rg + int64_t(blk) * 4 * kBlkBytes;
        const uint8_t* vb = rg + nblk * 4 * kBlkBytes + int64_t(blk) * 4 * kBlkBytes;
#pragma unroll
        for (int tile = 0; tile < 2; ++tile)
#pragma unroll
            for (int st = 0; st < 4; ++st)
                r.k[4 * tile + st] = *reinterpret_cast<const uint4*>(
                    kb + ((tile * 4 + g) * 16 + j) * 64 + 16 * st);
#pragma unroll
        for (int c = 0; c < 8; ++c)
            r.v[c] = *reinterpret_cast<const uint4*>(vb + (g * 16 + j) * 128 + 16 * c);
    };
    // buffer loads: the lane offsets are fixed, the block offset is uniform
    // (an SGPR), so no address arithmetic runs per block
    auto load4 = [&](Blk4& r, const Rs& rs, int blk) {
        const int sb = blk * kBlkBytes;
        const int smb = blk * kMetaBlkBytes;
        r.k0 = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs.k, kofs(0), sb, 0));
        r.k1 = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs.k, kofs(1), sb, 0));
        r.v0 = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs.v, vofs, sb, 0));
        r.v1 = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs.v, vofs + 16, sb, 0));
        r.sk = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs.m, 16 * g, smb, 0));
        r.sv = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs.m, 64 + 16 * g, smb, 0));
        r.z = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rs.m, 128 + 8 * g, smb, 0));
        r.zr = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rs.m, 128 + 8 * (j >> 2), smb, 0));
    };
    // byte j % 4 of the row word holds the zero of key row j (tile 0) and
    // 16 + j (tile 1); only the first k group's lanes carry it
    const uint32_t zsh = 8 * (j & 3);
    const uint32_t zmask = g == 0 ? 0xfu : 0u;
    const float kS24 = kScale * 16777216.0f;
    const uint32_t c64 = __builtin_amdgcn_readfirstlane(0x64646464u);
    // one code per 16-bit half; held in a VGPR so that mask-and-or fuses
    // into one v_and_or_b32 with the exponent constant in an SGPR
    uint32_t nib;
    asm volatile("v_mov_b32 %0, 0x000f000f" : "=v"(nib));
    const uint32_t e64 = __builtin_amdgcn_readfirstlane(0x64006400u);
    // online softmax for query j over a block's 32 tokens; the accumulators
    // are rescaled only when the running maximum grows by more than 2^8
    // (probabilities stay below 256 in between). The maximum is one of the
    // scores, so its token's probability is exactly 1. Returns the fp16 P
    // operand.
    auto softmax = [&](const float (&zs)[8]) {
        float bm = zs[0];
#pragma unroll
        for (int e = 1; e < 8; ++e) bm = fmaxf(bm, zs[e]);
        bm = group_max(bm);
        const bool grow = bm > m + 8.0f;
        if (__ballot(grow) != 0) {
            const float fac = grow ? __builtin_amdgcn_exp2f(m - bm) : 1.0f;
            l *= fac;
#pragma unroll
            for (int c = 0; c < 8; ++c) o[c] = o[c] * fac;
            m = grow ? bm : m;
        }
        v8h pop;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float pe = __builtin_amdgcn_exp2f(zs[e] - m);
            l += pe;
            pop[e] = static_cast<_Float16>(pe);
        }
        return pop;
    };
    auto compute16 = [&](const Blk16& r, int blk) {
        const int tbase = blk * kBlk;
        auto valid = [&](int e) {
            const int tok = e < 4 ? 4 * g + e : 16 + 4 * g + (e - 4);
            return tbase + tok < len;
        };
        float zs[8];
#pragma unroll
        for (int tile = 0; tile < 2; ++tile) {
            v4f acc = v4f{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int st = 0; st < 4; ++st)
                acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(v8h, r.k[4 * tile + st]),
                                                             qop[st], acc, 0, 0, 0);
#pragma unroll
            for (int i = 0; i < 4; ++i) zs[4 * tile + i] = valid(4 * tile + i) ? acc[i] * kScale : -INFINITY;
        }
        const v8h pop = softmax(zs);
        // tokens past the context: their values are zeroed (any bits may be there)
        uint32_t keep[4];
#pragma unroll
        for (int pr = 0; pr < 4; ++pr)
            keep[pr] = (valid(2 * pr) ? 0x0000ffffu : 0u) | (valid(2 * pr + 1) ? 0xffff0000u : 0u);
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            const uint4 w = r.v[c];
            const uint4 vm = uint4{w.x & keep[0], w.y & keep[1], w.z & keep[2], w.w & keep[3]};
            o[c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(v8h, vm), pop, o[c], 0, 0, 0);
        }
    };
    auto compute4 = [&](const Blk4& r, int blk) {
        // tokens past the context occur only in a context's last block: the
        // masks are built there alone (a scalar branch), every other block
        // runs with all 32 tokens kept
        const int tbase = blk * kBlk;
        const bool partial = tbase + kBlk > len;
        auto valid = [&](int e) {
            const int tok = e < 4 ? 4 * g + e : 16 + 4 * g + (e - 4);
            return tbase + tok < len;
        };
        const uint32_t skw[4] = {r.sk.x, r.sk.y, r.sk.z, r.sk.w};
        // scores: S[token, query] = q~ . (u - z_k). The key codes enter the
        // MFMA as the fp16 subnormals u 2^-24 (their bit patterns, exact),
        // the zero point through the fifth MFMA; the sum times the token's
        // scale s_k (one mixed-precision multiply) is the 2^-24-scaled
        // score, then brought to the log2 domain (2^24 log2(e) / sqrt(D)).
        float zs[8];
#pragma unroll
        for (int tile = 0; tile < 2; ++tile) {
            v4f acc = v4f{0.0f, 0.0f, 0.0f, 0.0f};
            const uint4 kt = tile ? r.k1 : r.k0;
            const uint32_t kw[4] = {kt.x, kt.y, kt.z, kt.w};
#pragma unroll
            for (int st = 0; st < 4; ++st) {
                h2 u[4];
                unpack_tiny(kw[st], nib, u);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(join(u), qop[st], acc, 0, 0, 0);
            }
            const uint32_t zt = ((tile ? r.zr.y : r.zr.x) >> zsh) & zmask;
            const uint4 zrow = uint4{zt * 0x00800080u, zt << 7, 0u, 0u};
            acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(v8h, zrow), qz, acc, 0, 0, 0);
#pragma unroll
            for (int i = 0; i < 4; i += 2) {
                zs[4 * tile + i] = mul_f16<false>(acc[i], skw[2 * tile + i / 2]) * kS24;
                zs[4 * tile + i + 1] = mul_f16<true>(acc[i + 1], skw[2 * tile + i / 2]) * kS24;
            }
        }
        uint32_t svw[4] = {r.sv.x, r.sv.y, r.sv.z, r.sv.w};
        if (partial) {
#pragma unroll
            for (int e = 0; e < 8; ++e) zs[e] = valid(e) ? zs[e] : -INFINITY;
            // tokens past the context get value scale 0, whatever bits
            // their slot holds
#pragma unroll
            for (int pr = 0; pr < 4; ++pr)
                svw[pr] &= (valid(2 * pr) ? 0x0000ffffu : 0u) | (valid(2 * pr + 1) ? 0xffff0000u : 0u);
        }
        const v8h pop = softmax(zs);
        // values: sum_t p_t s_t (u_t - z_t). The token's scale rides on its
        // probability, P' = fp16(fp16(p) s), and the value operand is the
        // exact integer (1024 + u) - (1024 + z) = u - z: one packed
        // subtraction per two values, no per-value scaling. (Codes and zeros
        // in separate MFMA sums would save the subtractions but not the
        // accuracy: the two sums cancel where u ~ z, and their rounding then
        // exceeds the error bound of the exact difference.)
        const uint32_t zv03 = (r.z.x >> 4) & 0x0f0f0f0fu, zv47 = (r.z.y >> 4) & 0x0f0f0f0fu;
        // 1024 + z_v pairs: the zero bytes with 0x64 exponent bytes between
        h2 zz[4];
        zz[0] = __builtin_bit_cast(h2, __builtin_amdgcn_perm(c64, zv03, 0x04010400u));
        zz[1] = __builtin_bit_cast(h2, __builtin_amdgcn_perm(c64, zv03, 0x04030402u));
        zz[2] = __builtin_bit_cast(h2, __builtin_amdgcn_perm(c64, zv47, 0x04010400u));
        zz[3] = __builtin_bit_cast(h2, __builtin_amdgcn_perm(c64, zv47, 0x04030402u));
        v8h pv;
#pragma unroll
        for (int pr = 0; pr < 4; ++pr) {
            const h2 ps = h2{pop[2 * pr], pop[2 * pr + 1]} * __builtin_bit_cast(h2, svw[pr]);
            pv[2 * pr] = ps[0];
            pv[2 * pr + 1] = ps[1];
        }
        const uint32_t vw[8] = {r.v0.x, r.v0.y, r.v0.z, r.v0.w, r.v1.x, r.v1.y, r.v1.z, r.v1.w};
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            h2 u[4];
            unpack_1024(vw[c], nib, e64, u);
#pragma unroll
            for (int i = 0; i < 4; ++i) u[i] = u[i] - zz[i];
            o[c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(join(u), pv, o[c], 0, 0, 0);
        }
    };

    // a wave's state into merge slot `slot`: lane (j, g) holds query j,
    // dims 16 c + 4 g + i
    auto flush = [&](int slot) {
        float lt = l;
        lt += __shfl_xor(lt, 16, 64);
        lt += __shfl_xor(lt, 32, 64);
        if (g == 0) {
            sm[slot][wave][j] = m;
            sl[slot][wave][j] = lt;
        }
#pragma unroll
        for (int c = 0; c < 8; ++c)
#pragma unroll
            for (int i = 0; i < 4; ++i) so[slot][wave][j][16 * c + 4 * g + i] = o[c][i];
    };
    // the waves' states of slot `slot` merged by 256 threads (thread t:
    // query t / 16, 8 dims; G <= 16, so threads past the group hold no
    // query): the output of sequence b, or the partial of split sp
    auto merge = [&](int slot, int b, int h, int sp, int t) {
        const int jq = t >> 4;
        const int d0 = (t & 15) * 8;
        if (jq >= a.G) return;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < NW; ++w) M = fmaxf(M, sm[slot][w][jq]);
        float L = 0.0f, f[NW];
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            f[w] = M == -INFINITY ? 0.0f : exp2f(sm[slot][w][jq] - M);
            L += f[w] * sl[slot][w][jq];
        }
        float acc[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            acc[e] = 0.0f;
#pragma unroll
            for (int w = 0; w < NW; ++w) acc[e] += f[w] * so[slot][w][jq][d0 + e];
        }
        const int64_t row = int64_t(b) * a.H + h * a.G + jq;
        if (a.splits == 1) {
            uint32_t pk[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float x0 = L > 0.0f ? acc[2 * e] / L : 0.0f;
                const float x1 = L > 0.0f ? acc[2 * e + 1] / L : 0.0f;
                pk[e] = uint32_t(__half_as_ushort(__float2half_rn(x0))) |
                        (uint32_t(__half_as_ushort(__float2half_rn(x1))) << 16);
            }
            *reinterpret_cast<uint4*>(a.out + row * kD + d0) = uint4{pk[0], pk[1], pk[2], pk[3]};
        } else {
            float* pp = a.part + (row * a.splits + sp) * (kD + 4);
            *reinterpret_cast<float4*>(pp + d0) = float4{acc[0], acc[1], acc[2], acc[3]};
            *reinterpret_cast<float4*>(pp + d0 + 4) = float4{acc[4], acc[5], acc[6], acc[7]};
            if (d0 == 0) {
                pp[kD] = M;
                pp[kD + 1] = L;
            }
        }
    };

    // The 4-bit block loop: this wave's blocks are the stream indices
    // first, first + NW, ..., last (load_at / compute_at map an index to a
    // context and block). The loads of the next R - 1 are in flight while
    // one is computed; whole rounds of R blocks run unconditionally, and
    // the last R - 1 or fewer blocks are already in the ring when the
    // rounds end and are only computed. Every step issues its load (indices
    // past the wave's last are clamped to it: cache hits, never used). The
    // compiler is free to interleave one block's value MFMAs with the next
    // block's key unpacking (with scheduling barriers around each load,
    // which keep each block's loads together, the four 8-16K-token contexts
    // in 16 splits took 18.5 against 17.6 us; the other benchmarked batches
    // are level). The caller has already loaded ring[0] with block `first`
    // (issued before the query loads, so the two latencies overlap).
    static_assert(R == 2, "ring[0] is the caller's prologue load");
    auto block_loop = [&](Blk4 (&ring)[R], int first, int last, auto load_at, auto compute_at) {
        if (first > last) return;
        const int mine = (last - first) / NW + 1;   // blocks of this wave
        int b = first, i = 0;
        for (; i + R <= mine; i += R) {
#pragma unroll
            for (int s = 0; s < R; ++s) {
                load_at(ring[(s + R - 1) % R], min(b + (R - 1) * NW, last));
                compute_at(ring[s], b);
                b += NW;
            }
        }
#pragma unroll
        for (int s = 0; s < R - 1; ++s)
            if (i + s < mine) compute_at(ring[s], b + s * NW);
    };

  // one (sequence, KV head, split): the whole attention of its queries
  auto run = [&](const int b_in, const int h, const int sp) {
    // b comes from LDS in the paired schedule: the same in every lane
    const int b = __builtin_amdgcn_readfirstlane(b_in);
    const int blk0 = sp * a.bps;
    const int first = blk0 + wave;
    if constexpr (kF16) {
        len = __builtin_amdgcn_readfirstlane(clamped_len(b));
        const int nb = (len + kBlk - 1) / kBlk;
        const int blk1 = min(nb, blk0 + a.bps);
        if (a.splits > 1 && blk0 >= nb) return;
        set_query(b, h, qop, qsum);
        reset();
        // the fp16 cache (comparison point): two blocks, the next one's
        // loads in flight while one is computed
        const uint8_t* rg = region_base(b, h);
        Blk16 ra, rb;
        int bi = first;
        if (bi < blk1) load16(ra, rg, bi);
        for (; bi < blk1; bi += 2 * NW) {
            if (bi + NW < blk1) load16(rb, rg, bi + NW);
            compute16(ra, bi);
            if (bi + NW >= blk1) break;
            if (bi + 2 * NW < blk1) load16(ra, rg, bi + 2 * NW);
            compute16(rb, bi + NW);
        }
    } else {
        // the wave's first block, the query and the length all at once: the
        // block needs no length (a block of the region's capacity, clamped;
        // unused when the context ends before it)
        const Rs rs = region_rsrc(b, h);
        Blk4 ring[R];
        load4(ring[0], rs, min(first, int(nblk) - 1));
        set_query(b, h, qop, qsum);
        len = __builtin_amdgcn_readfirstlane(clamped_len(b));
        const int nb = (len + kBlk - 1) / kBlk;
        const int blk1 = min(nb, blk0 + a.bps);
        // a split past the end of its context writes nothing: the merge of
        // the splits reads only those that hold tokens
        if (a.splits > 1 && blk0 >= nb) return;
        qz = make_qz(qsum);
        reset();
        block_loop(ring, first, blk1 - 1, [&](Blk4& r, int blk) { load4(r, rs, blk); },
                   [&](const Blk4& r, int blk) { compute4(r, blk); });
    }
    flush(0);
    __syncthreads();
    merge(0, b, h, sp, threadIdx.x);
  };

  // the paired schedule's two contexts (A, then B; bB == bA: A alone) as one
  // stream of blocks over the workgroup's waves: a wave whose blocks cross
  // from A to B parks its A state in slot 0 and goes on with B's query;
  // both merges run at the end, on the two halves of the workgroup. The
  // lengths come from the ranking in LDS.
  auto run_pair = [&](const int bA_in, const int bB_in, const int lenA_in, const int lenB_in,
                      const int h) {
    const int bA = __builtin_amdgcn_readfirstlane(bA_in);
    const int bB = __builtin_amdgcn_readfirstlane(bB_in);
    const bool alone = bA == bB;
    const int lenA = __builtin_amdgcn_readfirstlane(lenA_in);
    const int lenB = alone ? 0 : __builtin_amdgcn_readfirstlane(lenB_in);
    const int nA = (lenA + kBlk - 1) / kBlk;
    const int nB = (lenB + kBlk - 1) / kBlk;
    const Rs rsA = region_rsrc(bA, h);
    const Rs rsB = region_rsrc(bB, h);
    auto load_at = [&](Blk4& r, int c) {
        if (c < nA) load4(r, rsA, c);
        else load4(r, rsB, c - nA);
    };
    // the wave's first block before the queries (clamped to the stream's
    // last, or block 0 of B when the pair holds no tokens: unused then)
    Blk4 ring[R];
    load_at(ring[0], min(wave, max(nA + nB - 1, 0)));
    v8h qopB[4];
    float qsumB;
    set_query(bB, h, qopB, qsumB);
    const v8h qzB = make_qz(qsumB);
    set_query(bA, h, qop, qsum);
    qz = make_qz(qsum);
    len = lenA;
    reset();
    bool inB = false;
    block_loop(
        ring, wave, nA + nB - 1, load_at,
        [&](const Blk4& r, int c) {
            if (c >= nA && !inB) {
                flush(0);
                reset();
#pragma unroll
                for (int st = 0; st < 4; ++st) qop[st] = qopB[st];
                qz = qzB;
                len = lenB;
                inB = true;
            }
            compute4(r, inB ? c - nA : c);
        });
    if (!inB) {
        flush(0);
        reset();
    }
    flush(1);
    __syncthreads();
    if (threadIdx.x < 256) merge(0, bA, h, 0, threadIdx.x);
    else if (!alone) merge(1, bB, h, 0, threadIdx.x - 256);
  };

    if (!a.paired) {
        // 4-bit cache, split-major: the splits of one (sequence, KV head) are
        // `regions` ids apart, so with a multiple of 8 regions they all run
        // on XCD region % 8 (ids are dealt to the XCDs round-robin), where the
        // one-wave merge workgroups of that region's rows run too (merge
        // workgroup i takes a row of a region r with r % 8 = i % 8), and the
        // partials are still in that XCD's L2 (Llama-3-8B-shaped, 4 x 8-16K
        // tokens: 22.6 -> 22.25 us). The fp16 cache keeps the splits of a
        // region adjacent (split-major costs it 50.4 -> 51.2 us).
        const int regions = a.B * a.Hkv;
        const int region = kF16 ? blockIdx.x / a.splits : blockIdx.x % regions;
        const int sp = kF16 ? blockIdx.x % a.splits : blockIdx.x / regions;
        run(region / a.Hkv, region % a.Hkv, sp);
        return;
    }
    // paired schedule: rank the contexts by length (longest first, ties by
    // index), then take ranks p and B - 1 - p
    for (int t = threadIdx.x; t < a.B; t += 64 * NW) rank_len[t] = clamped_len(t);
    __syncthreads();
    for (int t = threadIdx.x; t < a.B; t += 64 * NW) {
        const int lt = rank_len[t];
        int r = 0;
        for (int u = 0; u < a.B; ++u) {
            const int lu = rank_len[u];
            r += (lu > lt || (lu == lt && u < t)) ? 1 : 0;
        }
        by_rank[r] = t;
    }
    __syncthreads();
    const int p = blockIdx.x / a.Hkv;
    const int h = blockIdx.x % a.Hkv;
    if constexpr (kPairStream) {
        const int bA = by_rank[p], bB = by_rank[a.B - 1 - p];
        run_pair(bA, bB, rank_len[bA], rank_len[bB], h);
    } else {
        run(by_rank[p], h, 0);
        if (a.B - 1 - p != p) {
            __syncthreads();   // the merge buffers are reused
            run(by_rank[a.B - 1 - p], h, 0);
        }
    }
}

// Splits of one (sequence, query head) merged: one wave, 2 dims per lane;
// only the splits that hold tokens of the sequence are read. Up to 16 of
// them, every load is issued at once (one round trip); beyond that, lane s
// reads split s's maximum and sum, the weights come from wave reductions,
// and the partial outputs are read eight splits at a time.
__global__ void __launch_bounds__(256) kv4_combine_kernel(const float* __restrict__ part, int rows,
                                                          int H, int splits, int bps,
                                                          const int32_t* __restrict__ lens,
                                                          int max_len, int64_t C,
                                                          uint16_t* __restrict__ out, int xg) {
    const int lane = threadIdx.x & 63;
    int row = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (xg > 0) {
        // one wave per workgroup (xg = G): workgroup i merges a row of region
        // (i % 8) + 8 j, so it runs on that region's XCD
        const int j = blockIdx.x / 8;
        row = (int(blockIdx.x % 8) + 8 * (j / xg)) * xg + j % xg;
    }
    if (row >= rows) return;
    const int b = row / H;
    const int len = int(min(int64_t(max(min(lens[b], max_len), 0)), C));
    const int nb = (len + kBlk - 1) / kBlk;
    const int ns = min(splits, (nb + bps - 1) / bps);
    const float* pp = part + int64_t(row) * splits * (kD + 4);
    if (ns >= 1 && ns <= 16) {
        // up to 16 splits: every load (each split's maximum and sum, and the
        // lane's two dims of each partial output) in one round trip
        float2 v[16];
#pragma unroll
        for (int u = 0; u < 16; ++u)
            v[u] = *reinterpret_cast<const float2*>(pp + int64_t(min(u, ns - 1)) * (kD + 4) + 2 * lane);
        const float* q = pp + int64_t(min(lane, ns - 1)) * (kD + 4);
        const float mz = lane < ns ? q[kD] : -INFINITY;
        const float lz = q[kD + 1];
        float M = mz;
        for (int off = 32; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off, 64));
        const float f = lane < ns ? exp2f(mz - M) : 0.0f;
        float L = f * lz;
        for (int off = 32; off > 0; off >>= 1) L += __shfl_xor(L, off, 64);
        float o0 = 0.0f, o1 = 0.0f;
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            const float fu = __shfl(f, u, 64);
            if (u < ns) {
                o0 += fu * v[u].x;
                o1 += fu * v[u].y;
            }
        }
        const float x0 = L > 0.0f ? o0 / L : 0.0f, x1 = L > 0.0f ? o1 / L : 0.0f;
        *reinterpret_cast<uint32_t*>(out + int64_t(row) * kD + 2 * lane) =
            uint32_t(__half_as_ushort(__float2half_rn(x0))) |
            (uint32_t(__half_as_ushort(__float2half_rn(x1))) << 16);
        return;
    }
    float M = -INFINITY;
    for (int s0 = 0; s0 < ns; s0 += 64)
        if (s0 + lane < ns) M = fmaxf(M, pp[int64_t(s0 + lane) * (kD + 4) + kD]);
    for (int off = 32; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off, 64));
    float L = 0.0f, o0 = 0.0f, o1 = 0.0f;
    for (int s0 = 0; s0 < ns; s0 += 64) {
        float f = 0.0f, ls = 0.0f;
        if (s0 + lane < ns) {
            const float* q = pp + int64_t(s0 + lane) * (kD + 4);
            f = exp2f(q[kD] - M);
            ls = f * q[kD + 1];
        }
        for (int off = 32; off > 0; off >>= 1) ls += __shfl_xor(ls, off, 64);
        L += ls;
        const int n = min(64, ns - s0);
        for (int s1 = 0; s1 < n; s1 += 8) {
            float2 v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int ss = min(s1 + u, n - 1);
                v[u] = *reinterpret_cast<const float2*>(pp + int64_t(s0 + ss) * (kD + 4) + 2 * lane);
            }
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const float fu = __shfl(f, s1 + u, 64);
                if (s1 + u < n) {
                    o0 += fu * v[u].x;
                    o1 += fu * v[u].y;
                }
            }
        }
    }
    const float x0 = L > 0.0f ? o0 / L : 0.0f, x1 = L > 0.0f ? o1 / L : 0.0f;
    *reinterpret_cast<uint32_t*>(out + int64_t(row) * kD + 2 * lane) =
        uint32_t(__half_as_ushort(__float2half_rn(x0))) | (uint32_t(__half_as_ushort(__float2half_rn(x1))) << 16);
}

}  // namespace

int64_t kv4_cache_bytes(int64_t B, int64_t Hkv, int64_t C) { return B * Hkv * C * kRegionPerToken; }

// One workgroup per (sequence, KV head) when that gives ~512 workgroups
// (two rounds of 4-wave workgroups over the 256 CUs); fewer, longer
// contexts are cut into equal splits, at least one block per wave, merged by
// a second kernel. (Measured on MI355X: cutting every context into fixed
// 256-1024-token splits to even out ragged lengths is slower -- the
// per-workgroup query set-up and merge cost more than the imbalance.)
// The "kv4_splits" tuning key forces n splits. Unsplit batches of 2..256
// sequences whose pairs fit one per CU take the paired schedule (8-wave
// workgroups) when the longest context has 1024 tokens or more; the
// "kv4_paired" key set to "0" turns it off, set to "1" takes it whenever the
// batch allows it.
Kv4Plan plan_kv4(int64_t B, int64_t Hkv, int64_t max_len) {
    Kv4Plan p{};
    const int64_t nb = std::max<int64_t>(1, (max_len + kBlk - 1) / kBlk);
    const int64_t regions = std::max<int64_t>(1, B * Hkv);
    int64_t splits = (512 + regions - 1) / regions;
    // at most 32: the merge reads more than 16 splits in several rounds
    // (one context of 16K / 64K tokens on 8 KV heads: 64 splits 13.9 / 25.3
    // us, 32 splits 11.5 / 21.7 us)
    splits = std::max<int64_t>(1, std::min<int64_t>({splits, (nb + 3) / 4, int64_t(32)}));
    const std::string tune_splits = tuning(kTuneKv4Splits);
    if (!tune_splits.empty()) {
        const int v = std::atoi(tune_splits.c_str());
        if (v > 0) splits = std::min(v, 1 << 16);
    }
    p.splits = int(splits);
    p.bps = int(std::max<int64_t>(1, (nb + splits - 1) / splits));
    p.grid = B * Hkv * splits;
    p.waves = 4;
    // pairs as 8-wave workgroups, at most one per CU (more pairs than CUs
    // would run two contexts back to back per 4-wave workgroup, which costs
    // the fp16 cache more than it saves: 121 -> 133 us on 16 x 64 heads)
    // pairs only for contexts of 1024 tokens or more: the 8-wave pair
    // workgroups run one per CU, and short contexts gain more from the
    // 4-wave workgroups three to a CU (64 sequences of 128-512 tokens: 11.8
    // -> 9.6 us unpaired; of 512-2048: 21.8-22.2 paired, 22.4-22.9 not)
    const bool can_pair = splits == 1 && B >= 2 && B <= kPairMaxB && (B + 1) / 2 * Hkv <= 256;
    p.paired = can_pair && max_len >= 1024;
    const std::string tune_paired = tuning(kTuneKv4Paired);
    if (tune_paired == "0") p.paired = false;
    else if (tune_paired == "1") p.paired = can_pair;
    if (p.paired) {
        p.grid = (B + 1) / 2 * Hkv;
        p.waves = 8;
    }
    return p;
}

hipError_t launch_kv4_smooth(const uint16_t* k, int64_t T, int64_t Hkv, uint16_t* lam,
                             hipStream_t stream) {
    const int cols = int(Hkv * kD);
    return launch_kernel(kv4_smooth_kernel, dim3(unsigned((cols + 63) / 64)), dim3(256), 0, stream,
                         k, T, cols, lam);
}

hipError_t launch_kv4_append(const uint16_t* k, const uint16_t* v, int64_t B, int64_t Tn,
                             int64_t Hkv, const uint16_t* lam, const int32_t* start, uint8_t* cache,
                             int64_t C, hipStream_t stream) {
    const int64_t waves = B * Tn * Hkv;
    hipError_t e = launch_kernel(kv4_append_keys_kernel, dim3(unsigned((waves + 3) / 4)), dim3(256), 0,
                                 stream, k, v, int(B), int(Tn), int(Hkv), lam, start, cache, C);
    if (e != hipSuccess) return e;
    // blocks a run of Tn tokens can touch from any start
    const int nblk_touch = int((Tn + kBlk - 1) / kBlk + 1);
    const int64_t threads = B * Hkv * int64_t(nblk_touch) * 512;
    return launch_kernel(kv4_append_values_kernel, dim3(unsigned((threads + 255) / 256)), dim3(256), 0,
                         stream, v, int(B), int(Tn), int(Hkv), start, cache, C, nblk_touch);
}

int64_t kv4_workspace_bytes(const Kv4Plan& p, int64_t B, int64_t H) {
    return p.splits > 1 ? B * H * p.splits * (kD + 4) * int64_t(sizeof(float)) : 0;
}

// The fp16 cache takes its pairs in 4-wave workgroups: 66.4 against 73.4 us
// with 8 waves on the Llama-3-8B-shaped batch (64 sequences of 512-2048
// tokens), where the 4-bit cache needs the 8 waves (31.6 against 27.7 us).
template <bool kF16>
hipError_t launch_attention_kernel(const Kv4Plan& p, const AttnArgs& a, hipStream_t stream) {
    const dim3 grid(unsigned(p.grid));
    if constexpr (!kF16) {
        if (p.waves == 8)
            return launch_kernel(kv4_attention_kernel<false, 8>, grid, dim3(512), 0, stream, a);
    }
    return launch_kernel(kv4_attention_kernel<kF16, 4>, grid, dim3(256), 0, stream, a);
}

hipError_t launch_kv4_attention(const Kv4Plan& p, const uint16_t* q, int64_t B, int64_t H,
                                int64_t Hkv, const uint16_t* lam, const uint8_t* cache, int64_t C,
                                const int32_t* lens, int64_t max_len, uint16_t* out, float* part,
                                hipStream_t stream) {
    AttnArgs a{q, lam, cache, lens, out, part, C, int(B), int(H), int(Hkv), int(H / Hkv), p.splits,
               p.bps, int(max_len), p.paired ? 1 : 0};
    hipError_t e = launch_attention_kernel<false>(p, a, stream);
    if (e != hipSuccess || p.splits == 1) return e;
    const int rows = int(B * H);
    // one wave per workgroup, numbered so that row r's merge runs on the XCD
    // whose split workgroups wrote its partials (region r / G, split-major
    // above): 22.4 -> 22.0 us on 4 x 8-16K tokens against 4 rows per
    // workgroup; needs the regions in whole rounds of 8
    if ((B * Hkv) % 8 == 0)
        return launch_kernel(kv4_combine_kernel, dim3(unsigned(rows)), dim3(64), 0, stream,
                             (const float*)part, rows, int(H), p.splits, p.bps, lens, int(max_len),
                             C, out, int(H / Hkv));
    return launch_kernel(kv4_combine_kernel, dim3(unsigned((rows + 3) / 4)), dim3(256), 0, stream,
                         (const float*)part, rows, int(H), p.splits, p.bps, lens, int(max_len), C,
                         out, 0);
}

int64_t kv16_cache_bytes(int64_t B, int64_t Hkv, int64_t C) { return B * Hkv * C * 4 * kD; }

hipError_t launch_kv16_append(const uint16_t* k, const uint16_t* v, int64_t B, int64_t Tn,
                              int64_t Hkv, const int32_t* start, uint8_t* cache, int64_t C,
                              hipStream_t stream) {
    const int64_t waves = B * Tn * Hkv;
    return launch_kernel(kv16_append_kernel, dim3(unsigned((waves + 3) / 4)), dim3(256), 0, stream,
                         k, v, int(B), int(Tn), int(Hkv), start, cache, C);
}

hipError_t launch_kv16_attention(const Kv4Plan& p, const uint16_t* q, int64_t B, int64_t H,
                                 int64_t Hkv, const uint8_t* cache, int64_t C, const int32_t* lens,
                                 int64_t max_len, uint16_t* out, float* part, hipStream_t stream) {
    AttnArgs a{q, nullptr, cache, lens, out, part, C, int(B), int(H), int(Hkv), int(H / Hkv),
               p.splits, p.bps, int(max_len), p.paired ? 1 : 0};
    hipError_t e = launch_attention_kernel<true>(p, a, stream);
    if (e != hipSuccess || p.splits == 1) return e;
    const int rows = int(B * H);
    return launch_kernel(kv4_combine_kernel, dim3(unsigned((rows + 3) / 4)), dim3(256), 0, stream,
                         (const float*)part, rows, int(H), p.splits, p.bps, lens, int(max_len), C,
                         out, 0);
}

}  // namespace qoq
