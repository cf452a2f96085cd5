// Weight-streaming family of the W4A8 GEMM (gfx950): up to 64 tokens, where
// the HBM stream of packed weights bounds the GEMM.
//
// Main loop as in the other families (pages: velog notes on QServe,
// "Methods / 1) Algorithm: QoQ" and "Methods / 2) System: QServe"): packed
// UINT4 codes in MFMA operand order, one packed 16-bit multiply-add per 4
// weights inside the protective range, XOR 0x80 per byte to INT8,
// v_mfma_i32_32x32x32_i8 accumulating INT32 over the workgroup's K range.
//
// Work split: a workgroup of NW waves covers 32 MT tokens (all of them for
// the shapes it is planned for; grid z takes further row tiles) and
// 32 CB NW output columns over a range of K; wave w owns CB 32-column tiles.
//   * Activations are shared by all waves through LDS in chunks of CH
//     groups (4 MT fragments of 1 KiB per group), loaded by buffer loads
//     that write LDS directly, one chunk ahead into the other of two slots:
//     one barrier per chunk instead of one per group.
//   * Each wave streams its packed weights through a register ring PD
//     groups deep, continuously across chunks, so the HBM stream of a wave
//     never waits for the other waves.
//   * Split K: with `part`, workgroup row y of the grid covers groups
//     [y gps, (y + 1) gps) and stores exact INT32 partial sums for the
//     second kernel (integer addition: bit-identical to the unsplit sum).
#include "qoq_internal.hpp"
#include "kernel_common.hpp"

#include <hip/hip_fp16.h>

namespace qoq {
namespace {

// 16 bytes per lane from a buffer straight into LDS: lane l writes bytes
// 16 l .. 16 l + 15 after `lds` (the wave-uniform destination).
__device__ __forceinline__ void buffer_load_lds16(__amdgpu_buffer_rsrc_t rsrc, void* lds, int voffset,
                                                  int soffset) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (__attribute__((address_space(3))) void*)lds, 16,
                                             voffset, soffset, 0, 0);
}

// s_waitcnt immediate: at most n vector-memory operations of this wave
// outstanding (expcnt and lgkmcnt left at their maximum).
constexpr int vmcnt_imm(int n) { return 0x0f70 | (n & 0xf) | (((n >> 4) & 3) << 14); }

template <int MT, int CB, int NW, int PD, int CH>
__global__ void __launch_bounds__(64 * NW) gemm_stream_kernel(
    const int8_t* __restrict__ x8, const float* __restrict__ s_x, int M, int K,
    const uint8_t* __restrict__ nib, const uint8_t* __restrict__ rec, int ng8,
    const uint16_t* __restrict__ s1, int N, uint16_t* __restrict__ y,
    int32_t* __restrict__ acc_debug, int gps, int32_t* __restrict__ part) {
    constexpr int AF = 4 * MT;                    // A fragments per group
    constexpr int CF = CH * AF;                   // A fragments per chunk
    constexpr int FW = (CF + NW - 1) / NW;        // fragments per wave and chunk (at most)
    static_assert(CH % PD == 0, "ring depth divides the chunk");
    constexpr int kSlotBytes = CF * 1024;
    static_assert(2 * kSlotBytes <= 160 * 1024, "LDS slots above 160 KiB");
    __shared__ __attribute__((aligned(1024))) v4i As[2 * CF * 64];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int j = lane & 31;
    const int q = lane >> 5;
    const int c = lane & 15;
    const int ng = K >> 7;
    const int nbt = N >> 4;
    const int nbw = (blockIdx.x * NW + wave) * 2 * CB;   // this wave's first 16-column block
    const int g0 = blockIdx.y * gps;
    const int cnt = min(ng - g0, gps);            // >= 1 by the grid
    const int nch = (cnt + CH - 1) / CH;
    const int m0 = blockIdx.z * 32 * MT;

    const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
        (void*)x8, (short)0, int(act_bytes(M, K)), 0x00020000);
    const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
        (void*)nib, (short)0, nbt * ng * kBlockBytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t rr = __builtin_amdgcn_make_buffer_rsrc(
        (void*)rec, (short)0, nbt * ng8 * kRecChunkBytes, 0x00020000);
    // Chunk fragment fi = wave + NW u: group fi / AF of the chunk, fragment
    // f = fi % AF = (row tile f / 4, step f % 4); lane (j, q) reads row
    // 32 (f / 4) + j (rows at or beyond M read the last row, never stored),
    // inputs 32 (f % 4) + 16 q .. + 15 of the group.
    int a_off[FW], a_grp[FW];
#pragma unroll
    for (int u = 0; u < FW; ++u) {
        const int fi = min(wave + NW * u, CF - 1), f = fi % AF;
        a_off[u] = int(act_row_offset(min(m0 + 32 * (f >> 2) + j, M - 1), K)) + kActUnit * q +
                   2 * kActUnit * (f & 3);
        a_grp[u] = fi / AF;
    }
    auto load_chunk = [&](int slot, int ch) {
        char* base = reinterpret_cast<char*>(As) + slot * kSlotBytes;
#pragma unroll
        for (int u = 0; u < FW; ++u) {
            if (CF % NW != 0 && wave + NW * u >= CF) break;   // wave-uniform
            const int g = g0 + min(ch * CH + a_grp[u], cnt - 1);
            buffer_load_lds16(ra, base + (wave + NW * u) * 1024, a_off[u], g * kActGroupBytes);
        }
    };
    // B of 32-column tile t: lane (j, q) is column j, in block nbw + 2t + j/16
    // (clamped; never stored past N), packed lanes c + 16 q and c + 16 (q + 2).
    int b_off[CB], r_off[CB];
#pragma unroll
    for (int t = 0; t < CB; ++t) {
        const int blk = min(nbw + 2 * t + (j >> 4), nbt - 1);
        b_off[t] = blk * ng * kBlockBytes + (c + 16 * q) * 16;
        r_off[t] = (blk * ng8 * kBlockCols + c) * (kRecChunk * 2);
    }
    uint4 qn[PD][CB][2];
    uint32_t rs[PD][CB];
    auto load_b = [&](int p, int i) {
        const int g = g0 + min(i, cnt - 1);
#pragma unroll
        for (int t = 0; t < CB; ++t) {
            qn[p][t][0] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                rb, b_off[t], g * kBlockBytes, 0));
            qn[p][t][1] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                rb, b_off[t], g * kBlockBytes + 512, 0));
            rs[p][t] = __builtin_amdgcn_raw_buffer_load_b16(
                rr, r_off[t], (g >> 3) * kRecChunkBytes + (g & 7) * 2, 0);
        }
    };

    // epilogue scales, fetched now: rows 8 (r / 4) + 4 q + r % 4 of row tile
    // mt, column j of tile t
    float sw[CB];
#pragma unroll
    for (int t = 0; t < CB; ++t) sw[t] = h2f(s1[min(16 * nbw + 32 * t + j, N - 1)]);

    v16i acc[MT][CB];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int t = 0; t < CB; ++t)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[mt][t][r] = 0;

    auto compute = [&](int p, int slot, int gg) {
        const v4i* A = As + (slot * CF + gg * AF) * 64;
#pragma unroll
        for (int t = 0; t < CB; ++t) {
            v4i bq[4];
            dequant_block(qn[p][t][0], rs[p][t], bq[0], bq[2]);
            dequant_block(qn[p][t][1], rs[p][t], bq[1], bq[3]);
#pragma unroll
            for (int st = 0; st < 4; ++st)
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
                    acc[mt][t] = __builtin_amdgcn_mfma_i32_32x32x32_i8(A[(4 * mt + st) * 64 + lane],
                                                                      bq[st], acc[mt][t], 0, 0, 0);
        }
    };

    // Prologue: activations of chunk 0, then the weight ring.
    load_chunk(0, 0);
#pragma unroll
    for (int p = 0; p < PD; ++p) load_b(p, p);
    // Loads per group of the weight stream, issued after a chunk's
    // activation loads until the next chunk begins (the waits below count
    // only these, so the number of activation loads per wave may differ).
    constexpr int kB = 3 * CB;
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(PD * kB));
    __syncthreads();
    for (int ch = 0; ch < nch; ++ch) {
        const int slot = ch & 1;
        // the other slot was read in chunk ch - 1, which every wave has left
        // (the barrier before this chunk)
        load_chunk(slot ^ 1, ch + 1);
        __builtin_amdgcn_sched_barrier(0);
        const int i0 = ch * CH;
#pragma unroll
        for (int gg = 0; gg < CH; ++gg) {
            const int p = gg % PD;
            if (i0 + gg < cnt) compute(p, slot, gg);
            __builtin_amdgcn_sched_barrier(0);
            load_b(p, i0 + gg + PD);
            __builtin_amdgcn_sched_barrier(0);
        }
        // this wave's fragments of chunk ch + 1 (issued before the CH refills
        // of the weight ring), then the barrier publishes every wave's
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(CH * kB));
        __syncthreads();
    }
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));

    // Lane (j, q), register r of tile (mt, t) holds row 32 mt + 8 (r / 4) +
    // 4 q + r % 4, column 32 t + j of the wave's columns.
#pragma unroll
    for (int t = 0; t < CB; ++t) {
        const int n = 16 * nbw + 32 * t + j;
        if (n >= N) continue;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int m = m0 + 32 * mt + 8 * (r >> 2) + 4 * q + (r & 3);
                if (m >= M) continue;
                const int64_t o = int64_t(m) * N + n;
                const int32_t v = acc[mt][t][r];
                if (part) {
                    part[int64_t(blockIdx.y) * M * N + o] = v;
                    continue;
                }
                if (acc_debug) acc_debug[o] = v;
                y[o] = epilogue_value(v, s_x[m], sw[t]);
            }
    }
}

template <int MT, int CB, int NW, int PD, int CH>
hipError_t launch_one(const GemmPlan& p, const GemmArgs& a, int32_t* part, hipStream_t stream) {
    return launch_kernel(gemm_stream_kernel<MT, CB, NW, PD, CH>,
                         dim3(p.grid_x, p.splits, (a.M + 32 * MT - 1) / (32 * MT)),
                         dim3(64 * NW), 0, stream, a.x8, a.s_x, a.M, a.K, a.nib, a.rec, a.ng8,
                         a.s1, a.N, a.y, a.acc_debug, p.groups_per_split, part);
}

}  // namespace

// (MT, CB, NW, PD ring depth, CH groups per activation chunk)
#define QOQ_STREAM_CONFIGS(X)                                                        \
    X(2, 1, 8, 4, 8) X(2, 1, 8, 4, 4) X(2, 1, 6, 4, 8) X(2, 1, 4, 4, 8)              \
    X(2, 1, 8, 8, 8) X(2, 2, 8, 4, 8) X(2, 1, 12, 4, 8) X(1, 1, 8, 4, 8)             \
    X(1, 2, 8, 4, 8) X(2, 1, 16, 4, 8) X(2, 1, 3, 4, 8) X(1, 1, 4, 4, 8)             \
    X(2, 2, 4, 4, 8) X(2, 1, 6, 8, 8)

bool stream_config_exists(int mt, int cb, int nw, int pd, int ch) {
#define X(a, b, c, d, e) if (mt == a && cb == b && nw == c && pd == d && ch == e) return true;
    QOQ_STREAM_CONFIGS(X)
#undef X
    return false;
}

hipError_t launch_stream(const GemmPlan& p, const GemmArgs& a, int32_t* part, hipStream_t stream) {
#define X(A, B, C, D, E)                                                                 \
    if (p.mt == A && p.cb == B && p.nw == C && p.pd == D && p.pa == E)                   \
        return launch_one<A, B, C, D, E>(p, a, part, stream);
    QOQ_STREAM_CONFIGS(X)
#undef X
    return hipErrorInvalidConfiguration;
}

}  // namespace qoq
