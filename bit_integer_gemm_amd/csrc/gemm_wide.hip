// Wide-tile family of the W4A8 GEMM (gfx950): large token counts, where the
// INT8 matrix pipes bound the GEMM.
//
// Main loop (pages: velog notes on QServe, "Methods / 1) Algorithm: QoQ" and
// "Methods / 2) System: QServe"; "Part5 LLM部署技术" section 3): packed UINT4
// codes arrive in MFMA operand order; one packed 16-bit multiply-add per 4
// weights computes q4*s2 + (128 - z*s2) inside the protective range and
// XOR 0x80 per byte gives the INT8 weight ("subtraction after
// multiplication"); v_mfma_i32_32x32x32_i8 accumulates INT32 over all of K
// (or over the workgroup's K range, whose exact partial sums a second
// kernel adds). No partial sum is ever scaled.
//
// Work split: a workgroup of NW waves side by side along N computes a
// (32 MT) x (32 CB NW) tile; wave w owns CB 32-column tiles and all MT
// 32-row tiles, so every weight is dequantized once per workgroup.
//   * Activations: the 4 MT fragments of a group (32 rows x 32 inputs each,
//     1 KiB, lane l at 16 l) go straight from global memory into LDS with
//     buffer loads that write LDS (no VGPR staging, no LDS store
//     instructions), R - 1 groups ahead, into a ring of R slots. One barrier
//     per group: before it each wave waits for its own share of the next
//     group's fragments; after it the slot read two groups ago is free.
//   * Weights: each wave loads its packed fragments into a register ring
//     two groups deep and dequantizes them half a group ahead of the MFMAs
//     that use them: while the MFMAs of steps 0 and 2 of group i run, the
//     VALU unpacks steps 1 and 3 of group i; while those of steps 1 and 3
//     run, it unpacks steps 0 and 2 of group i + 1. Scheduling groups place
//     a few VALU instructions after every MFMA, so the matrix pipe and the
//     VALU of one SIMD work at the same time.
//   * Epilogue through LDS with 16-byte row-segment stores; XCD-aware
//     grouped tile order; split K as in the other tile family.
#include "qoq_internal.hpp"
#include "kernel_common.hpp"

#include <hip/hip_fp16.h>

namespace qoq {
namespace {

// 16 bytes per lane from a buffer straight into LDS: lane l writes bytes
// 16 l .. 16 l + 15 after `lds` (the wave-uniform destination).
__device__ __forceinline__ void buffer_load_lds16(__amdgpu_buffer_rsrc_t rsrc, void* lds, int voffset,
                                                  int soffset) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rsrc, (__attribute__((address_space(3))) void*)lds, 16, voffset, soffset,
        0, 0);
}

// s_waitcnt immediate that waits until at most n vector-memory operations of
// this wave are outstanding (expcnt and lgkmcnt left at their maximum).
constexpr int vmcnt_imm(int n) { return 0x0f70 | (n & 0xf) | (((n >> 4) & 3) << 14); }

template <int MT, int CB, int NW, int R, int MINB>
__global__ void __launch_bounds__(64 * NW, MINB) gemm_wide_kernel(
    const int8_t* __restrict__ x8, const float* __restrict__ s_x, int M, int K,
    const uint8_t* __restrict__ nib, const uint8_t* __restrict__ rec, int ng8,
    const uint16_t* __restrict__ s1, int N, uint16_t* __restrict__ y,
    int32_t* __restrict__ acc_debug, int gps, int32_t* __restrict__ part) {
    constexpr int AF = 4 * MT;                    // A fragments per group
    static_assert(AF % NW == 0, "every wave loads the same number of fragments");
    constexpr int AFW = AF / NW;                  // fragments per wave
    static_assert(R >= 3, "the ring needs a slot in flight beyond the two in use");
    constexpr int kSlotBytes = AF * 1024;
    constexpr int kRingBytes = R * kSlotBytes;
    constexpr int kStageBytes = NW * 32 * 32 * CB * 2;
    static_assert(kRingBytes <= 160 * 1024, "LDS ring above 160 KiB");
    __shared__ __attribute__((aligned(1024))) v4i lds_raw[(kRingBytes > kStageBytes ? kRingBytes : kStageBytes) / 16];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int j = lane & 31;
    const int q = lane >> 5;
    const int c = lane & 15;
    const int ng = K >> 7;
    const int nbt = N >> 4;
    constexpr int BM = 32 * MT, BNB = 2 * CB * NW;   // tile rows, tile 16-column blocks
    const int tiles_m = (M + BM - 1) / BM;
    const int tiles_n = (nbt + BNB - 1) / BNB;
    int tm, tn;
    tile_of(blockIdx.x, tiles_m, tiles_n, tm, tn);
    const int m0 = tm * BM;
    const int nbw = tn * BNB + wave * 2 * CB;     // this wave's first 16-column block
    const int g0 = blockIdx.y * gps;
    const int cnt = min(ng - g0, gps);            // >= 1 by the grid

    const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
        (void*)x8, (short)0, int(act_bytes(M, K)), 0x00020000);
    const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
        (void*)nib, (short)0, nbt * ng * kBlockBytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t rr = __builtin_amdgcn_make_buffer_rsrc(
        (void*)rec, (short)0, nbt * ng8 * kRecChunkBytes, 0x00020000);
    // A fragment f = (row tile f / 4, step f % 4): lane (j, q) reads row
    // m0 + 32 (f / 4) + j, inputs 32 (f % 4) + 16 q .. + 15 of the group, i.e.
    // row offset + 256 q + 512 (f % 4) + 2048 g in the activation tile layout;
    // rows at or beyond M read the last row (never stored). Wave w loads
    // fragments w, w + NW, ... of every group.
    int a_off[AFW];
#pragma unroll
    for (int u = 0; u < AFW; ++u) {
        const int f = wave + NW * u;
        a_off[u] = int(act_row_offset(min(m0 + 32 * (f >> 2) + j, M - 1), K)) + kActUnit * q +
                   2 * kActUnit * (f & 3);
    }
    // B of 32-column tile t: lane (j, q) is column j, in 16-column block
    // nbw + 2t + j / 16 (clamped; never stored past N), packed lanes c + 16 q
    // (steps 0, 2) and c + 16 (q + 2) (steps 1, 3).
    int b_off[CB], r_off[CB];
#pragma unroll
    for (int t = 0; t < CB; ++t) {
        const int blk = min(nbw + 2 * t + (j >> 4), nbt - 1);
        b_off[t] = blk * ng * kBlockBytes + (c + 16 * q) * 16;
        r_off[t] = (blk * ng8 * kBlockCols + c) * (kRecChunk * 2);
    }

    v16i acc[MT][CB];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int t = 0; t < CB; ++t)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[mt][t][r] = 0;

    // group i of the range (clamped to its last group past the end)
    auto grp = [&](int i) { return g0 + min(i, cnt - 1); };
    auto load_a = [&](int slot, int i) {
        const int g = grp(i);
        char* base = reinterpret_cast<char*>(lds_raw) + slot * kSlotBytes;
#pragma unroll
        for (int u = 0; u < AFW; ++u)
            buffer_load_lds16(ra, base + (wave + NW * u) * 1024, a_off[u], g * kActGroupBytes);
    };
    uint4 qn[3][CB][2];       // packed weights, group i in entry i % 3
    uint32_t rs[3][CB];       // its group records (s2, 128 - z s2)
    auto load_b = [&](int e, int i) {
        const int g = grp(i);
#pragma unroll
        for (int t = 0; t < CB; ++t) {
            qn[e][t][0] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                rb, b_off[t], g * kBlockBytes, 0));
            qn[e][t][1] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                rb, b_off[t], g * kBlockBytes + 512, 0));
            rs[e][t] = __builtin_amdgcn_raw_buffer_load_b16(
                rr, r_off[t], (g >> 3) * kRecChunkBytes + (g & 7) * 2, 0);
        }
    };
    // INT8 weights of the MFMA steps: bq[t][s] for step s of the current
    // group (steps 0 and 2 come from the low and high nibbles of the first
    // packed chunk, steps 1 and 3 from the second)
    v4i bq[CB][4];
    auto dequant_half = [&](int e, int h) {
#pragma unroll
        for (int t = 0; t < CB; ++t)
            dequant_block(qn[e][t][h], rs[e][t], bq[t][h], bq[t][h + 2]);
    };
    // The 32 x 32 MFMA steps of one group in the order (st 0, 2, then 1, 3) x
    // row tiles; A fragment k of that order is read from LDS PF fragments
    // before its MFMAs (a register ring of PF + 1), so the LDS latency hides
    // behind the MFMAs of the PF fragments before.
    constexpr int PF = 4;
    constexpr int NF = 4 * MT;                    // fragments (and MFMA groups) per group
    auto frag_index = [](int k) {                 // k -> (row tile, step) slot in LDS
        const int half = k / (2 * MT), r = k % (2 * MT);
        const int st = half + 2 * (r / MT);
        return 4 * (r % MT) + st;
    };
    auto frag_step = [](int k) {
        const int half = k / (2 * MT), r = k % (2 * MT);
        return half + 2 * (r / MT);
    };
    // Own loads that may stay in flight at the end of a step: those of the
    // R - 2 later steps, plus the weight loads issued after this wave's share
    // of the next group's fragments.
    constexpr int kLoadsPerStep = AFW + 3 * CB;
    constexpr int kAllowed = (R - 2) * kLoadsPerStep + 3 * CB;
    static_assert(kAllowed < 64, "vmcnt holds at most 63");
    constexpr int kValuTotal = 62 * CB;           // dequantization of one group (about)
    constexpr int kValuPer = (kValuTotal + NF * CB - 1) / (NF * CB);
    // Step i: the A fragments of group i + R - 1 go to the slot read in step
    // i - 1; then in one scheduling region the MFMAs of group i (steps 0, 2
    // with steps 1, 3 of group i dequantized alongside, then steps 1, 3 with
    // steps 0, 2 of group i + 1 dequantized alongside), a few VALU
    // instructions after every MFMA and each LDS read two fragments ahead;
    // then the packed weights of group i + 3 refill entry i % 3; finally
    // this wave's fragments of group i + 1 are waited for and the barrier
    // publishes them.
    auto step = [&](int i, int u, bool full) {
        load_a((u + R - 1) % R, i + R - 1);
        __builtin_amdgcn_sched_barrier(0);
        const int e = u % 3, en = (u + 1) % 3;
        if (full || i < cnt) {
            const v4i* A = lds_raw + (u % R) * (kSlotBytes / 16);
            v4i a[PF + 1];
#pragma unroll
            for (int k = 0; k < PF; ++k) a[k] = A[frag_index(k) * 64 + lane];
#pragma unroll
            for (int k = 0; k < NF; ++k) {
                if (k + PF < NF) a[(k + PF) % (PF + 1)] = A[frag_index(k + PF) * 64 + lane];
                const int st = frag_step(k), mt = (k % (2 * MT)) % MT;
#pragma unroll
                for (int t = 0; t < CB; ++t)
                    acc[mt][t] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[k % (PF + 1)], bq[t][st],
                                                                       acc[mt][t], 0, 0, 0);
                if (k == 0) dequant_half(e, 1);
                if (k == 2 * MT && (full || i + 1 < cnt)) dequant_half(en, 0);
            }
            __builtin_amdgcn_sched_group_barrier(0x100, PF, 0);                    // LDS reads
#pragma unroll
            for (int k = 0; k < NF; ++k) {
#pragma unroll
                for (int t = 0; t < CB; ++t) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);              // MFMA
                    __builtin_amdgcn_sched_group_barrier(0x002, kValuPer, 0);       // VALU
                }
                if (k + PF < NF) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0); // LDS read
            }
        }
        __builtin_amdgcn_sched_barrier(0);
        load_b(e, i + 3);
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(kAllowed));
        __syncthreads();
    };

    // prologue: fragments of groups 0 .. R - 2, packed weights of groups 0 .. 2
#pragma unroll
    for (int s = 0; s < R - 1; ++s) load_a(s, s);
    load_b(0, 0);
    load_b(1, 1);
    load_b(2, 2);
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(6 * CB));
    __builtin_amdgcn_sched_barrier(0);
    dequant_half(0, 0);
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));   // this wave's fragments of group 0
    __syncthreads();
    // unroll: a multiple of R (LDS slot) and of 3 (weight entry)
    constexpr int U = R % 3 == 0 ? R : 3 * R;
    int i0 = 0;
    for (; i0 + U <= cnt; i0 += U) {
#pragma unroll
        for (int u = 0; u < U; ++u) step(i0 + u, u, true);
    }
    if (i0 < cnt) {
#pragma unroll
        for (int u = 0; u < U; ++u) step(i0 + u, u, false);
    }
    // drain: no buffer load may still write LDS when the epilogue reuses it
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    __syncthreads();

    if (part) {   // split K: the exact partial sums
        int32_t* pz = part + int64_t(blockIdx.y) * M * N;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int t = 0; t < CB; ++t)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int m = m0 + 32 * mt + 8 * (r >> 2) + 4 * q + (r & 3);
                    const int n = 16 * nbw + 32 * t + j;
                    if (m < M && n < N) pz[int64_t(m) * N + n] = acc[mt][t][r];
                }
        return;
    }

    // Epilogue through LDS: per 32-row tile, each wave converts its
    // 32 x 32CB block to fp16 into a staging area, then writes it out as
    // 16-byte row segments. Lane (j, q), register r of tile (mt, t) holds
    // row 32mt + 8(r/4) + 4q + r%4, column 32t + j of the wave's columns.
    uint16_t* stage = reinterpret_cast<uint16_t*>(lds_raw) + wave * (32 * 32 * CB);
    const int n0w = 16 * nbw;
    float sw[CB];
#pragma unroll
    for (int t = 0; t < CB; ++t) sw[t] = h2f(s1[min(n0w + 32 * t + j, N - 1)]);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        float sxr[16];
#pragma unroll
        for (int r = 0; r < 16; ++r)
            sxr[r] = s_x[min(m0 + 32 * mt + 8 * (r >> 2) + 4 * q + (r & 3), M - 1)];
#pragma unroll
        for (int t = 0; t < CB; ++t)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = 8 * (r >> 2) + 4 * q + (r & 3);
                stage[row * (32 * CB) + 32 * t + j] = epilogue_value(acc[mt][t][r], sxr[r], sw[t]);
            }
        if (acc_debug) {
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

template <int MT, int CB, int NW, int R, int MINB>
hipError_t launch_one(const GemmPlan& p, const GemmArgs& a, int32_t* part, hipStream_t stream) {
    return launch_kernel(gemm_wide_kernel<MT, CB, NW, R, MINB>, dim3(p.grid_x, p.splits),
                         dim3(64 * NW), 0, stream, a.x8, a.s_x, a.M, a.K, a.nib, a.rec, a.ng8,
                         a.s1, a.N, a.y, a.acc_debug, p.groups_per_split, part);
}

}  // namespace

// (MT, CB, NW, R, workgroups per CU)
#define QOQ_WIDE_CONFIGS(X)                                                          \
    X(4, 2, 8, 3, 1) X(4, 2, 8, 4, 1) X(8, 1, 8, 3, 1) X(8, 1, 8, 4, 1)              \
    X(4, 1, 8, 4, 1) X(4, 2, 4, 4, 1) X(4, 1, 4, 4, 2) X(2, 1, 8, 4, 1)              \
    X(8, 2, 4, 3, 1) X(8, 2, 4, 4, 1)

bool wide_config_exists(int mt, int cb, int nw, int r, int minb) {
#define X(a, b, c, d, e) if (mt == a && cb == b && nw == c && r == d && minb == e) return true;
    QOQ_WIDE_CONFIGS(X)
#undef X
    return false;
}

hipError_t launch_wide(const GemmPlan& p, const GemmArgs& a, int32_t* part, hipStream_t stream) {
#define X(A, B, C, D, E)                                                                 \
    if (p.mt == A && p.cb == B && p.nw == C && p.pd == D && p.pa == E)                   \
        return launch_one<A, B, C, D, E>(p, a, part, stream);
    QOQ_WIDE_CONFIGS(X)
#undef X
    return hipErrorInvalidConfiguration;
}

}  // namespace qoq
