// K-split 32x32 family of the W4A8 GEMM (gfx950): mid-size token counts on
// layers with few output tiles.
//
// Main loop as in the other families (pages: velog notes on QServe,
// "Methods / 1) Algorithm: QoQ" and "Methods / 2) System: QServe"): packed
// UINT4 codes arrive in MFMA operand order, one packed 16-bit multiply-add
// per 4 weights computes q4*s2 + (128 - z*s2) inside the protective range,
// XOR 0x80 per byte gives the INT8 weight, and v_mfma_i32_32x32x32_i8
// accumulates INT32 over all of K. No partial sum is ever scaled.
//
// Work split: a workgroup owns a (32 MT) x (32 CB) output tile and all of K;
// its KW waves take contiguous ranges of the 128-input groups and each keeps
// PD groups of activation fragments and packed weights in flight in a
// register ring (loaded straight from global memory: nothing is shared
// between the waves, so there is no barrier in the main loop). A wave reads
// the group records of its whole range into its own LDS area once, with
// 16-byte loads, when the range spans at most 8 record chunks; longer ranges
// carry one 2-byte record load per group in the ring. The
// KW partial INT32 tiles are added in LDS (integer addition: the sum is the
// same in any order) and the epilogue writes the tile. Compared with the
// 16-row decode family this issues the full-rate 32x32x32 INT8 MFMA and
// dequantizes each weight fragment for 32 MT tokens; compared with the
// 32x32 tile family (K whole per wave, activations shared in LDS) it keeps
// the output tile small, so layers with few output columns still fill every
// CU without a second kernel.
#include "qoq_internal.hpp"
#include "kernel_common.hpp"

#include <hip/hip_fp16.h>

namespace qoq {
namespace {

// Record chunks (8 groups each) a wave stages in LDS; a range of up to
// kRecLdsMaxGroups groups starting anywhere spans at most that many.
constexpr int kRecLdsChunks = 8;
constexpr int kRecLdsMaxGroups = 8 * kRecLdsChunks - 7;

template <int MT, int CB, int KW, int PD, bool RL>
__global__ void __launch_bounds__(64 * KW) gemm_ksplit32_kernel(
    const int8_t* __restrict__ x8, const float* __restrict__ s_x, int M, int K,
    const uint8_t* __restrict__ nib, const uint8_t* __restrict__ rec, int ng8,
    const uint16_t* __restrict__ s1, int N, uint16_t* __restrict__ y,
    int32_t* __restrict__ acc_debug) {
    constexpr int T = MT * CB;                    // 32x32 accumulator tiles per wave
    // LDS for the cross-wave sum: at most 128 KiB; with more partial tiles
    // the upper half of the waves first folds into the lower half
    constexpr int KR = KW * T * 4096 <= 128 * 1024 ? KW : KW / 2;
    static_assert(KR * T * 4096 <= 128 * 1024, "LDS reduction buffer above 128 KiB");
    // RL: the group records of each wave's range staged in LDS (CB tiles x
    // 2 blocks x 8 record chunks of 256 bytes per wave), sharing the space
    // of the cross-wave sum, which only starts after every wave's loop
    constexpr int kRedInts = KR * T * 16 * 64;
    constexpr int kRecWaveU16 = CB * 2 * kRecLdsChunks * 128;
    constexpr int kRecInts = RL ? KW * kRecWaveU16 / 2 : 0;
    __shared__ __attribute__((aligned(16))) int red[kRedInts > kRecInts ? kRedInts : kRecInts];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int j = lane & 31;
    const int q = lane >> 5;
    const int c = lane & 15;
    const int ng = K >> 7;
    const int nbt = N >> 4;
    const int tiles_m = (M + 32 * MT - 1) / (32 * MT);
    const int tiles_n = (nbt + 2 * CB - 1) / (2 * CB);
    int tm, tn;
    tile_of(blockIdx.x, tiles_m, tiles_n, tm, tn);
    const int m0 = tm * 32 * MT;
    const int nb0 = tn * 2 * CB;                  // first 16-column block of the tile
    const int gpw = (ng + KW - 1) / KW;
    const int gb = min(ng, wave * gpw);
    const int cnt = min(ng, gb + gpw) - gb;

    const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
        (void*)x8, (short)0, int(act_bytes(M, K)), 0x00020000);
    const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
        (void*)nib, (short)0, nbt * ng * kBlockBytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t rr = __builtin_amdgcn_make_buffer_rsrc(
        (void*)rec, (short)0, nbt * ng8 * kRecChunkBytes, 0x00020000);
    // A operand of row tile mt, step st of group g: lane (j, q) takes row
    // m0 + 32 mt + j, inputs 32 st + 16 q .. + 15 of the group; in the
    // activation tile layout that is row offset + 256 q + 2048 g + 512 st.
    // Rows at or beyond M read the last row (never stored).
    int a_off[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
        a_off[mt] = int(act_row_offset(min(m0 + 32 * mt + j, M - 1), K)) + kActUnit * q;
    // B operand of column tile cb: lane (j, q) is column j of the tile, in
    // 16-column block nb0 + 2 cb + j / 16 (clamped: columns past N are
    // never stored); it loads packed lanes c + 16 q (steps 0, 2) and
    // c + 16 (q + 2) (steps 1, 3) of the block.
    int b_off[CB], r_off[CB];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
        const int blk = min(nb0 + 2 * cb + (j >> 4), nbt - 1);
        b_off[cb] = blk * ng * kBlockBytes + (c + 16 * q) * 16;
        r_off[cb] = (blk * ng8 * kBlockCols + c) * (kRecChunk * 2);
    }
    // RL: this wave's records in LDS, [cb][block of the tile][chunk - c0]
    // [channel][group % 8]; lane (j, q) reads its channel's entry
    uint16_t* rl = reinterpret_cast<uint16_t*>(red) + wave * kRecWaveU16;
    const int c0 = gb >> 3;
    auto rec_lds = [&](int cb, int g) {
        return uint32_t(rl[((cb * 2 + (j >> 4)) * kRecLdsChunks + (g >> 3) - c0) * 128 + c * 8 + (g & 7)]);
    };

    v16i acc[MT][CB];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[mt][cb][r] = 0;

    // Epilogue scales of this thread's outputs (see the end), fetched now so
    // the epilogue waits for no load: output quad e is four consecutive
    // columns of one row of the tile.
    constexpr int QUADS = T * 16 * 16;            // groups of 4 lanes per wave's tiles
    constexpr int IT = (QUADS + 64 * KW - 1) / (64 * KW);
    auto quad_row = [&](int e) {
        const int l4 = (e & 15) * 4, r = (e >> 4) & 15, t = e >> 8;
        return m0 + 32 * (t / CB) + 8 * (r >> 2) + 4 * (l4 >> 5) + (r & 3);
    };
    auto quad_col = [&](int e) {
        const int l4 = (e & 15) * 4, t = e >> 8;
        return 16 * nb0 + 32 * (t % CB) + (l4 & 31);
    };
    float esx[IT];
    uint2 esw[IT];
#pragma unroll
    for (int it = 0; it < IT; ++it) {
        const int e = min(int(threadIdx.x) + it * 64 * KW, QUADS - 1);
        esx[it] = s_x[min(quad_row(e), M - 1)];
        esw[it] = *reinterpret_cast<const uint2*>(s1 + min(quad_col(e), N - 4));
    }

    // Register ring: group i of the wave's range lives in stage i % PD; a
    // stage is consumed, then refilled with the group PD ahead. Loads past
    // the range repeat its last group (cache hits, never used), so every
    // load is unconditional and the compiler's waits cover one stage.
    // Dequantization is software-pipelined: while the MFMAs of group i run
    // on the INT8 weights of buffer i % 2, the VALU turns the packed codes of
    // group i + 1 into buffer (i + 1) % 2, interleaved one MFMA to a few
    // VALU instructions, so the SIMD's matrix pipe and VALU work at once.
    // Records: without RL each stage also carries its groups' 2-byte records,
    // loaded from global memory beside the codes (a vector-memory request per
    // record: measured at 9-10 % of the operand stream's time); with RL they
    // are read from LDS two groups ahead into a pair of registers.
    v4i av[PD][MT][4];
    uint4 qn[PD][CB][2];
    uint32_t rs[RL ? 2 : PD][CB];
    v4i bq[2][CB][4];
    auto load = [&](int p, int g) {
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) {
            qn[p][cb][0] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                rb, b_off[cb], g * kBlockBytes, 0));
            qn[p][cb][1] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                rb, b_off[cb], g * kBlockBytes + 512, 0));
            if constexpr (!RL)
                rs[p][cb] = __builtin_amdgcn_raw_buffer_load_b16(
                    rr, r_off[cb], (g >> 3) * kRecChunkBytes + (g & 7) * 2, 0);
        }
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int st = 0; st < 4; ++st)
                av[p][mt][st] = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(
                    ra, a_off[mt], g * kActGroupBytes + 2 * kActUnit * st, 0));
    };
    // dequantize stage p's codes into buffer b with record set r
    auto dequant = [&](int b, int p, int r) {
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) {
            dequant_block(qn[p][cb][0], rs[r][cb], bq[b][cb][0], bq[b][cb][2]);
            dequant_block(qn[p][cb][1], rs[r][cb], bq[b][cb][1], bq[b][cb][3]);
        }
    };
    auto read_rec = [&](int r, int g) {
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) rs[r][cb] = rec_lds(cb, g);
    };
    constexpr int kMfma = 4 * MT * CB;            // MFMAs per group
    constexpr int kValu = 62 * CB;                // dequantization VALU per group (about)
    constexpr int kValuPer = (kValu + kMfma - 1) / kMfma;
    auto mfmas = [&](int b, int p) {
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
#pragma unroll
            for (int st = 0; st < 4; ++st)
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
                    acc[mt][cb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(av[p][mt][st], bq[b][cb][st],
                                                                       acc[mt][cb], 0, 0, 0);
    };
    // Step i (u = i mod U, U a multiple of PD and of 2): MFMAs of group i
    // interleaved with the dequantization of group i + 1, then the refill of
    // group i's stage with group i + PD. Scheduling barriers pin the refill
    // after the step's MFMAs (left to itself the compiler sinks every refill
    // of an unrolled block to its end, and the next block then waits for
    // loads it has only just issued).
    auto step = [&](int i, int u, bool full) {
        const int p = u % PD, pn = (u + 1) % PD, b = u & 1;
        if (full || i < cnt) {
            // RL: the records of group i + 2 into the pair entry group i used
            if constexpr (RL) read_rec(b, gb + min(i + 2, cnt - 1));
            mfmas(b, p);
            if (full || i + 1 < cnt) dequant(b ^ 1, pn, RL ? b ^ 1 : pn);
#pragma unroll
            for (int k = 0; k < kMfma; ++k) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);          // one MFMA
                __builtin_amdgcn_sched_group_barrier(0x002, kValuPer, 0);   // then VALU
            }
        }
        __builtin_amdgcn_sched_barrier(0);
        if (full || i + PD < cnt) load(p, gb + min(i + PD, cnt - 1));
        __builtin_amdgcn_sched_barrier(0);
    };
    constexpr int U = PD % 2 == 0 ? PD : 2 * PD;
    if (cnt > 0) {
        uint4 stg[CB][2][2];
        if constexpr (RL) {
            // the range's record chunks c0 .. c0 + 7 (clamped) of the 2 CB
            // blocks: lane l takes 16 bytes of chunk c0 + l / 16 + 4 k
#pragma unroll
            for (int cb = 0; cb < CB; ++cb)
#pragma unroll
                for (int h2 = 0; h2 < 2; ++h2) {
                    const int blk = min(nb0 + 2 * cb + h2, nbt - 1);
#pragma unroll
                    for (int k = 0; k < 2; ++k) {
                        const int ch = min(c0 + (lane >> 4) + 4 * k, ng8 - 1);
                        stg[cb][h2][k] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                            rr, (blk * ng8 + ch) * kRecChunkBytes + (lane & 15) * 16, 0, 0));
                    }
                }
        }
#pragma unroll
        for (int p = 0; p < PD; ++p) load(p, gb + min(p, cnt - 1));
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (RL) {
#pragma unroll
            for (int cb = 0; cb < CB; ++cb)
#pragma unroll
                for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
                    for (int k = 0; k < 2; ++k)
                        *reinterpret_cast<uint4*>(rl + ((cb * 2 + h2) * kRecLdsChunks + (lane >> 4) + 4 * k) * 128 +
                                                  (lane & 15) * 8) = stg[cb][h2][k];
            // written by other lanes of this wave: order the wave's LDS
            // accesses (DS instructions of one wave complete in order)
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            read_rec(0, gb);
            read_rec(1, gb + min(1, cnt - 1));
        }
        __builtin_amdgcn_sched_barrier(0);
        dequant(0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
        int i0 = 0;
        for (; i0 + U <= cnt; i0 += U) {
#pragma unroll
            for (int u = 0; u < U; ++u) step(i0 + u, u, true);
        }
        if (i0 < cnt) {
#pragma unroll
            for (int u = 0; u < U; ++u) step(i0 + u, u, false);
        }
    }

    // RL: no wave may still read its records when the sum below reuses them
    if constexpr (RL) __syncthreads();

    // Add the KW partial tiles in LDS: wave w stores register r of tile t at
    // red[((w T + t) 16 + r) 64 + lane] (conflict-free), then each thread
    // sums four consecutive lanes (four consecutive output columns of one
    // row) over the waves and writes them with the epilogue. When the KW
    // tiles do not fit, waves KR..KW-1 first store theirs and waves 0..KR-1
    // add them to their registers.
    auto store_red = [&](int slot) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int cb = 0; cb < CB; ++cb)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    red[((slot * T + mt * CB + cb) * 16 + r) * 64 + lane] = acc[mt][cb][r];
    };
    if constexpr (KR < KW) {
        if (wave >= KR) store_red(wave - KR);
        __syncthreads();
        if (wave < KR) {
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int cb = 0; cb < CB; ++cb)
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        acc[mt][cb][r] += red[((wave * T + mt * CB + cb) * 16 + r) * 64 + lane];
        }
        __syncthreads();
    }
    if (wave < KR) store_red(wave);
    __syncthreads();
#pragma unroll
    for (int it = 0; it < IT; ++it) {
        const int e = int(threadIdx.x) + it * 64 * KW;
        if (QUADS % (64 * KW) != 0 && e >= QUADS) break;
        const int l4 = (e & 15) * 4;             // first lane of the quad
        const int r = (e >> 4) & 15;
        const int t = e >> 8;
        int4 sum = *reinterpret_cast<const int4*>(&red[(t * 16 + r) * 64 + l4]);
#pragma unroll
        for (int w = 1; w < KR; ++w) {
            const int4 v = *reinterpret_cast<const int4*>(&red[((w * T + t) * 16 + r) * 64 + l4]);
            sum.x += v.x;
            sum.y += v.y;
            sum.z += v.z;
            sum.w += v.w;
        }
        const int m = quad_row(e);
        const int n = quad_col(e);
        if (m >= M || n >= N) continue;          // N % 16 == 0: the quad is whole
        const float sx = esx[it];
        const int64_t o = int64_t(m) * N + n;
        if (acc_debug) {   // the debug buffer carries no alignment promise
            acc_debug[o] = sum.x;
            acc_debug[o + 1] = sum.y;
            acc_debug[o + 2] = sum.z;
            acc_debug[o + 3] = sum.w;
        }
        uint2 out;
        out.x = uint32_t(epilogue_value(sum.x, sx, h2f(uint16_t(esw[it].x & 0xffffu)))) |
                (uint32_t(epilogue_value(sum.y, sx, h2f(uint16_t(esw[it].x >> 16)))) << 16);
        out.y = uint32_t(epilogue_value(sum.z, sx, h2f(uint16_t(esw[it].y & 0xffffu)))) |
                (uint32_t(epilogue_value(sum.w, sx, h2f(uint16_t(esw[it].y >> 16)))) << 16);
        *reinterpret_cast<uint2*>(y + o) = out;   // y is 16-byte aligned, N % 16 == 0
    }
}

template <int MT, int CB, int KW, int PD>
hipError_t launch_one(const GemmPlan& p, const GemmArgs& a, hipStream_t stream) {
    // records in LDS when every wave's group range fits the staging area
    const int gpw = ((a.K >> 7) + KW - 1) / KW;
    if (gpw <= kRecLdsMaxGroups)
        return launch_kernel(gemm_ksplit32_kernel<MT, CB, KW, PD, true>, dim3(p.grid_x),
                             dim3(64 * KW), 0, stream, a.x8, a.s_x, a.M, a.K, a.nib, a.rec, a.ng8,
                             a.s1, a.N, a.y, a.acc_debug);
    return launch_kernel(gemm_ksplit32_kernel<MT, CB, KW, PD, false>, dim3(p.grid_x), dim3(64 * KW),
                         0, stream, a.x8, a.s_x, a.M, a.K, a.nib, a.rec, a.ng8, a.s1, a.N, a.y,
                         a.acc_debug);
}

}  // namespace

#define QOQ_KSPLIT32_CONFIGS(X)                                                      \
    X(1, 1, 8, 2) X(1, 2, 8, 2) X(2, 1, 8, 2) X(2, 2, 8, 2) X(4, 1, 8, 2)             \
    X(2, 2, 4, 2) X(4, 1, 4, 2) X(2, 1, 8, 4) X(1, 1, 16, 2) X(2, 3, 4, 2)            \
    X(1, 3, 8, 2) X(2, 2, 4, 3) X(2, 2, 4, 4) X(2, 3, 4, 3) X(2, 3, 4, 4)             \
    X(4, 1, 4, 3) X(4, 1, 4, 4) X(1, 1, 8, 4) X(1, 2, 8, 3) X(2, 1, 8, 3)

bool ksplit32_config_exists(int mt, int cb, int kw, int pd) {
#define X(a, b, c, d) if (mt == a && cb == b && kw == c && pd == d) return true;
    QOQ_KSPLIT32_CONFIGS(X)
#undef X
    return false;
}

hipError_t launch_ksplit32(const GemmPlan& p, const GemmArgs& a, hipStream_t stream) {
#define X(A, B, C, D) \
    if (p.mt == A && p.cb == B && p.kw == C && p.pd == D) return launch_one<A, B, C, D>(p, a, stream);
    QOQ_KSPLIT32_CONFIGS(X)
#undef X
    return hipErrorInvalidConfiguration;
}

}  // namespace qoq
