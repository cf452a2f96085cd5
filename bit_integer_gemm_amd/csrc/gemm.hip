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
#include "kernel_common.hpp"

#include <hip/hip_fp16.h>

#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <mutex>
#include <string>
#include <type_traits>

namespace qoq {
namespace {

// Decode family (M <= 64): weight streaming.
//
// A workgroup owns 16*MT tokens x CB column blocks (16 channels each) over
// the whole of K and splits K between its KW waves in contiguous group
// ranges. With TM > 1 row tiles, the TM workgroups of one column range are
// 8 workgroup ids apart, so they run on the same XCD (ids are dealt to the
// XCDs round-robin) at the same time and the second read of the weights
// hits that XCD's L2; splitting M halves the activation bytes each
// workgroup pulls from L2, which bounds M = 64. Each wave
// keeps PD groups of nibbles, records and activation fragments in flight
// (register ring), so the HBM stream never waits on the MFMAs. The KW partial
// INT32 accumulators are summed in LDS -- exact, so the result does not
// depend on KW -- and the workgroup writes its outputs with the epilogue.
// No partial sum ever leaves the workgroup: no global atomics, no fences.
template <int MT, int CB, int KW, int PD>
__global__ void __launch_bounds__(64 * KW) gemm_decode_kernel(
    const int8_t* __restrict__ x8, const float* __restrict__ s_x, int M, int K,
    const uint8_t* __restrict__ nib, const uint8_t* __restrict__ rec, int ng8,
    const uint16_t* __restrict__ s1, int N, uint16_t* __restrict__ y,
    int32_t* __restrict__ acc_debug, int TM) {
    static_assert(KW * MT * CB <= 64, "LDS reduction buffer above 64 KiB");
    __shared__ v4i red[KW * MT * CB * 64];
    const int lane = threadIdx.x & 63;
    // wave-uniform (scalar) so the group-range branches stay scalar
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int c = lane & 15;
    const int h = lane >> 4;
    const int ng = K >> 7;
    const int nbt = N >> 4;
    int tn = blockIdx.x, tm_id = 0;
    if (TM > 1) {
        const int q = blockIdx.x >> 3;
        tm_id = q % TM;
        tn = (q / TM) * 8 + (blockIdx.x & 7);
    }
    const int nb0 = tn * CB;
    const int m0 = 16 * MT * tm_id;
    const int gpw = (ng + KW - 1) / KW;
    const int gb = min(ng, wave * gpw);
    const int cnt = min(ng, gb + gpw) - gb;

    const uint8_t* bptr[CB];
    const uint8_t* rptr[CB];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
        const int64_t nbc = min(nb0 + cb, nbt - 1);
        bptr[cb] = nib + nbc * ng * kBlockBytes + lane * 16;
        rptr[cb] = rec + (nbc * ng8 * kBlockCols + c) * (kRecChunk * 2);
    }
    // Activations in the tile layout: the A operand of step s of group g for
    // row tile mt is 1 KiB at tile base + 2048 g + 1024 s, lane l at 16 l.
    // Rows at or beyond M read a valid row instead (the last one): an MFMA
    // row only feeds the same output row, and those rows are never stored.
    // Unpredicated loads keep the prefetch ring free of per-lane branches.
    const int8_t* aptr[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
        aptr[mt] = x8 + act_row_offset(min(m0 + 16 * mt + c, M - 1), K) + kActUnit * h;

    // Epilogue elements of this thread (see the end): their token and
    // channel scales are fetched now, so the epilogue waits for no load.
    // Output element e = (mt, r, h, cb, c) is token 16mt + 4h + r, channel
    // 16(nb0 + cb) + c; consecutive threads take consecutive channels.
    constexpr int E = MT * 16 * CB * 16;
    constexpr int EI = (E + 64 * KW - 1) / (64 * KW);
    float esx[EI], esw[EI];
#pragma unroll
    for (int it = 0; it < EI; ++it) {
        const int e = min(int(threadIdx.x) + it * 64 * KW, E - 1);
        const int cc = e & 15;
        const int t = e >> 4;
        const int cbi = t % CB;
        const int hh = (t / CB) & 3;
        const int rr = ((t / CB) >> 2) & 3;
        const int mt = (t / CB) >> 4;
        esx[it] = s_x[min(m0 + 16 * mt + 4 * hh + rr, M - 1)];
        esw[it] = h2f(s1[16 * min(nb0 + cbi, nbt - 1) + cc]);
    }

    v4i acc[MT][CB];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) acc[mt][cb] = v4i{0, 0, 0, 0};

    // Register ring of PD groups: group i of this wave lives in stage i % PD.
    // A stage is consumed, then immediately refilled with the group PD ahead,
    // so PD - 1 groups are always in flight while the MFMAs run. Loads are
    // unconditional (past the range they repeat the last group: cache hits,
    // never used) so the compiler's waits cover one stage at a time.
    // Group records: when every wave's range starts on a multiple of 8, one
    // 16-byte load per 8 groups (static slot in a loop unrolled by 8);
    // otherwise one 2-byte load per group.
    static_assert(8 % PD == 0, "ring depth must divide the record chunk");
    uint4 qn[PD][CB];
    uint32_t rs[PD][CB];
    v4i av[PD][MT][2];
    uint4 rc_cur[CB], rc_next[CB];
    const bool aligned = (gpw & 7) == 0;

    auto load = [&](int p, int g, bool per_group_rec) {
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
            qn[p][cb] = *reinterpret_cast<const uint4*>(bptr[cb] + int64_t(g) * kBlockBytes);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int s = 0; s < 2; ++s)
                av[p][mt][s] = *reinterpret_cast<const v4i*>(aptr[mt] + g * kActGroupBytes + 1024 * s);
        if (per_group_rec) {
#pragma unroll
            for (int cb = 0; cb < CB; ++cb)
                rs[p][cb] = *reinterpret_cast<const uint16_t*>(
                    rptr[cb] + (g >> 3) * (kBlockCols * kRecChunk * 2) + (g & 7) * 2);
        }
    };
    auto load_rec = [&](uint4 (&dst)[CB], int chunk) {
        chunk = min(chunk, (ng - 1) >> 3);
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
            dst[cb] = *reinterpret_cast<const uint4*>(rptr[cb] + chunk * (kBlockCols * kRecChunk * 2));
    };
    auto compute = [&](int p, uint32_t const (&rec)[CB]) {
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) {
            v4i b0, b1;
            dequant_block(qn[p][cb], rec[cb], b0, b1);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                acc[mt][cb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(av[p][mt][0], b0, acc[mt][cb], 0, 0, 0);
                acc[mt][cb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(av[p][mt][1], b1, acc[mt][cb], 0, 0, 0);
            }
        }
    };
    auto run = [&](auto chunked) {
        constexpr bool kChunked = decltype(chunked)::value;
        auto step = [&](int i, int u, bool full) {
            const int p = u % PD;
            if (full || i < cnt) {
                uint32_t rec[CB];
#pragma unroll
                for (int cb = 0; cb < CB; ++cb) rec[cb] = kChunked ? record_of(rc_cur[cb], u) : rs[p][cb];
                compute(p, rec);
            }
            // in the final (guarded) block only the loads still needed are issued
            if (full || i + PD < cnt) load(p, gb + min(i + PD, cnt - 1), !kChunked);
            if (kChunked && u == 7) {
#pragma unroll
                for (int cb = 0; cb < CB; ++cb) rc_cur[cb] = rc_next[cb];
                load_rec(rc_next, ((gb + i + 1) >> 3) + 1);
            }
        };
        if (kChunked) {
            load_rec(rc_cur, gb >> 3);
            load_rec(rc_next, (gb >> 3) + 1);
        }
        if (cnt >= PD) {
#pragma unroll
            for (int p = 0; p < PD; ++p) load(p, gb + p, !kChunked);
        } else {
#pragma unroll
            for (int p = 0; p < PD; ++p)
                if (p < cnt) load(p, gb + p, !kChunked);
        }
        int i0 = 0;
        for (; i0 + 8 <= cnt; i0 += 8) {
#pragma unroll
            for (int u = 0; u < 8; ++u) step(i0 + u, u, true);
        }
        if (i0 < cnt) {
#pragma unroll
            for (int u = 0; u < 8; ++u) step(i0 + u, u, false);
        }
    };
    if (cnt > 0) {
        if (aligned) run(std::true_type{});
        else run(std::false_type{});
    }

    // Sum the KW partial accumulators in LDS, then the epilogue.
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) red[((wave * MT + mt) * CB + cb) * 64 + lane] = acc[mt][cb];
    __syncthreads();
    const int* redi = reinterpret_cast<const int*>(red);
#pragma unroll
    for (int it = 0; it < EI; ++it) {
        const int e = int(threadIdx.x) + it * 64 * KW;
        if (e >= E) break;
        const int cc = e & 15;
        int t = e >> 4;
        const int cbi = t % CB;
        t /= CB;
        const int hh = t & 3;
        const int rr = (t >> 2) & 3;
        const int mt = t >> 4;
        const int m = m0 + 16 * mt + 4 * hh + rr;
        const int nbi = nb0 + cbi;
        if (m >= M || nbi >= nbt) continue;
        const int l = cc + 16 * hh;
        int32_t sum = 0;
#pragma unroll
        for (int w = 0; w < KW; ++w) sum += redi[(((w * MT + mt) * CB + cbi) * 64 + l) * 4 + rr];
        const int n = 16 * nbi + cc;
        if (acc_debug) acc_debug[int64_t(m) * N + n] = sum;
        y[int64_t(m) * N + n] = epilogue_value(sum, esx[it], esw[it]);
    }
}

// Shared-activation family (any M): a workgroup of NW waves covers
// 16*MT tokens x 16*CB*NW channels over the whole of K. Wave w owns CB column
// blocks and all MT row tiles, so every weight is dequantized exactly once
// per workgroup and no B operand is shared. The INT8 activations of each
// group (MT x 2 MFMA A fragments of 1 KiB) are staged in LDS once per
// workgroup -- each wave fetches a share of the fragments into a register
// ring P groups ahead and writes them to one of two LDS slots -- and all
// waves read them from there. One barrier per group.
//
// Split K: when `part` is given, workgroup z covers only the groups
// [z * gps, (z + 1) * gps) (gps a multiple of 8, so the record chunks stay
// aligned) and stores its exact INT32 sums to part[z][m][n] instead of the
// epilogue; splitk_epilogue_kernel adds the splits (integer addition, so the
// result equals the unsplit sum bit for bit) and applies the epilogue. This
// fills the chip for shapes with few column blocks and a long K.
template <int MT, int CB, int NW, int P>
__global__ void __launch_bounds__(64 * NW) gemm_lds_kernel(
    const int8_t* __restrict__ x8, const float* __restrict__ s_x, int M, int K,
    const uint8_t* __restrict__ nib, const uint8_t* __restrict__ rec, int ng8,
    const uint16_t* __restrict__ s1, int N, uint16_t* __restrict__ y,
    int32_t* __restrict__ acc_debug, int gps, int32_t* __restrict__ part) {
    constexpr int AF = 2 * MT;                    // A fragments per group
    constexpr int AFW = (AF + NW - 1) / NW;       // fragments fetched per wave
    static_assert(P >= 2 && P % 2 == 0, "ring depth must be even");
    __shared__ v4i As[2][AF][64];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int c = lane & 15;
    const int h = lane >> 4;
    const int ng = K >> 7;
    const int nbt = N >> 4;
    const int nb0 = (blockIdx.x * NW + wave) * CB;
    const int m0 = blockIdx.y * 16 * MT;
    // this workgroup's group range [g0, g0 + cnt); cnt >= 1 by the grid
    const int g0 = blockIdx.z * gps;
    const int cnt = min(ng - g0, gps);
    const int glast = g0 + cnt - 1;

    const uint8_t* bptr[CB];
    const uint8_t* rptr[CB];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
        const int64_t nbc = min(nb0 + cb, nbt - 1);
        bptr[cb] = nib + nbc * ng * kBlockBytes + lane * 16;
        rptr[cb] = rec + (nbc * ng8 * kBlockCols + c) * (kRecChunk * 2);
    }
    // fragment f = wave + NW*j -> (row tile f >> 1, MFMA step f & 1), 1 KiB
    // contiguous in the activation tile layout; rows at or beyond M read the
    // last row (never stored)
    const int8_t* aptr[AFW];
#pragma unroll
    for (int j = 0; j < AFW; ++j) {
        const int f = min(wave + NW * j, AF - 1);
        const int row = min(m0 + 16 * (f >> 1) + c, M - 1);
        aptr[j] = x8 + act_row_offset(row, K) + 1024 * (f & 1) + kActUnit * h;
    }
    auto owns = [&](int j) { return wave + NW * j < AF; };

    v4i acc[MT][CB];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) acc[mt][cb] = v4i{0, 0, 0, 0};

    uint4 qn[P][CB];
    v4i ar[P][AFW];
    // group records: one 16-byte load per lane brings 8 groups of its
    // channel; the loop is unrolled by 8 so the group's slot is static
    uint4 rc_cur[CB], rc_next[CB];
    auto load_rec = [&](uint4 (&dst)[CB], int chunk) {
        chunk = min(chunk, glast >> 3);
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
            dst[cb] = *reinterpret_cast<const uint4*>(rptr[cb] + chunk * (kBlockCols * kRecChunk * 2));
    };

    auto load_b = [&](int p, int g) {
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
            qn[p][cb] = *reinterpret_cast<const uint4*>(bptr[cb] + int64_t(g) * kBlockBytes);
    };
    auto load_a = [&](int p, int g) {
#pragma unroll
        for (int j = 0; j < AFW; ++j)
            ar[p][j] = *reinterpret_cast<const v4i*>(aptr[j] + int64_t(g) * kActGroupBytes);
    };
    auto stage_a = [&](int slot, int p) {
#pragma unroll
        for (int j = 0; j < AFW; ++j)
            if (owns(j)) As[slot][wave + NW * j][lane] = ar[p][j];
    };
    auto compute = [&](int slot, int p, int u) {
        v4i b[CB][2];
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
            dequant_block(qn[p][cb], record_of(rc_cur[cb], u), b[cb][0], b[cb][1]);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const v4i a0 = As[slot][2 * mt][lane];
            const v4i a1 = As[slot][2 * mt + 1][lane];
#pragma unroll
            for (int cb = 0; cb < CB; ++cb) {
                acc[mt][cb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a0, b[cb][0], acc[mt][cb], 0, 0, 0);
                acc[mt][cb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a1, b[cb][1], acc[mt][cb], 0, 0, 0);
            }
        }
    };
    // One group step (i counts from the range start; groups are g0 + i).
    // Every global load is unconditional -- groups past the range's last one
    // are clamped to it (cache hits, never used) -- and only LDS staging and
    // compute are guarded, so the compiler's waits cover exactly one stage
    // of each ring and never drain them.
    auto step = [&](int i, int u, bool full) {
        const int p = u % P;
        const int pn = (p + 1) % P;
        if (i + 1 < cnt) stage_a((p + 1) & 1, pn);
        load_a(pn, g0 + min(i + 1 + P, cnt - 1));
        if (full || i < cnt) compute(p & 1, p, u);
        load_b(p, g0 + min(i + P, cnt - 1));
        if (u == 7) {
#pragma unroll
            for (int cb = 0; cb < CB; ++cb) rc_cur[cb] = rc_next[cb];
            load_rec(rc_next, ((g0 + i + 1) >> 3) + 1);
        }
        __syncthreads();
    };

    // Prologue: stage the range's first group, then issue the loads in the
    // same order the steady state issues them (as if steps -P..-1 had run),
    // so the loop is entered with the rings in their steady-state shape.
    load_rec(rc_cur, g0 >> 3);
    load_rec(rc_next, (g0 >> 3) + 1);
    load_a(0, g0);
    stage_a(0, 0);
#pragma unroll
    for (int j = -P; j < 0; ++j) {
        load_a((j + 1 + P) % P, g0 + min(j + 1 + P, cnt - 1));
        load_b((j + P) % P, g0 + min(j + P, cnt - 1));
    }
    __syncthreads();
    static_assert(8 % P == 0, "ring depth must divide the record chunk");
    int i0 = 0;
    for (; i0 + 8 <= cnt; i0 += 8) {
#pragma unroll
        for (int u = 0; u < 8; ++u) step(i0 + u, u, true);
    }
    if (i0 < cnt) {
#pragma unroll
        for (int u = 0; u < 8; ++u) step(i0 + u, u, false);
    }

    int32_t* pz = part ? part + int64_t(blockIdx.z) * M * N : nullptr;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
        if (nb0 + cb >= nbt) continue;
        const int n = 16 * (nb0 + cb) + c;
        const float sw = pz ? 0.f : h2f(s1[n]);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int m = m0 + 16 * mt + 4 * h + r;
                if (m >= M) continue;
                const int32_t v = acc[mt][cb][r];
                if (pz) {
                    pz[int64_t(m) * N + n] = v;
                    continue;
                }
                if (acc_debug) acc_debug[int64_t(m) * N + n] = v;
                y[int64_t(m) * N + n] = epilogue_value(v, s_x[m], sw);
            }
    }
}

// Second pass of a split-K GEMM: thread t sums the S INT32 partials of
// outputs 4t .. 4t + 3 (one row, N % 16 == 0) in split order and applies the
// epilogue.
__global__ void __launch_bounds__(256) splitk_epilogue_kernel(
    const int32_t* __restrict__ part, int S, int M, int N, const float* __restrict__ s_x,
    const uint16_t* __restrict__ s1, uint16_t* __restrict__ y, int32_t* __restrict__ acc_debug) {
    const int64_t t = int64_t(blockIdx.x) * 256 + threadIdx.x;
    const int64_t MN = int64_t(M) * N;
    if (4 * t >= MN) return;
    const int m = int(4 * t / N);
    const int n = int(4 * t - int64_t(m) * N);
    int4 sum = *reinterpret_cast<const int4*>(part + 4 * t);
    for (int z = 1; z < S; ++z) {
        const int4 v = *reinterpret_cast<const int4*>(part + z * MN + 4 * t);
        sum.x += v.x;
        sum.y += v.y;
        sum.z += v.z;
        sum.w += v.w;
    }
    if (acc_debug) {   // the debug buffer carries no alignment promise
        acc_debug[4 * t] = sum.x;
        acc_debug[4 * t + 1] = sum.y;
        acc_debug[4 * t + 2] = sum.z;
        acc_debug[4 * t + 3] = sum.w;
    }
    const float sx = s_x[m];
    uint2 out;
    out.x = uint32_t(epilogue_value(sum.x, sx, h2f(s1[n]))) |
            (uint32_t(epilogue_value(sum.y, sx, h2f(s1[n + 1]))) << 16);
    out.y = uint32_t(epilogue_value(sum.z, sx, h2f(s1[n + 2]))) |
            (uint32_t(epilogue_value(sum.w, sx, h2f(s1[n + 3]))) << 16);
    *reinterpret_cast<uint2*>(y + 4 * t) = out;   // y is 16-byte aligned
}

// 32x32 tile family (large M), built on v_mfma_i32_32x32x32_i8 (the
// 16x16x64 INT8 form issues at half the rate on gfx950). A workgroup of four
// waves side by side along N computes a (32*MT) x (128*CB) tile over the
// whole of K; wave w owns CB 32-column tiles and all MT 32-row tiles.
//   * A (activations) of each group is staged once per workgroup in LDS, in
//     32x32x32 fragment order: fragment (mt, s) holds, for lane l, the 16
//     bytes x8[32mt + l%32][32s + 16(l/32) ...]; waves read them back with
//     conflict-free 16-byte LDS reads. Two slots: group i+1 is staged while
//     group i is consumed.
//   * B (weights) comes straight from the packed buffer: for a 32-column
//     tile, lane l (column l%32 of the tile, k-half q = l/32) loads the
//     16-byte chunks of packed-block lanes c+16q and c+16(q+2) (c = l%16 in
//     the block of its 16 columns); low nibbles of the two chunks are MFMA
//     steps 0 and 1 of the group, high nibbles steps 2 and 3 -- the layout
//     written for the 16x16x64 form serves this instruction unchanged.
//   * Buffer loads: per-lane VGPR offsets fixed for the whole loop, the
//     group and step offsets uniform in SGPRs; rows of A past M read the
//     last row (those outputs are never stored).
//   * Register budget is kept under 256 (accumulators in AGPRs, shallow
//     rings) so two workgroups share a CU: one's barrier waits, LDS latency
//     and dequantization bursts are covered by the other's MFMAs.
//   * Epilogue through LDS with 16-byte row-segment stores.
//   * Split K (as in the shared-activation family): with `part` given,
//     workgroup row y of the grid covers groups [y * gps, (y + 1) * gps) and
//     stores its INT32 sums to part[y][m][n] for splitk_epilogue_kernel.
template <int MT, int CB, int PB, int MINB, int NW>
__global__ void __launch_bounds__(64 * NW, MINB) gemm_tile32_kernel(
    const int8_t* __restrict__ x8, const float* __restrict__ s_x, int M, int K,
    const uint8_t* __restrict__ nib, const uint8_t* __restrict__ rec, int ng8,
    const uint16_t* __restrict__ s1, int N, uint16_t* __restrict__ y,
    int32_t* __restrict__ acc_debug, int gps, int32_t* __restrict__ part) {
    constexpr int AF = 4 * MT;                    // A fragments per group
    constexpr int AFW = (AF + NW - 1) / NW;       // fetched per wave
    static_assert(AF * 2 <= 64, "LDS slots above 64 KiB");
    static_assert(PB == 1 || PB == 2 || PB == 4 || PB == 8, "weight ring depth divides 8");
    // two slots of A fragments; the epilogue reuses the space to stage NW
    // blocks of 32 x 32CB fp16 outputs
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
    constexpr int BM = 32 * MT, BNB = 2 * CB * NW;   // tile rows, tile 16-column blocks
    const int tiles_m = (M + BM - 1) / BM;
    const int tiles_n = (nbt + BNB - 1) / BNB;
    int tm, tn;
    tile_of(blockIdx.x, tiles_m, tiles_n, tm, tn);
    const int m0 = tm * BM;
    const int nbw = tn * BNB + wave * 2 * CB;     // this wave's first 16-column block
    // this workgroup's group range [g0, g0 + cnt); cnt >= 1 by the grid
    const int g0 = blockIdx.y * gps;
    const int cnt = min(ng - g0, gps);
    const int glast = g0 + cnt - 1;

    const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
        (void*)x8, (short)0, int(act_bytes(M, K)), 0x00020000);
    const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
        (void*)nib, (short)0, nbt * ng * kBlockBytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t rr = __builtin_amdgcn_make_buffer_rsrc(
        (void*)rec, (short)0, nbt * ng8 * (kBlockCols * kRecChunk * 2), 0x00020000);
    // A fragment f = (32-row tile f / 4, step f % 4) of group g: lanes 0-31
    // take rows 0-31 of the tile at inputs 32 (f % 4) .. +15, lanes 32-63 the
    // next 16 inputs; in the tile layout that is two 512-byte runs. Wave w
    // fetches and stages fragments w, w + NW, ... Rows at or beyond M read the
    // last row (never stored).
    int a_lane[AFW], a_soff[AFW];
#pragma unroll
    for (int u = 0; u < AFW; ++u) {
        const int f = min(wave + NW * u, AF - 1);
        a_lane[u] = int(act_row_offset(min(m0 + 32 * (f >> 2) + j, M - 1), K)) + kActUnit * q;
        a_soff[u] = 2 * kActUnit * (f & 3);
    }
    auto owns = [&](int u) { return wave + NW * u < AF; };
    int b_lane[CB], r_lane[CB];
#pragma unroll
    for (int t = 0; t < CB; ++t) {
        const int blk = min(nbw + 2 * t + (j >> 4), nbt - 1);
        b_lane[t] = blk * ng * kBlockBytes + (c + 16 * q) * 16;
        r_lane[t] = (blk * ng8 * kBlockCols + c) * (kRecChunk * 2);
    }

    v16i acc[MT][CB];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int t = 0; t < CB; ++t)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[mt][t][r] = 0;

    // activation fragments of the next kAr groups to stage: group g in
    // entry g % kAr, fetched kAr steps before it is staged
    constexpr int kAr = 2;
    v4i ar[kAr][AFW];
    uint4 qn[PB][CB][2];    // packed weights: group g in entry g % PB
    // group records: one 16-byte load per lane brings 8 groups of its
    // channel; the loop is unrolled by 8 so the group's slot is static
    uint4 rc_cur[CB], rc_next[CB];
    auto load_rec = [&](uint4 (&dst)[CB], int chunk) {
        chunk = min(chunk, glast >> 3);
#pragma unroll
        for (int t = 0; t < CB; ++t)
            dst[t] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                rr, r_lane[t], chunk * (kBlockCols * kRecChunk * 2), 0));
    };

    // i counts groups from the range start; past its end the last group is
    // loaded again (cache hits, never used)
    auto load_a = [&](int e, int i) {
        const int g = g0 + min(i, cnt - 1);
#pragma unroll
        for (int u = 0; u < AFW; ++u) {
            const int soff = g * kActGroupBytes + a_soff[u];
            ar[e][u] = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(ra, a_lane[u], soff, 0));
        }
    };
    auto stage_a = [&](int slot, int e) {
#pragma unroll
        for (int u = 0; u < AFW; ++u)
            if (owns(u)) As[slot][wave + NW * u][lane] = ar[e][u];
    };
    auto load_b = [&](int p, int i) {
        const int g = g0 + min(i, cnt - 1);
#pragma unroll
        for (int t = 0; t < CB; ++t) {
            qn[p][t][0] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                rb, b_lane[t], g * kBlockBytes, 0));
            qn[p][t][1] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                rb, b_lane[t], g * kBlockBytes + 512, 0));
        }
    };
    // Step i: stage A(i+1), fetch A(i+1+kAr) into its entry, dequantize
    // B(i) and refill its entry with group i+PB, then the MFMAs of group i.
    auto step = [&](int i, int u, bool full) {
        if (i + 1 < cnt) stage_a((u + 1) & 1, (u + 1) % kAr);
        load_a((u + 1) % kAr, i + 1 + kAr);
        v4i bq[CB][4];
#pragma unroll
        for (int t = 0; t < CB; ++t) {
            const uint32_t rec_u = record_of(rc_cur[t], u);
            dequant_block(qn[u % PB][t][0], rec_u, bq[t][0], bq[t][2]);
            dequant_block(qn[u % PB][t][1], rec_u, bq[t][1], bq[t][3]);
        }
        load_b(u % PB, i + PB);
        if (u == 7) {
#pragma unroll
            for (int t = 0; t < CB; ++t) rc_cur[t] = rc_next[t];
            load_rec(rc_next, ((g0 + i + 1) >> 3) + 1);
        }
        if (full || i < cnt) {
#pragma unroll
            for (int st = 0; st < 4; ++st)
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    const v4i a = As[u & 1][4 * mt + st][lane];
#pragma unroll
                    for (int t = 0; t < CB; ++t)
                        acc[mt][t] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, bq[t][st], acc[mt][t], 0, 0, 0);
                }
        }
        __syncthreads();
    };

    // prologue, in steady-state issue order
    load_rec(rc_cur, g0 >> 3);
    load_rec(rc_next, (g0 >> 3) + 1);
#pragma unroll
    for (int e = 0; e < kAr; ++e) load_a(e, e);
#pragma unroll
    for (int p = 0; p < PB; ++p) load_b(p, p);
    stage_a(0, 0);
    load_a(0, kAr);
    __syncthreads();
    constexpr int U = 8;    // unroll: one record chunk; a multiple of PB, 2 and kAr
    static_assert(U % PB == 0, "ring depth must divide the record chunk");
    int i0 = 0;
    for (; i0 + U <= cnt; i0 += U) {
#pragma unroll
        for (int u = 0; u < U; ++u) step(i0 + u, u, true);
    }
    if (i0 < cnt) {
#pragma unroll
        for (int u = 0; u < U; ++u) step(i0 + u, u, false);
    }

    if (part) {   // split K: the exact partial sums, 32 consecutive columns per lane group
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

    // Epilogue through LDS: per 32-row tile, each wave converts its 32 x 32CB
    // block to fp16 into a staging area (reusing the A slots), then writes it
    // out as 16-byte row segments. Lane (j, q), register r of tile (mt, t)
    // holds row 32mt + 8(r/4) + 4q + r%4, column 32t + j of the wave's columns.
    __syncthreads();
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
        // 32 rows x 4CB chunks of 16 bytes
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

// Generic family (any M): a workgroup of 4 waves, wave w owns CB column
// blocks and MT row tiles over the whole of K. Kept for shapes no tuned
// family covers.
template <int MT, int CB>
__global__ void __launch_bounds__(256) gemm_generic_kernel(
    const int8_t* __restrict__ x8, const float* __restrict__ s_x, int M, int K,
    const uint8_t* __restrict__ nib, const uint8_t* __restrict__ rec, int ng8,
    const uint16_t* __restrict__ s1, int N, uint16_t* __restrict__ y,
    int32_t* __restrict__ acc_debug) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int c = lane & 15;
    const int h = lane >> 4;
    const int ng = K >> 7;
    const int nbt = N >> 4;
    const int nb_first = (blockIdx.x * 4 + wave) * CB;
    const int m0 = blockIdx.y * 16 * MT;

    int nbc[CB];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) nbc[cb] = min(nb_first + cb, nbt - 1);
    const int8_t* arow[MT];
    bool aval[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        const int r = m0 + 16 * mt + c;
        aval[mt] = r < M;
        arow[mt] = x8 + act_row_offset(aval[mt] ? r : 0, K) + kActUnit * h;
    }
    v4i acc[MT][CB];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) acc[mt][cb] = v4i{0, 0, 0, 0};

    for (int g = 0; g < ng; ++g) {
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
                a[mt][s] = aval[mt] ? *reinterpret_cast<const v4i*>(arow[mt] + int64_t(g) * kActGroupBytes + 1024 * s)
                                    : v4i{0, 0, 0, 0};
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) {
            v4i b0, b1;
            dequant_block(q[cb], sb[cb], b0, b1);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                acc[mt][cb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[mt][0], b0, acc[mt][cb], 0, 0, 0);
                acc[mt][cb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[mt][1], b1, acc[mt][cb], 0, 0, 0);
            }
        }
    }
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
}

// Per-token INT8 codes of V fp16 activations (V/2 words, two per word),
// V bytes in input order, with the activation quantizer's arithmetic: the
// fp32 product with the token's inv = fp32(127/absmax), rounded half to even.
//   * The product is formed as fma(x, inv, 0): one rounding of the exact
//     product, as a plain fp32 multiply (a zero product may come out +0
//     instead of -0; its code is 0 either way).
//   * The quantizer's clamp to +-127 never acts here: |x| <= absmax gives
//     |x * inv| <= 127 (1 + 2^-24), which rounds to at most 127. So the codes
//     equal the quantizer's for every finite input.
//   * Rounding adds 1.5 * 2^23: in [2^23, 2^24) the fp32 spacing is 1, the
//     addition rounds to nearest even, and the low byte of the sum is the
//     code in two's complement.
template <int V>
__device__ __forceinline__ void act_codes(const uint32_t (&w)[V / 2], float inv,
                                          uint32_t (&out)[(V + 3) / 4]) {
    uint32_t b[V];
#pragma unroll
    for (int i = 0; i < V / 2; ++i) {
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
            const float p = __builtin_fmaf(h2f(uint16_t(hf ? w[i] >> 16 : w[i] & 0xffffu)), inv, 0.0f);
            b[2 * i + hf] = __builtin_bit_cast(uint32_t, p + 12582912.0f);
        }
    }
    // gather low bytes: perm(b1, b0) = [b0 b1 0 0]; two of those -> 4 bytes
    if constexpr (V == 2) {
        out[0] = __builtin_amdgcn_perm(b[1], b[0], 0x0c0c0400u);
    } else {
#pragma unroll
        for (int i = 0; i < V / 4; ++i)
            out[i] = __builtin_amdgcn_perm(__builtin_amdgcn_perm(b[4 * i + 3], b[4 * i + 2], 0x0c0c0400u),
                                           __builtin_amdgcn_perm(b[4 * i + 1], b[4 * i], 0x0c0c0400u),
                                           0x05040100u);
    }
}

// Fused family (M <= 16): per-token activation quantization inside the GEMM.
//
// For a handful of tokens the activation quantizer is a separate launch of
// almost no work; here every workgroup quantizes the tokens itself. The
// split of work is the decode family's with one 16-row tile: a workgroup
// owns one column block over all of K, its KW waves split K into ranges of
// at most kFusedGroups groups, and every load of a wave (packed weights,
// group records, fp16 activations) is issued up front.
//   * Only the M real tokens are quantized, spread over all 64 lanes: per
//     group, lane l takes V consecutive inputs, V * (l % (128/V)) onward, of
//     token l / (128/V) + (V/2) t for each of T rounds (V = 2 for one token,
//     4 for two, else 8; token rows past M repeat the last token).
//   * Token absmax: per-lane partial maxima on the fp16 magnitude bits, a
//     shuffle reduction over the lanes of a token, one LDS slot per (wave,
//     token), then a max over the waves (exact in any order).
//   * Codes go to a per-wave LDS area (groups x tokens x 128 bytes) and are
//     read back in the A-operand lane order of v_mfma_i32_16x16x64_i8 (lane
//     (c, h): token c, 16 bytes at 16h of each half-group).
//   * The KW partial accumulators are summed in LDS and the epilogue uses
//     s_x = absmax / 127 as the quantizer stores it: outputs equal the
//     two-call path's bit for bit.
template <int V, int T, int KW, int CB>
__global__ void __launch_bounds__(64 * KW) gemm_fused_small_kernel(
    const uint16_t* __restrict__ x, int M, int K,
    const uint8_t* __restrict__ nib, const uint8_t* __restrict__ rec, int ng8,
    const uint16_t* __restrict__ s1, int N, uint16_t* __restrict__ y,
    int32_t* __restrict__ acc_debug) {
    constexpr int GM = kFusedGroups;
    constexpr int LPR = kGroup / V;           // lanes per token row
    constexpr int RR = 64 / LPR;              // token rows per round
    constexpr int ROWS = RR * T;              // token rows held (>= M)
    static_assert(ROWS <= 16, "at most one 16-row tile");
    __shared__ v4i red[KW * CB * 64];
    __shared__ __attribute__((aligned(16))) uint8_t aq[KW][GM * ROWS * kGroup];
    __shared__ uint32_t pmax[KW][ROWS];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int c = lane & 15;
    const int h = lane >> 4;
    const int ng = K >> 7;
    const int nbt = N >> 4;
    const int nb0 = blockIdx.x * CB;              // first of the CB column blocks
    const int gpw = (ng + KW - 1) / KW;           // <= GM (checked by the launch plan)
    const int gb = min(ng, wave * gpw);
    const int cnt = min(ng, gb + gpw) - gb;

    const uint8_t* bptr[CB];
    const uint8_t* rptr[CB];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
        const int64_t nbc = min(nb0 + cb, nbt - 1);   // past N: never stored
        bptr[cb] = nib + nbc * ng * kBlockBytes + lane * 16;
        rptr[cb] = rec + (nbc * ng8 * kBlockCols + c) * (kRecChunk * 2);
    }
    // the channel scales of this thread's epilogue elements, fetched now
    constexpr int EI = (256 * CB + 64 * KW - 1) / (64 * KW);
    float esw[EI];
#pragma unroll
    for (int it = 0; it < EI; ++it) {
        const int e = min(int(threadIdx.x) + it * 64 * KW, 256 * CB - 1);
        esw[it] = h2f(s1[16 * min(nb0 + (e >> 8), nbt - 1) + (e & 15)]);
    }
    const int qj = lane % LPR;                    // V-value chunk within the group
    int qrow[T];
#pragma unroll
    for (int t = 0; t < T; ++t) qrow[t] = min(lane / LPR + RR * t, M - 1);

    // Activations first, so the absmax waits only for them while the weights
    // are still in flight. Loads are unconditional -- groups past the wave's
    // range repeat its last group (cache hits, never used) -- so the
    // compiler's waits count exactly the loads issued.
    uint32_t xv[T][GM][V / 2];
    uint4 qn[GM][CB];
    uint32_t rs[GM][CB];
#pragma unroll
    for (int i = 0; i < GM; ++i) {
        {
            const int g = min(gb + i, ng - 1);
#pragma unroll
            for (int t = 0; t < T; ++t) {
                const uint16_t* src = x + int64_t(qrow[t]) * K + g * kGroup + V * qj;
                if constexpr (V == 8) {
                    const uint4 v = *reinterpret_cast<const uint4*>(src);
                    xv[t][i][0] = v.x; xv[t][i][1] = v.y; xv[t][i][2] = v.z; xv[t][i][3] = v.w;
                } else if constexpr (V == 4) {
                    const uint2 v = *reinterpret_cast<const uint2*>(src);
                    xv[t][i][0] = v.x; xv[t][i][1] = v.y;
                } else {
                    xv[t][i][0] = *reinterpret_cast<const uint32_t*>(src);
                }
            }
        }
    }
#pragma unroll
    for (int i = 0; i < GM; ++i) {
        {
            const int g = min(gb + i, ng - 1);
#pragma unroll
            for (int cb = 0; cb < CB; ++cb) {
                qn[i][cb] = *reinterpret_cast<const uint4*>(bptr[cb] + int64_t(g) * kBlockBytes);
                rs[i][cb] = *reinterpret_cast<const uint16_t*>(
                    rptr[cb] + (g >> 3) * (kBlockCols * kRecChunk * 2) + (g & 7) * 2);
            }
        }
    }
    // token absmax on the magnitude bits (for finite fp16 their order is
    // |x|'s), two 16-bit lanes at a time
#pragma unroll
    for (int t = 0; t < T; ++t) {
        us2 m2 = us2{0, 0};
#pragma unroll
        for (int i = 0; i < GM; ++i) {
            if (i < cnt) {
#pragma unroll
                for (int j = 0; j < V / 2; ++j)
                    m2 = __builtin_elementwise_max(m2, __builtin_bit_cast(us2, xv[t][i][j] & 0x7fff7fffu));
            }
        }
        uint32_t mb = max(uint32_t(m2[0]), uint32_t(m2[1]));
#pragma unroll
        for (int off = LPR / 2; off > 0; off >>= 1)
            mb = max(mb, uint32_t(__shfl_xor(int(mb), off, LPR)));
        // lanes past M hold the last token: same maximum, same slot
        if (qj == 0) pmax[wave][qrow[t]] = mb;
    }
    __syncthreads();
    float inv[T];
#pragma unroll
    for (int t = 0; t < T; ++t) {
        uint32_t mm = 0;
#pragma unroll
        for (int w = 0; w < KW; ++w) mm = max(mm, pmax[w][qrow[t]]);
        const float a = h2f(uint16_t(mm));
        inv[t] = a > 0.0f ? float(kActMax) / a : 0.0f;
    }

    // quantize the wave's whole K range into its LDS area, then read it back
    // in operand order (written by other lanes of this wave: order the wave's
    // LDS accesses; DS instructions of one wave complete in order)
    uint8_t* my = aq[wave];
#pragma unroll
    for (int i = 0; i < GM; ++i) {
        if (i < cnt) {
#pragma unroll
            for (int t = 0; t < T; ++t) {
                uint32_t code[(V + 3) / 4];
                act_codes<V>(xv[t][i], inv[t], code);
                uint8_t* dst = my + (i * ROWS + qrow[t]) * kGroup + V * qj;
                if constexpr (V == 8) *reinterpret_cast<uint2*>(dst) = uint2{code[0], code[1]};
                else if constexpr (V == 4) *reinterpret_cast<uint32_t*>(dst) = code[0];
                else *reinterpret_cast<uint16_t*>(dst) = uint16_t(code[0]);
            }
        }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const int arow = min(c, M - 1);
    v4i acc[CB];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) acc[cb] = v4i{0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < GM; ++i) {
        if (i < cnt) {
            const uint8_t* src = my + (i * ROWS + arow) * kGroup + 16 * h;
            const v4i a0 = *reinterpret_cast<const v4i*>(src);
            const v4i a1 = *reinterpret_cast<const v4i*>(src + 64);
#pragma unroll
            for (int cb = 0; cb < CB; ++cb) {
                v4i b0, b1;
                dequant_block(qn[i][cb], rs[i][cb], b0, b1);
                acc[cb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a0, b0, acc[cb], 0, 0, 0);
                acc[cb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a1, b1, acc[cb], 0, 0, 0);
            }
        }
    }

    // sum the KW partial accumulators in LDS, then the epilogue (column
    // block cb, token 4h + r, channel 16 (nb0 + cb) + c for lane (c, h),
    // register r)
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) red[(wave * CB + cb) * 64 + lane] = acc[cb];
    __syncthreads();
    const int* redi = reinterpret_cast<const int*>(red);
#pragma unroll
    for (int it = 0; it < EI; ++it) {
        const int e = int(threadIdx.x) + it * 64 * KW;
        if (e >= 256 * CB) break;
        const int cc = e & 15;
        const int hh = (e >> 4) & 3;
        const int rr = (e >> 6) & 3;
        const int cb = e >> 8;
        const int m = 4 * hh + rr;
        if (m >= M || nb0 + cb >= nbt) continue;
        const int l = cc + 16 * hh;
        int32_t sum = 0;
        uint32_t mm = 0;
#pragma unroll
        for (int w = 0; w < KW; ++w) {
            sum += redi[((w * CB + cb) * 64 + l) * 4 + rr];
            mm = max(mm, pmax[w][m]);
        }
        const float am = h2f(uint16_t(mm));
        const float sx = am > 0.0f ? am / float(kActMax) : 0.0f;
        const int n = 16 * (nb0 + cb) + cc;
        if (acc_debug) acc_debug[int64_t(m) * N + n] = sum;
        y[int64_t(m) * N + n] = epilogue_value(sum, sx, esw[it]);
    }
}

int64_t round_up(int64_t v, int64_t a) { return (v + a - 1) / a * a; }

using Args = GemmArgs;

// Second pass of a split-K launch: partial sums [splits][M][N] -> y.
hipError_t launch_splitk_epilogue(const GemmPlan& p, const Args& a, const int32_t* part,
                                  hipStream_t stream) {
    const int64_t quads = int64_t(a.M) * a.N / 4;
    return launch_kernel(splitk_epilogue_kernel, dim3(unsigned((quads + 255) / 256)), dim3(256), 0,
                         stream, part, p.splits, a.M, a.N, a.s_x, a.s1, a.y, a.acc_debug);
}

template <int MT, int CB, int KW, int PD>
hipError_t launch_decode(const GemmPlan& p, const Args& a, hipStream_t stream) {
    return launch_kernel(gemm_decode_kernel<MT, CB, KW, PD>, dim3(p.grid_x), dim3(64 * KW), 0,
                         stream, a.x8, a.s_x, a.M, a.K, a.nib, a.rec, a.ng8, a.s1, a.N, a.y,
                         a.acc_debug, p.grid_y);
}

template <int MT, int CB, int NW, int P>
hipError_t launch_lds(const GemmPlan& p, const Args& a, void* ws, hipStream_t stream) {
    int32_t* part = p.splits > 1 ? static_cast<int32_t*>(ws) : nullptr;
    if (p.splits > 1 && part == nullptr) return hipErrorInvalidValue;
    hipError_t e = launch_kernel(gemm_lds_kernel<MT, CB, NW, P>, dim3(p.grid_x, p.grid_y, p.splits),
                                 dim3(64 * NW), 0, stream, a.x8, a.s_x, a.M, a.K, a.nib, a.rec,
                                 a.ng8, a.s1, a.N, a.y, a.acc_debug, p.groups_per_split, part);
    if (e != hipSuccess || p.splits == 1) return e;
    return launch_splitk_epilogue(p, a, part, stream);
}

template <int MT, int CB, int PB, int MINB, int NW>
hipError_t launch_tile32(const GemmPlan& p, const Args& a, void* ws, hipStream_t stream) {
    int32_t* part = p.splits > 1 ? static_cast<int32_t*>(ws) : nullptr;
    if (p.splits > 1 && part == nullptr) return hipErrorInvalidValue;
    const hipError_t e = launch_kernel(gemm_tile32_kernel<MT, CB, PB, MINB, NW>,
                                       dim3(p.grid_x, p.splits), dim3(64 * NW), 0, stream, a.x8,
                                       a.s_x, a.M, a.K, a.nib, a.rec, a.ng8, a.s1, a.N, a.y,
                                       a.acc_debug, p.groups_per_split, part);
    if (e != hipSuccess || p.splits == 1) return e;
    return launch_splitk_epilogue(p, a, part, stream);
}

template <int MT, int CB>
hipError_t launch_generic(const GemmPlan& p, const Args& a, hipStream_t stream) {
    return launch_kernel(gemm_generic_kernel<MT, CB>, dim3(p.grid_x, p.grid_y), dim3(256), 0,
                         stream, a.x8, a.s_x, a.M, a.K, a.nib, a.rec, a.ng8, a.s1, a.N, a.y,
                         a.acc_debug);
}

// Every compiled decode configuration: (MT, CB, KW, PD).
#define QOQ_DECODE_CONFIGS(X)                                                        \
    X(1, 1, 16, 2) X(1, 1, 8, 2) X(1, 2, 8, 2) X(1, 2, 4, 2) X(1, 4, 4, 2)            \
    X(1, 4, 2, 2) X(1, 8, 2, 2) X(1, 1, 16, 4) X(1, 2, 8, 4) X(1, 4, 4, 4)            \
    X(2, 1, 16, 2) X(2, 1, 8, 2) X(2, 2, 8, 2) X(2, 2, 4, 2) X(2, 4, 4, 2)            \
    X(2, 4, 2, 2) X(2, 8, 2, 2) X(2, 2, 8, 4) X(2, 4, 4, 4)                           \
    X(4, 1, 8, 2) X(4, 2, 8, 2) X(4, 2, 4, 2) X(4, 4, 4, 2) X(4, 4, 2, 2)             \
    X(4, 4, 4, 4) X(4, 1, 8, 4) X(2, 1, 8, 4) X(1, 1, 8, 4) X(2, 1, 16, 4)

// Every compiled shared-activation configuration: (MT, CB, NW, P).
#define QOQ_LDS_CONFIGS(X)                                                           \
    X(1, 1, 4, 2) X(1, 2, 4, 2) X(1, 1, 8, 2) X(1, 2, 8, 2) X(1, 4, 4, 2)             \
    X(2, 1, 4, 2) X(2, 2, 4, 2) X(2, 1, 8, 2) X(2, 2, 8, 2) X(2, 4, 4, 2)             \
    X(4, 1, 4, 2) X(4, 2, 4, 2) X(4, 1, 8, 2) X(4, 2, 8, 2) X(4, 4, 4, 2)             \
    X(4, 1, 4, 4) X(4, 2, 4, 4) X(4, 1, 8, 4) X(4, 2, 8, 4)                           \
    X(8, 2, 4, 2) X(8, 4, 4, 2) X(16, 2, 4, 2) X(16, 4, 4, 2) X(8, 2, 8, 2)             \
    X(4, 1, 6, 4) X(4, 2, 6, 4) X(4, 1, 12, 4) X(4, 1, 12, 2) X(4, 1, 16, 2)            \
    X(1, 1, 6, 4) X(1, 1, 12, 4) X(2, 1, 6, 4) X(2, 1, 12, 4) X(4, 1, 12, 8)             \
    X(4, 1, 8, 8) X(4, 1, 6, 8) X(4, 2, 6, 8) X(4, 1, 4, 8)

bool lds_config_exists(int mt, int cb, int nw, int pp) {
#define X(a, b, c, d) if (mt == a && cb == b && nw == c && pp == d) return true;
    QOQ_LDS_CONFIGS(X)
#undef X
    return false;
}

// Every compiled 32x32 tile configuration: (MT, CB, PB, workgroups per CU,
// waves per workgroup).
#define QOQ_TILE32_CONFIGS(X)                                                        \
    X(4, 2, 2, 2, 4) X(4, 2, 1, 2, 4) X(4, 1, 2, 2, 4) X(2, 2, 2, 2, 4) X(2, 1, 2, 2, 4)   \
    X(8, 1, 1, 2, 4) X(4, 2, 2, 1, 4) X(8, 1, 2, 1, 4) X(8, 2, 2, 1, 4) X(2, 1, 2, 3, 4)   \
    X(4, 1, 2, 3, 4) X(2, 1, 4, 2, 4) X(2, 1, 8, 2, 4) X(2, 2, 4, 2, 4) X(2, 1, 4, 3, 4)   \
    X(2, 1, 8, 1, 4) X(2, 2, 8, 1, 4) X(4, 1, 4, 2, 4) X(1, 1, 4, 3, 4) X(1, 1, 2, 3, 4)   \
    X(1, 1, 8, 2, 4) X(1, 1, 4, 4, 4) X(2, 1, 4, 1, 6) X(2, 1, 2, 1, 6) X(2, 1, 4, 1, 8)   \
    X(2, 1, 2, 1, 8) X(2, 1, 4, 1, 3) X(2, 1, 4, 2, 3) X(1, 1, 4, 1, 6) X(2, 1, 8, 1, 6)   \
    X(4, 1, 2, 1, 8) X(4, 2, 2, 1, 8)

bool tile32_config_exists(int mt, int cb, int pb, int minb, int nw) {
#define X(a, b, c, d, e) if (mt == a && cb == b && pb == c && minb == d && nw == e) return true;
    QOQ_TILE32_CONFIGS(X)
#undef X
    return false;
}

bool decode_config_exists(int mt, int cb, int kw, int pd) {
#define X(a, b, c, d) if (mt == a && cb == b && kw == c && pd == d) return true;
    QOQ_DECODE_CONFIGS(X)
#undef X
    return false;
}

}  // namespace

// Launch plan (defaults chosen from sweeps on MI355X over the workload
// shapes; the "gemm" tuning key (qoq_set_tuning) "<family>,<params>"
// overrides it for A/B runs, host-side only; a value naming no compiled
// configuration makes the call fail before anything is launched):
//   M <= 64, N <= 8192:  decode family -- K split over the waves of a
//                        workgroup, one or two column blocks per workgroup;
//                        for 32 < M <= 64, N >= 4096 and K >= 16384 the
//                        shared-activation family with K split over
//                        workgroups instead;
//   32 < M <= 64, 18432 <= N <= 30720, K >= 4096: K-split 32x32 family,
//                        64 x 96 tiles;
//   M <= 64, N  > 8192:  shared-activation family -- activations staged in
//                        LDS, waves side by side along N (K split in two for
//                        32 < M <= 64, N < 32768 and K >= 8192);
//   128 < M <= 256, N <= 8192: K-split 32x32 family (64-row tiles, K split
//                        over the 4 waves of a workgroup);
//   64 < M <= 128, N <= 4096, K <= 4096: decode family, 64-row tiles;
//   M  > 64:             wide-tile family (256 x 256 tiles of 8 waves) when
//                        they fill whole rounds of the CUs, or for deep,
//                        narrow shapes (N <= 8192, K >= 16384: K in two
//                        ranges); otherwise the 32x32 tile family: 128 x 256
//                        tiles of 8 waves for short, narrow shapes, else tiles
//                        sized so that ~2 workgroups per CU exist (down to
//                        32 x 128 for few, short tiles), with K split when
//                        fewer tiles than CUs remain.
// Split K keeps INT32 partial sums [splits][M][N] in the workspace.
GemmPlan plan_gemm(int64_t M, int64_t N, int64_t K) {
    GemmPlan p{};
    const int64_t nbt = N / kBlockCols;
    const int64_t ng = K / kGroup;
    p.splits = 1;
    p.groups_per_split = int(ng);
    p.ws_bytes = 0;
    p.mt = M <= 16 ? 1 : (M <= 32 ? 2 : 4);
    // 32-bit buffer offsets: the fast families need the nibble and x8 buffer
    // sizes below 2^31
    const bool small_offsets = N * K / 2 < (int64_t(1) << 31) && act_bytes(M, K) < (int64_t(1) << 31);
    if (!small_offsets) {
        p.kind = 0;
        p.mt = M <= 16 ? 1 : (M <= 32 ? 2 : 4);
        p.cb = 2;
    } else if (M > 32 && M <= 64 && nbt >= 256 && nbt <= 512 && ng >= 128) {
        // long K over few column blocks: the shared-activation family split
        // over K, about one workgroup of 8 waves per CU
        p.kind = 2; p.cb = 1; p.kw = 8; p.pd = 4;
        p.splits = int(std::min<int64_t>(std::max<int64_t>(256 / ((nbt + 7) / 8), 1), ng / 32));
    } else if (M > 32 && M <= 64 && nbt >= 1152 && nbt <= 1920 && ng >= 64) {
        // 33-64 tokens on layers of 18432-30720 columns and K >= 8192
        // (Qwen1.5-72B qkv at M = 64): K-split 32x32 family, 64 x 96 tiles
        // (about one per CU), 4 waves splitting K, rings of 3 groups
        // (31.3-31.7 -> 27.1 us against the shared-activation family with K
        // in two ranges); with K = 4096 the shared-activation family is
        // faster (Llama-3-8B gate+up at M = 48: 26.5 -> 18.7 us)
        p.kind = 5; p.mt = 2; p.cb = 3; p.kw = 4; p.pd = 3;
    } else if (M > 8 && M <= 16 && nbt >= 1152 && nbt <= 1920 && ng >= 64) {
        // 9-16 tokens on the same layers: K-split 32x32 family, 32 x 96
        // tiles, 8 waves splitting K (Qwen1.5-72B qkv at M = 16: 27.6 ->
        // 22.0 us against the shared-activation family)
        p.kind = 5; p.mt = 1; p.cb = 3; p.kw = 8; p.pd = 2;
    } else if (M <= 64 && nbt <= 512) {
        p.kind = 1;
        // up to 16 tokens, two 16-column blocks per workgroup once that
        // still gives 256 workgroups (Qwen1.5-72B down at M = 16: 27.4 ->
        // 22.6 us; Llama-3-8B down, 256 blocks, keeps one: 9.9 against 12.4)
        if (p.mt == 1) { p.cb = nbt >= 512 ? 2 : 1; p.kw = 8; p.pd = 4; }
        else if (p.mt == 2) { p.cb = 1; p.kw = 8; p.pd = 4; }
        else if (nbt >= 512) { p.cb = 2; p.kw = 4; p.pd = 2; }
        else if (nbt % 16 == 0) { p.mt = 2; p.cb = 2; p.kw = 8; p.pd = 4; }   // two row tiles
        else { p.cb = 1; p.kw = 8; p.pd = 4; }
        while (p.kw > 2 && ng < 2 * p.kw) p.kw /= 2;
        if (!decode_config_exists(p.mt, p.cb, p.kw, p.pd)) { p.cb = 1; p.kw = 8; p.pd = 2; }
    } else if ((M > 128 && M <= 256 && nbt <= 512) ||
               (M > 64 && M <= 128 && nbt <= 512 && ng <= 32)) {
        // narrow layers at 129-256 tokens (Llama-3-8B qkv / o / down at
        // M = 256): K-split 32x32 family, 64-row tiles of 64 or 96 columns
        // (whichever is closer to one workgroup per CU), 4 waves splitting
        // K, rings of 3 groups (o 12.8 -> 10.5 us, qkv 16.9 -> 13.2 us,
        // down 32.0 -> 26.5 us against the previous rules); at 65-128
        // tokens only for short K (Llama-3-8B o / qkv at M = 96: 12.0 ->
        // 9.9 us, 14.9 -> 10.0 us; down keeps the rules below: 21.5 against
        // 23.9 us)
        p.kind = 5; p.mt = 2; p.kw = 4; p.pd = 3;
        const int64_t rows = (M + 63) / 64;
        p.cb = rows * ((nbt + 3) / 4) > 256 && rows * ((nbt + 5) / 6) >= 192 ? 3 : 2;
    } else if (M <= 64) {
        p.kind = 2;
        p.cb = 1;
        // waves per workgroup, ring depth; up to 16 tokens on the widest
        // layers two 16-column blocks per wave (Qwen1.5-72B gate+up at
        // M = 16: 45.6 -> 40.1 us against 12 waves of one)
        if (nbt >= 2048 && p.mt == 1) { p.cb = 2; p.kw = 8; p.pd = 2; }
        else if (nbt >= 2048) { p.kw = 12; p.pd = 2; }
        else if (p.mt == 4 && ng >= 64) { p.kw = 16; p.pd = 2; p.splits = 2; }
        else { p.kw = 8; p.pd = 4; }
        if (!lds_config_exists(p.mt, p.cb, p.kw, p.pd)) { p.kw = 8; p.pd = 2; p.splits = 1; }
    } else {
        p.kind = 4;
        p.pa = 2;   // workgroups per CU
        p.nw = 4;
        const int64_t rows128 = (M + 127) / 128;
        const int64_t t42 = rows128 * ((nbt + 15) / 16);       // 128 x 256 tiles
        const int64_t t22 = ((M + 63) / 64) * ((nbt + 15) / 16);
        // A 256 x 256 tile (one per CU) takes about the time of two 128 x 256
        // tiles: the wide tiles when their rounds over the CUs take no more
        // of that time than the 128 x 256 tiles' rounds (past 128 tokens).
        // Measured (us, wide / 32x32-family tiles): Llama-3-8B gate+up at
        // M = 512 60.3 / 77.9, qkv at M = 2048 54.1 / 66.3; Qwen1.5-72B
        // gate+up at M = 192 105.7 / 123.4, qkv at M = 512 99.9 / 114.0 and
        // M = 2048 337.8 / 342.0, down at M = 2048 320.7 / 364.4; fewer tiles
        // than that stay on the 32x32 family (Llama-3-8B o and down at
        // M = 2048: 47.6-48.3 / 38.8, 132.8 / 114.6).
        // Deep, narrow layers with fewer tiles than CUs keep K in two ranges
        // (the rule below; Qwen1.5-72B down at M = 1024, 128 tiles: 182 us
        // against 192-197 in one).
        const int64_t t256 = ((M + 255) / 256) * ((nbt + 15) / 16);
        auto rounds = [](int64_t t) { return (t + 255) / 256; };
        const bool deep_narrow = M >= 512 && N <= 8192 && t42 >= 256 && ng >= 128;
        // (only where 256-row tiles pad M no further than 128-row ones: at
        // M = 320 and 384 they lose, qkv 78.1 -> 101.5 us, gate+up 56.5 ->
        // 61.7 and 60.0 -> 63.0 us)
        const bool same_rows = M % 256 == 0 || M % 256 > 128;
        const bool wide_fills = M > 128 && same_rows && 2 * rounds(t256) <= rounds(t42) &&
                                !(deep_narrow && t256 < 256);
        if (wide_fills) {
            // wide-tile family: 256 x 256 tiles of 8 waves, activations
            // staged by direct LDS loads three groups deep (Qwen1.5-72B
            // gate+up at M = 1024: 344-359 -> 330-347 us against 128 x 512
            // tiles of the 32x32 family)
            p.kind = 6; p.mt = 8; p.cb = 1; p.nw = 8; p.pd = 3; p.pa = 1;
        }
        else if (deep_narrow) {
            // deep and narrow: wide-tile family, 256 x 256 tiles, K in two
            // ranges (Qwen1.5-72B down at M = 1024: 192-197 -> 182 us)
            p.kind = 6; p.mt = 8; p.cb = 1; p.nw = 8; p.pd = 3; p.pa = 1; p.splits = 2;
        }
        else if (M >= 512 && N <= 8192 && t42 >= 256) { p.mt = 4; p.cb = 1; p.pd = 2; p.pa = 1; p.nw = 8; }
        else if (t42 >= 512) { p.mt = 4; p.cb = 2; p.pd = 2; }
        else if (M > 128 && M <= 256 && t42 >= 192) {
            // 129-256 tokens on a wide layer: two rows of 128 x 256 tiles,
            // 8 waves, one per CU for most CUs -- the 128-row tile
            // dequantizes each weight for twice the tokens of the 64-row one
            // (Llama-3-8B gate_up at M = 256: 38.9 -> 36.0 us); below 129
            // tokens it would leave rows of the tile idle
            p.mt = 4; p.cb = 1; p.pd = 2; p.pa = 1; p.nw = 8;
        }
        else if (t22 >= 384) { p.mt = 2; p.cb = 1; p.pd = 2; p.pa = 1; p.nw = 8; }   // 64 x 256, 8 waves
        else if (((M + 63) / 64) * ((nbt + 7) / 8) < 160 && ng < 64) {
            p.mt = 1; p.cb = 1; p.pd = 4; p.pa = 3;   // 32 x 128 tiles: twice the workgroups
        }
        else { p.mt = 2; p.cb = 1; p.pd = 4; }
        // 32x32-family tiles under one workgroup per CU and a long K: split K
        // to about two per CU (the wide tiles split only by the rule above)
        const int64_t tiles = ((M + 32 * p.mt - 1) / (32 * p.mt)) *
                              ((nbt + 2 * p.cb * p.nw - 1) / (2 * p.cb * p.nw));
        if (p.kind == 4 && tiles < 256 && ng >= 64 && p.splits == 1)
            p.splits = int(std::min<int64_t>((512 + tiles - 1) / tiles, ng / 16));
    }
    const std::string tune = tuning(kTuneGemm);
    if (!tune.empty()) {
        const char* env = tune.c_str();
        {
            int a = 0, b = 0, c = 0, d = 0, e = 4, sp = 1;
            char fam[16] = {0};
            const int nf =
                std::sscanf(env, "%15[a-z0-9],%d,%d,%d,%d,%d,%d", fam, &a, &b, &c, &d, &e, &sp);
            const std::string f(fam);
            p.kind = -1;   // an override that names no compiled configuration is an error
            if (f == "decode" && nf == 5 && M <= 256 && decode_config_exists(a, b, c, d)) {
                p.kind = 1; p.mt = a; p.cb = b; p.kw = c; p.pd = d;
            } else if (f == "lds" && (nf == 5 || nf == 6) && lds_config_exists(a, b, c, d) &&
                       (nf == 5 || (e >= 1 && e <= 64))) {
                p.kind = 2; p.mt = a; p.cb = b; p.kw = c; p.pd = d;
                p.splits = nf == 6 ? e : 1;
            } else if (f == "tile32" && (nf == 5 || nf == 6 || nf == 7) && small_offsets &&
                       tile32_config_exists(a, b, c, d, e) && sp >= 1 && sp <= 64) {
                p.kind = 4; p.mt = a; p.cb = b; p.pd = c; p.pa = d; p.nw = e;
                p.splits = nf == 7 ? sp : 1;
            } else if (f == "stream" && (nf == 6 || nf == 7) && small_offsets &&
                       stream_config_exists(a, b, c, d, e) && sp >= 1 && sp <= 64) {
                p.kind = 7; p.mt = a; p.cb = b; p.nw = c; p.pd = d; p.pa = e;
                p.splits = nf == 7 ? sp : 1;
            } else if (f == "wide" && (nf == 6 || nf == 7) && small_offsets &&
                       wide_config_exists(a, b, c, d, e) && sp >= 1 && sp <= 64) {
                p.kind = 6; p.mt = a; p.cb = b; p.nw = c; p.pd = d; p.pa = e;
                p.splits = nf == 7 ? sp : 1;
            } else if (f == "ksplit" && nf == 5 && small_offsets && ksplit32_config_exists(a, b, c, d)) {
                p.kind = 5; p.mt = a; p.cb = b; p.kw = c; p.pd = d;
            } else if (f == "generic" && nf >= 3 && (a == 1 || a == 2 || a == 4) && b == 2) {
                p.kind = 0; p.mt = a; p.cb = b;
            }
            if (p.kind < 0) return p;
        }
    }
    if (p.kind == 1) {
        // grid_y: row tiles, folded into the 1-D grid (the XCD pairing needs
        // the column tiles in whole rounds of 8)
        const int64_t tn = (nbt + p.cb - 1) / p.cb;
        p.grid_y = int((M + 16 * p.mt - 1) / (16 * p.mt));
        if (p.grid_y > 1 && tn % 8 != 0) { p.kind = -1; return p; }
        p.grid_x = int(tn * p.grid_y);
    } else if (p.kind == 5) {
        p.grid_x = int(((M + 32 * p.mt - 1) / (32 * p.mt)) * ((nbt + 2 * p.cb - 1) / (2 * p.cb)));
        p.grid_y = 1;
    } else if (p.kind == 7) {
        p.grid_x = int((nbt + 2 * p.cb * p.nw - 1) / (2 * p.cb * p.nw));
        p.grid_y = int((M + 32 * p.mt - 1) / (32 * p.mt));
    } else if (p.kind == 4 || p.kind == 6) {
        const int64_t tm = (M + 32 * p.mt - 1) / (32 * p.mt);
        const int64_t tn = (nbt + 2 * p.cb * p.nw - 1) / (2 * p.cb * p.nw);
        p.grid_x = int(tm * tn);
        p.grid_y = 1;
    } else if (p.kind == 2) {
        p.grid_x = int((nbt + p.cb * p.kw - 1) / (p.cb * p.kw));
        p.grid_y = int((M + 16 * p.mt - 1) / (16 * p.mt));
    } else {
        p.grid_x = int((nbt + 4 * p.cb - 1) / (4 * p.cb));
        p.grid_y = int((M + 16 * p.mt - 1) / (16 * p.mt));
    }
    if (p.kind == 2 || p.kind == 4 || p.kind == 6 || p.kind == 7) {
        // split K into whole record chunks of 8 groups; the partial sums
        // [splits][M][N] live in the workspace
        const int64_t want = std::max(1, p.splits);
        const int64_t gps = std::min(ng, round_up((ng + want - 1) / want, 8));
        p.groups_per_split = int(gps);
        p.splits = int((ng + gps - 1) / gps);
        if (p.splits > 1) p.ws_bytes = int64_t(p.splits) * M * N * 4;
    }
    return p;
}

hipError_t launch_gemm(const GemmPlan& p, const int8_t* x8, const float* s_x, int64_t M, int64_t K,
                       const uint8_t* packed, const uint16_t* s1, int64_t N, uint16_t* y,
                       int32_t* acc_debug, void* ws, hipStream_t stream) {
    const PackedLayout L = packed_layout(N, K);
    const Args a{x8, s_x, int(M), int(K), packed, packed + L.rec_offset, int(L.ng8), s1, int(N),
                 y, acc_debug};
    if (p.kind == 1) {
#define X(A, B, C, D) \
    if (p.mt == A && p.cb == B && p.kw == C && p.pd == D) return launch_decode<A, B, C, D>(p, a, stream);
        QOQ_DECODE_CONFIGS(X)
#undef X
        return hipErrorInvalidConfiguration;
    }
    if (p.kind == 5) return launch_ksplit32(p, a, stream);
    if (p.kind == 6 || p.kind == 7) {
        int32_t* part = p.splits > 1 ? static_cast<int32_t*>(ws) : nullptr;
        if (p.splits > 1 && part == nullptr) return hipErrorInvalidValue;
        const hipError_t e = p.kind == 6 ? launch_wide(p, a, part, stream)
                                         : launch_stream(p, a, part, stream);
        if (e != hipSuccess || p.splits == 1) return e;
        return launch_splitk_epilogue(p, a, part, stream);
    }
    if (p.kind == 4) {
#define X(A, B, C, D, E)                                                              \
    if (p.mt == A && p.cb == B && p.pd == C && p.pa == D && p.nw == E)                    \
        return launch_tile32<A, B, C, D, E>(p, a, ws, stream);
        QOQ_TILE32_CONFIGS(X)
#undef X
        return hipErrorInvalidConfiguration;
    }
    if (p.kind == 2) {
#define X(A, B, C, D) \
    if (p.mt == A && p.cb == B && p.kw == C && p.pd == D) return launch_lds<A, B, C, D>(p, a, ws, stream);
        QOQ_LDS_CONFIGS(X)
#undef X
        return hipErrorInvalidConfiguration;
    }
    switch (p.mt) {
        case 1: return launch_generic<1, 2>(p, a, stream);
        case 2: return launch_generic<2, 2>(p, a, stream);
        default: return launch_generic<4, 2>(p, a, stream);
    }
}

// Fused entry point: one launch of the fused family (each wave's K range
// must fit kFusedGroups groups: K <= 8192 with 16 waves) when the repeated
// quantization stays small against the quantizer launch it saves. Every
// workgroup of one column block quantizes all M x K activations, so the
// launch quantizes R = M K ceil(N / 16) values in all:
//   * up to 12 tokens (9-12 only for K >= 4096): fused while R <= 64e6;
//     otherwise two launches;
//   * one column block per workgroup up to 4 tokens; from 5 tokens two
//     (half the workgroups, half of R) once R > 16e6 or, past 8 tokens,
//     N > 4096.
// Measured in HIP graphs against the quantizer + GEMM launches (us, fused /
// two launches): K = 4096, N = 4096: M = 8 5.9 / 7.3, M = 12 6.8 / 7.6;
// N = 6144, M = 9-12: 8.5 / 9.4 (two blocks); N = 14336: M = 8 11.0 / 15.8,
// M = 12 12.7 / 15.9 (two blocks); N = 28672: M = 8 17.7 / 18.3 (two
// blocks), M = 9-12 two launches (18.3 against 19.5-19.9); K = 8192:
// N = 8192 and 10240, M = 9-12 15.3 / 15.9 and 25.4 / 26.2 (two blocks);
// N = 24576, M = 4 26.9 / 30.9 but M = 8 two launches (30.3 against 36.5 with
// two blocks, 48.7 with one); N = 49152, M = 4 and 8 two launches (48.4
// against 52.1, 48.6 against 68-92). Other shapes run the quantizer into the
// workspace, then the GEMM.
// (The fused kernel takes up to 16 tokens when forced.)
// The "gemm" tuning value "fused,KW" forces the fused kernel with KW waves;
// any other family forces the two-call path with that GEMM configuration.
LinearPlan plan_linear(int64_t M, int64_t N, int64_t K) {
    LinearPlan p{};
    p.valid = true;
    const int64_t ng = K / kGroup;
    const bool fits = M <= 16 && N * K / 2 < (int64_t(1) << 31) &&
                      M * K * 2 < (int64_t(1) << 31) && ng <= int64_t(kFusedGroups) * 16;
    // values quantized over all workgroups (only up to 16 tokens matter)
    const int64_t quantized = M <= 16 ? M * K * ((N + kBlockCols - 1) / kBlockCols) : 0;
    const bool pays = M <= 12 && (M <= 8 || K >= 4096) && quantized <= 64000000;
    int kw = ng <= 4 * kFusedGroups ? 4 : (ng <= 8 * kFusedGroups ? 8 : 16);
    bool fused = fits && pays;
    // column blocks per fused workgroup
    int fcb = M > 4 && (quantized > 16000000 || (M > 8 && N > 4096)) ? 2 : 1;
    const std::string tune = tuning(kTuneGemm);
    if (!tune.empty()) {
        const char* env = tune.c_str();
        {
            int a = 0;
            char fam[16] = {0};
            int cbf = 1;
            const int nf = std::sscanf(env, "%15[a-z0-9],%d,%d", fam, &a, &cbf);
            if (std::string(fam) == "fused") {
                fused = true;
                kw = a;
                fcb = cbf;
                if ((nf != 2 && nf != 3) || !fits || (a != 4 && a != 8 && a != 16) ||
                    (cbf != 1 && cbf != 2) || ng > int64_t(kFusedGroups) * a ||
                    (cbf == 2 && a == 16 && M > 12)) {   // not built: LDS above 160 KiB
                    p.valid = false;
                    return p;
                }
            } else {
                fused = false;
            }
        }
    }
    if (fused) {
        p.fused = true;
        p.kw = kw;
        p.fcb = fcb;
        p.grid_x = int((N / kBlockCols + fcb - 1) / fcb);
        p.ws_bytes = 0;
        return p;
    }
    p.fused = false;
    p.gemm = plan_gemm(M, N, K);
    if (p.gemm.kind < 0) {
        p.valid = false;
        return p;
    }
    p.x8_offset = 0;
    p.sx_offset = round_up(act_bytes(M, K), 256);
    p.gemm_ws_offset = round_up(p.sx_offset + 4 * M, 256);
    p.ws_bytes = p.gemm_ws_offset + p.gemm.ws_bytes;
    return p;
}

template <int V, int T, int CB>
hipError_t launch_fused_vtc(const LinearPlan& p, const uint16_t* x, int M, int K, const uint8_t* nib,
                            const uint8_t* rec, int ng8, const uint16_t* s1, int N, uint16_t* y,
                            int32_t* acc_debug, hipStream_t stream) {
    switch (p.kw) {
        case 4:
            return launch_kernel(gemm_fused_small_kernel<V, T, 4, CB>, dim3(p.grid_x), dim3(256), 0,
                                 stream, x, M, K, nib, rec, ng8, s1, N, y, acc_debug);
        case 8:
            return launch_kernel(gemm_fused_small_kernel<V, T, 8, CB>, dim3(p.grid_x), dim3(512), 0,
                                 stream, x, M, K, nib, rec, ng8, s1, N, y, acc_debug);
        case 16:
            // 16 waves of 16 token rows and two column blocks need more than
            // the 160 KiB of LDS: not built
            if constexpr (T == 4 && CB == 2) return hipErrorInvalidConfiguration;
            else
                return launch_kernel(gemm_fused_small_kernel<V, T, 16, CB>, dim3(p.grid_x),
                                     dim3(1024), 0, stream, x, M, K, nib, rec, ng8, s1, N, y,
                                     acc_debug);
        default:
            return hipErrorInvalidConfiguration;
    }
}

template <int V, int T>
hipError_t launch_fused_vt(const LinearPlan& p, const uint16_t* x, int M, int K, const uint8_t* nib,
                           const uint8_t* rec, int ng8, const uint16_t* s1, int N, uint16_t* y,
                           int32_t* acc_debug, hipStream_t stream) {
    if (p.fcb == 2)
        return launch_fused_vtc<V, T, 2>(p, x, M, K, nib, rec, ng8, s1, N, y, acc_debug, stream);
    return launch_fused_vtc<V, T, 1>(p, x, M, K, nib, rec, ng8, s1, N, y, acc_debug, stream);
}

hipError_t launch_linear_fused(const LinearPlan& p, const uint16_t* x, int64_t M, int64_t K,
                               const uint8_t* packed, const uint16_t* s1, int64_t N, uint16_t* y,
                               int32_t* acc_debug, hipStream_t stream) {
    const PackedLayout L = packed_layout(N, K);
    const uint8_t* rec = packed + L.rec_offset;
    const int m = int(M), k = int(K), n = int(N), ng8 = int(L.ng8);
    if (m == 1) return launch_fused_vt<2, 1>(p, x, m, k, packed, rec, ng8, s1, n, y, acc_debug, stream);
    if (m == 2) return launch_fused_vt<4, 1>(p, x, m, k, packed, rec, ng8, s1, n, y, acc_debug, stream);
    switch ((m + 3) / 4) {
        case 1: return launch_fused_vt<8, 1>(p, x, m, k, packed, rec, ng8, s1, n, y, acc_debug, stream);
        case 2: return launch_fused_vt<8, 2>(p, x, m, k, packed, rec, ng8, s1, n, y, acc_debug, stream);
        case 3: return launch_fused_vt<8, 3>(p, x, m, k, packed, rec, ng8, s1, n, y, acc_debug, stream);
        case 4: return launch_fused_vt<8, 4>(p, x, m, k, packed, rec, ng8, s1, n, y, acc_debug, stream);
        default: return hipErrorInvalidConfiguration;
    }
}

}  // namespace qoq

// Scratch memory of the allocation-free GEMM entry point: a fixed device
// array of this library (one copy per GPU, held until the process ends)
// that stands in for the caller's workspace. Host code never passes the
// array's name to a kernel (on the host it is only a stand-in for the
// symbol): its device address is looked up once per device with
// hipGetSymbolAddress and kept in scratch_addr.
static __device__ __align__(256) uint8_t scratch[qoq::kStaticScratchBytes];

namespace qoq {
namespace {
constexpr int kMaxScratchDevices = 64;
std::mutex scratch_mu;
void* scratch_addr[kMaxScratchDevices] = {};
}  // namespace

hipError_t static_scratch(hipStream_t stream, void** out) {
    *out = nullptr;
    int cur = 0;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    int dev = cur;
    if (stream != nullptr) {
        e = hipStreamGetDevice(stream, &dev);
        if (e != hipSuccess) return e;
    }
    if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(scratch_mu);
    if (scratch_addr[dev] == nullptr) {
        // the lookup runs with the stream's device current
        if (dev != cur && (e = hipSetDevice(dev)) != hipSuccess) return e;
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (dev != cur) {
            const hipError_t r = hipSetDevice(cur);
            if (e == hipSuccess) e = r;
        }
        if (e != hipSuccess) return e;
        if (p == nullptr) return hipErrorInvalidSymbol;
        scratch_addr[dev] = p;
    }
    *out = scratch_addr[dev];
    return hipSuccess;
}

}  // namespace qoq
