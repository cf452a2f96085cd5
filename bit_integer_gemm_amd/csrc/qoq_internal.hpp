// Internal declarations shared by the translation units of libqoq.
//
// Packed-weight layout, version 1 (what qoq_pack_weights writes and the
// GEMM kernels read). N output channels, K inputs, groups of 128 inputs:
//
//   NB  = N / 16           column blocks of 16 output channels
//   NG  = K / 128          groups per channel
//   NG8 = ceil(NG / 8)     record chunks of 8 groups
//
//   nibbles  [NB][NG][64 lanes][16 bytes]       at byte 0
//       The 1 KiB block (nb, g) is exactly the B operand of two
//       v_mfma_i32_16x16x64_i8 steps for channels 16nb..16nb+15 and inputs
//       128g..128g+127: lane l (channel 16nb + (l & 15), quarter h = l >> 4)
//       owns 16 bytes; byte b holds the code of input 128g + 16h + b in its
//       low nibble (first MFMA step, k in [0, 64) of the group) and of input
//       128g + 64 + 16h + b in its high nibble (second step, k in [64, 128)).
//       A wave fetches its fragments for one group with one 16-byte load per
//       lane at base + 16 * lane, and `w & 0x0F0F0F0F` / `(w >> 4) &
//       0x0F0F0F0F` put the codes of each 32-bit word directly into the byte
//       order of the operand registers: no other address arithmetic and no
//       byte permutes in the main loop (compute-aware reordering).
//   records  [NB][NG8][16 channels][8 groups][2 bytes]   after the nibbles
//       (s2, 128 - z*s2) as two uint8 per (channel, group); one 16-byte load
//       gives a lane the records of 8 consecutive groups of its channel.
//       Entries for groups >= NG are zero.
//
// Activation tile layout, version 1 (what the activation quantizer writes and
// the GEMM kernels read): code (m, k) of x8 at byte
//   ((m >> 4) * (K >> 4) + (k >> 4)) * 256 + (m & 15) * 16 + (k & 15),
// i.e. row m starts at (m >> 4) * 16K + (m & 15) * 16 and its 16-byte chunk
// j sits 256 bytes after chunk j - 1. Group g of a 16-row tile is 2 KiB
// contiguous; its half s (inputs 64s .. 64s + 63) is the 1 KiB A operand of
// one v_mfma_i32_16x16x64_i8 step, lane l at byte 16 l. Rows past M in the
// last tile are never written or read (loads clamp the row to M - 1).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <string>
#include <tuple>
#include <utility>

namespace qoq {

// Launch through hipLaunchKernel so the status of this very launch is
// returned (not whatever an unrelated earlier call left behind).
template <typename... KArgs, typename Tuple, size_t... I>
hipError_t launch_tuple(void (*kernel)(KArgs...), dim3 grid, dim3 block, size_t shmem,
                        hipStream_t stream, Tuple& args, std::index_sequence<I...>) {
    void* argv[sizeof...(I) + 1] = {static_cast<void*>(&std::get<I>(args))..., nullptr};
    return hipLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, argv, shmem,
                           stream);
}

template <typename... KArgs, typename... Args>
hipError_t launch_kernel(void (*kernel)(KArgs...), dim3 grid, dim3 block, size_t shmem,
                         hipStream_t stream, Args&&... args) {
    static_assert(sizeof...(KArgs) == sizeof...(Args), "kernel argument count");
    std::tuple<KArgs...> tup(std::forward<Args>(args)...);
    return launch_tuple(kernel, grid, block, shmem, stream, tup,
                        std::index_sequence_for<KArgs...>{});
}

// Plan overrides for measurements and tests (qoq_set_tuning): the value of
// a key, or "" when it is unset. Read by the planners on the host.
enum TuningKey { kTuneGemm = 0, kTuneVariant, kTuneKv4Splits, kTuneKv4Paired, kTuneCount };
std::string tuning(TuningKey key);

constexpr int kGroup = 128;
constexpr int kBlockCols = 16;
constexpr int kBlockBytes = 1024;
constexpr int kRecChunk = 8;
constexpr int kRecChunkBytes = kBlockCols * kRecChunk * 2;  // 256
constexpr int kProtect = 119;   // level-1 protective range
constexpr int kActMax = 127;    // activation code bound
constexpr int kFusedGroups = 4;  // fused kernel: groups of K held per wave
constexpr int kActTileRows = 16;
constexpr int kActUnit = 256;                          // 16 rows x 16 bytes
constexpr int kActGroupBytes = kActUnit * kGroup / 16; // 2048: one group of a row tile

// Bytes of the x8 buffer (activation tile layout) for M rows of K inputs.
__host__ __device__ inline int64_t act_bytes(int64_t M, int64_t K) {
    return (M + kActTileRows - 1) / kActTileRows * kActTileRows * K;
}

// Byte offset of the first code of row m (valid on host and device).
__host__ __device__ inline int64_t act_row_offset(int64_t m, int64_t K) {
    return (m >> 4) * 16 * K + (m & 15) * 16;
}

struct PackedLayout {
    int64_t nb, ng, ng8;
    int64_t nib_bytes;
    int64_t rec_offset;
    int64_t rec_bytes;
    int64_t total;
};

inline PackedLayout packed_layout(int64_t N, int64_t K) {
    PackedLayout L;
    L.nb = N / kBlockCols;
    L.ng = K / kGroup;
    L.ng8 = (L.ng + kRecChunk - 1) / kRecChunk;
    L.nib_bytes = L.nb * L.ng * kBlockBytes;
    L.rec_offset = L.nib_bytes;
    L.rec_bytes = L.nb * L.ng8 * kRecChunkBytes;
    L.total = L.nib_bytes + L.rec_bytes;
    return L;
}

// Launch plan of the GEMM for one shape (host side, shared by the
// workspace-size query and the launcher).
struct GemmPlan {
    int kind;           // 0: generic, 1: decode (K split over waves), 2: shared-activation,
                        // 4: 32x32 tile (large M), 5: K-split 32x32 (K over waves),
                        // 6: wide tile (activations to LDS by direct loads),
                        // 7: weight streaming (activation chunks in LDS)
    int mt;             // 16-row MFMA tiles per wave
    int cb;             // 16-column blocks per wave
    int kw;             // decode: waves splitting K; shared-activation: waves per workgroup
    int pd;             // weight groups kept in flight per wave (register ring depth)
    int pa;             // 32x32 tile: workgroups per CU the kernel is built for
    int nw;             // 32x32 tile: waves per workgroup (side by side along N)
    int grid_x, grid_y;
    int splits;             // shared-activation family: workgroups along K (grid z)
    int groups_per_split;   // a multiple of 8 unless it is all of K
    int64_t ws_bytes;       // int32 partial sums [splits][M][N]; 0 when splits == 1
};

GemmPlan plan_gemm(int64_t M, int64_t N, int64_t K);

// Kernel arguments shared by the GEMM families (packed buffer split into its
// nibble and record regions).
struct GemmArgs {
    const int8_t* x8;
    const float* s_x;
    int M, K;
    const uint8_t* nib;
    const uint8_t* rec;
    int ng8;
    const uint16_t* s1;
    int N;
    uint16_t* y;
    int32_t* acc_debug;
};

// K-split 32x32 family (gemm_ksplit.hip): plan kind 5, (mt, cb, kw, pd).
bool ksplit32_config_exists(int mt, int cb, int kw, int pd);
hipError_t launch_ksplit32(const GemmPlan& p, const GemmArgs& a, hipStream_t stream);

// Wide-tile family (gemm_wide.hip): plan kind 6, (mt, cb, nw, R = pd ring
// slots, pa workgroups per CU); `part` = split-K partial sums or null.
bool wide_config_exists(int mt, int cb, int nw, int r, int minb);
hipError_t launch_wide(const GemmPlan& p, const GemmArgs& a, int32_t* part, hipStream_t stream);

// Weight-streaming family (gemm_stream.hip): plan kind 7, (mt, cb, nw, pd
// ring depth, pa = groups per activation chunk); `part` as above.
bool stream_config_exists(int mt, int cb, int nw, int pd, int ch);
hipError_t launch_stream(const GemmPlan& p, const GemmArgs& a, int32_t* part, hipStream_t stream);

// Launch plan of the fused entry point (activation quantization + GEMM):
// either one fused launch (small M) or the quantizer into a workspace
// followed by the GEMM.
struct LinearPlan {
    bool valid;         // false: the "gemm" tuning names no usable configuration
    bool fused;         // one launch, every workgroup quantizes the tokens itself
    int kw;             // fused: waves splitting K
    int fcb;            // fused: 16-column blocks per workgroup (1 or 2)
    int grid_x;
    int64_t x8_offset, sx_offset, gemm_ws_offset;   // workspace carve-up (two-call path)
    int64_t ws_bytes;
    GemmPlan gemm;      // two-call path
};

LinearPlan plan_linear(int64_t M, int64_t N, int64_t K);

// Allocation-free GEMM: the library's own scratch array stands in for the
// workspace. static_scratch returns its device address on the stream's
// device (looked up on first use per device, then cached).
constexpr int64_t kStaticScratchBytes = int64_t(64) << 20;
hipError_t static_scratch(hipStream_t stream, void** out);

// Comparison GEMMs (W8A8 per-channel, W4A4 per-group with partial-sum
// scaling) on the 32x32 tile skeleton.
constexpr int kVariantW8A8 = 1;
constexpr int kVariantW4A4 = 2;
constexpr int kVariantW4A16 = 3;
struct VariantPlan {
    bool valid;         // false: the "variant" tuning names no compiled configuration
    int fmt;
    int mt, cb, pb, pa, nw;
    int grid_x;
};
VariantPlan plan_variant(int fmt, int64_t M, int64_t N, int64_t K);
int64_t w4a4_rows_padded(int64_t M);
int64_t w4a4_act_bytes(int64_t M, int64_t K);

// Launchers (enqueue only; return the launch status).
hipError_t launch_pack(const float* W, int64_t N, int64_t K, uint8_t* packed, uint16_t* s1,
                       uint8_t* cq4, int8_t* cs2, uint8_t* cz, bool from_canonical,
                       hipStream_t stream);
hipError_t launch_quantize_act(const uint16_t* x, int64_t M, int64_t K, int8_t* x8, float* s_x,
                               hipStream_t stream);
hipError_t launch_gemm(const GemmPlan& plan, const int8_t* x8, const float* s_x, int64_t M,
                       int64_t K, const uint8_t* packed, const uint16_t* s1, int64_t N,
                       uint16_t* y, int32_t* acc_debug, void* workspace, hipStream_t stream);
hipError_t launch_w8a8_pack(const float* W, int64_t N, int64_t K, uint8_t* packed, uint16_t* s,
                            hipStream_t stream);
hipError_t launch_w4a4_pack(const float* W, int64_t N, int64_t K, uint8_t* packed,
                            hipStream_t stream);
hipError_t launch_w4a16_pack(const float* W, int64_t N, int64_t K, uint8_t* packed,
                             hipStream_t stream);
hipError_t launch_w4a16_gemm(const VariantPlan& p, const uint16_t* x, int64_t M, int64_t K,
                             const uint8_t* packed, int64_t N, uint16_t* y, hipStream_t stream);
hipError_t launch_w4a4_quantize_act(const uint16_t* x, int64_t M, int64_t K, uint8_t* act,
                                    hipStream_t stream);
hipError_t launch_w8a8_gemm(const VariantPlan& p, const int8_t* x8, const float* s_x, int64_t M,
                            int64_t K, const uint8_t* packed, const uint16_t* s, int64_t N,
                            uint16_t* y, int32_t* acc_debug, hipStream_t stream);
hipError_t launch_w4a4_gemm(const VariantPlan& p, const uint8_t* act, int64_t M, int64_t K,
                            const uint8_t* packed, int64_t N, uint16_t* y, hipStream_t stream);
// KV4 decode attention (4-bit KV cache, SmoothAttention scaling)
// Largest KV cache capacity (tokens per sequence) the entry points accept.
constexpr int64_t kKv4MaxCapacity = int64_t(1) << 24;

struct Kv4Plan {
    int splits;        // workgroups per (sequence, KV head), context split evenly
    int bps;           // 32-token blocks per split
    int waves;         // waves per workgroup (4 or 8)
    bool paired;       // workgroups take two sequences of complementary length rank
    int64_t grid;
};
int64_t kv4_cache_bytes(int64_t B, int64_t Hkv, int64_t C);
Kv4Plan plan_kv4(int64_t B, int64_t Hkv, int64_t max_len);
hipError_t launch_kv4_smooth(const uint16_t* k, int64_t T, int64_t Hkv, uint16_t* lam,
                             hipStream_t stream);
hipError_t launch_kv4_append(const uint16_t* k, const uint16_t* v, int64_t B, int64_t Tn,
                             int64_t Hkv, const uint16_t* lam, const int32_t* start, uint8_t* cache,
                             int64_t C, hipStream_t stream);
int64_t kv4_workspace_bytes(const Kv4Plan& p, int64_t B, int64_t H);
hipError_t launch_kv4_attention(const Kv4Plan& p, const uint16_t* q, int64_t B, int64_t H,
                                int64_t Hkv, const uint16_t* lam, const uint8_t* cache, int64_t C,
                                const int32_t* lens, int64_t max_len, uint16_t* out, float* part,
                                hipStream_t stream);

int64_t kv16_cache_bytes(int64_t B, int64_t Hkv, int64_t C);
hipError_t launch_kv16_append(const uint16_t* k, const uint16_t* v, int64_t B, int64_t Tn,
                              int64_t Hkv, const int32_t* start, uint8_t* cache, int64_t C,
                              hipStream_t stream);
hipError_t launch_kv16_attention(const Kv4Plan& p, const uint16_t* q, int64_t B, int64_t H,
                                 int64_t Hkv, const uint8_t* cache, int64_t C, const int32_t* lens,
                                 int64_t max_len, uint16_t* out, float* part, hipStream_t stream);

hipError_t launch_linear_fused(const LinearPlan& plan, const uint16_t* x, int64_t M, int64_t K,
                               const uint8_t* packed, const uint16_t* s1, int64_t N, uint16_t* y,
                               int32_t* acc_debug, hipStream_t stream);

}  // namespace qoq
