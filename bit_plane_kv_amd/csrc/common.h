// Internal declarations shared by the libfathom.so sources (not part of the C-ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "fathom.h"

namespace fathom {

constexpr int kD = FATHOM_D;                 // channels per head
constexpr int kPlanes = FATHOM_PLANES;       // 4 planes per channel
constexpr int kMaxPlanesPerHead = kD * kPlanes;  // 512
constexpr int kGroupBits = 8;                // planes per matrix-core byte operand
constexpr int kMaxGroups = kMaxPlanesPerHead / kGroupBits;  // 64
constexpr int kKBlockGroups = 4;             // groups summed by one i8 MFMA (K = 32)
constexpr int kMaxKBlocks = kMaxGroups / kKBlockGroups;     // 16
constexpr int kDigits = 4;                   // signed base-256 digits per weight

// ---------------------------------------------------------------------------------
// Scan workspace, per head: a meta block, then per K-block (4 groups of 8 planes) and
// per wave lane one record of the MFMA operands that lane supplies.
//   meta: int32 n_planes, n_groups, n_kblocks, pad; float C[8] (constant term of each
//   query); float S[8] (power-of-two weight unit of each query); uint32 plane[512]
//   (c*4 + j, channels ascending, planes ascending within a channel).
//   record (kblock, lane), lane = 16*kb + 4*w + s:  uint32 row of plane s and of plane
//   s+4 of group 4*kblock + kb (kSkipRow: no plane, load nothing), then for each set of
//   4 queries the 8 bytes of A row (lane & 15) = (query 4*set + ((lane & 15) >> 2),
//   digit lane & 3) over that group's 8 planes.  QS = 1 (G <= 4): 16 bytes; QS = 2: 32.
// ---------------------------------------------------------------------------------
constexpr size_t kMetaBytes = 4096;
constexpr uint32_t kSkipRow = 0xFFFFFFFFu;
struct ScanMeta {
    int32_t n_planes;
    int32_t n_groups;
    int32_t n_kblocks;
    int32_t pad;
    float C[FATHOM_MAX_G];
    float S[FATHOM_MAX_G];
    uint32_t plane[kMaxPlanesPerHead];
};
static_assert(sizeof(ScanMeta) <= kMetaBytes, "meta block");

inline int query_sets(int G) { return G <= 4 ? 1 : 2; }
inline size_t scan_rec_bytes_per_head(int G) {
    return (size_t)kMaxKBlocks * 64 * 16 * query_sets(G);
}
inline size_t scan_ws_bytes(int H, int G) {
    return (size_t)H * (kMetaBytes + scan_rec_bytes_per_head(G));
}

// ---------------------------------------------------------------------------------
// Store-build workspace: min/max partials [H][nchunk][2][d] fp32, then the integer
// code sums [H][d][2] uint64.
// ---------------------------------------------------------------------------------
constexpr int kMinMaxTokens = 2048;
inline int minmax_chunks(int n) { return (n + kMinMaxTokens - 1) / kMinMaxTokens; }
inline size_t quantize_ws_bytes(int H, int n) {
    size_t mm = (size_t)H * minmax_chunks(n) * 2 * kD * sizeof(float);
    mm = (mm + 255) / 256 * 256;
    return mm + (size_t)H * kD * 2 * sizeof(uint64_t);
}

// ---------------------------------------------------------------------------------
// Top-k: rows longer than one chunk are reduced level by level; each level keeps the
// top min(k, chunk) (value, index) candidates of every chunk, in index order.
// ---------------------------------------------------------------------------------
constexpr int kTopkChunk = FATHOM_TOPK_CHUNK;
struct TopkLevels {
    int n_levels;       // candidate levels (0 when the row fits one chunk)
    int64_t count[8];   // candidates per row after level l
};
TopkLevels topk_levels(int n, int k);
size_t topk_ws_bytes(int R, int n, int k);

// ---------------------------------------------------------------------------------
// Launchers (each returns the launch's hipError_t).
// ---------------------------------------------------------------------------------
hipError_t launch_quantize_store(const float *keys, int H, int n, const fathom_store &st,
                                 void *ws, hipStream_t s);
hipError_t launch_plan(const fathom_store &st, const float *q, int G, int B,
                       uint8_t *depth, hipStream_t s);
hipError_t launch_plan_fixed(const fathom_store &st, int n_channels, uint8_t *depth,
                             hipStream_t s);
hipError_t launch_scan_prepare(const fathom_store &st, const float *q, int G,
                               const uint8_t *depth, void *ws, hipStream_t s);
hipError_t launch_plan_prepare(const fathom_store &st, const float *q, int G, int B,
                               uint8_t *depth, void *ws, hipStream_t s);
hipError_t launch_scan_main(const fathom_store &st, int G, float *scores, void *ws,
                            hipStream_t s);
hipError_t launch_scan_extract(const fathom_store &st, const float *q, int G,
                               const uint8_t *depth, float *scores, hipStream_t s);
hipError_t launch_topk(const float *scores, int R, int n, int k, int32_t *idx, void *ws,
                       hipStream_t s);
hipError_t launch_sparse_attn(const float *q, const uint16_t *K, const uint16_t *V, int H,
                              int G, int n, const int32_t *idx, int k, float sm_scale,
                              uint16_t *out, hipStream_t s);
hipError_t launch_stream_read(const void *src, size_t bytes, uint64_t *sink,
                              hipStream_t s);
hipError_t launch_stream_runs(const void *src, size_t run_bytes, size_t stride_bytes,
                              size_t n_runs, uint64_t *sink, hipStream_t s);

// ---------------------------------------------------------------------------------
// Device helpers
// ---------------------------------------------------------------------------------
__device__ __forceinline__ float bf16_bits_to_float(uint32_t h16) {
    return __uint_as_float(h16 << 16);
}

__device__ __forceinline__ uint16_t float_to_bf16_bits(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu))
        return (uint16_t)((u >> 16) | 0x0040u);
    u += 0x7fffu + ((u >> 16) & 1u);  // round to nearest, ties to even
    return (uint16_t)(u >> 16);
}

// Map launch block b of nb onto a logical block so that logical blocks
// [x*nb/8, (x+1)*nb/8) all run on XCD x: hardware hands consecutive block ids to the
// 8 XCDs round-robin.  Blocks beyond the largest multiple of 8 keep their id.
__device__ __forceinline__ int xcd_remap(int b, int nb) {
    const int per = nb >> 3;
    if (b >= per * 8) return b;
    return (b & 7) * per + (b >> 3);
}

}  // namespace fathom
