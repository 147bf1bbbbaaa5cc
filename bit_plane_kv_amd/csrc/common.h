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
constexpr int kGroupBits = 8;                // planes per lookup-table group
constexpr int kMaxGroups = kMaxPlanesPerHead / kGroupBits;  // 64
constexpr int kLutEntries = 1 << kGroupBits;  // 256

// ---------------------------------------------------------------------------------
// Scan workspace, per head:  a meta block (plane list, constant term, counts) and the
// lookup tables.  meta: int32 n_planes, int32 n_groups, int32 pad[2], float C[8],
// uint32 plane[512] (c*4 + j, channels ascending, planes ascending within a channel;
// entries past n_planes repeat the group's first plane so reads stay in bounds).
// lut: [kMaxGroups][256][gp] fp32, gp = G padded to 1, 2, 4 or 8.
// ---------------------------------------------------------------------------------
constexpr size_t kMetaBytes = 4096;
struct ScanMeta {
    int32_t n_planes;
    int32_t n_groups;
    int32_t pad[2];
    float C[FATHOM_MAX_G];
    uint32_t plane[kMaxPlanesPerHead];
};
static_assert(sizeof(ScanMeta) <= kMetaBytes, "meta block");

inline int padded_g(int G) { return G <= 1 ? 1 : G <= 2 ? 2 : G <= 4 ? 4 : 8; }
inline size_t scan_lut_bytes_per_head(int G) {
    return (size_t)kMaxGroups * kLutEntries * padded_g(G) * sizeof(float);
}
inline size_t scan_ws_bytes(int H, int G) {
    return (size_t)H * (kMetaBytes + scan_lut_bytes_per_head(G));
}
// meta blocks first (H * kMetaBytes), then the tables
inline ScanMeta *scan_meta(void *ws, int h) {
    return reinterpret_cast<ScanMeta *>(static_cast<char *>(ws) + (size_t)h * kMetaBytes);
}
inline float *scan_lut(void *ws, int H, int G, int h) {
    return reinterpret_cast<float *>(static_cast<char *>(ws) + (size_t)H * kMetaBytes +
                                     (size_t)h * scan_lut_bytes_per_head(G));
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
hipError_t launch_scan_main(const fathom_store &st, int G, float *scores, void *ws,
                            hipStream_t s);
hipError_t launch_topk(const float *scores, int R, int n, int k, int32_t *idx, void *ws,
                       hipStream_t s);
hipError_t launch_sparse_attn(const float *q, const uint16_t *K, const uint16_t *V, int H,
                              int G, int n, const int32_t *idx, int k, float sm_scale,
                              uint16_t *out, hipStream_t s);
hipError_t launch_stream_read(const void *src, size_t bytes, uint64_t *sink,
                              hipStream_t s);

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
