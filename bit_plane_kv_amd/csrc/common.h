// Internal declarations shared by the libfathom.so sources (not part of the C-ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stddef.h>
#include <stdint.h>

#include "fathom.h"

// Whole-wave reductions of the device library (DPP row operations, the result in every
// lane): cheaper than a butterfly of cross-lane shuffles.
extern "C" __device__ __attribute__((const)) unsigned int __ockl_wfred_add_u32(unsigned int);
extern "C" __device__ __attribute__((const)) unsigned int __ockl_wfred_min_u32(unsigned int);
extern "C" __device__ __attribute__((const)) unsigned int __ockl_wfred_max_u32(unsigned int);
extern "C" __device__ __attribute__((const)) unsigned long long __ockl_wfred_add_u64(
    unsigned long long);
extern "C" __device__ __attribute__((const)) double __ockl_wfred_max_f64(double);

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
//   meta: int32 n_planes, n_groups, n_kblocks; uint32 redo (head 0's only: the row
//   chunks the filtered select hands to the full select); float C[8] (constant term of each
//   query); float S[8] (power-of-two weight unit of each query); uint32 tkey[8]
//   (candidate threshold of each query as an order key, 0: keep every key); uint32
//   cnt[8] (candidates the filtering scan kept per query); uint32 plane[512]
//   (c*4 + j, channels ascending, planes ascending within a channel); uint32
//   cnt_exact[8] (candidates whose exact score clears the threshold, counted by the
//   select); uint32 ovf (bit g: a 256-token block of query g had more candidates than
//   its record area holds); int32 xthr[8][8] (the filter's integer thresholds, below);
//   uint32 attn_done[8] (workgroups of query g's split attention that have finished);
//   uint32 sel_done[8] (chunk selects of query g's row that have finished, rows of several
//   chunks).
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
    uint32_t redo;
    float C[FATHOM_MAX_G];
    float S[FATHOM_MAX_G];
    uint32_t tkey[FATHOM_MAX_G];
    uint32_t cnt[FATHOM_MAX_G];
    uint32_t plane[kMaxPlanesPerHead];
    uint32_t cnt_exact[FATHOM_MAX_G];
    uint32_t ovf;
    int32_t xthr[FATHOM_MAX_G][8];
    uint32_t attn_done[FATHOM_MAX_G];
    uint32_t sel_done[FATHOM_MAX_G];
};
static_assert(sizeof(ScanMeta) <= kMetaBytes, "meta block");

inline int query_sets(int G) { return G <= 4 ? 1 : 2; }
inline size_t scan_rec_bytes_per_head(int G) {
    return (size_t)kMaxKBlocks * 64 * 16 * query_sets(G);
}
inline size_t scan_ws_bytes(int H, int G) {
    return (size_t)H * (kMetaBytes + scan_rec_bytes_per_head(G));
}

// Candidate filter.  Each row (head, query) has a threshold score T.  The filtering
// scan decides in integers which tokens may clear it: with the digit sums of a token's
// score (bit m of its byte), X = D2 + 256 D3 bounds the score to within the largest
// possible contribution of the two low digits plus fp32 rounding, so the test
// X >= xthr[g][m] (X <= xthr[g][7] for m = 7, whose byte value is negative) keeps every
// token whose score is >= T and a few more.  A kept token's record -- int32 X and the
// low part R = D0 + 256 D1 (int32: heads of more than 480 planes, where that sum could
// overflow, keep no records and have all their rows rescored) -- goes, in token order, to the
// front of its 256-token block of a [H][G][cand_stride(n)] area of 4-byte words (at
// most kBlockRecords records a block, 64 when a head has at most 4 queries; a block with
// more sets the row's ovf bit), and
// bit i of word w of a [H][G][ceil(n/32)] uint32 mask marks token 32w + i as kept.
// The select turns each record into the scan's exact fp32 score and counts the
// candidates whose score is >= T: with at least k of them the row's k-th largest score
// is >= T, so every winner was kept; a row with fewer (or with ovf set) is rescored.
constexpr int kFilterBlockWords = 8;  // words per compaction block (256 tokens)
constexpr int kBlockRecords = 128;    // 8-byte records in a block's 256 4-byte words
__host__ __device__ inline int64_t cand_stride(int64_t n) { return (n + 255) / 256 * 256; }
constexpr int kSampleRuns = 8;        // threshold sample: runs of 4 words per head
constexpr int kSampleRunWords = 4;
constexpr int kSampleWords = kSampleRuns * kSampleRunWords;  // 32 words: 1024 tokens

// First word of sample run r (0 .. kSampleRuns-1) of a row of W words: every word of a
// short row, else runs spread evenly over it, 16-byte aligned.
__host__ __device__ inline int sample_run_word(int r, int W) {
    return W <= kSampleWords ? kSampleRunWords * r
                             : kSampleRunWords *
                                   (int)(((long)r * (W / kSampleRunWords - 1)) / (kSampleRuns - 1));
}
// Tokens the sample covers.
__host__ __device__ inline int sample_tokens(int n) {
    const int W = (n + 31) / 32;
    if (W <= kSampleWords) return n;
    const int end = 32 * (sample_run_word(kSampleRuns - 1, W) + kSampleRunWords);
    return kSampleWords * 32 - (end > n ? end - n : 0);
}
// Rank m of the sampled key kept as the threshold: the least m with
// n (m - 5 sqrt(m)) / S >= k (S sampled tokens); 0 when it exceeds S (no threshold).
__host__ __device__ inline int sample_rank(int n, int k) {
    const int S = sample_tokens(n);
    const double x = 0.5 * (5.0 + sqrt(25.0 + 4.0 * (double)k * (double)S / (double)n));
    const double m = ceil(x * x);
    return m > (double)S ? 0 : (int)m;
}
inline size_t cand_bytes(int H, int G, int n) {
    return (size_t)H * G * (size_t)cand_stride(n) * sizeof(float);
}
inline size_t filter_mask_bytes(int H, int G, int n) {
    return (size_t)H * G * (size_t)((n + 31) / 32) * sizeof(uint32_t);
}
// the select's list of row chunks for the full select: two uint32 per chunk (a chunk is
// listed by its own select, and again when its row of several chunks falls short)
inline size_t filter_redo_bytes(int H, int G, int n) {
    return (size_t)H * G * (size_t)((n + FATHOM_TOPK_CHUNK - 1) / FATHOM_TOPK_CHUNK) * 8;
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
                       uint8_t *depth, hipStream_t s, uint32_t *zero = nullptr);
hipError_t launch_plan_fixed(const fathom_store &st, int n_channels, uint8_t *depth,
                             hipStream_t s);
// k > 0: also sample the candidate thresholds for a top-k of k (0: no filtering)
hipError_t launch_scan_prepare(const fathom_store &st, const float *q, int G,
                               const uint8_t *depth, int k, void *ws, hipStream_t s);
hipError_t launch_plan_prepare(const fathom_store &st, const float *q, int G, int B, int k,
                               uint8_t *depth, void *ws, hipStream_t s);
// masks == nullptr: every score to `scores`; else the candidate filter (see above)
hipError_t launch_scan_main(const fathom_store &st, int G, float *scores, void *ws,
                            hipStream_t s, uint32_t *masks = nullptr);
// A decode step's plan, prepare and filtering scan in one kernel (k_front_fused): when the
// heads have one query set, rows of one top-k chunk and at most 256 (head, super-step)
// pairs.  The same outputs as launch_plan_prepare + launch_scan_main with the filter,
// except that the rows' kept counts and overflow bits in the workspace are not set.
bool front_fused_applies(const fathom_store &st, int G);
hipError_t launch_front_fused(const fathom_store &st, const float *q, int G, int B, int k,
                              uint8_t *depth, void *ws, float *cand, uint32_t *masks,
                              hipStream_t s);
hipError_t launch_scan_extract(const fathom_store &st, const float *q, int G,
                               const uint8_t *depth, float *scores, hipStream_t s);
hipError_t launch_pack_nibbles(const fathom_store &st, uint8_t *nib, hipStream_t s);
hipError_t launch_quantize_groups(const float *keys, int64_t head_stride,
                                  const fathom_gstore &gs, int g0, int g1, hipStream_t s);
// host_planes: the planes are pinned host memory (longer reads per tile)
hipError_t launch_scan_grouped(const fathom_gstore &gs, const float *q, const uint8_t *depth,
                               int G, float *scores, bool host_planes, hipStream_t s);
hipError_t launch_scan_nibble(const uint8_t *nib, const float *scale, const float *zero, int H,
                              int n, const float *q, int G, float *scores, hipStream_t s);
hipError_t launch_topk(const float *scores, int R, int n, int k, int32_t *idx, void *ws,
                       hipStream_t s);
// top-k of the filtering scan's candidates (rows = H*G); rows that kept fewer than k
// are rescored from the store and the prepared scan workspace
hipError_t launch_topk_filtered(const fathom_store &st, int G, const float *cand,
                                const uint32_t *masks, void *scan_ws, uint32_t *redo_list,
                                int k, int32_t *idx, void *ws, hipStream_t s);
// rows of one chunk, at most 256 of them, small k: the select of the filtering scan's
// candidates runs one workgroup a row and finishes every row itself
bool filtered_direct_applies(int R, int n, int k);
// the same select fused with the attention of each row, for as many rows as fill the
// device's CUs once (filtered_attend_applies); idx still receives the winners
bool filtered_attend_applies(int R, int n, int k);
// the partial results of a step's split attention over R query rows (0 above 256 rows,
// where a row is one workgroup)
size_t attn_part_bytes(int R);
hipError_t launch_topk_filtered_attend(const fathom_store &st, int G, const float *cand,
                                       const uint32_t *masks, void *scan_ws, int k,
                                       int32_t *idx, const float *q, const uint16_t *K,
                                       const uint16_t *V, float sm_scale, uint16_t *out,
                                       float *part, hipStream_t s);
hipError_t launch_sparse_attn(const float *q, const uint16_t *K, const uint16_t *V, int H,
                              int G, int n, const int32_t *idx, int k, float sm_scale,
                              uint16_t *out, hipStream_t s);
// the same inside a decode step: few rows split over several workgroups a row, with the
// parts in `part` (attn_part_bytes(H*G)) and row (h, g)'s counter at count + h * cstride + g
// (zero before the launch); the same results as launch_sparse_attn
hipError_t launch_sparse_attn_split(const float *q, const uint16_t *K, const uint16_t *V,
                                    int H, int G, int n, const int32_t *idx, int k,
                                    float sm_scale, uint16_t *out, float *part,
                                    uint32_t *count, int cstride, hipStream_t s);
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

// Order-preserving 32-bit key of a score (-0 ranks as +0); key 0 is below every
// non-NaN value.
__device__ __forceinline__ uint32_t order_key(float v) {
    uint32_t u = __float_as_uint(v);
    if (u == 0x80000000u) u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
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
