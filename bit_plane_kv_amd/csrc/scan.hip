// The key scan: approximate scores of every key from the planes its head's plan reads.
//
// Sources: the blog's "The first fix" (score every key, keep the top k), "Bit planes"
// (a t-plane prefix is the t-bit quantizer with the same scale), "How each query picks
// its own depth" (each channel read to its own depth), "Where this does not work"
// (with the index in GPU memory, extracting bits costs integer work per bit).
//
// Arithmetic.  With m = p 2^(4-t) + h(t) (bin midpoint, h(t) = (2^(4-t) - 1)/2) and p
// the t-plane prefix, p 2^(4-t) = sum_{j<t} bit_j 2^(3-j), so
//   score_g(i) = C_g + sum over the head's planes (c, j) of bit_cj(i) * q_gc s_c 2^(3-j),
//   C_g = sum_c q_gc (z_c + s_c h(t_c)).
// The B planes of a head are cut into groups of 8; for each group a 256-entry table
// holds, for every 8-bit pattern, the sum of the weights of the planes whose bit is set.
// A token then costs one table lookup per group (per query: G adds) instead of one add
// per plane: the integer work per byte of planes -- what bounds the HBM-resident scan
// -- is a byte gather plus an 8x8 bit transpose per 8 tokens and 8 planes.
#include "common.h"

namespace fathom {
namespace {

// ---------------------------------------------------------------------------------
// prepare: plane list, constant term and lookup tables of one head (one workgroup)
// ---------------------------------------------------------------------------------
template <int GP>
__global__ __launch_bounds__(256) void k_scan_prepare(
    const float *__restrict__ q, const uint8_t *__restrict__ depth,
    const float *__restrict__ scale, const float *__restrict__ zero, int H, int G,
    char *__restrict__ ws) {
    __shared__ int tc[kD];
    __shared__ int off[kD + 1];
    __shared__ double wt[GP][kMaxPlanesPerHead];
    __shared__ double red[GP][kD];
    const int h = blockIdx.x, tid = threadIdx.x, lane = tid & 63;
    ScanMeta *meta = reinterpret_cast<ScanMeta *>(ws + (size_t)h * kMetaBytes);
    float *lut = reinterpret_cast<float *>(ws + (size_t)H * kMetaBytes +
                                           (size_t)h * kMaxGroups * kLutEntries * GP *
                                               sizeof(float));
    if (tid < kD) tc[tid] = min((int)depth[(size_t)h * kD + tid], kPlanes);
    __syncthreads();
    if (tid < 64) {  // one wave: exclusive prefix sum of the depths, 2 channels a lane
        const int a = tc[2 * lane], b = tc[2 * lane + 1];
        int inc = a + b;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int t = __shfl_up(inc, o, 64);
            if (lane >= o) inc += t;
        }
        const int ex = inc - a - b;
        off[2 * lane] = ex;
        off[2 * lane + 1] = ex + a;
        if (lane == 63) off[kD] = inc;
    }
    __syncthreads();
    const int nplanes = off[kD];
    const int ngroups = (nplanes + kGroupBits - 1) / kGroupBits;
    if (tid < kD) {
        const int c = tid, t = tc[c], o = off[c];
        const double s = (double)scale[(size_t)h * kD + c];
        const double z = (double)zero[(size_t)h * kD + c];
        const double hm = (double)((16 >> t) - 1) * 0.5;  // bin-midpoint offset h(t)
        for (int j = 0; j < t; ++j) meta->plane[o + j] = (uint32_t)(c * kPlanes + j);
#pragma unroll
        for (int g = 0; g < GP; ++g) {
            const double qv = g < G ? (double)q[((size_t)h * G + g) * kD + c] : 0.0;
            for (int j = 0; j < t; ++j) wt[g][o + j] = (qv * s) * (double)(8 >> j);
            red[g][c] = qv * (z + s * hm);  // this channel's share of C_g
        }
    }
    __syncthreads();
    // pad the last group with a valid plane so the scan's loads stay in bounds
    if (tid < ngroups * kGroupBits - nplanes) {
        meta->plane[nplanes + tid] = meta->plane[nplanes - 1 < 0 ? 0 : nplanes - 1];
#pragma unroll
        for (int g = 0; g < GP; ++g) wt[g][nplanes + tid] = 0.0;
    }
    for (int s2 = kD / 2; s2 > 0; s2 >>= 1) {  // C_g: fixed-order tree sum over channels
        if (tid < s2) {
#pragma unroll
            for (int g = 0; g < GP; ++g) red[g][tid] += red[g][tid + s2];
        }
        __syncthreads();
    }
    if (tid < FATHOM_MAX_G) meta->C[tid] = tid < G ? (float)red[tid < GP ? tid : 0][0] : 0.0f;
    if (tid == 0) {
        meta->n_planes = nplanes;
        meta->n_groups = ngroups;
    }
    // tables: entry (group, pattern) = sum of the weights of the planes set in pattern
    for (int e = tid; e < ngroups * kLutEntries; e += 256) {
        const int grp = e >> 8, pat = e & (kLutEntries - 1);
        float v[GP];
#pragma unroll
        for (int g = 0; g < GP; ++g) {
            double a = 0.0;
#pragma unroll
            for (int r = 0; r < kGroupBits; ++r)
                a += ((pat >> r) & 1) ? wt[g][grp * kGroupBits + r] : 0.0;
            v[g] = (float)a;
        }
        float *dst = lut + (size_t)e * GP;
        if constexpr (GP == 1) {
            dst[0] = v[0];
        } else if constexpr (GP == 2) {
            *reinterpret_cast<float2 *>(dst) = make_float2(v[0], v[1]);
        } else {
#pragma unroll
            for (int g = 0; g < GP; g += 4)
                *reinterpret_cast<float4 *>(dst + g) = make_float4(v[g], v[g + 1], v[g + 2], v[g + 3]);
        }
    }
}

// ---------------------------------------------------------------------------------
// main scan
// ---------------------------------------------------------------------------------
// 8x8 bit-matrix transpose: byte r of (lo: rows 0-3, hi: rows 4-7) is row r, bit c of
// that byte is column c; afterwards byte c holds column c.
__device__ __forceinline__ void transpose8x8(uint32_t &lo, uint32_t &hi) {
    uint32_t t;
    t = (lo ^ (lo >> 7)) & 0x00AA00AAu;
    lo = lo ^ t ^ (t << 7);
    t = (hi ^ (hi >> 7)) & 0x00AA00AAu;
    hi = hi ^ t ^ (t << 7);
    t = (lo ^ (lo >> 14)) & 0x0000CCCCu;
    lo = lo ^ t ^ (t << 14);
    t = (hi ^ (hi >> 14)) & 0x0000CCCCu;
    hi = hi ^ t ^ (t << 14);
    t = ((lo >> 4) ^ hi) & 0x0F0F0F0Fu;
    hi = hi ^ t;
    lo = lo ^ (t << 4);
}

constexpr int kScanThreads = 256;
constexpr int kTokensPerLane = 16;                                     // half a word
constexpr int kTileWords = kScanThreads * kTokensPerLane / 32;         // 128 words
constexpr int kLdsBudget = 48 * 1024;                                  // tables per batch

template <int GP>
struct Lut;
template <>
struct Lut<1> {
    static __device__ __forceinline__ void add(float (&a)[1], const float *p) { a[0] += p[0]; }
};
template <>
struct Lut<2> {
    static __device__ __forceinline__ void add(float (&a)[2], const float *p) {
        const float2 v = *reinterpret_cast<const float2 *>(p);
        a[0] += v.x;
        a[1] += v.y;
    }
};
template <>
struct Lut<4> {
    static __device__ __forceinline__ void add(float (&a)[4], const float *p) {
        const float4 v = *reinterpret_cast<const float4 *>(p);
        a[0] += v.x;
        a[1] += v.y;
        a[2] += v.z;
        a[3] += v.w;
    }
};
template <>
struct Lut<8> {
    static __device__ __forceinline__ void add(float (&a)[8], const float *p) {
        const float4 v = *reinterpret_cast<const float4 *>(p);
        const float4 u = *reinterpret_cast<const float4 *>(p + 4);
        a[0] += v.x;
        a[1] += v.y;
        a[2] += v.z;
        a[3] += v.w;
        a[4] += u.x;
        a[5] += u.y;
        a[6] += u.z;
        a[7] += u.w;
    }
};

// Lane layout: lane L of wave w reads word (tile*128 + w*32 + L%32) of every plane in a
// group and scores that word's tokens 16*(L/32) .. 16*(L/32)+15; both halves of a word
// read the same address (one 128-byte line per wave per plane).
// Loads one group's 8 plane words for this lane's word.  ids are uniform (SGPRs).
__device__ __forceinline__ void load_group(const uint32_t *__restrict__ hp,
                                           const uint32_t (&ids)[kGroupBits],
                                           int word_stride, int gwc,
                                           uint32_t (&w)[kGroupBits]) {
#pragma unroll
    for (int r = 0; r < kGroupBits; ++r)
        w[r] = hp[(size_t)ids[r] * (size_t)word_stride + gwc];
}

// Uniform read of a group's 8 plane ids from LDS (every lane reads the same address).
__device__ __forceinline__ void lds_ids(const uint32_t *lids, int gi,
                                        uint32_t (&ids)[kGroupBits]) {
    const uint4 a = reinterpret_cast<const uint4 *>(lids)[2 * gi];
    const uint4 b = reinterpret_cast<const uint4 *>(lids)[2 * gi + 1];
    ids[0] = __builtin_amdgcn_readfirstlane(a.x);
    ids[1] = __builtin_amdgcn_readfirstlane(a.y);
    ids[2] = __builtin_amdgcn_readfirstlane(a.z);
    ids[3] = __builtin_amdgcn_readfirstlane(a.w);
    ids[4] = __builtin_amdgcn_readfirstlane(b.x);
    ids[5] = __builtin_amdgcn_readfirstlane(b.y);
    ids[6] = __builtin_amdgcn_readfirstlane(b.z);
    ids[7] = __builtin_amdgcn_readfirstlane(b.w);
}

template <int GP>
__device__ __forceinline__ void lookup_add(const uint32_t (&x)[4], int m0, const float *lg,
                                           float (&acc)[kTokensPerLane][GP]) {
    // 8 table reads in flight, then the adds
    float e[8][GP];
#pragma unroll
    for (int m = 0; m < 8; ++m) {
        const uint32_t pat = (x[(m0 + m) >> 2] >> (8 * ((m0 + m) & 3))) & 0xFFu;
        const float *p = lg + pat * GP;
#pragma unroll
        for (int g = 0; g < GP; g += (GP >= 4 ? 4 : GP)) {
            if constexpr (GP >= 4) {
                const float4 v = *reinterpret_cast<const float4 *>(p + g);
                e[m][g] = v.x;
                e[m][g + 1] = v.y;
                e[m][g + 2] = v.z;
                e[m][g + 3] = v.w;
            } else if constexpr (GP == 2) {
                const float2 v = *reinterpret_cast<const float2 *>(p);
                e[m][0] = v.x;
                e[m][1] = v.y;
            } else {
                e[m][0] = p[0];
            }
        }
    }
#pragma unroll
    for (int m = 0; m < 8; ++m)
#pragma unroll
        for (int g = 0; g < GP; ++g) acc[m0 + m][g] += e[m][g];
}

template <int GP>
__device__ __forceinline__ void process_group(const uint32_t (&w)[kGroupBits],
                                              uint32_t sel_pair, const float *lg,
                                              float (&acc)[kTokensPerLane][GP]) {
    const uint32_t t01 = __builtin_amdgcn_perm(w[1], w[0], sel_pair);
    const uint32_t t23 = __builtin_amdgcn_perm(w[3], w[2], sel_pair);
    const uint32_t t45 = __builtin_amdgcn_perm(w[5], w[4], sel_pair);
    const uint32_t t67 = __builtin_amdgcn_perm(w[7], w[6], sel_pair);
    uint32_t x[4];
    x[0] = __builtin_amdgcn_perm(t23, t01, 0x05040100u);  // tokens 0-7: rows 0-3
    x[1] = __builtin_amdgcn_perm(t67, t45, 0x05040100u);  //             rows 4-7
    x[2] = __builtin_amdgcn_perm(t23, t01, 0x07060302u);  // tokens 8-15: rows 0-3
    x[3] = __builtin_amdgcn_perm(t67, t45, 0x07060302u);  //              rows 4-7
    transpose8x8(x[0], x[1]);
    transpose8x8(x[2], x[3]);
    lookup_add<GP>(x, 0, lg, acc);
    lookup_add<GP>(x, 8, lg, acc);
}

// Lane layout: lane L of wave w reads word (tile*128 + w*32 + L%32) of every plane in a
// group and scores that word's tokens 16*(L/32) .. 16*(L/32)+15; both halves of a word
// read the same address (one 128-byte line per wave per plane).  The plane words of the
// next two groups are in flight while a group is transposed and looked up; the plane
// ids of a batch sit in LDS next to its tables.
template <int GP>
__global__ __launch_bounds__(kScanThreads) void k_scan_main(
    const uint32_t *__restrict__ planes, int n, int word_stride, int G, int H,
    int tiles_per_head, const char *__restrict__ ws, float *__restrict__ scores) {
    extern __shared__ float4 lds_v4[];  // 16-byte aligned: tables, then plane ids
    constexpr int kBatchGroups = kLdsBudget / (kLutEntries * GP * (int)sizeof(float));
    float *lds = reinterpret_cast<float *>(lds_v4);
    uint32_t *lids = reinterpret_cast<uint32_t *>(lds_v4 + kBatchGroups * kLutEntries * GP / 4);
    const int lb = xcd_remap(blockIdx.x, gridDim.x);
    const int h = lb / tiles_per_head, tile = lb - h * tiles_per_head;
    const ScanMeta *meta = reinterpret_cast<const ScanMeta *>(ws + (size_t)h * kMetaBytes);
    const float *lut = reinterpret_cast<const float *>(
        ws + (size_t)H * kMetaBytes +
        (size_t)h * kMaxGroups * kLutEntries * GP * sizeof(float));
    // clamped so that any workspace content keeps every read inside this head's data
    const int ngroups = min(max(meta->n_groups, 0), kMaxGroups);
    const uint32_t *pids = meta->plane;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, half = lane >> 5;
    const int W = (n + 31) >> 5;
    const int gw = tile * kTileWords + wave * 32 + (lane & 31);
    const int gwc = min(gw, W - 1);  // lanes past the end re-read the last word
    const uint32_t *hp = planes + (size_t)h * kMaxPlanesPerHead * word_stride;
    // byte selectors: pairs (w_a, w_b) -> [a.b(2h), b.b(2h), a.b(2h+1), b.b(2h+1)]
    const uint32_t sel_pair = half ? 0x07030602u : 0x05010400u;

    float acc[kTokensPerLane][GP];
#pragma unroll
    for (int g = 0; g < GP; ++g) {
        const float c0 = g < G ? meta->C[g] : 0.0f;
#pragma unroll
        for (int m = 0; m < kTokensPerLane; ++m) acc[m][g] = c0;
    }

    for (int gb0 = 0; gb0 < ngroups; gb0 += kBatchGroups) {
        const int gcount = min(kBatchGroups, ngroups - gb0);
        uint32_t wa[kGroupBits], wb[kGroupBits];
        {
            uint32_t ida[kGroupBits], idb[kGroupBits];
#pragma unroll
            for (int r = 0; r < kGroupBits; ++r) {
                ida[r] = pids[gb0 * kGroupBits + r] & (kMaxPlanesPerHead - 1);
                idb[r] = pids[min(gb0 + 1, gb0 + gcount - 1) * kGroupBits + r] &
                         (kMaxPlanesPerHead - 1);
            }
            load_group(hp, ida, word_stride, gwc, wa);
            load_group(hp, idb, word_stride, gwc, wb);
        }
        __syncthreads();
        {
            const float4 *src =
                reinterpret_cast<const float4 *>(lut + (size_t)gb0 * kLutEntries * GP);
            const int nvec = gcount * kLutEntries * GP / 4;
            for (int e = tid; e < nvec; e += kScanThreads) lds_v4[e] = src[e];
            for (int e = tid; e < gcount * kGroupBits; e += kScanThreads)
                lids[e] = pids[gb0 * kGroupBits + e] & (kMaxPlanesPerHead - 1);
        }
        __syncthreads();
        for (int gi = 0; gi < gcount; gi += 2) {
            uint32_t ida[kGroupBits], idb[kGroupBits];
            lds_ids(lids, min(gi + 2, gcount - 1), ida);
            lds_ids(lids, min(gi + 3, gcount - 1), idb);
            process_group<GP>(wa, sel_pair, lds + gi * kLutEntries * GP, acc);
            load_group(hp, ida, word_stride, gwc, wa);
            if (gi + 1 < gcount)
                process_group<GP>(wb, sel_pair, lds + (gi + 1) * kLutEntries * GP, acc);
            load_group(hp, idb, word_stride, gwc, wb);
        }
    }

    const int tok0 = gw * 32 + half * kTokensPerLane;
    if (tok0 >= n) return;
    const bool full = (tok0 + kTokensPerLane <= n) && ((n & 3) == 0);
#pragma unroll
    for (int g = 0; g < GP; ++g) {
        if (g >= G) break;
        float *out = scores + ((size_t)h * G + g) * n + tok0;
        if (full) {
#pragma unroll
            for (int m = 0; m < kTokensPerLane; m += 4)
                *reinterpret_cast<float4 *>(out + m) =
                    make_float4(acc[m][g], acc[m + 1][g], acc[m + 2][g], acc[m + 3][g]);
        } else {
#pragma unroll
            for (int m = 0; m < kTokensPerLane; ++m)
                if (tok0 + m < n) out[m] = acc[m][g];
        }
    }
}

template <int GP>
hipError_t launch_main_gp(const fathom_store &st, int G, float *scores, const char *ws,
                          hipStream_t s) {
    const int W = (st.n_tokens + 31) >> 5;
    const int tiles = (W + kTileWords - 1) / kTileWords;
    const int nblocks = st.n_heads * tiles;
    constexpr int kBatchGroups = kLdsBudget / (kLutEntries * GP * (int)sizeof(float));
    const size_t lds = (size_t)kBatchGroups * kLutEntries * GP * sizeof(float) +
                       (size_t)kBatchGroups * kGroupBits * sizeof(uint32_t);
    hipLaunchKernelGGL(k_scan_main<GP>, dim3(nblocks), dim3(kScanThreads), lds, s,
                       st.planes, st.n_tokens, st.word_stride, G, st.n_heads, tiles, ws,
                       scores);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_scan_prepare(const fathom_store &st, const float *q, int G,
                               const uint8_t *depth, void *ws, hipStream_t s) {
    char *w = static_cast<char *>(ws);
    const dim3 grid(st.n_heads), block(256);
    switch (padded_g(G)) {
    case 1: hipLaunchKernelGGL(k_scan_prepare<1>, grid, block, 0, s, q, depth, st.scale, st.zero, st.n_heads, G, w); break;
    case 2: hipLaunchKernelGGL(k_scan_prepare<2>, grid, block, 0, s, q, depth, st.scale, st.zero, st.n_heads, G, w); break;
    case 4: hipLaunchKernelGGL(k_scan_prepare<4>, grid, block, 0, s, q, depth, st.scale, st.zero, st.n_heads, G, w); break;
    default: hipLaunchKernelGGL(k_scan_prepare<8>, grid, block, 0, s, q, depth, st.scale, st.zero, st.n_heads, G, w); break;
    }
    return hipGetLastError();
}

hipError_t launch_scan_main(const fathom_store &st, int G, float *scores, void *ws,
                            hipStream_t s) {
    const char *w = static_cast<const char *>(ws);
    switch (padded_g(G)) {
    case 1: return launch_main_gp<1>(st, G, scores, w, s);
    case 2: return launch_main_gp<2>(st, G, scores, w, s);
    case 4: return launch_main_gp<4>(st, G, scores, w, s);
    default: return launch_main_gp<8>(st, G, scores, w, s);
    }
}

}  // namespace fathom
