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

// Shape of the main kernel.  A workgroup of 8 waves scores a tile of 128 words (4096
// tokens) of one head.  In a wave, the 4 lanes of a quad share one 32-token word: lane
// (4w + s) loads planes s and s+4 of word w, a 4x4 byte transpose across the quad gives
// every lane byte s (8 tokens) of all 8 planes of the group, and lane (4w + s) scores
// tokens 8s .. 8s+7 of the word.  Each lane thus issues 2 loads per group of 8 planes.
constexpr int kScanThreads = 512;
constexpr int kWordsPerWave = 16;
constexpr int kTileWords = (kScanThreads / 64) * kWordsPerWave;  // 128 words
constexpr int kTokensPerLane = 8;
constexpr int kInflight = 4;   // table reads issued before their adds
constexpr int kPrefetch = 4;   // groups of plane words in flight per lane
constexpr int kLdsBudget = 48 * 1024;  // tables per batch (LDS also stages the scores)

// Byte transpose across a quad: lane s holds word M_s; afterwards byte p of lane s's
// result is byte s of M_p (p = 0..3).  Two butterfly stages, each one DPP move of the
// partner's word and one byte permute.
__device__ __forceinline__ uint32_t quad_byte_transpose(uint32_t m, int s) {
    const uint32_t p = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0x4E, 0xF, 0xF, false);
    const uint32_t a = __builtin_amdgcn_perm(p, m, s < 2 ? 0x05040100u : 0x03020706u);
    const uint32_t q = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)a, 0xB1, 0xF, 0xF, false);
    return __builtin_amdgcn_perm(q, a, (s & 1) ? 0x03070105u : 0x06020400u);
}

// Adds the table entries of tokens m0 .. m0+kInflight-1 (reads first, then adds).
template <int GP>
__device__ __forceinline__ void lookup_add(const uint32_t (&x)[2], int m0, const float *lg,
                                           float (&acc)[kTokensPerLane][GP]) {
    float e[kInflight][GP];
#pragma unroll
    for (int m = 0; m < kInflight; ++m) {
        const uint32_t pat = (x[(m0 + m) >> 2] >> (8 * ((m0 + m) & 3))) & 0xFFu;
        const float *p = lg + pat * GP;
        if constexpr (GP >= 4) {
#pragma unroll
            for (int g = 0; g < GP; g += 4) {
                const float4 v = *reinterpret_cast<const float4 *>(p + g);
                e[m][g] = v.x;
                e[m][g + 1] = v.y;
                e[m][g + 2] = v.z;
                e[m][g + 3] = v.w;
            }
        } else if constexpr (GP == 2) {
            const float2 v = *reinterpret_cast<const float2 *>(p);
            e[m][0] = v.x;
            e[m][1] = v.y;
        } else {
            e[m][0] = p[0];
        }
    }
#pragma unroll
    for (int m = 0; m < kInflight; ++m)
#pragma unroll
        for (int g = 0; g < GP; ++g) acc[m0 + m][g] += e[m][g];
}

// One group: quad byte transposes give x[0] = byte s of planes 0-3 and x[1] = planes
// 4-7 (an 8x8 bit block: 8 planes x 8 tokens); the bit transpose turns byte m into
// token m's 8-plane pattern; then the table lookups.
template <int GP>
__device__ __forceinline__ void process_group(const uint32_t (&w)[2], int s, const float *lg,
                                              float (&acc)[kTokensPerLane][GP]) {
    uint32_t x[2];
    x[0] = quad_byte_transpose(w[0], s);
    x[1] = quad_byte_transpose(w[1], s);
    transpose8x8(x[0], x[1]);
#pragma unroll
    for (int m0 = 0; m0 < kTokensPerLane; m0 += kInflight) lookup_add<GP>(x, m0, lg, acc);
}

// Issues this lane's two plane-word loads of group gi (row offsets of the batch's planes
// are staged in LDS, in words).
__device__ __forceinline__ void issue_group(const uint32_t *lane_base, const uint64_t *lrow,
                                            int gi, int s, uint32_t (&w)[2]) {
    const uint64_t r0 = lrow[gi * kGroupBits + s];
    const uint64_t r1 = lrow[gi * kGroupBits + s + 4];
    w[0] = lane_base[r0];
    w[1] = lane_base[r1];
}

template <int GP>
__global__ __launch_bounds__(kScanThreads) void k_scan_main(
    const uint32_t *__restrict__ planes, int n, int word_stride, int G, int H,
    int tiles_per_head, const char *__restrict__ ws, float *__restrict__ scores) {
    extern __shared__ float4 lds_v4[];  // 16-byte aligned: tables, then plane rows
    constexpr int kBatchGroups = kLdsBudget / (kLutEntries * GP * (int)sizeof(float));
    float *lds = reinterpret_cast<float *>(lds_v4);
    uint64_t *lrow =
        reinterpret_cast<uint64_t *>(lds_v4 + kBatchGroups * kLutEntries * GP / 4);
    const int lb = xcd_remap(blockIdx.x, gridDim.x);
    const int h = lb / tiles_per_head, tile = lb - h * tiles_per_head;
    const ScanMeta *meta = reinterpret_cast<const ScanMeta *>(ws + (size_t)h * kMetaBytes);
    const float *lut = reinterpret_cast<const float *>(
        ws + (size_t)H * kMetaBytes +
        (size_t)h * kMaxGroups * kLutEntries * GP * sizeof(float));
    // clamped so that any workspace content keeps every read inside this head's data
    const int ngroups = min(max(meta->n_groups, 0), kMaxGroups);
    const uint32_t *pids = meta->plane;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int s = lane & 3;  // quad position: byte of the word = tokens 8s .. 8s+7
    const int W = (n + 31) >> 5;
    const int gw = tile * kTileWords + wave * kWordsPerWave + (lane >> 2);
    const int gwc = min(gw, W - 1);  // lanes past the end re-read the last word
    const uint32_t *lane_base = planes + (size_t)h * kMaxPlanesPerHead * word_stride + gwc;

    float acc[kTokensPerLane][GP];
#pragma unroll
    for (int g = 0; g < GP; ++g) {
        const float c0 = g < G ? meta->C[g] : 0.0f;
#pragma unroll
        for (int m = 0; m < kTokensPerLane; ++m) acc[m][g] = c0;
    }

    for (int gb0 = 0; gb0 < ngroups; gb0 += kBatchGroups) {
        const int gcount = min(kBatchGroups, ngroups - gb0);
        __syncthreads();  // the previous batch's tables are no longer read
        {
            const float4 *src =
                reinterpret_cast<const float4 *>(lut + (size_t)gb0 * kLutEntries * GP);
            const int nvec = gcount * kLutEntries * GP / 4;
            for (int e = tid; e < nvec; e += kScanThreads) lds_v4[e] = src[e];
            for (int e = tid; e < gcount * kGroupBits; e += kScanThreads)
                lrow[e] = (uint64_t)(pids[gb0 * kGroupBits + e] & (kMaxPlanesPerHead - 1)) *
                          (uint64_t)word_stride;
        }
        __syncthreads();
        uint32_t buf[kPrefetch][2];
#pragma unroll
        for (int u = 0; u < kPrefetch; ++u) issue_group(lane_base, lrow, min(u, gcount - 1), s, buf[u]);
        for (int gi = 0; gi < gcount; gi += kPrefetch) {
#pragma unroll
            for (int u = 0; u < kPrefetch; ++u) {
                if (gi + u < gcount)
                    process_group<GP>(buf[u], s, lds + (gi + u) * kLutEntries * GP, acc);
                issue_group(lane_base, lrow, min(gi + u + kPrefetch, gcount - 1), s, buf[u]);
            }
        }
    }

    // Scores leave through LDS so that every store instruction writes 1 KB of one row:
    // each wave stages its 512 tokens for two queries at a time in its own 4 KB.
    __syncthreads();  // all table reads of the workgroup are done
    float *stage = lds + wave * 2 * 512;
    const int wtok0 = (tile * kTileWords + wave * kWordsPerWave) * 32;  // wave's first token
    const int pos = (lane >> 2) * 32 + s * kTokensPerLane;             // lane's first token
#pragma unroll
    for (int g0 = 0; g0 < GP; g0 += 2) {
        if (g0 >= G) break;
#pragma unroll
        for (int gg = 0; gg < 2 && g0 + gg < GP; ++gg) {
            float *d = stage + gg * 512 + pos;
            *reinterpret_cast<float4 *>(d) =
                make_float4(acc[0][g0 + gg], acc[1][g0 + gg], acc[2][g0 + gg], acc[3][g0 + gg]);
            *reinterpret_cast<float4 *>(d + 4) =
                make_float4(acc[4][g0 + gg], acc[5][g0 + gg], acc[6][g0 + gg], acc[7][g0 + gg]);
        }
        __builtin_amdgcn_wave_barrier();  // the wave's staged rows are complete
#pragma unroll
        for (int gg = 0; gg < 2; ++gg) {
            const int g = g0 + gg;
            if (g >= G) break;
            float *row = scores + ((size_t)h * G + g) * n;
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                const int t = half * 256 + lane * 4;  // token within the wave's 512
                const float4 v = *reinterpret_cast<const float4 *>(stage + gg * 512 + t);
                const int tok = wtok0 + t;
                if (tok + 4 <= n && (n & 3) == 0) {
                    *reinterpret_cast<float4 *>(row + tok) = v;
                } else {
                    if (tok < n) row[tok] = v.x;
                    if (tok + 1 < n) row[tok + 1] = v.y;
                    if (tok + 2 < n) row[tok + 2] = v.z;
                    if (tok + 3 < n) row[tok + 3] = v.w;
                }
            }
        }
        __builtin_amdgcn_wave_barrier();  // reads done before the next pair is staged
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
                       (size_t)kBatchGroups * kGroupBits * sizeof(uint64_t);
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
