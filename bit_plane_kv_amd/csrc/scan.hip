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
__global__ __launch_bounds__(256) void k_scan_prepare(
    const float *__restrict__ q, const uint8_t *__restrict__ depth,
    const float *__restrict__ scale, const float *__restrict__ zero, int H, int G, int gp,
    char *__restrict__ ws) {
    __shared__ int tc[kD];
    __shared__ int off[kD + 1];
    __shared__ double wt[FATHOM_MAX_G][kMaxPlanesPerHead];
    const int h = blockIdx.x, tid = threadIdx.x;
    ScanMeta *meta = reinterpret_cast<ScanMeta *>(ws + (size_t)h * kMetaBytes);
    float *lut = reinterpret_cast<float *>(ws + (size_t)H * kMetaBytes +
                                           (size_t)h * kMaxGroups * kLutEntries * gp *
                                               sizeof(float));
    if (tid < kD) tc[tid] = min((int)depth[(size_t)h * kD + tid], kPlanes);
    __syncthreads();
    if (tid == 0) {
        int a = 0;
        for (int c = 0; c < kD; ++c) {
            off[c] = a;
            a += tc[c];
        }
        off[kD] = a;
    }
    __syncthreads();
    const int nplanes = off[kD];
    const int ngroups = (nplanes + kGroupBits - 1) / kGroupBits;
    if (tid < kD) {
        const int c = tid, t = tc[c], o = off[c];
        const double s = (double)scale[(size_t)h * kD + c];
        for (int j = 0; j < t; ++j) {
            meta->plane[o + j] = (uint16_t)(c * kPlanes + j);
            for (int g = 0; g < G; ++g) {
                const double qv = (double)q[((size_t)h * G + g) * kD + c];
                wt[g][o + j] = (qv * s) * (double)(8 >> j);  // q s 2^(3-j), exact
            }
        }
    }
    if (tid < FATHOM_MAX_G) {
        float cg = 0.0f;
        if (tid < G) {
            double a = 0.0;
            for (int c = 0; c < kD; ++c) {
                const int t = tc[c];
                const double hm = (double)((16 >> t) - 1) * 0.5;  // bin-midpoint offset
                const double khat0 = (double)zero[(size_t)h * kD + c] +
                                     (double)scale[(size_t)h * kD + c] * hm;
                a += (double)q[((size_t)h * G + tid) * kD + c] * khat0;
            }
            cg = (float)a;
        }
        meta->C[tid] = cg;
    }
    if (tid == 0) {
        meta->n_planes = nplanes;
        meta->n_groups = ngroups;
    }
    __syncthreads();
    for (int e = tid; e < ngroups * kLutEntries; e += 256) {
        const int grp = e >> 8, pat = e & (kLutEntries - 1);
        for (int g = 0; g < gp; ++g) {
            double a = 0.0;
            for (int r = 0; r < kGroupBits; ++r) {
                const int b = grp * kGroupBits + r;
                if (b < nplanes && ((pat >> r) & 1)) a += wt[g < G ? g : 0][b];
            }
            lut[(size_t)e * gp + g] = g < G ? (float)a : 0.0f;
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
template <int GP>
__global__ __launch_bounds__(kScanThreads) void k_scan_main(
    const uint32_t *__restrict__ planes, int n, int word_stride, int G, int H,
    int tiles_per_head, const char *__restrict__ ws, float *__restrict__ scores) {
    extern __shared__ float4 lds_v4[];  // 16-byte aligned table storage
    float *lds = reinterpret_cast<float *>(lds_v4);
    constexpr int kBatchGroups = kLdsBudget / (kLutEntries * GP * (int)sizeof(float));
    const int lb = xcd_remap(blockIdx.x, gridDim.x);
    const int h = lb / tiles_per_head, tile = lb - h * tiles_per_head;
    const ScanMeta *meta = reinterpret_cast<const ScanMeta *>(ws + (size_t)h * kMetaBytes);
    const float *lut = reinterpret_cast<const float *>(
        ws + (size_t)H * kMetaBytes +
        (size_t)h * kMaxGroups * kLutEntries * GP * sizeof(float));
    const int nplanes = meta->n_planes, ngroups = meta->n_groups;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, half = lane >> 5;
    const int W = (n + 31) >> 5;
    const int gw = tile * kTileWords + wave * 32 + (lane & 31);
    const bool wvalid = gw < W;
    const uint32_t *ph = planes + (size_t)h * kMaxPlanesPerHead * word_stride + gw;
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
        __syncthreads();
        {
            const float4 *src =
                reinterpret_cast<const float4 *>(lut + (size_t)gb0 * kLutEntries * GP);
            float4 *dst = reinterpret_cast<float4 *>(lds);
            const int nvec = gcount * kLutEntries * GP / 4;
            for (int e = tid; e < nvec; e += kScanThreads) dst[e] = src[e];
        }
        __syncthreads();
        for (int gi = 0; gi < gcount; ++gi) {
            const int pbase = (gb0 + gi) * kGroupBits;
            const int pc = min(kGroupBits, nplanes - pbase);
            uint32_t w[kGroupBits];
#pragma unroll
            for (int r = 0; r < kGroupBits; ++r) {
                uint32_t v = 0u;
                if (r < pc && wvalid)
                    v = ph[(size_t)meta->plane[pbase + r] * word_stride];
                w[r] = v;
            }
            const uint32_t t01 = __builtin_amdgcn_perm(w[1], w[0], sel_pair);
            const uint32_t t23 = __builtin_amdgcn_perm(w[3], w[2], sel_pair);
            const uint32_t t45 = __builtin_amdgcn_perm(w[5], w[4], sel_pair);
            const uint32_t t67 = __builtin_amdgcn_perm(w[7], w[6], sel_pair);
            uint32_t x[4];
            x[0] = __builtin_amdgcn_perm(t23, t01, 0x05040100u);  // tokens 0-3 (rows 0-3)
            x[1] = __builtin_amdgcn_perm(t67, t45, 0x05040100u);  // rows 4-7
            x[2] = __builtin_amdgcn_perm(t23, t01, 0x07060302u);  // tokens 8-15, rows 0-3
            x[3] = __builtin_amdgcn_perm(t67, t45, 0x07060302u);
            transpose8x8(x[0], x[1]);
            transpose8x8(x[2], x[3]);
            const float *lg = lds + gi * kLutEntries * GP;
#pragma unroll
            for (int m = 0; m < kTokensPerLane; ++m) {
                const uint32_t pat = (x[m >> 2] >> (8 * (m & 3))) & 0xFFu;
                Lut<GP>::add(acc[m], lg + pat * GP);
            }
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
    const size_t lds = (size_t)kBatchGroups * kLutEntries * GP * sizeof(float);
    hipLaunchKernelGGL(k_scan_main<GP>, dim3(nblocks), dim3(kScanThreads), lds, s,
                       st.planes, st.n_tokens, st.word_stride, G, st.n_heads, tiles, ws,
                       scores);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_scan_prepare(const fathom_store &st, const float *q, int G,
                               const uint8_t *depth, void *ws, hipStream_t s) {
    hipLaunchKernelGGL(k_scan_prepare, dim3(st.n_heads), dim3(256), 0, s, q, depth, st.scale,
                       st.zero, st.n_heads, G, padded_g(G), static_cast<char *>(ws));
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
