// The key scan: approximate scores of every key from the planes its head's plan reads.
//
// Sources: the blog's "The first fix" (score every key, keep the top k), "Bit planes"
// (a t-plane prefix is the t-bit quantizer with the same scale), "How each query picks
// its own depth" (each channel read to its own depth), "Where this does not work"
// (with the index in GPU memory, extracting bits costs integer work per bit).
//
// Arithmetic.  With m = p 2^(4-t) + h(t) (bin midpoint, h(t) = (2^(4-t) - 1)/2) and p
// the t-plane prefix, p 2^(4-t) = sum_{j<t} bit_j 2^(3-j), so
//   score_g(i) = C_g + sum over the head's planes P = (c, j) of bit_P(i) * w_gP,
//   w_gP = q_gc s_c 2^(3-j),   C_g = sum_c q_gc (z_c + s_c h(t_c)).
// The sum over planes is the product of the token-by-plane bit matrix and the
// plane-by-query weight matrix, so it runs on the matrix cores in int8: each weight
// becomes an integer count of a per-query unit S_g = 2^(e_g - 30) (e_g: the binary
// exponent just above the largest |w_gP| of the head, so the error is at most 2^-31 of
// the largest weight), written as 4 signed base-256 digits.  One 16x16x64 i8 MFMA takes
// 16 rows = 4 queries x 4 digits, K = 64 planes (8 groups of 8) and 16 columns = 16
// tokens whose plane bits are bytes; the int32 sums are exact, and one fp32 combine per
// score gives C_g + S_g * sum_d 256^d D_d.  For each 16-column block a lane turns words of
// 16 planes into its operand with four byte transposes across its quad and one mask per
// 4 bytes for each of the 8 token bits; no table lookups.
#include <algorithm>
#include <mutex>

#include "common.h"
#include "plan_device.h"
#include "scan_device.h"

namespace fathom {
namespace {

// ---------------------------------------------------------------------------------
// prepare: plane list, constant terms, weight units and MFMA operand records of one
// head (one workgroup)
// ---------------------------------------------------------------------------------
// One K-pair: w[h][p][pos] = word pos of plane s (p = 0) / s+4 (p = 1) of group q + 4h.
// kHi: the upper 4 groups exist; without them their operand bytes are zero and their
// words are neither transposed nor masked.
template <int QS, bool kFirst, bool kHi, int NP = 2>
__device__ __forceinline__ void mma_kpair(const uint32_t (&w)[2][2][NP], const v4i (&A)[QS],
                                          int s, bool hi, v4i (&acc)[NP][8][QS]) {
    const uint32_t hi_mask = hi ? 0xFFFFFFFFu : 0u;
#pragma unroll
    for (int pos = 0; pos < NP; ++pos) {
        uint32_t x[2][2];  // [half][planes 0-3 / 4-7]
#pragma unroll
        for (int h = 0; h < (kHi ? 2 : 1); ++h) {
            x[h][0] = quad_byte_transpose(w[h][0][pos], s);
            x[h][1] = quad_byte_transpose(w[h][1][pos], s);
        }
#pragma unroll
        for (int m = 0; m < 8; ++m) {
            const uint32_t mask = 0x01010101u << m;
            const uint32_t mhi = mask & hi_mask;
            const v4i b = kHi ? v4i{(int)(x[0][0] & mask), (int)(x[0][1] & mask),
                                    (int)(x[1][0] & mhi), (int)(x[1][1] & mhi)}
                              : v4i{(int)(x[0][0] & mask), (int)(x[0][1] & mask), 0, 0};
#pragma unroll
            for (int set = 0; set < QS; ++set) {
                const v4i c = kFirst ? v4i{0, 0, 0, 0} : acc[pos][m][set];
                acc[pos][m][set] = __builtin_amdgcn_mfma_i32_16x16x64_i8(A[set], b, c, 0, 0, 0);
            }
        }
    }
}

// One pass of a K-pair of the scan from operand dwords read with the LDS transpose read:
// x[h][p] = byte s (8 tokens) of planes 4p .. 4p+3 of group q + 4h.
template <int QS, bool kFirst>
__device__ __forceinline__ void mma_pass_x(const uint32_t (&x)[2][2], const v4i (&A)[QS],
                                           uint32_t hi_mask, v4i (&acc)[8][QS]) {
#pragma unroll
    for (int m = 0; m < 8; ++m) {
        const uint32_t mask = 0x01010101u << m;
        const uint32_t mhi = mask & hi_mask;
        const v4i b = v4i{(int)(x[0][0] & mask), (int)(x[0][1] & mask), (int)(x[1][0] & mhi),
                          (int)(x[1][1] & mhi)};
#pragma unroll
        for (int set = 0; set < QS; ++set) {
            const v4i c = kFirst ? v4i{0, 0, 0, 0} : acc[m][set];
            acc[m][set] = __builtin_amdgcn_mfma_i32_16x16x64_i8(A[set], b, c, 0, 0, 0);
        }
    }
}

// NP words per lane (2 in the scan; 1 in the threshold sample of a 512-thread prepare)
template <int QS, int NP = 2>
__device__ __forceinline__ void mma_item(const uint32_t (&w)[2][2][NP], const v4i (&A)[QS], int s,
                                         bool first, bool hi, v4i (&acc)[NP][8][QS]) {
    if (first) mma_kpair<QS, true, true, NP>(w, A, s, hi, acc);
    else mma_kpair<QS, false, true, NP>(w, A, s, hi, acc);
}

// Candidate thresholds of one head (NT threads: 256 or 512).  A guess of each query's score
// quantile from a sample of the head's tokens (sample_run_word): the sampled tokens are
// scored exactly as the scan scores them -- the same operand records, matrix-core digit
// sums and fp32 combine -- and the sample_rank-th largest sampled key is the threshold,
// about five standard deviations of the sample quantile above the k the select needs.
// Only the count of kept tokens decides correctness, and the select checks it.  The
// sampled words of up to 128 planes (two K-pairs) at a time are staged in LDS, 16 bytes
// per (plane, run), all in flight together (those of the first 128 planes are loaded by
// sample_issue as soon as the plane list is known); each wave then takes its share of
// the sampled words (8 of 4 waves, 4 of 8) the way a scan wave takes its 8 words of a
// super-step.
constexpr int kSamplePlanes = 128;
static_assert(kSampleWords == 32, "32 sampled words: 8 a wave of 4, 4 a wave of 8");

// Loads (plane p0 + e / 8, run e % 8), e = tid + NT u, of the head's plane list pl
// (np planes from p0).  Every load is unconditional -- a plane past the list reads the
// store's row 0, a run past a short row the row's first 16 bytes -- so that the
// compiler keeps them all in flight; sample_stage drops those values.
template <int NT>
constexpr int sample_per() { return kSamplePlanes * kSampleRuns / NT; }  // loads a thread

template <int NT>
__device__ __forceinline__ void sample_issue(const uint32_t *__restrict__ hp, int W,
                                             int word_stride, const uint32_t *pl, int p0,
                                             int np, uint4 (&v)[sample_per<NT>()]) {
    constexpr int SP = sample_per<NT>();
    uint32_t row[SP];
#pragma unroll
    for (int u = 0; u < SP; ++u) {  // every list read first (p0 + p < 512 always)
        const int p = (threadIdx.x + NT * u) / kSampleRuns;
        row[u] = pl[p0 + p];
    }
#pragma unroll
    for (int u = 0; u < SP; ++u) {
        const int e = threadIdx.x + NT * u;
        const int p = e / kSampleRuns, r = e % kSampleRuns;
        const int w0 = sample_run_word(r, W);
        // a run that starts below W lies in the row (word_stride >= 4 * ceil(W / 4))
        v[u] = *reinterpret_cast<const uint4 *>(hp + (size_t)(p < np ? row[u] : 0u) * word_stride +
                                                (w0 < W ? w0 : 0));
    }
}
// Writes the loaded values of real (plane, run) pairs to sw; a run past a short row is
// zero.  Rows of sw past np keep whatever they hold: their planes have zero weights.
template <int NT>
__device__ __forceinline__ void sample_stage(const uint4 (&v)[sample_per<NT>()], int W, int np,
                                             uint32_t (*sw)[kSampleWords]) {
#pragma unroll
    for (int u = 0; u < sample_per<NT>(); ++u) {
        const int e = threadIdx.x + NT * u;
        const int p = e / kSampleRuns, r = e % kSampleRuns;
        const bool live = sample_run_word(r, W) < W;
        if (p < np)
            *reinterpret_cast<uint4 *>(&sw[p][kSampleRunWords * r]) =
                live ? v[u] : make_uint4(0u, 0u, 0u, 0u);
    }
}

// The m-th largest (m >= 1) of the wave's 64 N keys with its low 12 bits cleared (the
// top 20 bits suffice for a guess), bit by bit from the top: the largest such T with at
// least m keys >= T.
template <int N>
__device__ __forceinline__ uint32_t rank_top_bits(const uint32_t (&kk)[N], uint32_t m) {
    uint32_t T = 0u;
    for (int b = 31; b >= 12; --b) {
        const uint32_t cand = T | (1u << b);
        uint32_t c = 0u;
#pragma unroll
        for (int e = 0; e < N; ++e) c += (uint32_t)__popcll(__ballot(kk[e] >= cand));
        if (c >= m) T = cand;
    }
    return T;
}

// rank_top_bits of the total (<= 64 N) keys compacted at the front of buf (zero keys
// count for nothing: every candidate is at least 2^12).
template <int N>
__device__ __forceinline__ uint32_t rank_top_bits_buf(const uint32_t *buf, uint32_t total,
                                                      uint32_t m, int lane) {
    uint32_t kk[N];
#pragma unroll
    for (int e = 0; e < N; ++e) kk[e] = (uint32_t)lane + 64u * e < total ? buf[lane + 64 * e] : 0u;
    return rank_top_bits(kk, m);
}

// rank_top_bits of the wave's 1024 sampled keys, searched over fewer keys: with L the
// same search over the two largest keys of each lane (m <= 128), at least m keys are
// >= L, so the m-th largest key is too, and every count the search compares with m is
// the same over the keys >= L as over all of them (below L both are >= m).  When at
// most 256 keys are >= L they are compacted into buf (this wave's 1024 words of LDS)
// and searched one to four a lane; otherwise all 16 a lane are.
__device__ __forceinline__ uint32_t sample_quantile(const uint32_t (&kk)[16], uint32_t m,
                                                    int lane, uint32_t *buf) {
    if (m > 128u) return rank_top_bits(kk, m);
    uint32_t top[2] = {0u, 0u};  // the lane's largest and second largest key
#pragma unroll
    for (int e = 0; e < 16; ++e) {
        top[1] = max(top[1], min(top[0], kk[e]));
        top[0] = max(top[0], kk[e]);
    }
    const uint32_t L = rank_top_bits(top, m);
    uint32_t c = 0u;
#pragma unroll
    for (int e = 0; e < 16; ++e) c += kk[e] >= L;
    uint32_t inc = c;  // inclusive prefix over the lanes
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const uint32_t t = (uint32_t)__shfl_up((int)inc, o, 64);
        if (lane >= o) inc += t;
    }
    const uint32_t total = (uint32_t)__shfl((int)inc, 63, 64);
    if (total > 256u) return rank_top_bits(kk, m);
    uint32_t pos = inc - c;
#pragma unroll
    for (int e = 0; e < 16; ++e)
        if (kk[e] >= L) buf[pos++] = kk[e];
    if (total <= 64u) return rank_top_bits_buf<1>(buf, total, m, lane);
    if (total <= 128u) return rank_top_bits_buf<2>(buf, total, m, lane);
    return rank_top_bits_buf<4>(buf, total, m, lane);
}

// la: the head's A operand halves [K-block][lane][QS] (8 bytes, as in the records);
// C, S: each query's constant term and weight unit as the scan reads them.
template <int QS, int NT>
__device__ __forceinline__ void sample_thresholds(const uint32_t *__restrict__ planes, int n,
                                                  int word_stride, int k, int h,
                                                  int nplanes, int nkb, const uint32_t *pl,
                                                  const uint4 (&first)[sample_per<NT>()],
                                                  const uint2 *la, const float *C,
                                                  const float *S, uint32_t *tk,
                                                  ScanMeta *meta) {
    constexpr int kST = kSampleWords * 32;  // sampled tokens per query
    // the staged words and, once they are used, the sampled keys share one buffer
    __shared__ __align__(16) uint32_t sbuf[kSamplePlanes * kSampleWords];
    static_assert(kSamplePlanes * kSampleWords >= 4 * kST, "sample keys");
    uint32_t(*sw)[kSampleWords] = reinterpret_cast<uint32_t(*)[kSampleWords]>(sbuf);
    uint32_t(*skey)[kST] = reinterpret_cast<uint32_t(*)[kST]>(sbuf);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int s = lane & 3, wq = (lane >> 2) & 3, jq = lane >> 4;
    const int W = (n + 31) >> 5;
    const uint32_t m = (uint32_t)sample_rank(n, k);
    const uint32_t *hp = planes + (size_t)h * kMaxPlanesPerHead * word_stride;
    const int npr = (nkb + 1) >> 1;  // K-pairs (nkb >= 1)
    constexpr int WPW = kSampleWords / (NT / 64);  // sampled words a wave: 8 or 4
    constexpr int NP = WPW / 4;                    // words a lane: 2 or 1
    v4i acc[NP][8][QS];
    for (int kp0 = 0; kp0 < npr; kp0 += 2) {  // batches of two K-pairs (128 planes)
        const int p0 = 64 * kp0;
        const int np = max(0, min(kSamplePlanes, nplanes - p0));
        if (kp0) __syncthreads();  // the previous batch is no longer read
        if (kp0 == 0) {
            sample_stage<NT>(first, W, np, sw);
        } else {
            uint4 v[sample_per<NT>()];
            sample_issue<NT>(hp, W, word_stride, pl, p0, np, v);
            sample_stage<NT>(v, W, np, sw);
        }
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            const int kp = kp0 + kk;
            if (kp >= npr) break;
            const bool hi = 2 * kp + 1 < nkb;  // upper 4 groups of the K-pair exist
            uint32_t w[2][2][NP];
#pragma unroll
            for (int hh = 0; hh < 2; ++hh)
#pragma unroll
                for (int pp = 0; pp < 2; ++pp)
#pragma unroll
                    for (int pos = 0; pos < NP; ++pos)
                        w[hh][pp][pos] =
                            sw[64 * kk + 8 * (jq + 4 * hh) + s + 4 * pp][WPW * wave + NP * wq + pos];
            v4i A[QS];
#pragma unroll
            for (int set = 0; set < QS; ++set) {
                const uint2 alo = la[((2 * kp) * 64 + lane) * QS + set];
                const uint2 ahi = hi ? la[((2 * kp + 1) * 64 + lane) * QS + set] : make_uint2(0u, 0u);
                A[set] = v4i{(int)alo.x, (int)alo.y, (int)ahi.x, (int)ahi.y};
            }
            mma_item<QS, NP>(w, A, s, kp == 0, hi, acc);
        }
    }
    const bool small = nkb < kMaxKBlocks;
#pragma unroll
    for (int set = 0; set < QS; ++set) {
        __syncthreads();  // the staged words (or the previous set's keys) are no longer read
        const int g = 4 * set + jq;
#pragma unroll
        for (int pos = 0; pos < NP; ++pos) {
            const int i = WPW * wave + NP * wq + pos;  // sampled word
            const int word = sample_run_word(i / kSampleRunWords, W) + i % kSampleRunWords;
#pragma unroll
            for (int mm = 0; mm < 8; ++mm) {
                const float v = combined_score<QS>(acc[pos][mm][set], mm, C[g], S[g], small);
                const bool valid = word < W && 32 * word + 8 * s + mm < n;
                skey[jq][32 * i + 8 * s + mm] = valid ? order_key(v) : 0u;
            }
        }
        __syncthreads();
        if (wave < 4) {  // wave gq: the m-th largest sampled key of query 4*set + gq
            const int gq = wave;
            constexpr int kPerLane = kST / 64;
            uint32_t kk[kPerLane];
#pragma unroll
            for (int e = 0; e < kPerLane; ++e) kk[e] = skey[gq][lane + 64 * e];
            // the wave's own row of skey, now in registers, holds the compacted keys
            const uint32_t T = m > 0u ? sample_quantile(kk, m, lane, skey[gq]) : 0u;
            if (lane == 0) {
                if (meta) meta->tkey[4 * set + gq] = T;
                tk[4 * set + gq] = T;
            }
        }
    }
}

// The filter's integer threshold for the tokens at bit m of their byte (see the
// candidate filter in common.h).  With b = 2^m (-128 for m = 7), the token's score is
// C + S (65536 X + R) / b, |R S / b| <= S rb (rb: the query's sum over planes of
// |D0 + 256 D1| of its weights), and the scan's fp32 arithmetic is off the exact value
// by less than 2^-22 (|C| + S mabs + S rb).  So a score >= T needs
// 65536 X S / b >= T - C - eps - S rb, eps = 2^-20 (|C| + |T| + S mabs + S rb): for
// b > 0 X >= that bound * b / (65536 S), for b < 0 X <= it.  One more unit of slack
// covers the rounding of the bound itself.  live == false (no such query): keep none;
// tkey 0: keep all.
__device__ __forceinline__ int32_t filter_threshold(bool live, uint32_t tkey, float Cf, float Sf,
                                                    double rbs, double mabs, int m) {
    const bool neg = m == 7;
    if (!live) return neg ? INT32_MIN : INT32_MAX;
    if (tkey == 0u) return neg ? INT32_MAX : INT32_MIN;
    const double T = (double)__uint_as_float((tkey & 0x80000000u) ? (tkey ^ 0x80000000u) : ~tkey);
    const double C = (double)Cf, S = (double)Sf;
    const double srb = rbs * S, w = mabs * S;
    const double eps = ldexp(fabs(C) + fabs(T) + w + srb, -20);
    const double bound = (T - C) - eps - srb;
    const double q = bound * (neg ? -128.0 : (double)(1 << m)) / (65536.0 * S);
    const double t = neg ? floor(q) + 1.0 : ceil(q) - 1.0;
    if (t <= (double)INT32_MIN) return INT32_MIN;
    if (t >= (double)INT32_MAX) return INT32_MAX;
    return (int32_t)t;
}

// Inputs of the prepare step a thread reads (thread t: channel t mod 128): the head's
// queries, scale and zero, loaded together at the start of a kernel.
template <int QS>
struct PrepIn {
    float q[4 * QS];
    float s, z;
};
template <int QS>
__device__ __forceinline__ void load_prep_in(const float *__restrict__ q,
                                             const float *__restrict__ scale,
                                             const float *__restrict__ zero, int G, int h,
                                             PrepIn<QS> &in) {
    // unconditional loads (channel and query clamped) so that all are in flight
    // together; the values a thread does not need are never used or zeroed
    const int c = (int)threadIdx.x & (kD - 1);
#pragma unroll
    for (int g = 0; g < 4 * QS; ++g) in.q[g] = q[((size_t)h * G + min(g, G - 1)) * kD + c];
    in.s = scale[(size_t)h * kD + c];
    in.z = zero[(size_t)h * kD + c];
#pragma unroll
    for (int g = 0; g < 4 * QS; ++g) in.q[g] = g < G ? in.q[g] : 0.0f;
}

// Body of the prepare step for head h; tc[c] (LDS, complete) holds the channel depths.
// NT threads: 512 for one query set, 256 for two (whose registers allow no more).  pl
// (kMaxPlanesPerHead words) and la (the A operands, kMaxKBlocks * 64 * QS) are LDS the
// caller provides; they hold the plane list and the operand halves on return, xthr_lds
// (if given) the filter thresholds [query][m].  Only a writer stores the head's meta
// block and records.  Returns the head's number of planes.
template <int QS, int NT>
__device__ __forceinline__ int prepare_head(const PrepIn<QS> &in, const int *tc, int H,
                                            int G, const uint32_t *__restrict__ planes, int n,
                                            int word_stride, int k, char *__restrict__ ws,
                                            int h, uint32_t *pl, uint2 *la,
                                            int32_t *xthr_lds, bool writer) {
    constexpr int NQ = 4 * QS;
    constexpr int NW = NT / 64;                       // waves
    constexpr int QT = NT / kD;                       // threads per channel
    constexpr int WPQ = NW / NQ > 1 ? NW / NQ : 1;    // waves per query in the weight pass
    __shared__ int off[kD + 1];
    __shared__ double wt[NQ][kMaxPlanesPerHead];
    __shared__ double red[NQ][kD];
    __shared__ double amx[NQ][kD];
    __shared__ double csum[NQ];
    __shared__ double inv_unit[NQ];
    __shared__ double unit[NQ];
    __shared__ float cf[NQ], sf[NQ];             // C_g and S_g as the scan reads them
    const int tid = threadIdx.x, lane = tid & 63;
    ScanMeta *meta = reinterpret_cast<ScanMeta *>(ws + (size_t)h * kMetaBytes);
    uint32_t *rec = reinterpret_cast<uint32_t *>(ws + (size_t)H * kMetaBytes +
                                                 (size_t)h * kMaxKBlocks * 64 * 16 * QS);
    __shared__ unsigned long long rbi[NQ], mai[NQ];  // digit-sum bounds, summed by waves
    if (tid < NQ) rbi[tid] = mai[tid] = 0ull;
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
    // at least one K-block, so that a head with no planes still writes its constants
    const int nkb = max(1, (ngroups + kKBlockGroups - 1) / kKBlockGroups);
    {   // thread t: channel t mod 128, queries t / 128, t / 128 + QT, ...
        const int c = tid & (kD - 1), half = tid >> 7, t = tc[c], o = off[c];
        const double s = (double)in.s;
        const double z = (double)in.z;
        const double hm = (double)((16 >> t) - 1) * 0.5;  // bin-midpoint offset h(t)
        if (!half)
            for (int j = 0; j < t; ++j) pl[o + j] = (uint32_t)(c * kPlanes + j);
#pragma unroll
        for (int g = 0; g < NQ; ++g) {
            if (g % QT != half) continue;
            const double qv = (double)in.q[g];
            for (int j = 0; j < t; ++j) wt[g][o + j] = (qv * s) * (double)(8 >> j);
            red[g][c] = qv * (z + s * hm);  // this channel's share of C_g
            amx[g][c] = t > 0 ? fabs((qv * s) * 8.0) : 0.0;  // its largest |weight|
        }
    }
    __syncthreads();
    // the threshold sample's first loads go out now and land during the work below
    uint4 first[sample_per<NT>()];
    if (k > 0)
        sample_issue<NT>(planes + (size_t)h * kMaxPlanesPerHead * word_stride, (n + 31) >> 5,
                         word_stride, pl, 0, min(nplanes, kSamplePlanes), first);
    // C_g (a sum over the channels) and the weight unit of each query (from the largest
    // |weight|): wave v takes queries v, v + 4.  Lane l first adds channels l and l + 64,
    // then a butterfly over the lanes halves the distance each step, so lane 0 adds the
    // same pairs in the same order as a halving tree over the 128 channels.
    for (int g = tid >> 6; g < NQ; g += NW) {
        double sum = red[g][lane] + red[g][lane + 64];
        double mx = fmax(amx[g][lane], amx[g][lane + 64]);
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) sum += __shfl_xor(sum, o, 64);
        mx = __ockl_wfred_max_f64(mx);
        if (lane == 0) {
            csum[g] = sum;
            int e = 0;
            frexp(mx, &e);  // mx < 2^e
            unit[g] = mx > 0.0 ? ldexp(1.0, e - 30) : 1.0;
            // a power of two: multiplying by its inverse divides exactly
            inv_unit[g] = mx > 0.0 ? ldexp(1.0, 30 - e) : 1.0;
        }
    }
    __syncthreads();
    // each weight as an integer count of its query's unit, biased by 128 (1 + 256 +
    // 65536) so that its signed base-256 digits are plain bytes (weight_byte); written
    // over the weight it comes from.  The same pass sums, per query, |M| and
    // |D0 + 256 D1| of M's digits (the part of a weight the filter's integer test does
    // not see): integer sums, exact in any order.  WPQ waves share a query's planes.
    long long(*Mu)[kMaxPlanesPerHead] = reinterpret_cast<long long(*)[kMaxPlanesPerHead]>(wt);
    for (int gw = tid >> 6; gw < NQ * WPQ; gw += NW) {
        const int g = gw % NQ, wp = gw / NQ;
        long long r = 0, a = 0;
        for (int p = lane + 64 * wp; p < nplanes; p += 64 * WPQ) {
            const long long u = (g < G ? llrint(wt[g][p] * inv_unit[g]) : 0LL) + kDigitBias;
            Mu[g][p] = u;
            const int d0 = (int)(int8_t)(uint8_t)weight_byte(u, 0);
            const int d1 = (int)(int8_t)(uint8_t)weight_byte(u, 1);
            const int dl = d0 + 256 * d1;
            r += dl < 0 ? -dl : dl;
            a += u >= kDigitBias ? u - kDigitBias : kDigitBias - u;
        }
        r = (long long)__ockl_wfred_add_u64((unsigned long long)r);  // both sums are >= 0
        a = (long long)__ockl_wfred_add_u64((unsigned long long)a);
        if (lane == 0) {
            atomicAdd(&rbi[g], (unsigned long long)r);
            atomicAdd(&mai[g], (unsigned long long)a);
        }
    }
    if (writer) {
        for (int p = tid; p < nplanes; p += NT) meta->plane[p] = pl[p];
        if (tid < FATHOM_MAX_G) {
            meta->C[tid] = tid < G ? (float)csum[tid] : 0.0f;
            meta->S[tid] = tid < G ? (float)unit[tid] : 0.0f;
        }
    }
    if (tid < NQ) {
        cf[tid] = tid < G ? (float)csum[tid] : 0.0f;
        sf[tid] = tid < G ? (float)unit[tid] : 0.0f;
    }
    if (writer && tid == 0) {
        meta->n_planes = nplanes;
        meta->n_groups = ngroups;
        meta->n_kblocks = nkb;
        meta->redo = 0u;
    }
    __syncthreads();
    // operand records: lane ln of K-block kbl serves group 4*kbl + (ln >> 4)
    for (int e = tid; e < nkb * 64; e += NT) {
        const int kbl = e >> 6, ln = e & 63;
        const int grp = kbl * kKBlockGroups + (ln >> 4);
        const int s = ln & 3, r = ln & 15;
        const int p0 = grp * kGroupBits + s, p1 = p0 + 4;
        uint32_t *dst = rec + (size_t)e * 4 * QS;
        if (writer) {
            dst[0] = p0 < nplanes ? pl[p0] : kSkipRow;
            dst[1] = p1 < nplanes ? pl[p1] : kSkipRow;
        }
#pragma unroll
        for (int set = 0; set < QS; ++set) {
            const int g = 4 * set + (r >> 2), dg = r & 3;
            uint32_t wlo = 0, whi = 0;
#pragma unroll
            for (int i = 0; i < kGroupBits; ++i) {
                const int p = grp * kGroupBits + i;
                const uint32_t byte = weight_byte(p < nplanes ? Mu[g][p] : kDigitBias, dg);
                if (i < 4) wlo |= byte << (8 * i);
                else whi |= byte << (8 * (i - 4));
            }
            if (writer) {
                dst[2 + 2 * set] = wlo;
                dst[3 + 2 * set] = whi;
            }
            la[e * QS + set] = make_uint2(wlo, whi);
        }
        if (QS == 2 && writer) dst[6] = dst[7] = 0;
    }
    if (writer) {
        if (tid < FATHOM_MAX_G) {
            meta->cnt[tid] = 0u;
            meta->cnt_exact[tid] = 0u;
            meta->attn_done[tid] = 0u;
            meta->sel_done[tid] = 0u;
        }
        if (tid == 0) meta->ovf = 0u;
    }
    if (k <= 0) {
        if (writer && tid < FATHOM_MAX_G) meta->tkey[tid] = 0u;
        return nplanes;
    }
    __shared__ uint32_t tk[NQ];
    sample_thresholds<QS, NT>(planes, n, word_stride, k, h, nplanes, nkb, pl, first, la, cf, sf,
                              tk, writer ? meta : nullptr);
    __syncthreads();  // the thresholds and the sums are complete
    if (tid < NQ * 8) {
        const int g = tid >> 3, m = tid & 7;
        const int32_t x = filter_threshold(g < G, tk[g], cf[g], sf[g], (double)rbi[g],
                                           (double)mai[g], m);
        if (writer) meta->xthr[g][m] = x;
        if (xthr_lds) xthr_lds[tid] = x;
    }
    if (writer && tid >= NQ * 8 && tid < FATHOM_MAX_G * 8) meta->xthr[tid >> 3][tid & 7] = 0;
    return nplanes;
}

// Threads of a prepare workgroup: 512 for one query set (its 212 registers allow two
// waves a SIMD), 256 for two.
template <int QS>
constexpr int prep_threads() { return QS == 1 ? 512 : 256; }

template <int QS>
__global__ __launch_bounds__(prep_threads<QS>()) void k_scan_prepare(
    const float *__restrict__ q, const uint8_t *__restrict__ depth,
    const float *__restrict__ scale, const float *__restrict__ zero, int H, int G,
    const uint32_t *__restrict__ planes, int n, int word_stride, int k,
    char *__restrict__ ws) {
    __shared__ int tc[kD];
    const int h = blockIdx.x, tid = threadIdx.x;
    PrepIn<QS> in;
    load_prep_in<QS>(q, scale, zero, G, h, in);
    const int t = depth[(size_t)h * kD + min(tid, kD - 1)];
    if (tid < kD) tc[tid] = min(t, kPlanes);
    __syncthreads();
    __shared__ uint32_t pl[kMaxPlanesPerHead];
    __shared__ uint2 la[kMaxKBlocks * 64 * QS];
    prepare_head<QS, prep_threads<QS>()>(in, tc, H, G, planes, n, word_stride, k, ws, h, pl, la,
                                         nullptr, true);
}

// A decode step's plan and prepare in one kernel: the depths stay in LDS between them
// (and are also written to `depth`).  Every input of both is loaded up front.
template <int QS>
__global__ __launch_bounds__(prep_threads<QS>()) void k_plan_prepare(
    const float *__restrict__ q, const float *__restrict__ var,
    const float *__restrict__ scale, const float *__restrict__ zero, int H, int G, int B,
    const uint32_t *__restrict__ planes, int n, int word_stride, int k,
    uint8_t *__restrict__ depth, char *__restrict__ ws) {
    __shared__ int tc[kD];
    const int h = blockIdx.x, tid = threadIdx.x;
    PrepIn<QS> in;
    load_prep_in<QS>(q, scale, zero, G, h, in);
    float qp[FATHOM_MAX_G], vp;
    constexpr int NT = prep_threads<QS>();
    plan_load<NT>(q, var, G, h, qp, vp);
    plan_from<NT>(qp, vp, G, B, tc);
    if (tid < kD) depth[(size_t)h * kD + tid] = (uint8_t)tc[tid];
    __shared__ uint32_t pl[kMaxPlanesPerHead];
    __shared__ uint2 la[kMaxKBlocks * 64 * QS];
    prepare_head<QS, NT>(in, tc, H, G, planes, n, word_stride, k, ws, h, pl, la, nullptr, true);
}

// ---------------------------------------------------------------------------------
// main scan
// ---------------------------------------------------------------------------------
// Shape.  A workgroup of kWaves waves scores one super-step -- 256 tokens (8 words) per
// wave, 8*kWaves words of one head -- at a time, K-pair by K-pair: 8 groups of 8 planes,
// the K of one 16x16x64 i8 MFMA.  For each K-pair the waves copy its 64 plane rows,
// 32*kWaves contiguous bytes (whole cache lines) each, straight from global memory
// into an LDS tile, 16 bytes a lane; after a barrier, wave v takes words 8v .. 8v+7 of
// all 64 rows from the tile in two passes t of 4 words.  One LDS transpose read
// (ds_read_b64_tr_b8: within each 16 lanes, lane i < 8 receives byte i of the 8 bytes
// each even lane 2j read, lane 8 + i byte i of those of the odd lanes 2j + 1) per pass
// and K-block half h: lane 16*q + 2*j + p of the 16 reads 8 bytes (2 words) of plane j of
// group q + 4h, words 8v + 4t + 2p and the next, so that lane 16*q + 4*w + s receives
// byte s of word 8v + 4t + w of the group's 8 planes -- bit m of byte i is plane i's bit
// of token 8s + m of that word.  Masking bit m of every byte makes the MFMA column of that
// token (byte values 0 / 2^m, and -128 for m = 7, divided out in the combine).  The MFMA
// output lane 16*j + 4*w + s then holds query j's 4 digit sums for that token.  kTiles
// tiles rotate, so the copies of the next K-pairs are in flight while one is used.
#ifndef FATHOM_SCAN_WAVES
#define FATHOM_SCAN_WAVES 8
#endif
constexpr int kWaves = FATHOM_SCAN_WAVES;     // waves per workgroup (8 or 16)
static_assert(kWaves == 8 || kWaves == 16, "workgroup shape: rows of at least 16 chunks");
constexpr int kScanThreads = 64 * kWaves;
constexpr int kSuperWords = 8 * kWaves;       // words per super-step
constexpr int kRowChunks = kSuperWords / 4;   // 16-byte chunks of a row per super-step
constexpr int kCopyRows = 64 / kRowChunks;    // rows one copy instruction moves
constexpr int kRowBytes = 16 * kRowChunks;    // one row of a super-step in the tile
constexpr int kGroupBytes = 8 * kRowBytes;    // a group's 8 rows
constexpr int kTileBytes = 8 * kGroupBytes;   // one K-pair
#ifndef FATHOM_SCAN_TILES
#define FATHOM_SCAN_TILES 3
#endif
#ifndef FATHOM_SCAN_ROUNDS
#define FATHOM_SCAN_ROUNDS 1
#endif
#ifndef FATHOM_SCAN_WAVES_PER_EU
#define FATHOM_SCAN_WAVES_PER_EU 4
#endif
constexpr int kTiles = FATHOM_SCAN_TILES;
static_assert(kTiles >= 2 && kTiles <= 6, "tile ring");
constexpr uint32_t kNoRow = 0xFFFFFFFFu;
// Filter records a 256-token block may hold, and the LDS a wave stages them in beyond
// the tile ring (the filtering combine below).
template <int QS>
constexpr int block_records() { return QS == 1 ? 64 : kBlockRecords; }
constexpr uint32_t kRunOvf = 0x80000000u;  // a run's kept count: the row overflowed
template <int QS>
constexpr size_t stage_bytes_per_wave() { return QS == 1 ? 0 : (size_t)4 * QS * kBlockRecords * 8; }

// Chunk c of row i of group g sits in 16-byte slot c ^ tile_swz(g, i) of the row: one
// transpose read takes chunk 2v + t of the 8 rows of groups g and g + 1 (lanes 0-31; g
// even) or g + 2 and g + 3, and the xor puts those 16 chunks of each half-wave on 16
// different slots, i.e. all banks once.
__device__ __forceinline__ int tile_swz(int g, int i) { return 8 * (g & 1) + i; }

// LDS per head slot: A operand halves [K-block of 4 groups][lane][QS] (8 bytes); the
// rows the copies read, [K-pair][row r of a K-block half][half] (kWide: row index or
// kNoRow; otherwise the row's byte offset from the head's first row, absent rows
// pointing at a row the head reads anyway); the filter thresholds [query][m]; then,
// after both head slots, the tile ring.
template <int QS>
constexpr size_t lds_rows_off() { return (size_t)kMaxKBlocks * 64 * QS * 8; }
template <int QS>
constexpr size_t lds_xthr_off() { return lds_rows_off<QS>() + (size_t)kMaxKBlocks * 32 * 4; }
template <int QS>
constexpr size_t lds_head_bytes() {
    return lds_xthr_off<QS>() + (size_t)FATHOM_MAX_G * 8 * 4;
}
template <int QS>
constexpr size_t scan_lds_bytes() {
    static_assert(kMaxKBlocks * 64 % kScanThreads == 0, "records a thread");
    return 2 * lds_head_bytes<QS>() + (size_t)kTiles * kTileBytes + (size_t)kScanThreads * 8 +
           (size_t)kWaves * stage_bytes_per_wave<QS>();
}

// score = C + (D0 + 256 D1 + 65536 (D2 + 256 D3)) * S / (byte value of bit m); the
// digit sums of a head with at most 480 planes fit D0 + 256 D1 in int32.
template <int QS>
__device__ __forceinline__ void combine_store(const v4i (&acc)[2][8][QS], const float (&Cq)[QS],
                                              const float (&Sq)[QS], bool small, int G, int jq,
                                              int s, int wi, int n, float *hscores) {
#pragma unroll
    for (int set = 0; set < QS; ++set) {
        const int g = 4 * set + jq;
        if (g >= G) continue;
        float *row = hscores + (size_t)g * n;
#pragma unroll
        for (int pos = 0; pos < 2; ++pos) {
            float v[8];
#pragma unroll
            for (int m = 0; m < 8; ++m) {
                const v4i d = acc[pos][m][set];
                const float lo = small ? (float)(d[0] + d[1] * 256)
                                       : fmaf((float)d[1], 256.0f, (float)d[0]);
                const float hi = (float)(d[2] + d[3] * 256);
                const float f = fmaf(hi, 65536.0f, lo);
                const float mult = m < 7 ? Sq[set] * (1.0f / (float)(1 << m))
                                         : Sq[set] * (-1.0f / 128.0f);
                v[m] = fmaf(f, mult, Cq[set]);
            }
            const int tok = (wi + 4 * pos) * 32 + 8 * s;
            if ((n & 3) == 0 && tok + 8 <= n) {
                *reinterpret_cast<float4 *>(row + tok) = make_float4(v[0], v[1], v[2], v[3]);
                *reinterpret_cast<float4 *>(row + tok + 4) = make_float4(v[4], v[5], v[6], v[7]);
            } else {
#pragma unroll
                for (int m = 0; m < 8; ++m)
                    if (tok + m < n) row[tok + m] = v[m];
            }
        }
    }
}

// The filtering form of the combine (the candidate filter in common.h): per token the
// integer test X = D2 + 256 D3 against the row's threshold for its bit m, then the
// records of the tokens that pass go to the front of the wave's 256-token block (words
// wb .. wb+7) of the row's record area, with the block's 8 mask words; the row's count
// of kept tokens grows by the block's.  Within a block the records are in token order
// (pass pos, then w: lane 4w + s of a query's 16 holds byte s of word wb + 4 pos + w).  A
// block with more than block_records<QS>() candidates sets the row's ovf bit (its records are
// then incomplete and the row is rescored), as does every row of a head of more than
// 480 planes (!small: R would not fit int32).  xt: the lane's query's thresholds (keep
// none for a query past G); ragged: the super-step reaches past token n.  kWide: 64-bit
// record addresses; otherwise 32-bit byte offsets from hcand.  The lane's row's kept count
// and ovf bit (kRunOvf) are accumulated in cnt (per query set) and added to the row by
// the caller at the end of its run.
// The records are first gathered in LDS, block by block (query block b = 4 set + j: the
// first 2 QS blocks at stage_lo, the others at stage_hi): every lane writes one 8-byte
// record per token without
// a branch, a kept token's to its place in the block and the others to the lane's own
// slot `dummy`; then each query's 16 lanes copy their block out, 16 records a store, so
// that a few stores of whole runs replace one store per kept token position.  With one
// query set the stage is the wave's two 1 KiB areas of the tile its next copies will
// fill, 64 records a block; with two, an 8 KiB area of its own, 128 a block (the two-set
// scan runs one workgroup per CU, so the LDS is there).
template <int QS, bool kWide>
__device__ __forceinline__ void combine_filter(const v4i (&acc)[2][8][QS], const int (&xt)[QS][8],
                                               bool ragged, bool small, int G, int jq, int s,
                                               int wq, int lane, int wi, int n, int64_t cstride,
                                               char *hcand, uint32_t *hmask, uint32_t (&cnt)[QS],
                                               lds_char *stage_lo, lds_char *stage_hi,
                                               lds_char *dummy) {
    constexpr int kStage = block_records<QS>();
    const int W = (n + 31) >> 5;
    const int wb = wi - wq;       // first word of the block
    const uint32_t below = (1u << (8 * s)) - 1u;  // bits of the quad's lower lanes
#pragma unroll
    for (int set = 0; set < QS; ++set) {
        const int g = 4 * set + jq;
        const bool live = g < G;  // the same for a query's 16 lanes
        if (!small) {
            cnt[set] |= kRunOvf;
            continue;
        }
        const size_t blk_bytes = ((size_t)g * cstride + (size_t)wb * 32) * 4;
        const int sb = set * 4 + jq;  // this lane's query block
        lds_char *stage = (sb < 2 * QS ? stage_lo : stage_hi) + (sb % (2 * QS)) * kStage * 8;
        uint32_t base = 0u;       // records of the block's earlier words
#pragma unroll
        for (int pos = 0; pos < 2; ++pos) {
            int xp[8];
#pragma unroll
            for (int m = 0; m < 8; ++m) xp[m] = xt[set][m];
            if (ragged) {  // tokens >= n keep nothing
                const int left = n - ((wi + 4 * pos) * 32 + 8 * s);
#pragma unroll
                for (int m = 0; m < 8; ++m)
                    if (m >= left) xp[m] = m < 7 ? INT32_MAX : INT32_MIN;
            }
            bool keep[8];
            uint32_t bits = 0u;
#pragma unroll
            for (int m = 0; m < 8; ++m) {
                const int X = acc[pos][m][set][2] + acc[pos][m][set][3] * 256;
                keep[m] = m < 7 ? X >= xp[m] : X <= xp[7];
                bits |= (uint32_t)keep[m] << m;
            }
            // the quad's 4 bytes make the mask word
            uint32_t x = bits << (8 * s);
            x |= (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0xB1, 0xF, 0xF, false);
            x |= (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x4E, 0xF, 0xF, false);
            const uint32_t t = (uint32_t)__popc(x);  // this quad's word
            // inclusive prefix over the 4 quads of the query's 16 lanes (one DPP row):
            // row_shr 4 and 8, lanes shifted in from outside the row read 0
            uint32_t inc = t + (uint32_t)__builtin_amdgcn_update_dpp(0, (int)t, 0x114, 0xF, 0xF, true);
            inc += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)inc, 0x118, 0xF, 0xF, true);
            // and the inclusive suffix (row_shl 4 and 8): together the row's total
            uint32_t suf = t + (uint32_t)__builtin_amdgcn_update_dpp(0, (int)t, 0x104, 0xF, 0xF, true);
            suf += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)suf, 0x108, 0xF, 0xF, true);
            const uint32_t r = base + inc - t + (uint32_t)__popc(x & below);
            base += inc + suf - t;
            if (live && s == 0 && wi + 4 * pos < W) hmask[(size_t)g * W + wi + 4 * pos] = x;
            if (live) {
                {
                    uint32_t k = r;  // record index in the block
#pragma unroll
                    for (int m = 0; m < 8; ++m) {
                        const v4i d = acc[pos][m][set];
                        // past the block's room the record lands in its last slot: such a
                        // block overflowed, and its records are never copied out
                        lds_char *a = keep[m] ? stage + 8u * min(k, (uint32_t)kStage - 1u) : dummy;
                        *reinterpret_cast<lds_v2i *>(a) = v2i{d[2] + d[3] * 256, d[0] + d[1] * 256};
                        k += keep[m] ? 1u : 0u;
                    }
                }
            }
        }
        // the staged records out: lane i of the query's 16 copies records i, i + 16, ...
        const uint32_t staged = live && base <= (uint32_t)kStage ? base : 0u;
        for (uint32_t k = (uint32_t)(lane & 15); __builtin_amdgcn_ballot_w64(k < staged) != 0;
             k += 16u) {
            if (k < staged) {
                const v2i sv = *reinterpret_cast<const lds_v2i *>(stage + 8u * k);
                const int2 rv = make_int2(sv.x, sv.y);
                if constexpr (kWide) reinterpret_cast<int2 *>(hcand + blk_bytes)[k] = rv;
                else *reinterpret_cast<int2 *>(hcand + ((uint32_t)blk_bytes + 8u * k)) = rv;
            }
        }
        cnt[set] += base | (base > (uint32_t)kStage ? kRunOvf : 0u);
    }
}

// Global -> LDS copy of 16 bytes a lane: lane l's bytes land at LDS byte address
// m0 + 16 l (m0 the same for the whole wave).  Written as inline assembly so that the
// compiler's own wait insertion does not treat every later LDS read as depending on it
// (it cannot tell the tiles apart); the tile reads wait for it explicitly.
// m0 is a reserved register: it is saved and restored around the copy, so the statement
// leaves it as it found it.  copy16_to_lds takes a 64-bit address per lane;
// copy16_to_lds_off a base address common to the wave plus a 32-bit byte offset per
// lane (no 64-bit arithmetic per copy).
__device__ __forceinline__ void copy16_to_lds(const uint32_t *src, uint32_t m0) {
    uint32_t saved;
    __asm__ volatile(
        "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %1, off\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(src), "s"(__builtin_amdgcn_readfirstlane(m0))
        : "memory");
}
__device__ __forceinline__ void copy16_to_lds_off(const char *base, uint32_t off, uint32_t m0) {
    uint32_t saved;
    __asm__ volatile(
        "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %3\n\tglobal_load_lds_dwordx4 %1, %2\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(off), "s"(base), "s"(__builtin_amdgcn_readfirstlane(m0))
        : "memory");
}

// Work split.  The (head, super-step) pairs of a launch are numbered head-major;
// workgroup w takes a run of `run` consecutive ones.  With `flat`, runs are cut without
// regard to heads (one run per resident workgroup; a run is at most one head long, so
// it touches at most two heads); otherwise a run never leaves its head.
struct ScanSplit {
    int nss;           // super-steps per head
    int run;           // super-steps per workgroup
    int wgs_per_head;  // !flat: workgroups per head
    int flat;
};

template <int QS>
__device__ __forceinline__ void load_head_consts(const ScanMeta *meta, int G, int jq,
                                                 float (&C)[QS], float (&S)[QS]) {
#pragma unroll
    for (int set = 0; set < QS; ++set) {
        const int g = 4 * set + jq;
        C[set] = g < G ? meta->C[g] : 0.0f;
        S[set] = g < G ? meta->S[g] : 0.0f;
    }
}

// The plan and prepare inputs of the fused front (k_front_fused).
struct FrontIn {
    const float *q, *var, *scale, *zero;
    int B, k;
    uint8_t *depth;  // the plan, written by each head's first workgroup
};

// Body of the scan kernels.  kWide: a head's 512 rows span 4 GiB or more, so the copies
// take 64-bit addresses per lane; otherwise 32-bit byte offsets from the head's first row.
// kFused (k_front_fused): the workgroup first plans and prepares its head itself (every
// workgroup of a head computes the same plan, records and thresholds; the head's first
// one also stores them for the select) and builds its LDS from that instead of loading
// the records; its run is one super-step, and it adds no kept counts to the rows (the
// select of one-chunk rows takes them from the masks).
template <int QS, bool kWide, bool kFilter, bool kFused>
__device__ __forceinline__ void scan_body(
    const uint32_t *__restrict__ planes, int n, int word_stride, int G, int H, ScanSplit sp,
    const char *__restrict__ ws, float *__restrict__ scores, uint32_t *__restrict__ masks,
    const FrontIn &fz) {
    static_assert(!kFused || (QS == 1 && kFilter && !kWide && kScanThreads == 512),
                  "the fused front: one query set, filtering, 512 threads");
    extern __shared__ uint4 lds_u4[];
    char *lds = reinterpret_cast<char *>(lds_u4);
    lds_char *lds3 = (lds_char *)lds_u4;
    constexpr size_t kHeadBytes = lds_head_bytes<QS>();
    constexpr size_t kRowsOff = lds_rows_off<QS>();
    constexpr size_t kXthrOff = lds_xthr_off<QS>();
    const uint32_t lds_base = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char *)lds;
    const uint32_t tiles_base = lds_base + 2 * (uint32_t)kHeadBytes;
    const int nss = sp.nss;
    const int lb = xcd_remap(blockIdx.x, gridDim.x);
    long a, b;  // this workgroup's run of (head, super-step) pairs
    if (sp.flat) {
        a = (long)lb * sp.run;
        b = min(a + (long)sp.run, (long)H * nss);
    } else {
        const int h = lb / sp.wgs_per_head, c = lb - h * sp.wgs_per_head;
        a = (long)h * nss + (long)c * sp.run;
        b = min(a + (long)sp.run, (long)(h + 1) * nss);
    }
    const int h0 = (int)(a / nss);
    const int h1 = (int)((b - 1) / nss);  // h0 or h0 + 1
    const ScanMeta *meta0 = reinterpret_cast<const ScanMeta *>(ws + (size_t)h0 * kMetaBytes);
    const ScanMeta *meta1 = reinterpret_cast<const ScanMeta *>(ws + (size_t)h1 * kMetaBytes);
    const int tid = threadIdx.x;
    int nkb0, nkb1;  // 4-group K-blocks of the two heads
    if constexpr (kFused) {
        __shared__ int tc[kD];
        PrepIn<1> in;
        load_prep_in<1>(fz.q, fz.scale, fz.zero, G, h0, in);
        float qp[FATHOM_MAX_G], vp;
        plan_load<kScanThreads>(fz.q, fz.var, G, h0, qp, vp);
        plan_from<kScanThreads>(qp, vp, G, fz.B, tc);
        const bool writer = a == (long)h0 * nss;  // the head's first super-step
        if (writer && fz.depth && tid < kD) fz.depth[(size_t)h0 * kD + tid] = (uint8_t)tc[tid];
        // the plane list goes to the first tile (free until the first copies), the A
        // operands and thresholds to head slot 0, where the scan reads them
        uint32_t *plist = reinterpret_cast<uint32_t *>(lds + 2 * kHeadBytes);
        const int np = prepare_head<1, kScanThreads>(
            in, tc, H, G, planes, n, word_stride, fz.k, const_cast<char *>(ws), h0, plist,
            reinterpret_cast<uint2 *>(lds), reinterpret_cast<int32_t *>(lds + kXthrOff), writer);
        __syncthreads();
        const int ngroups = (np + kGroupBits - 1) / kGroupBits;
        nkb0 = nkb1 = min(max(1, (ngroups + kKBlockGroups - 1) / kKBlockGroups), kMaxKBlocks);
        // the row table as the records give it: row r of K-block kb is plane r & 7 of
        // group 4 kb + (r >> 3); absent rows read the head's first planned row
        uint32_t *lrow = reinterpret_cast<uint32_t *>(lds + kRowsOff);
        const uint32_t dead = np > 0 ? plist[0] * (uint32_t)word_stride * 4u : 0u;
        const int nk2 = 2 * ((nkb0 + 1) >> 1);
        for (int e = tid; e < nk2 * 32; e += kScanThreads) {
            const int kb = e >> 5, r = e & 31;
            const int p = (kKBlockGroups * kb + (r >> 3)) * kGroupBits + (r & 7);
            lrow[((kb >> 1) * 32 + r) * 2 + (kb & 1)] =
                kb < nkb0 && p < np ? plist[p] * (uint32_t)word_stride * 4u : dead;
        }
        __syncthreads();
    } else {
    // clamped so that any workspace content keeps every read inside the head's data
    nkb0 = min(max(meta0->n_kblocks, 1), kMaxKBlocks);
    nkb1 = min(max(meta1->n_kblocks, 1), kMaxKBlocks);
    // The head slots' LDS from the operand records.  Every record of the kMaxKBlocks a
    // head may have is loaded, unconditionally and in the same round as the K-block counts
    // above (the ones past a head's count are dropped), so that one memory latency, not
    // two, precedes the first copies.  Record e = 64 kb + ln holds in its first two words
    // the rows of planes s and s + 4 of group 4 kb + (ln >> 4), s = ln & 3, when
    // (ln & 15) < 4: row r = 8 (ln >> 4) + s and r + 4 of K-block kb.
    constexpr int kRecPer = kMaxKBlocks * 64 / kScanThreads;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        if (k && h1 == h0) break;
        const int hk = k ? h1 : h0, nk = k ? nkb1 : nkb0;
        const uint4 *grec = reinterpret_cast<const uint4 *>(
            ws + (size_t)H * kMetaBytes + (size_t)hk * kMaxKBlocks * 64 * 16 * QS);
        uint4 rec[kRecPer][QS];
#pragma unroll
        for (int u = 0; u < kRecPer; ++u)
#pragma unroll
            for (int set = 0; set < QS; ++set)
                rec[u][set] = grec[(size_t)(tid + kScanThreads * u) * QS + set];
        const uint32_t first_row = reinterpret_cast<const uint32_t *>(grec)[0];
        int32_t xk = 0;
        if constexpr (kFilter) {
            const ScanMeta *mk = k ? meta1 : meta0;
            if (tid < FATHOM_MAX_G * 8) xk = mk->xthr[tid >> 3][tid & 7];
        }
        uint2 *la = reinterpret_cast<uint2 *>(lds + k * kHeadBytes);
        uint32_t *lrow = reinterpret_cast<uint32_t *>(lds + k * kHeadBytes + kRowsOff);
        const uint32_t dead = kWide ? kNoRow
                                    : (first_row < (uint32_t)kMaxPlanesPerHead
                                           ? first_row * (uint32_t)word_stride * 4u : 0u);
        const int nk2 = 2 * ((nk + 1) >> 1);
#pragma unroll
        for (int u = 0; u < kRecPer; ++u) {
            const int e = tid + kScanThreads * u, kb = e >> 6, ln = e & 63;
            if (kb < nk) {
                la[e * QS] = make_uint2(rec[u][0].z, rec[u][0].w);
                if constexpr (QS == 2) la[e * QS + 1] = make_uint2(rec[u][1].x, rec[u][1].y);
            }
            if (kb < nk2 && (ln & 15) < 4) {
                const int r = 8 * (ln >> 4) + (ln & 3);
#pragma unroll
                for (int hf = 0; hf < 2; ++hf) {
                    const uint32_t p = hf ? rec[u][0].y : rec[u][0].x;
                    uint32_t v = dead;
                    if (kb < nk && p < (uint32_t)kMaxPlanesPerHead)
                        v = kWide ? p : p * (uint32_t)word_stride * 4u;
                    lrow[((kb >> 1) * 32 + r + 4 * hf) * 2 + (kb & 1)] = v;
                }
            }
        }
        if constexpr (kFilter) {
            int32_t *lx = reinterpret_cast<int32_t *>(lds + k * kHeadBytes + kXthrOff);
            if (tid < FATHOM_MAX_G * 8) lx[tid] = xk;
        }
    }
    __syncthreads();
    }

    const int lane = tid & 63, wave = tid >> 6;
    const int s = lane & 3, wq = (lane >> 2) & 3, jq = lane >> 4;
    const size_t head_words = (size_t)kMaxPlanesPerHead * word_stride;
    float C0[QS], S0[QS], C1[QS], S1[QS];
    if constexpr (!kFilter) {  // only the full scores use them
        load_head_consts<QS>(meta0, G, jq, C0, S0);
        load_head_consts<QS>(meta1, G, jq, C1, S1);
    }
    const bool small = max(nkb0, nkb1) < kMaxKBlocks;
    const int npr0 = (nkb0 + 1) >> 1, npr1 = (nkb1 + 1) >> 1;  // K-pairs per super-step
    // super-steps of the run, counted from a: [0, h1rel) in head h0, [h1rel, len) in h1
    const int len = (int)(b - a);
    const int h1rel = (int)min((long)len, (long)(h0 + 1) * nss - a);
    const int ss0 = (int)(a - (long)h0 * nss);  // super-step of head h0 at run start
    const int nitems = h1rel * npr0 + (len - h1rel) * npr1;

    // copy engine: item = (super-step, K-pair); per K-pair half (4 groups) this lane
    // moves chunk c of row r of the half: r = 8*cgrp + crow, c = cchunk
    const int cgrp = wave / (kWaves / 4);
    const int crow = (wave % (kWaves / 4)) * kCopyRows + lane / kRowChunks;
    const int cchunk = (lane % kRowChunks) ^ tile_swz(cgrp, crow);
    const int crr = 8 * cgrp + crow;  // row of a K-block half
    const uint32_t cdst = (uint32_t)(cgrp * kGroupBytes +
                                     (wave % (kWaves / 4)) * kCopyRows * kRowChunks * 16);
    // last 16-byte chunk of a row: chunks past the row's end read it instead
    const uint32_t last_chunk = (uint32_t)(word_stride - 4) * 4u;
    int iss = 0, ipr = 0, fi = 0;
    auto issue = [&]() {
        const int k = iss >= h1rel ? 1 : 0;
        const int hh = k ? h1 : h0;
        const int ss = k ? iss - h1rel : ss0 + iss;
        const uint2 ro = *reinterpret_cast<const uint2 *>(
            lds + k * kHeadBytes + kRowsOff + ((size_t)ipr * 32 + crr) * 8);
        const uint32_t tile = tiles_base + (uint32_t)((fi % kTiles) * kTileBytes) + cdst;
        if constexpr (kWide) {
            const int word = ss * kSuperWords + 4 * cchunk;
            const uint32_t *hbase = planes + (size_t)hh * head_words + min(word, word_stride - 4);
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                const uint32_t row = half ? ro.y : ro.x;
                // absent rows all fetch the store's first 16 bytes
                const uint32_t *src =
                    row != kNoRow ? hbase + (size_t)row * (size_t)word_stride : planes;
                copy16_to_lds(src, tile + (uint32_t)(half * 4 * kGroupBytes));
            }
        } else {
            const char *hbase = reinterpret_cast<const char *>(planes + (size_t)hh * head_words);
            const uint32_t chunk = min((uint32_t)(ss * kSuperWords + 4 * cchunk) * 4u, last_chunk);
            copy16_to_lds_off(hbase, ro.x + chunk, tile);
            copy16_to_lds_off(hbase, ro.y + chunk, tile + (uint32_t)(4 * kGroupBytes));
        }
        ++fi;
        if (++ipr == (k ? npr1 : npr0)) {
            ipr = 0;
            ++iss;
        }
    };
    for (int u = 0; u < kTiles - 1; ++u)
        if (fi < nitems) issue();

    v4i acc[2][8][QS];
    int pss = 0, ppr = 0;  // item being used
    // this lane's transpose-read source: plane j of group q (+ 4h), words 4t + 2p and
    // 4t + 2p + 1 of the wave's 8, i.e. the low or high 8 bytes of chunk 2v + t
    const int qgrp = lane >> 4;               // operand group q (and q + 4)
    const int trj = (lane & 15) >> 1;
    const uint32_t trsrc0 = (uint32_t)(qgrp * kGroupBytes + trj * kRowBytes + 8 * (lane & 1));
    // A super-step's scores are combined after the barrier of the next item, before
    // that item's copies are issued: its stores then precede the newest copies in the
    // wave's memory-instruction order, and the wait for the next tile (vmcnt(2): all but
    // the newest copies) covers them rather than copies just issued.  pk: head slot of
    // the pending combine (-1: none), pss_c: its super-step in the run.
    int pk = -1, pss_c = 0;
    uint32_t cnt0[QS], cnt1[QS];  // per head slot: kept counts and kRunOvf
#pragma unroll
    for (int set = 0; set < QS; ++set) cnt0[set] = cnt1[set] = 0u;
    uint32_t ptile = 0u;  // LDS address of the tile of the pending super-step's last item
    auto combine = [&]() {
        const int k = pk;
        const int hh = k ? h1 : h0;
        const int nk = k ? nkb1 : nkb0;
        const int ssh = k ? pss_c - h1rel : ss0 + pss_c;  // super-step within the head
        const int wi = (ssh * kWaves + wave) * 8 + wq;  // this lane's word of pass 0
        if constexpr (kFilter) {
            // this lane's queries' thresholds, from the head's LDS slot
            const int32_t *lx = reinterpret_cast<const int32_t *>(lds + k * kHeadBytes + kXthrOff);
            int xt[QS][8];
#pragma unroll
            for (int set = 0; set < QS; ++set) {
                const int4 x0 = *reinterpret_cast<const int4 *>(lx + (4 * set + jq) * 8);
                const int4 x1 = *reinterpret_cast<const int4 *>(lx + (4 * set + jq) * 8 + 4);
                xt[set][0] = x0.x; xt[set][1] = x0.y; xt[set][2] = x0.z; xt[set][3] = x0.w;
                xt[set][4] = x1.x; xt[set][5] = x1.y; xt[set][6] = x1.z; xt[set][7] = x1.w;
            }
            const int64_t cs = cand_stride(n);
            const bool ragged = (ssh + 1) * kSuperWords * 32 > n;
            // stage and dummy slots: this wave's two 1 KiB copy areas of the tile its
            // next copies will fill (every wave is done reading that tile)
            // the stage: with one query set this wave's two 1 KiB copy areas of the tile
            // its next copies will fill (every wave is done reading it); with two, its
            // own area after the lanes' dummy slots
            lds_char *tiles_end = lds3 + (tiles_base - lds_base) + kTiles * kTileBytes;
            lds_char *stage = QS == 1 ? lds3 + (ptile - lds_base) + cdst
                                      : tiles_end + kScanThreads * 8 + wave * stage_bytes_per_wave<QS>();
            lds_char *stage_hi = stage + (QS == 1 ? 4 * kGroupBytes : 4096);
            uint32_t c[QS];
#pragma unroll
            for (int set = 0; set < QS; ++set) c[set] = 0u;
            combine_filter<QS, kWide>(
                acc, xt, ragged, nk < kMaxKBlocks, G, jq, s, wq, lane, wi, n, cs,
                reinterpret_cast<char *>(scores + (size_t)hh * G * cs),
                masks + (size_t)hh * G * ((n + 31) >> 5), c, stage, stage_hi, tiles_end + 8 * tid);
#pragma unroll
            for (int set = 0; set < QS; ++set) {  // count bits stay below kRunOvf
                cnt0[set] |= k ? 0u : c[set] & kRunOvf;
                cnt0[set] += k ? 0u : c[set] & ~kRunOvf;
                cnt1[set] |= k ? c[set] & kRunOvf : 0u;
                cnt1[set] += k ? c[set] & ~kRunOvf : 0u;
            }
        } else {
            // the head's constants, picked element by element: choosing between the two
            // arrays as a whole made them addressable, i.e. scratch memory
            float Ck[QS], Sk[QS];
#pragma unroll
            for (int set = 0; set < QS; ++set) {
                Ck[set] = k ? C1[set] : C0[set];
                Sk[set] = k ? S1[set] : S0[set];
            }
            combine_store<QS>(acc, Ck, Sk, small, G, jq, s, wi, n, scores + (size_t)hh * G * n);
        }
        pk = -1;
    };
    for (int f = 0; f < nitems; ++f) {
        // this wave's copies of item f have landed (2 copies per later item in flight;
        // the stores of a combine, issued before the newest copies, are waited for too)
        if (fi - f - 1 == kTiles - 2) {
            if constexpr (kTiles == 2) __builtin_amdgcn_s_waitcnt(0x0F70);
            if constexpr (kTiles == 3) __builtin_amdgcn_s_waitcnt(0x0F72);
            if constexpr (kTiles == 4) __builtin_amdgcn_s_waitcnt(0x0F74);
            if constexpr (kTiles == 5) __builtin_amdgcn_s_waitcnt(0x0F76);
            if constexpr (kTiles == 6) __builtin_amdgcn_s_waitcnt(0x0F78);
        } else {
            __builtin_amdgcn_s_waitcnt(0x0F70);
        }
        __asm__ volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();  // ... and every wave's; tile f-1 is free again
        __asm__ volatile("" ::: "memory");
        if (pk >= 0) combine();
        if (fi < nitems) issue();
        const int k = pss >= h1rel ? 1 : 0;
        const int nk = k ? nkb1 : nkb0;
        const bool hi = 2 * ppr + 1 < nk;  // upper 4 groups of the K-pair exist
        char *t = lds + 2 * kHeadBytes + (f % kTiles) * kTileBytes + trsrc0;
        const uint32_t hi_mask = hi ? 0xFFFFFFFFu : 0u;
        const uint2 *la = reinterpret_cast<const uint2 *>(lds + k * kHeadBytes);
        v4i A[QS];
#pragma unroll
        for (int set = 0; set < QS; ++set) {
            const uint2 alo = la[((2 * ppr) * 64 + lane) * QS + set];
            const uint2 ahi = hi ? la[((2 * ppr + 1) * 64 + lane) * QS + set] : make_uint2(0u, 0u);
            A[set] = v4i{(int)alo.x, (int)alo.y, (int)ahi.x, (int)ahi.y};
        }
#pragma unroll
        for (int tp = 0; tp < 2; ++tp) {
            const int slot = (2 * wave + tp) ^ tile_swz(qgrp, trj);  // groups q and q + 4 alike
            uint32_t x[2][2];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const v2i r = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                    (__attribute__((address_space(3))) v2i *)(t + h * 4 * kGroupBytes + 16 * slot));
                x[h][0] = (uint32_t)r.x;
                x[h][1] = (uint32_t)r.y;
            }
            if (ppr == 0) mma_pass_x<QS, true>(x, A, hi_mask, acc[tp]);
            else mma_pass_x<QS, false>(x, A, hi_mask, acc[tp]);
        }
        if (++ppr == (k ? npr1 : npr0)) {
            pk = k;
            pss_c = pss;
            ptile = tiles_base + (uint32_t)((f % kTiles) * kTileBytes);
            ppr = 0;
            ++pss;
        }
    }
    if (pk >= 0) combine();
    if constexpr (kFilter && !kFused) {  // the run's kept counts and overflow bits into its rows
        if ((lane & 15) == 0) {
#pragma unroll
            for (int k = 0; k < 2; ++k) {
                if (k && h1 == h0) break;
                ScanMeta *mh = reinterpret_cast<ScanMeta *>(const_cast<char *>(ws) +
                                                            (size_t)(k ? h1 : h0) * kMetaBytes);
#pragma unroll
                for (int set = 0; set < QS; ++set) {
                    const int g = 4 * set + jq;
                    const uint32_t c = k ? cnt1[set] : cnt0[set];
                    if (g < G && (c & ~kRunOvf)) atomicAdd(mh->cnt + g, c & ~kRunOvf);
                    if (g < G && (c & kRunOvf)) atomicOr(&mh->ovf, 1u << g);
                }
            }
        }
    }
}

template <int QS, bool kWide, bool kFilter>
__global__ __launch_bounds__(kScanThreads)
__attribute__((amdgpu_waves_per_eu(QS == 1 ? FATHOM_SCAN_WAVES_PER_EU : 2))) void k_scan_main(
    const uint32_t *__restrict__ planes, int n, int word_stride, int G, int H, ScanSplit sp,
    const char *__restrict__ ws, float *__restrict__ scores, uint32_t *__restrict__ masks) {
    scan_body<QS, kWide, kFilter, false>(planes, n, word_stride, G, H, sp, ws, scores, masks,
                                         FrontIn{});
}

constexpr long kFrontMaxGroups = 256;  // (head, super-step) workgroups of the fused front

// A decode step's front for few heads of one-chunk rows: plan, prepare and filtering scan
// in one kernel, one workgroup per (head, super-step).  It saves the scan's reload of the
// records and a launch; the prepare work is repeated by each workgroup of a head.
__global__ __launch_bounds__(kScanThreads)
__attribute__((amdgpu_waves_per_eu(FATHOM_SCAN_WAVES_PER_EU))) void k_front_fused(
    const uint32_t *__restrict__ planes, int n, int word_stride, int G, int H, ScanSplit sp,
    char *__restrict__ ws, float *__restrict__ cand, uint32_t *__restrict__ masks, FrontIn fz) {
    scan_body<1, false, true, true>(planes, n, word_stride, G, H, sp, ws, cand, masks, fz);
}

// Resident workgroups of a kernel instance over the device (asked once per device).
template <int QS, bool kWide, bool kFilter>
int resident_slots() {
    static std::mutex mu;
    static int slots[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
    std::lock_guard<std::mutex> lock(mu);
    if (!slots[dev]) {
        int per_cu = 0, cus = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu,
                                                         k_scan_main<QS, kWide, kFilter>,
                                                         kScanThreads,
                                                         scan_lds_bytes<QS>()) != hipSuccess ||
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) !=
                hipSuccess)
            return 0;
        slots[dev] = std::max(1, per_cu) * std::max(1, cus);
    }
    return slots[dev];
}

template <int QS, bool kWide, bool kFilter>
hipError_t launch_main_qs(const fathom_store &st, int G, float *scores, const char *ws,
                          uint32_t *masks, hipStream_t s) {
    const int W = (st.n_tokens + 31) >> 5;
    ScanSplit sp;
    sp.nss = (W + kSuperWords - 1) / kSuperWords;
    const long total = (long)st.n_heads * sp.nss;
    int slots = resident_slots<QS, kWide, kFilter>();
    if (slots <= 0) slots = 1024;
    slots *= FATHOM_SCAN_ROUNDS;
    sp.run = (int)std::max(1L, (total + slots - 1) / slots);
    sp.flat = sp.run <= sp.nss;
    if (!sp.flat) sp.run = sp.nss;
    sp.wgs_per_head = (sp.nss + sp.run - 1) / sp.run;
    const long nblocks = sp.flat ? (total + sp.run - 1) / sp.run
                                 : (long)st.n_heads * sp.wgs_per_head;
    hipLaunchKernelGGL((k_scan_main<QS, kWide, kFilter>), dim3((unsigned)nblocks),
                       dim3(kScanThreads), scan_lds_bytes<QS>(), s, st.planes, st.n_tokens,
                       st.word_stride, G, st.n_heads, sp, ws, scores, masks);
    return hipGetLastError();
}

template <int QS>
hipError_t launch_main_q(const fathom_store &st, int G, float *scores, const char *ws,
                         uint32_t *masks, hipStream_t s) {
    // byte offsets within a head's 512 rows fit 32 bits?
    const bool wide = (uint64_t)kMaxPlanesPerHead * (uint64_t)st.word_stride * 4u > 0xFFFFFFFFull;
    if (masks)
        return wide ? launch_main_qs<QS, true, true>(st, G, scores, ws, masks, s)
                    : launch_main_qs<QS, false, true>(st, G, scores, ws, masks, s);
    return wide ? launch_main_qs<QS, true, false>(st, G, scores, ws, nullptr, s)
                : launch_main_qs<QS, false, false>(st, G, scores, ws, nullptr, s);
}

}  // namespace

hipError_t launch_scan_prepare(const fathom_store &st, const float *q, int G,
                               const uint8_t *depth, int k, void *ws, hipStream_t s) {
    char *w = static_cast<char *>(ws);
    const dim3 grid(st.n_heads);
    if (query_sets(G) == 1)
        hipLaunchKernelGGL(k_scan_prepare<1>, grid, dim3(prep_threads<1>()), 0, s, q, depth,
                           st.scale, st.zero, st.n_heads, G, st.planes, st.n_tokens,
                           st.word_stride, k, w);
    else
        hipLaunchKernelGGL(k_scan_prepare<2>, grid, dim3(prep_threads<2>()), 0, s, q, depth,
                           st.scale, st.zero, st.n_heads, G, st.planes, st.n_tokens,
                           st.word_stride, k, w);
    return hipGetLastError();
}

hipError_t launch_plan_prepare(const fathom_store &st, const float *q, int G, int B, int k,
                               uint8_t *depth, void *ws, hipStream_t s) {
    char *w = static_cast<char *>(ws);
    const dim3 grid(st.n_heads);
    if (query_sets(G) == 1)
        hipLaunchKernelGGL(k_plan_prepare<1>, grid, dim3(prep_threads<1>()), 0, s, q, st.var,
                           st.scale, st.zero, st.n_heads, G, B, st.planes, st.n_tokens,
                           st.word_stride, k, depth, w);
    else
        hipLaunchKernelGGL(k_plan_prepare<2>, grid, dim3(prep_threads<2>()), 0, s, q, st.var,
                           st.scale, st.zero, st.n_heads, G, B, st.planes, st.n_tokens,
                           st.word_stride, k, depth, w);
    return hipGetLastError();
}

hipError_t launch_scan_main(const fathom_store &st, int G, float *scores, void *ws,
                            hipStream_t s, uint32_t *masks) {
    const char *w = static_cast<const char *>(ws);
    return query_sets(G) == 1 ? launch_main_q<1>(st, G, scores, w, masks, s)
                              : launch_main_q<2>(st, G, scores, w, masks, s);
}

bool front_fused_applies(const fathom_store &st, int G) {
    const int W = (st.n_tokens + 31) >> 5;
    const long nss = (W + kSuperWords - 1) / kSuperWords;
    const bool wide = (uint64_t)kMaxPlanesPerHead * (uint64_t)st.word_stride * 4u > 0xFFFFFFFFull;
    return query_sets(G) == 1 && !wide && st.n_tokens <= kTopkChunk &&
           (long)st.n_heads * nss <= kFrontMaxGroups;
}

hipError_t launch_front_fused(const fathom_store &st, const float *q, int G, int B, int k,
                              uint8_t *depth, void *ws, float *cand, uint32_t *masks,
                              hipStream_t s) {
    if (!front_fused_applies(st, G)) return hipErrorInvalidValue;
    const int W = (st.n_tokens + 31) >> 5;
    ScanSplit sp;
    sp.nss = (W + kSuperWords - 1) / kSuperWords;
    sp.run = 1;
    sp.flat = 0;
    sp.wgs_per_head = sp.nss;
    FrontIn fz{q, st.var, st.scale, st.zero, B, k, depth};
    hipLaunchKernelGGL(k_front_fused, dim3((unsigned)(st.n_heads * sp.nss)), dim3(kScanThreads),
                       scan_lds_bytes<1>(), s, st.planes, st.n_tokens, st.word_stride, G,
                       st.n_heads, sp, static_cast<char *>(ws), cand, masks, fz);
    return hipGetLastError();
}

}  // namespace fathom
