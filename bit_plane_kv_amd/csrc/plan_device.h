// Device body of the per-head plan, shared by the plan kernel and the fused
// plan-and-prepare kernel of a decode step (one 256-thread workgroup per head).
//
// Source: the blog's "How each query picks its own depth" -- a channel's importance is
// the share of score variance it carries; one more bit on a channel cuts its error in
// proportion to importance / 4^(bits already spent); important channels get all four
// planes, marginal ones one, useless ones none.  Glonce: variance-weighted importance.
//
// The greedy form (B times, give a plane to the channel with the largest w_c 4^-t_c,
// equal values to the lower channel index) takes exactly the first B of the 4d items
// (c, t) ordered by key w_c 4^-t descending, then c ascending, then t ascending, because
// each channel's keys fall with t.  So depth_c = #{t : rank(c, t) < B}, rank = the
// number of items before (c, t) in that order.
//
// The ranks come from the channels alone.  With the channels sorted by (w descending,
// c ascending) and pos(X, c) = #{c' : w_c' > X, or w_c' = X and c' < c} (a search in
// that order), item (c', t') comes before (c, t) exactly when channel c' comes
// before (X, c) for X = w_c 4^(t' - t) (an exact scaling), except that the items of a
// channel with w_c = 0 are all equal and ordered by t.  Hence
//   rank(c, t) = sum over t' = 0..3 of pos(w_c 4^(t' - t), c)  (+ t when w_c = 0),
// seven searches per channel (t' - t = -3 .. 3).
#pragma once

#include "common.h"

namespace fathom {

// Importance of a channel from its G query values and its variance: w_c =
// (sum_g q_gc^2) * var_c in fp64; each square is exact, the sum runs over g ascending,
// then one product (no fused operations).
__device__ __forceinline__ double plan_importance(const float (&qc)[FATHOM_MAX_G], float v,
                                                  int G) {
    double sq = 0.0;
#pragma unroll
    for (int g = 0; g < FATHOM_MAX_G; ++g) {
        if (g < G) {
            const double x = (double)qc[g];
            sq = sq + x * x;
        }
    }
    return sq * (double)v;
}

// The channel a thread plans: NT / 128 threads per channel (NT = 256 or 512).
template <int NT>
__device__ __forceinline__ int plan_channel() { return (int)threadIdx.x / (NT / kD); }

// Loads the plan's inputs of this thread's channel: its G queries and its variance.
// Every load is unconditional (query clamped to a real one) so that all of them are in
// flight together; the unused values are zeroed afterwards.
template <int NT>
__device__ __forceinline__ void plan_load(const float *__restrict__ q,
                                          const float *__restrict__ var, int G, int h,
                                          float (&qp)[FATHOM_MAX_G], float &vp) {
    const int c = plan_channel<NT>();
#pragma unroll
    for (int g = 0; g < FATHOM_MAX_G; ++g) qp[g] = q[((size_t)h * G + min(g, G - 1)) * kD + c];
    vp = var[(size_t)h * kD + c];
#pragma unroll
    for (int g = 0; g < FATHOM_MAX_G; ++g) qp[g] = g < G ? qp[g] : 0.0f;
}

// Whole plan of head h from the loaded inputs: each channel's depth to cnt[0..127]
// (LDS); NT threads (256 or 512: 2 or 4 a channel); ends with a barrier, so cnt is
// complete for every thread.
//
// Importances are compared by their bit patterns: for non-negative doubles (-0 is made
// +0) the unsigned 64-bit order of the bits is the numeric order and equal bits are
// equal values, so each comparison is one integer compare.  The order's tie rule (lower
// channel first) only matters between equal importances; they are found by counting
// the channels at each strict rank (the number of larger importances), and only the
// channels that share one count the lower channels they tie with.
template <int NT>
__device__ __forceinline__ void plan_from(const float (&qp)[FATHOM_MAX_G], float vp, int G,
                                          int B, int *cnt) {
    constexpr int TPC = NT / kD;  // threads per channel: 2 or 4
    static_assert(TPC == 2 || TPC == 4, "2 or 4 threads a channel");
    __shared__ __align__(16) unsigned long long wkey[kD];  // by channel
    __shared__ __align__(16) unsigned long long skey[kD];  // in (w desc, c asc) order
    __shared__ int sch[kD];                                // the channel at each place
    __shared__ int nrank[kD];                              // channels per strict rank
    const int tid = threadIdx.x, c = plan_channel<NT>(), part = tid % TPC;
    const double w = plan_importance(qp, vp, G) + 0.0;  // -0 -> +0
    const unsigned long long bw = (unsigned long long)__double_as_longlong(w);
    if (part == 0) wkey[c] = bw;
    else if (part == 1) nrank[c] = 0;
    __syncthreads();
    // strict rank: each of the channel's threads counts the larger importances in its
    // share of the channels
    constexpr int kShare = kD / TPC;
    int r0 = 0, r1 = 0;
#pragma unroll
    for (int o = kShare * part; o < kShare * part + kShare; o += 2) {
        const ulonglong2 x = *reinterpret_cast<const ulonglong2 *>(&wkey[o]);
        r0 += x.x > bw;
        r1 += x.y > bw;
    }
    int strict = r0 + r1;
#pragma unroll
    for (int o = 1; o < TPC; o <<= 1) strict += __shfl_xor(strict, o, 64);
    if (part == 0) atomicAdd(&nrank[strict], 1);
    __syncthreads();
    int rank = strict;
    if (nrank[strict] > 1) {  // equal importances: the lower channels come first
        int before = 0;       // (all threads of the channel take this branch)
        for (int o = part; o < c; o += TPC) before += wkey[o] == bw;
#pragma unroll
        for (int o = 1; o < TPC; o <<= 1) before += __shfl_xor(before, o, 64);
        rank += before;
    }
    if (part == 0) {
        skey[rank] = bw;
        sch[rank] = c;
    }
    __syncthreads();
    // P[j + 3] = pos(w 4^j, c), j = -3 .. 3.  j = 0 is the channel's own rank; the other
    // six are shared by the channel's threads (2 threads: j = -3..-1 and 1..3; 4 threads:
    // -3, -2 | -1 | 1 | 2, 3).  Channels before (X, c) form a prefix of the sorted order:
    // its length is found from the last key of each group of 16 (the same 8 keys for
    // every thread), then by four halving steps inside the group, then past the channels
    // whose importance equals X and whose index is lower.
    constexpr int NS = 6 / TPC + (TPC == 4 ? 1 : 0);  // searches a thread: 3 or 2
    int js[NS];
#pragma unroll
    for (int i = 0; i < NS; ++i) {
        if (TPC == 2) js[i] = part ? i + 1 : i - 3;
        else js[i] = part == 0 ? i - 3 : part == 3 ? i + 2 : (i == 0 ? (part == 1 ? -1 : 1) : 0);
    }
    unsigned long long bx[NS];
    int pos[NS];
#pragma unroll
    for (int i = 0; i < NS; ++i) {
        const double X = ldexp(w, 2 * js[i]);
        bx[i] = (unsigned long long)__double_as_longlong(X);
        pos[i] = 0;
    }
    constexpr int kSeg = 16;
#pragma unroll
    for (int b = 0; b < kD / kSeg; ++b) {
        const unsigned long long last = skey[kSeg * b + kSeg - 1];
#pragma unroll
        for (int i = 0; i < NS; ++i) pos[i] += kSeg * (last > bx[i]);
    }
#pragma unroll
    for (int step = kSeg / 2; step > 0; step >>= 1) {
#pragma unroll
        for (int i = 0; i < NS; ++i) {
            const unsigned long long e = skey[min(pos[i] + step - 1, kD - 1)];
            if (pos[i] < kD && e > bx[i]) pos[i] += step;
        }
    }
#pragma unroll
    for (int i = 0; i < NS; ++i) {
        if (pos[i] < kD && skey[pos[i]] == bx[i]) {
            while (pos[i] < kD && skey[pos[i]] == bx[i] && sch[pos[i]] < c) ++pos[i];
        }
    }
    int P[7];
    P[3] = rank;
    const int base = (int)(threadIdx.x & 63) & ~(TPC - 1);  // the channel's first lane
    if (TPC == 2) {
#pragma unroll
        for (int i = 0; i < 3; ++i) {
            P[i] = __shfl(pos[i], base, 64);          // j = i - 3
            P[i + 4] = __shfl(pos[i], base + 1, 64);  // j = i + 1
        }
    } else {
        P[0] = __shfl(pos[0], base, 64);      // -3
        P[1] = __shfl(pos[1], base, 64);      // -2
        P[2] = __shfl(pos[0], base + 1, 64);  // -1
        P[4] = __shfl(pos[0], base + 2, 64);  // 1
        P[5] = __shfl(pos[0], base + 3, 64);  // 2
        P[6] = __shfl(pos[1], base + 3, 64);  // 3
    }
    int depth = 0;
#pragma unroll
    for (int t = 0; t < kPlanes; ++t) {
        int r = w == 0.0 ? t : 0;
#pragma unroll
        for (int tp = 0; tp < kPlanes; ++tp) r += P[tp - t + 3];
        depth += r < B;
    }
    if (part == 0) cnt[c] = depth;
    __syncthreads();
}

}  // namespace fathom
