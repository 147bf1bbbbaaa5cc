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
// c ascending) and pos(X, c) = #{c' : w_c' > X, or w_c' = X and c' < c} (a binary search
// in that order), item (c', t') comes before (c, t) exactly when channel c' comes
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

// The channel a thread plans: two threads per channel.
__device__ __forceinline__ int plan_channel() { return (int)(threadIdx.x >> 1); }

// Loads the plan's inputs of this thread's channel: its G queries and its variance.
// Every load is unconditional (query clamped to a real one) so that all of them are in
// flight together; the unused values are zeroed afterwards.
__device__ __forceinline__ void plan_load(const float *__restrict__ q,
                                          const float *__restrict__ var, int G, int h,
                                          float (&qp)[FATHOM_MAX_G], float &vp) {
    const int c = plan_channel();
#pragma unroll
    for (int g = 0; g < FATHOM_MAX_G; ++g) qp[g] = q[((size_t)h * G + min(g, G - 1)) * kD + c];
    vp = var[(size_t)h * kD + c];
#pragma unroll
    for (int g = 0; g < FATHOM_MAX_G; ++g) qp[g] = g < G ? qp[g] : 0.0f;
}

// Whole plan of head h from the loaded inputs: each channel's depth to cnt[0..127]
// (LDS); 256 threads; ends with a barrier, so cnt is complete for every thread.
__device__ __forceinline__ void plan_from(const float (&qp)[FATHOM_MAX_G], float vp, int G,
                                          int B, int *cnt) {
    struct Entry {  // a channel in sorted order
        double w;
        int c, pad;
    };
    __shared__ double wsh[kD];
    __shared__ Entry srt[kD];
    const int tid = threadIdx.x, c = plan_channel(), half = tid & 1;
    const double w = plan_importance(qp, vp, G);
    if (!half) wsh[c] = w;
    __syncthreads();
    // the channel's place in (w descending, c ascending): each thread counts half
    int rank = 0;
#pragma unroll 8
    for (int o = 64 * half; o < 64 * half + 64; ++o) {
        const double x = wsh[o];
        rank += (x > w) || (x == w && o < c);
    }
    rank += __shfl_xor(rank, 1, 64);
    if (!half) srt[rank] = Entry{w, c, 0};
    __syncthreads();
    // pos(w 4^j, c): thread half 0 searches j = -3 .. 0, half 1 j = 1 .. 3 (j = 4 is a
    // dummy), all four at once: the length of the prefix of the sorted channels that
    // comes before (X, c), found by steps of 128, 64, .., 1 (0 .. 128 channels)
    double X[4];
    int pos[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        X[s] = ldexp(w, 2 * (half ? s + 1 : s - 3));
        pos[s] = 0;
    }
#pragma unroll
    for (int step = kD; step > 0; step >>= 1) {
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            if (pos[s] + step <= kD) {
                const Entry e = srt[pos[s] + step - 1];
                if (e.w > X[s] || (e.w == X[s] && e.c < c)) pos[s] += step;
            }
        }
    }
    // P[j + 3] = pos(w 4^j, c) for j = -3 .. 3, from both threads of the channel
    int P[7];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        const int other = __shfl_xor(pos[s], 1, 64);
        const int lo = half ? other : pos[s];   // j = s - 3
        const int hi = half ? pos[s] : other;   // j = s + 1
        P[s] = lo;
        if (s < 3) P[s + 4] = hi;
    }
    int depth = 0;
#pragma unroll
    for (int t = 0; t < kPlanes; ++t) {
        int r = w == 0.0 ? t : 0;
#pragma unroll
        for (int tp = 0; tp < kPlanes; ++tp) r += P[tp - t + 3];
        depth += r < B;
    }
    if (!half) cnt[c] = depth;
    __syncthreads();
}

}  // namespace fathom
