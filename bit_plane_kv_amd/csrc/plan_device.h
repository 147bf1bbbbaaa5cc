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
// each channel's keys fall with t.  The body sorts those 512 items (bitonic network in
// LDS) and counts, per channel, the items among the first B.
#pragma once

#include "common.h"

namespace fathom {

// item a precedes item b: larger key first, then lower item number (= c*4 + t)
__device__ __forceinline__ bool plan_precedes(uint64_t ka, int ia, uint64_t kb, int ib) {
    return ka > kb || (ka == kb && ia < ib);
}

// Writes the depth of each of head h's channels to cnt[0..127] (LDS); 256 threads.
// Ends with a barrier, so cnt is complete for every thread.
__device__ __forceinline__ void plan_head(const float *__restrict__ q,
                                          const float *__restrict__ var, int G, int B, int h,
                                          int *cnt) {
    __shared__ uint64_t key[kMaxPlanesPerHead];
    __shared__ int16_t item[kMaxPlanesPerHead];
    const int tid = threadIdx.x;
    if (tid < kD) {
        // w_c = (sum_g q_gc^2) * var_c in fp64; each square is exact, the sum runs
        // over g ascending, then one product (no fused operations in this build)
        double sq = 0.0;
        for (int g = 0; g < G; ++g) {
            const double v = (double)q[((size_t)h * G + g) * kD + tid];
            sq = sq + v * v;
        }
        const double w = sq * (double)var[(size_t)h * kD + tid];
        // keys are >= +0, so their bit patterns order like the values
#pragma unroll
        for (int t = 0; t < kPlanes; ++t) {
            key[tid * kPlanes + t] = (uint64_t)__double_as_longlong(ldexp(w, -2 * t));
            item[tid * kPlanes + t] = (int16_t)(tid * kPlanes + t);
        }
        cnt[tid] = 0;
    }
    __syncthreads();
    // bitonic sort of 512 items into "precedes" order; 256 threads, one pair each
    for (int size = 2; size <= kMaxPlanesPerHead; size <<= 1) {
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            const int lo = 2 * tid - (tid & (stride - 1));
            const int hi = lo + stride;
            const bool ascending = (lo & size) == 0;  // "ascending" = precedes order
            const uint64_t ka = key[lo], kb = key[hi];
            const int ia = item[lo], ib = item[hi];
            const bool swap =
                ascending ? plan_precedes(kb, ib, ka, ia) : plan_precedes(ka, ia, kb, ib);
            if (swap) {
                key[lo] = kb;
                key[hi] = ka;
                item[lo] = (int16_t)ib;
                item[hi] = (int16_t)ia;
            }
            __syncthreads();
        }
    }
    for (int p = tid; p < B; p += 256) atomicAdd(&cnt[item[p] / kPlanes], 1);
    __syncthreads();
}

}  // namespace fathom
