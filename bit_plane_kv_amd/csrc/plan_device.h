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
// each channel's keys fall with t.  The body sorts those 512 items (a bitonic network)
// and counts, per channel, the items among the first B.
//
// Sort layout: item i = 4c + t; wave v holds items 128v .. 128v+127, lane l items
// 128v + l (register 0) and 128v + 64 + l (register 1).  Compare-exchanges of stride
// < 64 pair lanes of one wave (shuffles), stride 64 pairs a lane's two registers, and
// only the strides 128 and 256 (three stages) go through LDS with a barrier.
#pragma once

#include "common.h"

namespace fathom {

// item a precedes item b: larger key first, then lower item number (= c*4 + t)
__device__ __forceinline__ bool plan_precedes(uint64_t ka, int ia, uint64_t kb, int ib) {
    return ka > kb || (ka == kb && ia < ib);
}

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

// Position i of the sorted order keeps, from the pair (mine, the partner at i ^ stride),
// the item that comes first when i is the lower position of an ascending block or the
// upper of a descending one, else the other.
__device__ __forceinline__ void plan_keep(uint64_t &k, int &it, uint64_t ok, int oi, int i,
                                          int stride, int size) {
    const bool want_first = ((i & stride) == 0) == ((i & size) == 0);
    const bool mine_first = plan_precedes(k, it, ok, oi);
    if (want_first != mine_first) {
        k = ok;
        it = oi;
    }
}

// Sorts the 512 items of one head and writes each channel's depth (the number of its
// items among the first B) to cnt[0..127] (LDS); 256 threads.  wc[r] is the importance
// of the channel of this thread's item r (see the layout above).  Ends with a barrier,
// so cnt is complete for every thread.
__device__ __forceinline__ void plan_sort(const double (&wc)[2], int B, int *cnt) {
    __shared__ uint64_t xk[2][kMaxPlanesPerHead];
    __shared__ int xi[2][kMaxPlanesPerHead];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    if (tid < kD) cnt[tid] = 0;  // complete after the first cross-wave stage's barrier
    uint64_t k[2];
    int it[2];
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        it[r] = 128 * wave + 64 * r + lane;
        // keys are >= +0, so their bit patterns order like the values; w 4^-t is exact
        k[r] = (uint64_t)__double_as_longlong(ldexp(wc[r], -2 * (it[r] & 3)));
    }
    int buf = 0;
#pragma unroll
    for (int size = 2; size <= kMaxPlanesPerHead; size <<= 1) {
#pragma unroll
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            if (stride >= 128) {  // across waves, through LDS (two buffers alternate)
#pragma unroll
                for (int r = 0; r < 2; ++r) {
                    const int i = 128 * wave + 64 * r + lane;
                    xk[buf][i] = k[r];
                    xi[buf][i] = it[r];
                }
                __syncthreads();
#pragma unroll
                for (int r = 0; r < 2; ++r) {
                    const int i = 128 * wave + 64 * r + lane;
                    plan_keep(k[r], it[r], xk[buf][i ^ stride], xi[buf][i ^ stride], i, stride,
                              size);
                }
                buf ^= 1;
            } else if (stride == 64) {  // a lane's two registers
                const int i = 128 * wave + lane;
                const uint64_t k0 = k[0];
                const int i0 = it[0];
                plan_keep(k[0], it[0], k[1], it[1], i, 64, size);
                plan_keep(k[1], it[1], k0, i0, i + 64, 64, size);
            } else {  // lanes of one wave
#pragma unroll
                for (int r = 0; r < 2; ++r) {
                    const int i = 128 * wave + 64 * r + lane;
                    const uint64_t ok = (uint64_t)__shfl_xor((long long)k[r], stride, 64);
                    const int oi = __shfl_xor(it[r], stride, 64);
                    plan_keep(k[r], it[r], ok, oi, i, stride, size);
                }
            }
        }
    }
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        const int i = 128 * wave + 64 * r + lane;  // position in the sorted order
        if (i < B) atomicAdd(&cnt[it[r] >> 2], 1);
    }
    __syncthreads();
}

// The channel of this thread's sort item r (see the layout above).
__device__ __forceinline__ int plan_item_channel(int r) {
    return (128 * (threadIdx.x >> 6) + 64 * r + (threadIdx.x & 63)) >> 2;
}

// Loads the plan's inputs for this thread's two sort items: the G queries and the
// variance of each item's channel.
__device__ __forceinline__ void plan_load(const float *__restrict__ q,
                                          const float *__restrict__ var, int G, int h,
                                          float (&qp)[2][FATHOM_MAX_G], float (&vp)[2]) {
    // every load is unconditional (index clamped to a real query) so that all of them
    // are in flight together; the unused values are zeroed afterwards
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        const int c = plan_item_channel(r);
#pragma unroll
        for (int g = 0; g < FATHOM_MAX_G; ++g)
            qp[r][g] = q[((size_t)h * G + min(g, G - 1)) * kD + c];
        vp[r] = var[(size_t)h * kD + c];
    }
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
        for (int g = 0; g < FATHOM_MAX_G; ++g) qp[r][g] = g < G ? qp[r][g] : 0.0f;
}

// Whole plan of head h from the loaded inputs: depths to cnt[0..127] (LDS); 256
// threads; ends with a barrier.
__device__ __forceinline__ void plan_from(const float (&qp)[2][FATHOM_MAX_G],
                                          const float (&vp)[2], int G, int B, int *cnt) {
    double wc[2];
#pragma unroll
    for (int r = 0; r < 2; ++r) wc[r] = plan_importance(qp[r], vp[r], G);
    plan_sort(wc, B, cnt);
}

}  // namespace fathom
