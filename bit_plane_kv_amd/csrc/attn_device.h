// Device body of the exact attention over the winners' bf16 K/V rows (blog, "The first
// fix": compute attention over just those k tokens; reading the values for k tokens).
//
// One workgroup per (head, query).  A wave works on 8 winner rows at once, 8 lanes per
// row, 16 channels (32 bytes of K and of V) per lane; each of the NT / 8 row slots keeps
// an online softmax (running max, running sum, 128-wide output) over its rows, taken
// four at a time with every load of the four in flight together and one update of the
// running max per four rows.  At the end one wave finds the largest running max and each
// slot's factor; the slots' outputs are summed through LDS in two levels (NT / 128 groups
// of 16 slots, then the groups).
// Rows are gathered straight from HBM or from pinned host memory; the gather is
// memory-bound, so there is no matrix-core use.  With few rows (one layer of a decode
// step) a workgroup has 1024 threads, so that the 512 winners of a row need one round of
// index loads and one of K/V loads; with many (a batched step) it has 256, so that
// several workgroups share a CU and keep HBM busy.
#pragma once

#include "common.h"

namespace fathom {

__device__ __forceinline__ void unpack8(const uint4 u, float *f) {
    f[0] = bf16_bits_to_float(u.x & 0xFFFFu);
    f[1] = __uint_as_float(u.x & 0xFFFF0000u);
    f[2] = bf16_bits_to_float(u.y & 0xFFFFu);
    f[3] = __uint_as_float(u.y & 0xFFFF0000u);
    f[4] = bf16_bits_to_float(u.z & 0xFFFFu);
    f[5] = __uint_as_float(u.z & 0xFFFF0000u);
    f[6] = bf16_bits_to_float(u.w & 0xFFFFu);
    f[7] = __uint_as_float(u.w & 0xFFFF0000u);
}

// The attention of query row hg over its k winners, idx_of(r) giving the r-th winner's
// token index (an int32 array in global memory, or the select's winners in LDS).  NT
// threads (256 or 1024), one workgroup a row.
template <int NT, class Idx>
__device__ __forceinline__ void attend_row(const float *__restrict__ q,
                                           const uint16_t *__restrict__ K,
                                           const uint16_t *__restrict__ V, int G, int n,
                                           Idx idx_of, int k, float sm_scale,
                                           uint16_t *__restrict__ out, int hg) {
    constexpr int kSlots = NT / 8;              // rows in flight per workgroup
    constexpr int kParts = NT / kD;             // groups of slots in the merge
    constexpr int kSlotsPerPart = kSlots / kParts;  // 16
    __shared__ float so[kSlots][kD + 1];
    __shared__ float smax[kSlots], ssum[kSlots], sf[kSlots];
    __shared__ float po[kParts][kD];
    __shared__ float sL;
    const int h = hg / G;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int slot = wave * 8 + (lane >> 3), sub = lane & 7;

    float qv[16];
    {
        const float4 *qp = reinterpret_cast<const float4 *>(q + (size_t)hg * kD + sub * 16);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float4 t = qp[i];
            qv[4 * i] = t.x;
            qv[4 * i + 1] = t.y;
            qv[4 * i + 2] = t.z;
            qv[4 * i + 3] = t.w;
        }
    }
    float m = -INFINITY, l = 0.0f, o[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) o[i] = 0.0f;

    const uint16_t *Kh = K + (size_t)h * n * kD + sub * 16;
    const uint16_t *Vh = V + (size_t)h * n * kD + sub * 16;
    // four rows a slot at a time: their indices, then their K and V pieces, are loaded
    // together (a row past k or out of range reads row 0 and is then skipped), so that
    // each batch waits for two memory latencies instead of each row; the four rows then
    // update the slot's running softmax once
    for (int r0 = slot; r0 < k; r0 += 4 * kSlots) {
        int row[4];
        bool ok[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int r = r0 + u * kSlots;
            row[u] = r < k ? idx_of(r) : -1;
            ok[u] = (unsigned)row[u] < (unsigned)n;  // out-of-range index: skipped
        }
        uint4 kk[4][2], vv[4][2];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const size_t rr = ok[u] ? (size_t)row[u] : 0;
            const uint4 *kp = reinterpret_cast<const uint4 *>(Kh + rr * kD);
            const uint4 *vp = reinterpret_cast<const uint4 *>(Vh + rr * kD);
            kk[u][0] = kp[0];
            kk[u][1] = kp[1];
            vv[u][0] = vp[0];
            vv[u][1] = vp[1];
        }
        float sc[4];
        float mn = m;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            float kf[16];
            unpack8(kk[u][0], kf);
            unpack8(kk[u][1], kf + 8);
            float dot = 0.0f;
#pragma unroll
            for (int i = 0; i < 16; ++i) dot = fmaf(qv[i], kf[i], dot);
            dot += __shfl_xor(dot, 1, 64);
            dot += __shfl_xor(dot, 2, 64);
            dot += __shfl_xor(dot, 4, 64);
            sc[u] = ok[u] ? dot * sm_scale : -INFINITY;
            mn = fmaxf(mn, sc[u]);
        }
        if (mn == -INFINITY) continue;  // no row of this batch, none before it
        const float a = expf(m - mn);   // 0 while m is still -inf
        l *= a;
#pragma unroll
        for (int i = 0; i < 16; ++i) o[i] *= a;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const float b = expf(sc[u] - mn);  // 0 for a skipped row
            float vf[16];
            unpack8(vv[u][0], vf);
            unpack8(vv[u][1], vf + 8);
            l += b;
#pragma unroll
            for (int i = 0; i < 16; ++i) o[i] = fmaf(b, vf[i], o[i]);
        }
        m = mn;
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) so[slot][sub * 16 + i] = o[i];
    if (sub == 0) {
        smax[slot] = m;
        ssum[slot] = l;
    }
    __syncthreads();
    if (wave == 0) {  // the largest running max M, each slot's factor e^(m - M), and L
        float mx = -INFINITY;
        for (int s2 = lane; s2 < kSlots; s2 += 64) mx = fmaxf(mx, smax[s2]);
#pragma unroll
        for (int o2 = 32; o2 > 0; o2 >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o2, 64));
        float L = 0.0f;
        for (int s2 = lane; s2 < kSlots; s2 += 64) {
            const float f = smax[s2] == -INFINITY ? 0.0f : expf(smax[s2] - mx);
            sf[s2] = f;
            L += ssum[s2] * f;
        }
#pragma unroll
        for (int o2 = 32; o2 > 0; o2 >>= 1) L += __shfl_xor(L, o2, 64);
        if (lane == 0) sL = L;
    }
    __syncthreads();
    {   // group p of slots (p, p + kParts, ...): channel c's share of the output
        const int c = tid & (kD - 1), p = tid >> 7;
        float O = 0.0f;
#pragma unroll
        for (int j = 0; j < kSlotsPerPart; ++j) {
            const int s2 = p + kParts * j;
            O = fmaf(sf[s2], so[s2][c], O);
        }
        po[p][c] = O;
    }
    __syncthreads();
    if (tid < kD) {
        float O = 0.0f;
#pragma unroll
        for (int p = 0; p < kParts; ++p) O += po[p][tid];
        const float L = sL;
        const float res = L > 0.0f ? O / L : 0.0f;
        out[(size_t)hg * kD + tid] = float_to_bf16_bits(res);
    }
}

}  // namespace fathom
