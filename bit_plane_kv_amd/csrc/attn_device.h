// Device body of the exact attention over the winners' bf16 K/V rows (blog, "The first
// fix": compute attention over just those k tokens; reading the values for k tokens).
//
// A wave works on 8 winner rows at once, 8 lanes per row, 16 channels (32 bytes of K and
// of V) per lane; each row slot keeps an online softmax (running max, running sum,
// 128-wide output) over its rows, taken four at a time with every load of the four in
// flight together and one update of the running max per four rows.  Many rows (a batched
// step): one 256-thread workgroup a row, several to a CU to keep HBM busy, the slots
// merged through LDS.  Few rows (one layer of a decode step): the winners cut into one
// share a wave, merged in a fixed tree of partial results, so that the tree's groups can
// run in one workgroup or in several (the gather of one workgroup is bound by its CU's
// load rate).
// Rows are gathered straight from HBM or from pinned host memory; the gather is
// memory-bound, so there is no matrix-core use.
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

// The online softmax of one row slot (8 lanes, sub = lane & 7, 16 channels a lane) over
// the winners first, first + stride, ... below end: four rows at a time, their indices,
// then their K and V pieces, loaded together (a row past the end or out of range reads
// row 0 and is then skipped), so that each batch waits for two memory latencies instead
// of each row; the four rows then update the running max m, sum l and output o once.
template <class Idx>
__device__ __forceinline__ void slot_rows(const float (&qv)[16], const uint16_t *Kh,
                                          const uint16_t *Vh, int n, const Idx &idx_of,
                                          int first, int end, int stride, float sm_scale,
                                          float &m, float &l, float (&o)[16]) {
    for (int r0 = first; r0 < end; r0 += 4 * stride) {
        int row[4];
        bool ok[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int r = r0 + u * stride;
            row[u] = r < end ? idx_of(r) : -1;
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
}

// The lane's 16 channels of query row hg.
__device__ __forceinline__ void load_query(const float *q, int hg, int sub, float (&qv)[16]) {
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

// The result of a row's attention: channel c of out[hg] = O / L (0 when L = 0).
struct AttnToOut {
    uint16_t *out;
    int hg;
    __device__ void operator()(int c, float O, float L, float) const {
        out[(size_t)hg * kD + c] = float_to_bf16_bits(L > 0.0f ? O / L : 0.0f);
    }
};

// The attention of query row hg over its k winners, idx_of(r) giving the r-th winner's
// token index (an int32 array in global memory).  NT threads, one workgroup a row (many
// rows: a batched step): NT / 8 slots, slot s taking winners s, s + NT / 8, ...; at the end
// one wave finds the largest running max and each slot's factor, and the slots' outputs
// are summed through LDS in two levels (NT / 128 groups of 16 slots, then the groups).
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
    load_query(q, hg, sub, qv);
    float m = -INFINITY, l = 0.0f, o[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) o[i] = 0.0f;
    const uint16_t *Kh = K + (size_t)h * n * kD + sub * 16;
    const uint16_t *Vh = V + (size_t)h * n * kD + sub * 16;
    slot_rows(qv, Kh, Vh, n, idx_of, slot, k, kSlots, sm_scale, m, l, o);
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
        out[(size_t)hg * kD + tid] = float_to_bf16_bits(L > 0.0f ? O / L : 0.0f);
    }
}

// ---------------------------------------------------------------------------------
// Few rows (a layer of a decode step): a row's winners are cut into kShares equal shares,
// one a wave; kShareGroups groups of kShares / kShareGroups waves.  A wave attends its
// share (8 slots, merged by lane exchanges) to a partial result -- the unnormalised
// output O = sum_r e^(s_r - M) v_r, the weight sum L = sum_r e^(s_r - M) and the largest
// score M (-inf with no row) -- each group merges its waves' parts, and the groups' parts
// merge into the output.  One workgroup of 16 waves can do it all, or the groups can run
// in workgroups of their own and meet through memory: the same arithmetic in the same
// order either way, so the results are the same to the bit.
constexpr int kShares = 16;
constexpr int kShareGroups = 8;
constexpr int kSharesPerGroup = kShares / kShareGroups;
constexpr int kPartFloats = kD + 4;  // a partial result: O[128], L, M, two unused
static_assert(kShares % kShareGroups == 0 && kShareGroups * kD <= kShares * 64,
              "the one-workgroup form merges every group's channels at once");

// Share s of k winners: [s k / kShares, (s + 1) k / kShares).
__device__ __forceinline__ int share_begin(int k, int s) {
    return (int)((int64_t)k * s / kShares);
}

// Merges P partial results for channel c in order p = 0 .. P - 1: with M the largest of
// their scores, part p counts with the factor e^(M_p - M) (0 for a part with no row).
// ld(p, j) reads word j of part p.
template <int P, class Ld>
__device__ __forceinline__ void merge_parts(const Ld &ld, int c, float &O, float &L,
                                            float &M) {
    float Mp[P];
    M = -INFINITY;
#pragma unroll
    for (int p = 0; p < P; ++p) {
        Mp[p] = ld(p, kD + 1);
        M = fmaxf(M, Mp[p]);
    }
    O = 0.0f;
    L = 0.0f;
#pragma unroll
    for (int p = 0; p < P; ++p) {
        const float f = Mp[p] == -INFINITY ? 0.0f : expf(Mp[p] - M);
        L = fmaf(f, ld(p, kD), L);
        O = fmaf(f, ld(p, c), O);
    }
}

// The calling wave's share [b, e) of row hg's winners, as a partial result in dst (LDS).
template <class Idx>
__device__ __forceinline__ void attend_share(const float *__restrict__ q,
                                             const uint16_t *__restrict__ K,
                                             const uint16_t *__restrict__ V, int G, int n,
                                             const Idx &idx_of, int b, int e, float sm_scale,
                                             int hg, float *dst) {
    const int lane = threadIdx.x & 63, slot = lane >> 3, sub = lane & 7;
    const int h = hg / G;
    float qv[16];
    load_query(q, hg, sub, qv);
    float m = -INFINITY, l = 0.0f, o[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) o[i] = 0.0f;
    const uint16_t *Kh = K + (size_t)h * n * kD + sub * 16;
    const uint16_t *Vh = V + (size_t)h * n * kD + sub * 16;
    slot_rows(qv, Kh, Vh, n, idx_of, b + slot, e, 8, sm_scale, m, l, o);
    // the 8 slots (lanes sub, sub + 8, ..., sub + 56) merge by exchanges
    float M = m;
    M = fmaxf(M, __shfl_xor(M, 8, 64));
    M = fmaxf(M, __shfl_xor(M, 16, 64));
    M = fmaxf(M, __shfl_xor(M, 32, 64));
    const float f = m == -INFINITY ? 0.0f : expf(m - M);
    float L = l * f;
    L += __shfl_xor(L, 8, 64);
    L += __shfl_xor(L, 16, 64);
    L += __shfl_xor(L, 32, 64);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        float v = o[i] * f;
        v += __shfl_xor(v, 8, 64);
        v += __shfl_xor(v, 16, 64);
        v += __shfl_xor(v, 32, 64);
        o[i] = v;
    }
    if (slot == 0) {
#pragma unroll
        for (int i = 0; i < 16; ++i) dst[sub * 16 + i] = o[i];
        if (sub == 0) {
            dst[kD] = L;
            dst[kD + 1] = M;
        }
    }
}

// Group grp of row hg: its waves' shares attended by waves 0 .. kSharesPerGroup - 1 of
// the workgroup (the others idle), then merged by threads 0 .. kD - 1, which receive the
// group's part for channel tid as fin(tid, O, L, M).  Every thread of the workgroup calls
// it (it holds barriers).
template <class Idx, class Fin>
__device__ __forceinline__ void attend_group(const float *__restrict__ q,
                                             const uint16_t *__restrict__ K,
                                             const uint16_t *__restrict__ V, int G, int n,
                                             const Idx &idx_of, int k, int grp, float sm_scale,
                                             int hg, const Fin &fin) {
    __shared__ float wpart[kSharesPerGroup][kPartFloats];
    const int tid = threadIdx.x, wave = tid >> 6;
    if (wave < kSharesPerGroup) {
        const int s = grp * kSharesPerGroup + wave;
        attend_share(q, K, V, G, n, idx_of, share_begin(k, s), share_begin(k, s + 1),
                     sm_scale, hg, wpart[wave]);
    }
    __syncthreads();
    if (tid < kD) {
        float O, L, M;
        merge_parts<kSharesPerGroup>([](int p, int j) { return wpart[p][j]; }, tid, O, L, M);
        fin(tid, O, L, M);
    }
}

// Group grp of row hg in a workgroup of its own (blockIdx picks the group; every thread
// calls it): the group's part goes to prow[grp] (prow: the row's kShareGroups parts of
// kPartFloats floats) and the last of the row's groups to finish merges the parts into
// out[hg], with the arithmetic and order of attend_row_shares.  `count` is the row's
// counter, zero before the row's first group starts.
// The parts meet through device-scope stores and loads (written through to, and read from,
// the level of the memory system every CU sees), ordered by the count: each thread waits
// until its stores are done before the workgroup takes the count, and the count's last
// taker reads the parts after it.  A device-scope fence would do the same by writing back
// and invalidating the whole L2, which costs tens of microseconds here.
template <class Idx>
__device__ __forceinline__ void attend_group_split(const float *__restrict__ q,
                                                   const uint16_t *__restrict__ K,
                                                   const uint16_t *__restrict__ V, int G,
                                                   int n, const Idx &idx_of, int k, int grp,
                                                   float sm_scale, int hg, float *prow,
                                                   uint32_t *count, uint16_t *out) {
    __shared__ bool last;
    const int tid = threadIdx.x;
    float *mine = prow + grp * kPartFloats;
    attend_group(q, K, V, G, n, idx_of, k, grp, sm_scale, hg,
                 [mine](int c, float O, float L, float M) {
                     __hip_atomic_store(mine + c, O, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                     if (c == 0) {
                         __hip_atomic_store(mine + kD, L, __ATOMIC_RELAXED,
                                            __HIP_MEMORY_SCOPE_AGENT);
                         __hip_atomic_store(mine + kD + 1, M, __ATOMIC_RELAXED,
                                            __HIP_MEMORY_SCOPE_AGENT);
                     }
                 });
    __builtin_amdgcn_s_waitcnt(0);  // every store of this thread done
    __syncthreads();
    if (tid == 0) last = atomicAdd(count, 1u) == kShareGroups - 1;
    __syncthreads();
    if (!last) return;
    if (tid < kD) {
        float O, L, M;
        merge_parts<kShareGroups>(
            [prow](int p, int j) {
                return __hip_atomic_load(prow + p * kPartFloats + j, __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT);
            },
            tid, O, L, M);
        out[(size_t)hg * kD + tid] = float_to_bf16_bits(L > 0.0f ? O / L : 0.0f);
    }
}

// All groups of row hg in one workgroup of kShares waves, the output written to out[hg].
template <class Idx>
__device__ __forceinline__ void attend_row_shares(const float *__restrict__ q,
                                                  const uint16_t *__restrict__ K,
                                                  const uint16_t *__restrict__ V, int G, int n,
                                                  const Idx &idx_of, int k, float sm_scale,
                                                  uint16_t *__restrict__ out, int hg) {
    __shared__ float wpart[kShares][kPartFloats];
    __shared__ float gpart[kShareGroups][kPartFloats];
    const int tid = threadIdx.x, wave = tid >> 6;
    attend_share(q, K, V, G, n, idx_of, share_begin(k, wave), share_begin(k, wave + 1),
                 sm_scale, hg, wpart[wave]);
    __syncthreads();
    if (tid < kShareGroups * kD) {  // group tid / kD, channel tid % kD
        const int grp = tid / kD, c = tid % kD;
        float O, L, M;
        merge_parts<kSharesPerGroup>(
            [grp](int p, int j) { return wpart[grp * kSharesPerGroup + p][j]; }, c, O, L, M);
        gpart[grp][c] = O;
        if (c == 0) {
            gpart[grp][kD] = L;
            gpart[grp][kD + 1] = M;
        }
    }
    __syncthreads();
    if (tid < kD) {
        float O, L, M;
        merge_parts<kShareGroups>([](int p, int j) { return gpart[p][j]; }, tid, O, L, M);
        out[(size_t)hg * kD + tid] = float_to_bf16_bits(L > 0.0f ? O / L : 0.0f);
    }
}

}  // namespace fathom
