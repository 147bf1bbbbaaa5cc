// Exact attention over the winners' bf16 K/V rows (blog, "The first fix": compute
// attention over just those k tokens; reading the values for k tokens).
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
#include "common.h"

namespace fathom {
namespace {

constexpr int kSmallRows = 256;  // (head, query) rows up to which workgroups have 1024 threads

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

template <int NT>
__global__ __launch_bounds__(NT) void k_sparse_attn(
    const float *__restrict__ q, const uint16_t *__restrict__ K,
    const uint16_t *__restrict__ V, int G, int n, const int32_t *__restrict__ idx, int k,
    float sm_scale, uint16_t *__restrict__ out) {
    constexpr int kSlots = NT / 8;              // rows in flight per workgroup
    constexpr int kParts = NT / kD;             // groups of slots in the merge
    constexpr int kSlotsPerPart = kSlots / kParts;  // 16
    __shared__ float so[kSlots][kD + 1];
    __shared__ float smax[kSlots], ssum[kSlots], sf[kSlots];
    __shared__ float po[kParts][kD];
    __shared__ float sL;
    const int hg = blockIdx.x, h = hg / G;
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

    const int32_t *ix = idx + (size_t)hg * k;
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
            row[u] = r < k ? ix[r] : -1;
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

__global__ __launch_bounds__(256) void k_stream_read(const uint4 *__restrict__ src,
                                                     size_t nvec, uint64_t *__restrict__ sink) {
    uint32_t a = 0, b = 0, c = 0, d = 0;
    for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < nvec;
         i += (size_t)gridDim.x * 256) {
        const uint4 v = src[i];
        a ^= v.x;
        b ^= v.y;
        c ^= v.z;
        d ^= v.w;
    }
    const uint32_t x = a ^ b ^ c ^ d;
    if (x == 0x9E3779B9u) sink[0] = ((uint64_t)a << 32) | b;  // keeps the loads live
}

// Runs of run_vec 16-byte vectors, the r-th starting at src + r * stride bytes; the
// work-items walk all runs' vectors in order.  The index is 64-bit, so the stride
// over the grid cannot wrap it below `total` (total < 2^32 keeps the division cheap).
__global__ __launch_bounds__(256) void k_stream_runs(const char *__restrict__ src,
                                                     uint32_t run_vec, uint64_t stride,
                                                     uint64_t total, uint64_t *__restrict__ sink) {
    uint32_t a = 0, b = 0, c = 0, d = 0;
    for (uint64_t i = (uint64_t)blockIdx.x * 256u + threadIdx.x; i < total;
         i += (uint64_t)gridDim.x * 256u) {
        const uint32_t r = (uint32_t)i / run_vec, o = (uint32_t)i - r * run_vec;
        const uint4 v = *reinterpret_cast<const uint4 *>(src + r * stride + (uint64_t)o * 16u);
        a ^= v.x;
        b ^= v.y;
        c ^= v.z;
        d ^= v.w;
    }
    const uint32_t x = a ^ b ^ c ^ d;
    if (x == 0x9E3779B9u) sink[0] = ((uint64_t)a << 32) | b;  // keeps the loads live
}

}  // namespace

hipError_t launch_sparse_attn(const float *q, const uint16_t *K, const uint16_t *V, int H,
                              int G, int n, const int32_t *idx, int k, float sm_scale,
                              uint16_t *out, hipStream_t s) {
    if (H * G <= kSmallRows)
        hipLaunchKernelGGL(k_sparse_attn<1024>, dim3(H * G), dim3(1024), 0, s, q, K, V, G, n,
                           idx, k, sm_scale, out);
    else
        hipLaunchKernelGGL(k_sparse_attn<256>, dim3(H * G), dim3(256), 0, s, q, K, V, G, n,
                           idx, k, sm_scale, out);
    return hipGetLastError();
}

hipError_t launch_stream_read(const void *src, size_t bytes, uint64_t *sink,
                              hipStream_t s) {
    const size_t nvec = bytes / 16;
    const int grid = (int)std::min<size_t>((nvec + 255) / 256, 4096);
    hipLaunchKernelGGL(k_stream_read, dim3(std::max(grid, 1)), dim3(256), 0, s,
                       static_cast<const uint4 *>(src), nvec, sink);
    return hipGetLastError();
}

hipError_t launch_stream_runs(const void *src, size_t run_bytes, size_t stride_bytes,
                              size_t n_runs, uint64_t *sink, hipStream_t s) {
    const uint32_t run_vec = (uint32_t)(run_bytes / 16);
    const uint64_t total = (uint64_t)run_vec * (uint64_t)n_runs;  // < 2^32 (checked)
    const int grid = (int)std::min<uint64_t>((total + 255) / 256, 4096);
    hipLaunchKernelGGL(k_stream_runs, dim3(std::max(grid, 1)), dim3(256), 0, s,
                       static_cast<const char *>(src), run_vec, (uint64_t)stride_bytes, total,
                       sink);
    return hipGetLastError();
}

}  // namespace fathom
