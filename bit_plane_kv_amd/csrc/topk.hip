// Top-k select: the k largest scores of each row, equal scores to the lower token index,
// output ascending by index (blog, "The first fix": score every key, take the top k).
//
// One 1024-thread workgroup ranks one chunk of up to 32768 entries held in registers
// (32 consecutive positions per thread).  Radix select on order-preserving 32-bit keys
// (12 + 12 + 8 bit digits, LDS histograms) finds the k-th largest key T and how many
// entries equal to T are needed; a block-wide scan of (greater, equal) counts in
// position order then writes the winners in index order, taking the equal entries with
// the lowest positions.  Rows longer than a chunk are cut into chunks whose top
// min(k, chunk) survive as (value, index) candidates, in index order, for the next
// level, until one chunk remains.
#include "common.h"

namespace fathom {

TopkLevels topk_levels(int n, int k) {
    TopkLevels L{};
    int64_t count = n;
    const int64_t kk = std::min<int64_t>(k, kTopkChunk);
    while (count > kTopkChunk && L.n_levels < 8) {
        const int64_t nch = (count + kTopkChunk - 1) / kTopkChunk;
        count = (nch - 1) * kk + std::min<int64_t>(kk, count - (nch - 1) * kTopkChunk);
        L.count[L.n_levels++] = count;
    }
    return L;
}

// candidate buffers: per level, R rows of (stride = nchunks * kk) floats + int32
static int64_t level_stride(int64_t count_in, int k) {
    const int64_t nch = (count_in + kTopkChunk - 1) / kTopkChunk;
    return nch * std::min<int64_t>(k, kTopkChunk);
}

size_t topk_ws_bytes(int R, int n, int k) {
    const TopkLevels L = topk_levels(n, k);
    if (L.n_levels == 0) return 0;
    int64_t maxs = 0, cin = n;
    for (int l = 0; l < L.n_levels; ++l) {
        maxs = std::max(maxs, level_stride(cin, k));
        cin = L.count[l];
    }
    const size_t one = ((size_t)R * maxs * 8 + 255) / 256 * 256;
    return L.n_levels >= 2 ? 2 * one : one;
}

namespace {

constexpr int kThreads = 1024;
constexpr int kEPT = kTopkChunk / kThreads;  // 32

__device__ __forceinline__ uint32_t order_key(float v) {
    uint32_t u = __float_as_uint(v);
    if (u == 0x80000000u) u = 0u;  // -0 ranks as +0
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float key_value(uint32_t key) {
    return __uint_as_float((key & 0x80000000u) ? (key ^ 0x80000000u) : ~key);
}

__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v, int lane) {
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const uint32_t t = __shfl_up(v, o, 64);
        if (lane >= o) v += t;
    }
    return v;
}

// Exclusive prefix sum over the 1024 threads in thread order; *total = block sum.
__device__ uint32_t block_excl_scan(uint32_t v, uint32_t *sh, uint32_t *total) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const uint32_t inc = wave_incl_scan(v, lane);
    if (lane == 63) sh[wave] = inc;
    __syncthreads();
    if (wave == 0) {
        const uint32_t x = lane < 16 ? sh[lane] : 0u;
        const uint32_t xi = wave_incl_scan(x, lane);
        if (lane < 16) sh[lane] = xi - x;
        if (lane == 15) sh[16] = xi;
    }
    __syncthreads();
    const uint32_t r = sh[wave] + inc - v;
    *total = sh[16];
    __syncthreads();
    return r;
}

// One radix step over a set of keys: histogram of digit (key >> sh) & (nb - 1) of the
// keys whose top bits equal `prefix` (all keys when `all`), then find the bin holding
// the need-th largest.  Returns (via pick) the bin, the count above it and its count.
__device__ __forceinline__ void find_bin(uint32_t *hist, uint32_t *scan_sh, uint32_t *pick,
                                         int nb, uint32_t need) {
    const int tid = threadIdx.x;
    uint32_t c4[4];
    uint32_t local = 0u;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int b = nb - 1 - (4 * tid + e);  // thread t owns 4 bins, highest first
        c4[e] = b >= 0 ? hist[b] : 0u;
        local += c4[e];
    }
    uint32_t total;
    const uint32_t above = block_excl_scan(local, scan_sh, &total);
    if (above < need && need <= above + local) {
        uint32_t cum = above;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            if (cum < need && need <= cum + c4[e]) {
                pick[0] = (uint32_t)(nb - 1 - (4 * tid + e));
                pick[1] = cum;
                pick[2] = c4[e];
            }
            cum += c4[e];
        }
    }
    __syncthreads();
}

constexpr int kCandCap = 4096;  // threshold-bin entries refined in LDS

// kExplicit: input entries carry their own int32 index (candidate levels); otherwise
// the index is the position in the row.  kCandOut: write (value, index) candidates
// (at column chunk*kk of the output row) instead of final indices.
template <bool kExplicit, bool kCandOut>
__global__ __launch_bounds__(kThreads, 8) void k_topk_chunk(
    const float *__restrict__ vals, const int32_t *__restrict__ in_idx, int64_t row_len,
    int64_t in_stride, int row0, int k, float *__restrict__ out_val,
    int32_t *__restrict__ out_idx, int64_t out_stride) {
    __shared__ uint32_t hist[4096];
    __shared__ uint32_t cand[kCandCap];
    __shared__ uint32_t scan_sh[17];
    __shared__ uint32_t pick[3];
    __shared__ uint32_t ncand;
    const int tid = threadIdx.x;
    const int chunk = blockIdx.x;
    const int64_t row = (int64_t)row0 + blockIdx.y;
    const int64_t start = (int64_t)chunk * kTopkChunk;
    const int len = (int)min((int64_t)kTopkChunk, row_len - start);
    const int kr = min(k, len);
    const float *v = vals + row * in_stride + start;
    const int p0 = tid * kEPT;  // this thread's positions p0 .. p0+31
    const int nvalid = max(0, min(kEPT, len - p0));
    const uint32_t vmask = nvalid >= 32 ? 0xFFFFFFFFu : ((1u << nvalid) - 1u);

    uint32_t key[kEPT];
    if (((((uintptr_t)(v + p0)) & 15u) == 0) && nvalid == kEPT) {
#pragma unroll
        for (int e = 0; e < kEPT; e += 4) {
            const float4 f = *reinterpret_cast<const float4 *>(v + p0 + e);
            key[e] = order_key(f.x);
            key[e + 1] = order_key(f.y);
            key[e + 2] = order_key(f.z);
            key[e + 3] = order_key(f.w);
        }
    } else {
#pragma unroll
        for (int e = 0; e < kEPT; ++e) key[e] = e < nvalid ? order_key(v[p0 + e]) : 0u;
    }

    // ---- pass 1: top 12 bits of every key
    for (int b = tid; b < 4096; b += kThreads) hist[b] = 0u;
    if (tid == 0) ncand = 0u;
    __syncthreads();
    if (nvalid == kEPT) {
#pragma unroll
        for (int e = 0; e < kEPT; ++e) atomicAdd(&hist[key[e] >> 20], 1u);
    } else {
#pragma unroll
        for (int e = 0; e < kEPT; ++e)
            if (e < nvalid) atomicAdd(&hist[key[e] >> 20], 1u);
    }
    __syncthreads();
    find_bin(hist, scan_sh, pick, 4096, (uint32_t)kr);
    uint32_t prefix = pick[0];
    uint32_t need = (uint32_t)kr - pick[1];
    uint32_t in_bin = pick[2];
    int shift = 20;

    if (in_bin != need) {
        // The k-th largest key lies inside bin `prefix`; refine on its in_bin entries.
        const bool in_lds = in_bin <= (uint32_t)kCandCap;
        const int ncands = (int)in_bin;  // entries of the first bin (the list's length)
        if (in_lds) {  // compact the bin's keys into LDS (any order)
#pragma unroll
            for (int e = 0; e < kEPT; ++e) {
                if (((vmask >> e) & 1u) && (key[e] >> 20) == prefix)
                    cand[atomicAdd(&ncand, 1u)] = key[e];
            }
        }
        for (int pass = 1; pass < 3; ++pass) {
            const int sh = pass == 1 ? 8 : 0;
            const int nb = pass == 1 ? 4096 : 256;
            __syncthreads();  // previous readers of hist / pick are done
            for (int b = tid; b < 4096; b += kThreads) hist[b] = 0u;
            __syncthreads();
            if (in_lds) {
                for (int c = tid; c < ncands; c += kThreads) {
                    const uint32_t kv = cand[c];
                    if ((kv >> shift) == prefix) atomicAdd(&hist[(kv >> sh) & (nb - 1)], 1u);
                }
            } else {
#pragma unroll
                for (int e = 0; e < kEPT; ++e) {
                    if (((vmask >> e) & 1u) && (key[e] >> shift) == prefix)
                        atomicAdd(&hist[(key[e] >> sh) & (nb - 1)], 1u);
                }
            }
            __syncthreads();
            find_bin(hist, scan_sh, pick, nb, need);
            prefix = (prefix << (pass == 1 ? 12 : 8)) | pick[0];
            shift = sh;
            need -= pick[1];
            in_bin = pick[2];
            if (in_bin == need) break;  // every entry of the bin is a winner
        }
    }

    // ---- ordered output: greater entries all win; of the entries equal to the
    //      threshold prefix, the `need` lowest positions win.  Masks over the thread's
    //      32 positions, one packed scan, then the set bits in ascending order.
    uint32_t mgt = 0u, meq = 0u;
#pragma unroll
    for (int e = 0; e < kEPT; ++e) {
        const uint32_t kv = key[e] >> shift;
        mgt |= (uint32_t)(kv > prefix) << e;
        meq |= (uint32_t)(kv == prefix) << e;
    }
    mgt &= vmask;
    meq &= vmask;
    uint32_t total;
    const uint32_t before =
        block_excl_scan((uint32_t)__popc(mgt) | ((uint32_t)__popc(meq) << 16), scan_sh, &total);
    const uint32_t gtb = before & 0xFFFFu, eqb = before >> 16;
    const uint32_t r = need;
    // Equal entries of earlier threads that win, and this thread's that still win (the
    // lowest `take` bits of meq).  Written as a clamp followed by a subtraction that
    // cannot wrap: the form "eqb < r ? r - eqb : 0" was compiled (hipcc 7.2) into an
    // unconditional no-wrap subtraction, from which the clamp below was folded away.
    const uint32_t eq_won_before = min(eqb, r);
    const uint32_t eq_left = r - eq_won_before;
    uint32_t take = min(eq_left, (uint32_t)__popc(meq));
    uint32_t sel = mgt, m = meq;
    while (take > 0u) {
        const uint32_t low = m & (0u - m);
        sel |= low;
        m ^= low;
        --take;
    }
    int slot = (int)(gtb + eq_won_before);
    const int32_t *vi = kExplicit ? in_idx + row * in_stride + start : nullptr;
    while (sel != 0u) {
        const int e = __ffs(sel) - 1;
        sel &= sel - 1u;
        if (slot < kr) {
            const int p = p0 + e;
            const int32_t index = kExplicit ? vi[p] : (int32_t)(start + p);
            if (kCandOut) {
                const int64_t o =
                    row * out_stride + (int64_t)chunk * min(k, kTopkChunk) + slot;
                out_val[o] = key_value(key[e]);  // dynamic index: the key is re-read
                out_idx[o] = index;
            } else {
                out_idx[row * (int64_t)k + slot] = index;
            }
        }
        ++slot;
    }
}

template <bool kExplicit, bool kCandOut>
void launch_level(const float *vals, const int32_t *in_idx, int64_t len, int64_t in_stride,
                  int R, int k, float *out_val, int32_t *out_idx, int64_t out_stride,
                  hipStream_t s) {
    const int nch = (int)((len + kTopkChunk - 1) / kTopkChunk);
    for (int r0 = 0; r0 < R; r0 += 65535) {
        const int rows = std::min(65535, R - r0);
        hipLaunchKernelGGL((k_topk_chunk<kExplicit, kCandOut>), dim3(nch, rows),
                           dim3(kThreads), 0, s, vals, in_idx, len, in_stride, r0, k,
                           out_val, out_idx, out_stride);
    }
}

}  // namespace

hipError_t launch_topk(const float *scores, int R, int n, int k, int32_t *idx, void *ws,
                       hipStream_t s) {
    const TopkLevels L = topk_levels(n, k);
    if (L.n_levels == 0) {
        launch_level<false, false>(scores, nullptr, n, n, R, k, nullptr, idx, 0, s);
        return hipGetLastError();
    }
    const size_t one = topk_ws_bytes(R, n, k) / (L.n_levels >= 2 ? 2 : 1);
    char *buf[2] = {static_cast<char *>(ws), static_cast<char *>(ws) + one};
    int64_t cin = n, in_stride = n;
    const float *in_val = scores;
    const int32_t *in_i = nullptr;
    for (int l = 0; l < L.n_levels; ++l) {
        const int64_t os = level_stride(cin, k);
        float *ov = reinterpret_cast<float *>(buf[l & 1]);
        int32_t *oi = reinterpret_cast<int32_t *>(buf[l & 1] + (size_t)R * os * 4);
        if (l == 0)
            launch_level<false, true>(in_val, nullptr, cin, in_stride, R, k, ov, oi, os, s);
        else
            launch_level<true, true>(in_val, in_i, cin, in_stride, R, k, ov, oi, os, s);
        in_val = ov;
        in_i = oi;
        in_stride = os;
        cin = L.count[l];
    }
    launch_level<true, false>(in_val, in_i, cin, in_stride, R, k, nullptr, idx, 0, s);
    return hipGetLastError();
}

}  // namespace fathom
