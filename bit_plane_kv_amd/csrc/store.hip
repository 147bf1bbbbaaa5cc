// Store build: 4-bit per-channel quantization, MSB-first bit-plane packing with wave
// ballots, and the dequantized channel variance from exact integer code sums.
//
// Sources: the blog's "How to read fewer bits per key" (4-bit storage) and "Bit planes:
// how a partial read becomes a valid read" (plane 0 = most significant bit of every
// number, storage transposed channel-major); the Glonce summary (4-bit per-channel K
// cache stored as bit planes; variance-weighted importance).
#include "common.h"

namespace fathom {
namespace {

// ---- kernel A: min/max of each channel over a chunk of tokens --------------------
// keys [H][n][128]; partial [H][nchunk][2][128]
__global__ __launch_bounds__(256) void k_minmax_partial(const float *__restrict__ keys,
                                                        int n, int nchunk,
                                                        float *__restrict__ partial) {
    const int h = blockIdx.y, chunk = blockIdx.x;
    const int c = threadIdx.x & (kD - 1), sub = threadIdx.x >> 7;
    const int i0 = chunk * kMinMaxTokens;
    const int i1 = min(n, i0 + kMinMaxTokens);
    const float *base = keys + (size_t)h * n * kD + c;
    float mn = INFINITY, mx = -INFINITY;
    for (int i = i0 + sub; i < i1; i += 2) {
        float v = base[(size_t)i * kD];
        mn = fminf(mn, v);
        mx = fmaxf(mx, v);
    }
    __shared__ float smn[256], smx[256];
    smn[threadIdx.x] = mn;
    smx[threadIdx.x] = mx;
    __syncthreads();
    if (sub == 0) {
        mn = fminf(mn, smn[threadIdx.x + kD]);
        mx = fmaxf(mx, smx[threadIdx.x + kD]);
        float *out = partial + ((size_t)h * nchunk + chunk) * 2 * kD;
        out[c] = mn;
        out[kD + c] = mx;
    }
}

// ---- kernel B: s = (max - min)/15 and z = min per channel; clear the sums --------
__global__ __launch_bounds__(128) void k_minmax_final(const float *__restrict__ partial,
                                                      int nchunk, float *__restrict__ scale,
                                                      float *__restrict__ zero,
                                                      uint64_t *__restrict__ sums) {
    const int h = blockIdx.x, c = threadIdx.x;
    const float *p = partial + (size_t)h * nchunk * 2 * kD;
    float mn = p[c], mx = p[kD + c];
    for (int ch = 1; ch < nchunk; ++ch) {
        mn = fminf(mn, p[(size_t)ch * 2 * kD + c]);
        mx = fmaxf(mx, p[(size_t)ch * 2 * kD + kD + c]);
    }
    const float range = mx - mn;   // one fp32 subtraction
    const float s = range / 15.0f; // one correctly rounded fp32 division
    scale[(size_t)h * kD + c] = s;
    zero[(size_t)h * kD + c] = mn;
    sums[((size_t)h * kD + c) * 2 + 0] = 0;
    sums[((size_t)h * kD + c) * 2 + 1] = 0;
}

// ---- kernel C: quantize, ballot-pack the planes, accumulate integer code sums ----
// One workgroup = 4 waves = one 64-token tile at a time (wave w owns channels
// 32w .. 32w+31, lane = token).  Keys are staged through LDS so that global reads are
// coalesced rows; each (channel, plane) ballot yields two 32-token words.
constexpr int kQTileTokens = 64;
constexpr int kQTilesPerBlock = 8;  // 512 tokens per workgroup

__global__ __launch_bounds__(256) void k_quantize_pack(
    const float *__restrict__ keys, int n, const float *__restrict__ scale,
    const float *__restrict__ zero, uint32_t *__restrict__ planes, int word_stride,
    uint64_t *__restrict__ sums) {
    __shared__ float tile[kQTileTokens][kD + 1];
    const int h = blockIdx.y;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int W = (n + 31) >> 5;
    const float *kh = keys + (size_t)h * n * kD;
    uint32_t *ph = planes + (size_t)h * kD * kPlanes * word_stride;

    // this lane's channel parameters for the channels its wave owns (lane & 31)
    const int my_c = wave * 32 + (lane & 31);
    uint64_t acc1 = 0, acc2 = 0;

    for (int t = 0; t < kQTilesPerBlock; ++t) {
        const int tok0 = (blockIdx.x * kQTilesPerBlock + t) * kQTileTokens;
        if (tok0 >= n) break;
        __syncthreads();
        // cooperative coalesced load of [64 tokens][128 ch]
        for (int e = tid; e < kQTileTokens * kD; e += 256) {
            const int r = e >> 7, c = e & (kD - 1);
            const int i = tok0 + r;
            tile[r][c] = (i < n) ? kh[(size_t)i * kD + c] : 0.0f;
        }
        __syncthreads();
        const int i = tok0 + lane;
        const bool valid = i < n;
        const int w0 = tok0 >> 5;  // first of the two words this tile fills
        for (int cc = 0; cc < 32; ++cc) {
            const int c = wave * 32 + cc;
            const float s = scale[(size_t)h * kD + c];
            const float z = zero[(size_t)h * kD + c];
            uint32_t code = 0;
            if (s != 0.0f) {
                const float diff = tile[lane][c] - z;  // each step one fp32 operation
                const float u = diff / s;
                const float r = u + 0.5f;
                float f = floorf(r);
                f = fminf(fmaxf(f, 0.0f), 15.0f);
                code = (uint32_t)f;
            }
            uint64_t b[kPlanes];
#pragma unroll
            for (int j = 0; j < kPlanes; ++j)
                b[j] = __ballot(valid && ((code >> (3 - j)) & 1u));
            // exact code sums from the ballots: sum code = sum_j 2^(3-j) popc(b_j),
            // sum code^2 = sum_{j,j'} 2^(6-j-j') popc(b_j & b_j')
            uint64_t s1 = 0, s2 = 0;
#pragma unroll
            for (int j = 0; j < kPlanes; ++j) {
                s1 += (uint64_t)__popcll(b[j]) << (3 - j);
#pragma unroll
                for (int jj = 0; jj < kPlanes; ++jj)
                    s2 += (uint64_t)__popcll(b[j] & b[jj]) << (6 - j - jj);
            }
            if ((lane & 31) == cc) {
                acc1 += s1;
                acc2 += s2;
            }
            // lanes 0..7 store the 8 words: lane -> plane lane>>1, word w0 + (lane&1)
            if (lane < 8) {
                const int j = lane >> 1, half = lane & 1;
                const int w = w0 + half;
                uint64_t bj = b[0];
                if (j == 1) bj = b[1];
                if (j == 2) bj = b[2];
                if (j == 3) bj = b[3];
                if (w < W)
                    ph[((size_t)c * kPlanes + j) * word_stride + w] =
                        half ? (uint32_t)(bj >> 32) : (uint32_t)bj;
            }
        }
    }
    if (lane < 32) {
        atomicAdd((unsigned long long *)&sums[((size_t)h * kD + my_c) * 2 + 0],
                  (unsigned long long)acc1);
        atomicAdd((unsigned long long *)&sums[((size_t)h * kD + my_c) * 2 + 1],
                  (unsigned long long)acc2);
    }
}

// ---- kernel D: zero the words from ceil(n/32) up to word_stride ------------------
__global__ __launch_bounds__(256) void k_zero_tail(uint32_t *__restrict__ planes, int W,
                                                   int word_stride, size_t rows) {
    const int extra = word_stride - W;
    const size_t total = rows * (size_t)extra;
    for (size_t e = (size_t)blockIdx.x * 256 + threadIdx.x; e < total;
         e += (size_t)gridDim.x * 256) {
        const size_t r = e / extra, w = W + e % extra;
        planes[r * word_stride + w] = 0u;
    }
}

// ---- kernel E: var = s^2 (n S2 - S1^2) / n^2 in fp64, rounded once ---------------
__global__ __launch_bounds__(128) void k_var_final(const uint64_t *__restrict__ sums,
                                                   const float *__restrict__ scale, int n,
                                                   float *__restrict__ var) {
    const size_t hc = (size_t)blockIdx.x * kD + threadIdx.x;
    const int64_t s1 = (int64_t)sums[hc * 2 + 0];
    const int64_t s2 = (int64_t)sums[hc * 2 + 1];
    const int64_t num = (int64_t)n * s2 - s1 * s1;
    const double s = (double)scale[hc];
    const double v = (s * s) * (double)num / ((double)n * (double)n);
    var[hc] = (float)v;
}

}  // namespace

hipError_t launch_quantize_store(const float *keys, int H, int n, const fathom_store &st,
                                 void *ws, hipStream_t s) {
    const int nchunk = minmax_chunks(n);
    float *partial = static_cast<float *>(ws);
    size_t mm = (size_t)H * nchunk * 2 * kD * sizeof(float);
    mm = (mm + 255) / 256 * 256;
    uint64_t *sums = reinterpret_cast<uint64_t *>(static_cast<char *>(ws) + mm);

    hipLaunchKernelGGL(k_minmax_partial, dim3(nchunk, H), dim3(256), 0, s, keys, n, nchunk,
                       partial);
    hipLaunchKernelGGL(k_minmax_final, dim3(H), dim3(kD), 0, s, partial, nchunk, st.scale,
                       st.zero, sums);
    const int tokens_per_block = kQTileTokens * kQTilesPerBlock;
    const int nblk = (n + tokens_per_block - 1) / tokens_per_block;
    hipLaunchKernelGGL(k_quantize_pack, dim3(nblk, H), dim3(256), 0, s, keys, n, st.scale,
                       st.zero, st.planes, st.word_stride, sums);
    const int W = (n + 31) >> 5;
    if (st.word_stride > W) {
        const size_t rows = (size_t)H * kD * kPlanes;
        const size_t total = rows * (size_t)(st.word_stride - W);
        const int grid = (int)std::min<size_t>((total + 255) / 256, 65536);
        hipLaunchKernelGGL(k_zero_tail, dim3(grid), dim3(256), 0, s, st.planes, W,
                           st.word_stride, rows);
    }
    hipLaunchKernelGGL(k_var_final, dim3(H), dim3(kD), 0, s, sums, st.scale, n, st.var);
    return hipGetLastError();
}

}  // namespace fathom
