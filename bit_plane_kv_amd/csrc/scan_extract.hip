// Comparator scan: the same scores as the matrix-core scan, computed the way the blog's
// "Where this does not work" section describes the bit-plane scan's cost -- every bit
// extracted on the integer units (a bit-field extract and a shift-or per bit to rebuild
// each channel's code prefix), then one fp32 multiply-add per channel and query.  With P
// the channel's 4-bit value whose unread planes are zero, P = p 2^(4-t), so
//   score_g = C_g + sum over channels with t_c > 0 of fl32(q_gc s_c) * P_c,
//   C_g = sum_c q_gc (z_c + s_c h(t_c))  (fp64, rounded once).
// It exists to measure that integer work per byte on this chip; fathom_scan is the fast
// path.  One workgroup scores 2048 tokens (64 words) of one head.  Plane rows are staged
// in LDS a batch of channels at a time (256 contiguous bytes per row, 16-byte loads);
// each thread then owns byte s of word w -- 8 tokens -- and rebuilds their prefixes.
#include "common.h"

namespace fathom {
namespace {

constexpr int kExtThreads = 256;
constexpr int kExtWords = 64;        // words per workgroup tile (2048 tokens)
constexpr int kExtRowsMax = 96;      // plane rows staged at once
constexpr int kExtRowPad = kExtWords + 4;  // row stride in LDS words (16-byte aligned)

// Rebuilds P (plane j -> bit 3 - j) of one channel read to depth T for the thread's 8
// tokens and adds fl32(q s) * P to each query's sum.
template <int GP, int T>
__device__ __forceinline__ void channel_fma(const uint32_t (*words)[kExtRowPad], int o,
                                            int my_w, int my_s, const float (&a)[GP],
                                            float (&acc)[8][GP]) {
    uint32_t b[T];
#pragma unroll
    for (int j = 0; j < T; ++j) b[j] = words[o + j][my_w] >> (8 * my_s);
#pragma unroll
    for (int m = 0; m < 8; ++m) {
        uint32_t P = 0;
#pragma unroll
        for (int j = 0; j < T; ++j) P |= ((b[j] >> m) & 1u) << (3 - j);
        const float pf = (float)P;
#pragma unroll
        for (int g = 0; g < GP; ++g) acc[m][g] = fmaf(a[g], pf, acc[m][g]);
    }
}

template <int GP>
__global__ __launch_bounds__(kExtThreads) void k_scan_extract(
    const uint32_t *__restrict__ planes, int n, int word_stride, int G,
    const float *__restrict__ q, const uint8_t *__restrict__ depth,
    const float *__restrict__ scale, const float *__restrict__ zero,
    float *__restrict__ scores, int tiles_per_head) {
    __shared__ __align__(16) uint32_t words[kExtRowsMax][kExtRowPad];
    __shared__ float A[kD][GP];        // fl32(q_gc s_c)
    __shared__ int tc[kD];
    __shared__ int off[kD + 1];
    __shared__ uint16_t pl[kMaxPlanesPerHead];  // plane id (c*4 + j) of each read plane
    __shared__ double red[GP][kD];
    const int h = blockIdx.x / tiles_per_head, tile = blockIdx.x - h * tiles_per_head;
    const int tid = threadIdx.x, lane = tid & 63;
    if (tid < kD) tc[tid] = min((int)depth[(size_t)h * kD + tid], kPlanes);
    __syncthreads();
    if (tid < 64) {  // exclusive prefix sum of the depths, 2 channels a lane
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
    __syncthreads();  // off[] is complete
    if (tid < kD) {
        const int c = tid, t = tc[c];
        const float s = scale[(size_t)h * kD + c];
        const double hm = (double)((16 >> t) - 1) * 0.5;
        for (int j = 0; j < t; ++j) pl[off[c] + j] = (uint16_t)(c * kPlanes + j);
#pragma unroll
        for (int g = 0; g < GP; ++g) {
            const float qv = g < G ? q[((size_t)h * G + g) * kD + c] : 0.0f;
            A[c][g] = qv * s;
            red[g][c] = (double)qv * ((double)zero[(size_t)h * kD + c] + (double)s * hm);
        }
    }
    __syncthreads();
    for (int s2 = kD / 2; s2 > 0; s2 >>= 1) {  // C_g: fixed-order tree sum over channels
        if (tid < s2) {
#pragma unroll
            for (int g = 0; g < GP; ++g) red[g][tid] += red[g][tid + s2];
        }
        __syncthreads();
    }
    const int W = (n + 31) >> 5;
    const int w0 = tile * kExtWords;
    const uint32_t *hp = planes + (size_t)h * kMaxPlanesPerHead * word_stride;
    const int my_w = tid >> 2, my_s = tid & 3;  // this thread: byte my_s of word my_w
    float acc[8][GP];
#pragma unroll
    for (int g = 0; g < GP; ++g) {
        const float c0 = (float)red[g][0];
#pragma unroll
        for (int m = 0; m < 8; ++m) acc[m][g] = c0;
    }
    // channels in batches whose planes fit the staging area
    for (int c0 = 0; c0 < kD;) {
        int c1 = c0;
        while (c1 < kD && off[c1 + 1] - off[c0] <= kExtRowsMax) ++c1;
        const int r0 = off[c0], nr = off[c1] - r0;
        __syncthreads();  // the previous batch's words are no longer read
        // 16 lanes copy one row's 64 words
        for (int e = tid; e < nr * 16; e += kExtThreads) {
            const int r = e >> 4, v = e & 15;
            const int plane = pl[r0 + r];
            const int wv = w0 + 4 * v;
            uint4 x = make_uint4(0u, 0u, 0u, 0u);
            if (wv < word_stride)  // word_stride is a multiple of 4: the 16 bytes are in the row
                x = *reinterpret_cast<const uint4 *>(hp + (size_t)plane * word_stride + wv);
            *reinterpret_cast<uint4 *>(&words[r][4 * v]) = x;
        }
        __syncthreads();
        for (int c = c0; c < c1; ++c) {
            const int t = tc[c];
            const int o = off[c] - r0;
            float a[GP];
#pragma unroll
            for (int g = 0; g < GP; ++g) a[g] = A[c][g];
            // the channel's depth is the same for the whole workgroup: extract exactly
            // its t bits per token
            switch (t) {
            case 1: channel_fma<GP, 1>(words, o, my_w, my_s, a, acc); break;
            case 2: channel_fma<GP, 2>(words, o, my_w, my_s, a, acc); break;
            case 3: channel_fma<GP, 3>(words, o, my_w, my_s, a, acc); break;
            case 4: channel_fma<GP, 4>(words, o, my_w, my_s, a, acc); break;
            default: break;
            }
        }
        c0 = c1;
    }
    const int tok = (w0 + my_w) * 32 + 8 * my_s;
    if (w0 + my_w < W) {
#pragma unroll
        for (int g = 0; g < GP; ++g) {
            if (g >= G) break;
            float *row = scores + ((size_t)h * G + g) * n;
            if ((n & 3) == 0 && tok + 8 <= n) {
                *reinterpret_cast<float4 *>(row + tok) =
                    make_float4(acc[0][g], acc[1][g], acc[2][g], acc[3][g]);
                *reinterpret_cast<float4 *>(row + tok + 4) =
                    make_float4(acc[4][g], acc[5][g], acc[6][g], acc[7][g]);
            } else {
#pragma unroll
                for (int m = 0; m < 8; ++m)
                    if (tok + m < n) row[tok + m] = acc[m][g];
            }
        }
    }
}

template <int GP>
hipError_t launch_gp(const fathom_store &st, const float *q, int G, const uint8_t *depth,
                     float *scores, hipStream_t s) {
    const int W = (st.n_tokens + 31) >> 5;
    const int tiles = (W + kExtWords - 1) / kExtWords;
    hipLaunchKernelGGL(k_scan_extract<GP>, dim3(st.n_heads * tiles), dim3(kExtThreads), 0, s,
                       st.planes, st.n_tokens, st.word_stride, G, q, depth, st.scale, st.zero,
                       scores, tiles);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_scan_extract(const fathom_store &st, const float *q, int G,
                               const uint8_t *depth, float *scores, hipStream_t s) {
    if (G <= 1) return launch_gp<1>(st, q, G, depth, scores, s);
    if (G <= 2) return launch_gp<2>(st, q, G, depth, scores, s);
    if (G <= 4) return launch_gp<4>(st, q, G, depth, scores, s);
    return launch_gp<8>(st, q, G, depth, scores, s);
}

}  // namespace fathom
