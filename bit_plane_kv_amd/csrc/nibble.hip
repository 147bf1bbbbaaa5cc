// The plain 4-bit scan the pages measure the bit-plane scan against (blog, "Where this
// does not work": in GPU memory, extracting bits one by one costs more integer work per
// byte than reading each 4-bit number whole).  The ordinary layout is token-major, two
// channels a byte: byte j of token i = code(2j) | code(2j+1) << 4, d/2 = 64 bytes per
// token.  The scan reads every channel in full (t = 4, midpoint offset 0), so
//   score_g(i) = C_g + sum_c fl32(q_gc s_c) * code_c(i),   C_g = sum_c q_gc z_c
// (C_g in fp64 over channels in a fixed tree order, rounded once; the sum over channels
// in fp32, ascending).  It equals the bit-plane scan at B = 4d up to fp32 rounding.
#include "common.h"

namespace fathom {
namespace {

constexpr int kNibBytes = kD / 2;  // 64 bytes per token

// Planes -> nibbles.  A workgroup of 256 threads turns 4 words (128 tokens) of one head:
// thread (v, j) takes byte j of the 32 tokens of word 4*blk + v, reading the 4 planes of
// channels 2j and 2j+1, and writes one byte per token (64 consecutive threads write one
// token's 64 bytes).
__global__ __launch_bounds__(256) void k_pack_nibbles(const uint32_t *__restrict__ planes,
                                                      int n, int word_stride,
                                                      uint8_t *__restrict__ nib,
                                                      int blocks_per_head) {
    const int h = blockIdx.x / blocks_per_head, blk = blockIdx.x - h * blocks_per_head;
    const int v = threadIdx.x >> 6, j = threadIdx.x & 63;
    const int w = 4 * blk + v;
    const int W = (n + 31) >> 5;
    if (w >= W) return;
    const uint32_t *hp = planes + (size_t)h * kMaxPlanesPerHead * word_stride + w;
    uint32_t pl[2][kPlanes];
#pragma unroll
    for (int e = 0; e < 2; ++e)
#pragma unroll
        for (int p = 0; p < kPlanes; ++p)
            pl[e][p] = hp[(size_t)((2 * j + e) * kPlanes + p) * word_stride];
    uint8_t *out = nib + ((size_t)h * n + 32 * (size_t)w) * kNibBytes + j;
    const int ntok = min(32, n - 32 * w);
    for (int b = 0; b < ntok; ++b) {
        uint32_t code[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {  // plane 0 is the most significant bit
            code[e] = 0u;
#pragma unroll
            for (int p = 0; p < kPlanes; ++p) code[e] = (code[e] << 1) | ((pl[e][p] >> b) & 1u);
        }
        out[(size_t)b * kNibBytes] = (uint8_t)(code[0] | (code[1] << 4));
    }
}

// The scan.  One workgroup of 256 threads scores 512 tokens of one head, two a thread
// (tokens t and t + 256 of the block, so that stores stay coalesced).  The block's
// 32 KiB of codes are staged in LDS with coalesced 16-byte loads, one token per 17-word
// row (the odd stride keeps a wave's reads of one word of 64 tokens on distinct banks);
// then, word by word (8 channels), each thread splits its tokens' low and high nibbles
// with two masks, converts them with the byte-to-float instructions and adds
// A_gc = fl32(q_gc s_c) * code to each query's sum; A sits in LDS, read by broadcast.
constexpr int kNibTok = 512;           // tokens per workgroup
constexpr int kNibRow = kNibBytes / 4 + 1;  // LDS words per token row
template <int GP>
__global__ __launch_bounds__(256) void k_scan_nibble(
    const uint8_t *__restrict__ nib, const float *__restrict__ scale,
    const float *__restrict__ zero, int n, const float *__restrict__ q, int G,
    float *__restrict__ scores, int blocks_per_head) {
    __shared__ uint32_t tok[kNibTok * kNibRow];
    __shared__ __align__(16) float A[kD][GP];  // [channel][query]
    __shared__ double red[GP][kD];
    const int h = blockIdx.x / blocks_per_head, blk = blockIdx.x - h * blocks_per_head;
    const int tid = threadIdx.x;
    const int t0 = kNibTok * blk;  // first token of the block
    {   // stage the block's codes: 4 x 16 bytes per token, 8 a thread
        const uint4 *src = reinterpret_cast<const uint4 *>(nib + ((size_t)h * n + t0) * kNibBytes);
        uint4 v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int e = tid + 256 * u;  // 16-byte piece e: token e / 4, part e % 4
            v[u] = t0 + e / 4 < n ? src[e] : make_uint4(0u, 0u, 0u, 0u);
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int e = tid + 256 * u;
            uint32_t *row = tok + (e / 4) * kNibRow + 4 * (e % 4);
            row[0] = v[u].x;
            row[1] = v[u].y;
            row[2] = v[u].z;
            row[3] = v[u].w;
        }
    }
    if (tid < kD) {
        const int c = tid;
        const float s = scale[(size_t)h * kD + c];
        const double z = (double)zero[(size_t)h * kD + c];
#pragma unroll
        for (int g = 0; g < GP; ++g) {
            const float qv = g < G ? q[((size_t)h * G + g) * kD + c] : 0.0f;
            A[c][g] = qv * s;
            red[g][c] = (double)qv * z;
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
    float acc[2][GP];
#pragma unroll
    for (int g = 0; g < GP; ++g) acc[0][g] = acc[1][g] = (float)red[g][0];
    const uint32_t *r0 = tok + tid * kNibRow, *r1 = tok + (tid + 256) * kNibRow;
#pragma unroll 2
    for (int wd = 0; wd < kNibBytes / 4; ++wd) {  // word wd: channels 8 wd + 0..7
        const uint32_t w0 = r0[wd], w1 = r1[wd];
        const uint32_t lo[2] = {w0 & 0x0F0F0F0Fu, w1 & 0x0F0F0F0Fu};  // channels 8wd + 0,2,4,6
        const uint32_t hi[2] = {(w0 >> 4) & 0x0F0F0F0Fu, (w1 >> 4) & 0x0F0F0F0Fu};  // 1,3,5,7
#pragma unroll
        for (int b = 0; b < 4; ++b) {
#pragma unroll
            for (int odd = 0; odd < 2; ++odd) {
                const int c = 8 * wd + 2 * b + odd;  // ascending channel order
                float a[GP];
#pragma unroll
                for (int g = 0; g < GP; ++g) a[g] = A[c][g];
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    const float code = (float)(((odd ? hi[u] : lo[u]) >> (8 * b)) & 0xFFu);
#pragma unroll
                    for (int g = 0; g < GP; ++g) acc[u][g] = fmaf(a[g], code, acc[u][g]);
                }
            }
        }
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int i = t0 + tid + 256 * u;
        if (i >= n) continue;
#pragma unroll
        for (int g = 0; g < GP; ++g)
            if (g < G) scores[((size_t)h * G + g) * n + i] = acc[u][g];
    }
}

template <int GP>
void launch_gp(const uint8_t *nib, const float *scale, const float *zero, int H, int n,
               const float *q, int G, float *scores, hipStream_t s) {
    const int bph = (n + kNibTok - 1) / kNibTok;
    hipLaunchKernelGGL(k_scan_nibble<GP>, dim3(H * bph), dim3(256), 0, s, nib, scale, zero, n,
                       q, G, scores, bph);
}

}  // namespace

hipError_t launch_pack_nibbles(const fathom_store &st, uint8_t *nib, hipStream_t s) {
    const int W = (st.n_tokens + 31) / 32;
    const int bph = (W + 3) / 4;
    hipLaunchKernelGGL(k_pack_nibbles, dim3(st.n_heads * bph), dim3(256), 0, s, st.planes,
                       st.n_tokens, st.word_stride, nib, bph);
    return hipGetLastError();
}

hipError_t launch_scan_nibble(const uint8_t *nib, const float *scale, const float *zero, int H,
                              int n, const float *q, int G, float *scores, hipStream_t s) {
    if (G <= 1) launch_gp<1>(nib, scale, zero, H, n, q, G, scores, s);
    else if (G <= 2) launch_gp<2>(nib, scale, zero, H, n, q, G, scores, s);
    else if (G <= 4) launch_gp<4>(nib, scale, zero, H, n, q, G, scores, s);
    else launch_gp<8>(nib, scale, zero, H, n, q, G, scores, s);
    return hipGetLastError();
}

}  // namespace fathom
