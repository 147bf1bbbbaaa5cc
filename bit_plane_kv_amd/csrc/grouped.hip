// The grouped store: the same bit planes, with one fp16 scale and one fp16 zero per
// channel per 128-token group instead of one fp32 pair per channel -- 64 + 4 = 68 bytes
// per token per KV head, the index size the blog gives ("Where this does not work").
//
// * Build and decode-time append are one operation: (re)quantize whole groups.  A group
//   is quantized from its own tokens' min and max, so appending a token to a partial
//   group re-quantizes that group; the words of a group (4 per plane, 128 tokens) are
//   rewritten whole.  Per group and channel: s = (max - min)/15 and z = min in fp32, each
//   rounded to fp16 (nearest, ties to even); codes use the fp16 values,
//   code = clamp(floor((x - zf)/sf + 0.5), 0, 15), every step one fp32 operation.
// * The variance (the plan's importance) is recomputed from exact per-group code sums:
//   S = sum_G (n_G zf + sf S1_G), Q = sum_G (n_G zf^2 + 2 zf sf S1_G + sf^2 S2_G) in fp64
//   term by term, groups ascending, var = (n Q - S^2) / n^2 rounded once to fp32.
// * The scan reads a channel's planes to its depth as the bit-plane scan does, with each
//   group's fp16 scale and zero: score_g(i) = C_gG + sum_c fl32(q_gc sf_cG) P_c(i), P the
//   t-plane prefix times 2^(4-t), C_gG = sum_c q_gc (zf_cG + sf_cG h(t_c)) in fp64.
//   The matrix-core scan does not apply: its weights are shared by the 16 tokens of an
//   MFMA column block, which here would straddle two groups with different scales.
#include <hip/hip_fp16.h>

#include "common.h"

namespace fathom {
namespace {

constexpr int kGroup = FATHOM_GROUP;   // tokens per group: 4 words
constexpr int kGroupWords = kGroup / 32;

// One workgroup of 512 threads per (head, group): the group's keys (up to 128 tokens x
// 128 channels, 64 KiB) are staged in LDS with coalesced 16-byte loads, all in flight
// together; thread (w, c) then handles word w (32 tokens) of channel c.  The four
// words' minima and maxima are combined in token order with strict comparisons, which
// gives what one pass over the 128 tokens gives (the first of equal values is kept).
constexpr int kQThreads = kGroupWords * kD;  // 512
__global__ __launch_bounds__(kQThreads) void k_quantize_groups(
    const float *__restrict__ keys, int64_t head_stride, fathom_gstore gs, int g0) {
    __shared__ __align__(16) float tile[kGroup][kD];
    __shared__ float pmn[kGroupWords][kD], pmx[kGroupWords][kD];
    __shared__ int ps1[kGroupWords][kD], ps2[kGroupWords][kD];
    const int h = blockIdx.y, G = g0 + blockIdx.x;
    const int tid = threadIdx.x, w = tid / kD, c = tid - w * kD;
    const int n = gs.n_tokens;
    const int i0 = G * kGroup, nt = min(n, i0 + kGroup) - i0;  // tokens in the group
    // keys of this call start at token 128 g0
    const float4 *src = reinterpret_cast<const float4 *>(
        keys + (size_t)h * head_stride + (size_t)(i0 - g0 * kGroup) * kD);
    {
        constexpr int kPer = kGroup * kD / 4 / kQThreads;  // float4 loads per thread: 8
        float4 v[kPer];
        // unconditional loads (a slot past the group's tokens reads its last token's, and
        // is dropped), so that all of them are in flight together; nt >= 1
#pragma unroll
        for (int r = 0; r < kPer; ++r) {
            const int e = tid + kQThreads * r;  // float4 e: token e / 32, channels 4 (e % 32)..
            v[r] = src[min(e / (kD / 4), nt - 1) * (kD / 4) + e % (kD / 4)];
        }
#pragma unroll
        for (int r = 0; r < kPer; ++r) {
            const int e = tid + kQThreads * r;
            if (e / (kD / 4) < nt) reinterpret_cast<float4 *>(&tile[0][0])[e] = v[r];
        }
    }
    __syncthreads();
    const int nb = min(32, max(0, nt - 32 * w));  // this thread's tokens
    if (nb > 0) {
        float mn = tile[32 * w][c], mx = mn;
        for (int b = 1; b < nb; ++b) {
            const float v = tile[32 * w + b][c];
            if (v < mn) mn = v;  // plain comparisons: a -0 after a +0 keeps the +0
            if (v > mx) mx = v;
        }
        pmn[w][c] = mn;
        pmx[w][c] = mx;
    }
    __syncthreads();
    float mn = pmn[0][c], mx = pmx[0][c];
    for (int u = 1; u < kGroupWords && 32 * u < nt; ++u) {  // words in token order
        if (pmn[u][c] < mn) mn = pmn[u][c];
        if (pmx[u][c] > mx) mx = pmx[u][c];
    }
    const float range = mx - mn;
    const __half sh = __float2half_rn(range / 15.0f);
    const __half zh = __float2half_rn(mn);
    const float sf = __half2float(sh), zf = __half2float(zh);
    uint32_t word[kPlanes] = {0u, 0u, 0u, 0u};
    int s1 = 0, s2 = 0;
    for (int b = 0; b < nb; ++b) {
        uint32_t code = 0u;
        if (sf != 0.0f) {
            const float diff = tile[32 * w + b][c] - zf;
            const float u = diff / sf;
            const float r = u + 0.5f;
            const float f = fminf(fmaxf(floorf(r), 0.0f), 15.0f);
            code = (uint32_t)f;
        }
        s1 += (int)code;
        s2 += (int)(code * code);
#pragma unroll
        for (int j = 0; j < kPlanes; ++j) word[j] |= ((code >> (3 - j)) & 1u) << b;
    }
    uint32_t *prow = gs.planes + ((size_t)h * kD + c) * kPlanes * gs.word_stride;
#pragma unroll
    for (int j = 0; j < kPlanes; ++j) prow[(size_t)j * gs.word_stride + kGroupWords * G + w] = word[j];
    ps1[w][c] = s1;
    ps2[w][c] = s2;
    __syncthreads();
    if (w == 0) {
        const size_t t = ((size_t)h * kD + c) * gs.group_stride + G;
        gs.scale16[t] = __half_as_ushort(sh);
        gs.zero16[t] = __half_as_ushort(zh);
        gs.sums[2 * t] = ps1[0][c] + ps1[1][c] + ps1[2][c] + ps1[3][c];
        gs.sums[2 * t + 1] = ps2[0][c] + ps2[1][c] + ps2[2][c] + ps2[3][c];
    }
}

// Variance of every channel from its groups' code sums; one thread per (head, channel)
// sums the groups in ascending order (the order fixes the fp64 rounding).  The running
// sums over groups [0, P) are kept in prefix; when this call changed no group below P
// (P <= g0) the thread resumes from them, so an append adds one or two groups and the
// result equals the sum from group 0 bit for bit.  The prefix kept afterwards covers all
// groups but the last (the one a decode-time append changes).
__global__ __launch_bounds__(kD) void k_var_groups(fathom_gstore gs, int g0) {
    const int h = blockIdx.x, c = threadIdx.x;
    const int n = gs.n_tokens, ng = (n + kGroup - 1) / kGroup;
    const size_t hc = (size_t)h * kD + c, base = hc * gs.group_stride;
    int P = gs.prefix_groups[hc];
    double S = 0.0, Q = 0.0;
    if (P > 0 && P <= g0 && P < ng) {
        S = gs.prefix[2 * hc];
        Q = gs.prefix[2 * hc + 1];
    } else {
        P = 0;
    }
    for (int G = P; G < ng; ++G) {
        if (G == ng - 1 && G > 0 && G != P) {  // the sums before the last group
            gs.prefix[2 * hc] = S;
            gs.prefix[2 * hc + 1] = Q;
            gs.prefix_groups[hc] = G;
        }
        const double zf = (double)__half2float(__ushort_as_half(gs.zero16[base + G]));
        const double sf = (double)__half2float(__ushort_as_half(gs.scale16[base + G]));
        const int2 s12 = *reinterpret_cast<const int2 *>(gs.sums + 2 * (base + G));
        const double s1 = (double)s12.x, s2 = (double)s12.y;
        const double nG = (double)(min(n, (G + 1) * kGroup) - G * kGroup);
        S = S + nG * zf;
        S = S + sf * s1;
        Q = Q + nG * (zf * zf);
        Q = Q + 2.0 * zf * sf * s1;
        Q = Q + (sf * sf) * s2;
    }
    const double nn = (double)n;
    gs.var[hc] = (float)((nn * Q - S * S) / (nn * nn));
}

// ---------------------------------------------------------------------------------
// scan: one workgroup of 256 threads per 2048 tokens (64 words, 16 groups) of a head;
// channel rows staged in LDS a batch at a time; thread (w, s) owns byte s of word w,
// i.e. 8 tokens of group w / 4.
// ---------------------------------------------------------------------------------
constexpr int kGThreads = 256;
constexpr int kGWords = 64;
constexpr int kGGroups = kGWords / kGroupWords;  // 16
constexpr int kGRowsMax = 96;
constexpr int kGRowPad = kGWords + 4;

template <int GP>
__global__ __launch_bounds__(kGThreads) void k_scan_grouped(
    fathom_gstore gs, const float *__restrict__ q, const uint8_t *__restrict__ depth, int G,
    float *__restrict__ scores, int tiles_per_head) {
    __shared__ __align__(16) uint32_t words[kGRowsMax][kGRowPad];
    __shared__ float qs[GP][kD];
    __shared__ __half sgrp[kD][kGGroups];
    __shared__ __half zgrp[kD][kGGroups];
    __shared__ float cg[kGGroups][GP];
    __shared__ int tc[kD];
    __shared__ int off[kD + 1];
    __shared__ uint16_t pl[kMaxPlanesPerHead];
    const int h = blockIdx.x / tiles_per_head, tile = blockIdx.x - h * tiles_per_head;
    const int tid = threadIdx.x, lane = tid & 63;
    const int n = gs.n_tokens, W = (n + 31) >> 5;
    const int ng = (n + kGroup - 1) / kGroup;
    const int w0 = tile * kGWords, gb = w0 / kGroupWords;  // first word, first group
    // Every input load is unconditional (indices clamped into the head's tables) and
    // issued before any is used, so that they are all in flight together.
    constexpr int kQPer = (GP * kD + kGThreads - 1) / kGThreads;
    constexpr int kSPer = kD * kGGroups / kGThreads;  // 8
    const int tdep = depth[(size_t)h * kD + min(tid, kD - 1)];
    float qv[kQPer];
#pragma unroll
    for (int u = 0; u < kQPer; ++u) {
        const int e = min(tid + kGThreads * u, GP * kD - 1), g = e / kD, c = e - g * kD;
        qv[u] = q[((size_t)h * G + min(g, G - 1)) * kD + c];
    }
    uint16_t sv[kSPer], zv[kSPer];
#pragma unroll
    for (int u = 0; u < kSPer; ++u) {
        const int e = tid + kGThreads * u, c = e / kGGroups, gg = e - c * kGGroups;
        const size_t t = ((size_t)h * kD + c) * gs.group_stride + min(gb + gg, ng - 1);
        sv[u] = gs.scale16[t];
        zv[u] = gs.zero16[t];
    }
    if (tid < kD) tc[tid] = min(tdep, kPlanes);
#pragma unroll
    for (int u = 0; u < kQPer; ++u) {
        const int e = tid + kGThreads * u, g = e / kD, c = e - g * kD;
        if (e < GP * kD) qs[g][c] = g < G ? qv[u] : 0.0f;
    }
#pragma unroll
    for (int u = 0; u < kSPer; ++u) {
        const int e = tid + kGThreads * u, c = e / kGGroups, gg = e - c * kGGroups;
        sgrp[c][gg] = __ushort_as_half(sv[u]);
        zgrp[c][gg] = __ushort_as_half(zv[u]);
    }
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
    // C per (group, query): fp64 over channels ascending
    if (tid < kGGroups * GP) {
        const int gg = tid / GP, g = tid - gg * GP;
        double acc = 0.0;
        for (int c = 0; c < kD; ++c) {
            const double zf = (double)__half2float(zgrp[c][gg]);
            const double sf = (double)__half2float(sgrp[c][gg]);
            const double hm = (double)((16 >> tc[c]) - 1) * 0.5;
            acc += (double)qs[g][c] * (zf + sf * hm);
        }
        cg[gg][g] = (float)acc;
    }
    __syncthreads();
    if (tid < kD) {
        const int c = tid, t = tc[c];
        for (int j = 0; j < t; ++j) pl[off[c] + j] = (uint16_t)(c * kPlanes + j);
    }
    __syncthreads();
    const uint32_t *hp = gs.planes + (size_t)h * kMaxPlanesPerHead * gs.word_stride;
    const int my_w = tid >> 2, my_s = tid & 3;
    const int my_g = my_w / kGroupWords;  // group within the tile
    float acc[8][GP];
#pragma unroll
    for (int g = 0; g < GP; ++g) {
        const float c0 = cg[my_g][g];
#pragma unroll
        for (int m = 0; m < 8; ++m) acc[m][g] = c0;
    }
    for (int c0 = 0; c0 < kD;) {
        int c1 = c0;
        while (c1 < kD && off[c1 + 1] - off[c0] <= kGRowsMax) ++c1;
        const int r0 = off[c0], nr = off[c1] - r0;
        __syncthreads();  // the previous batch's words are no longer read
        if (nr > 0) {  // pl holds the batch's rows only when it has any (all depths 0:
                       // no row, no load)
            // the batch's rows, 16 bytes a load, all loads unconditional and in flight
            // together (a slot past the batch reads its last row, one past the row the
            // row's first 16 bytes, and is dropped)
            constexpr int kBPer = kGRowsMax * 16 / kGThreads;  // 6
            uint4 x[kBPer];
#pragma unroll
            for (int u = 0; u < kBPer; ++u) {
                const int e = tid + kGThreads * u, r = e >> 4, v = e & 15;
                const int wv = w0 + 4 * v;  // word_stride is a multiple of 4
                const int row = pl[r0 + min(r, nr - 1)];
                x[u] = *reinterpret_cast<const uint4 *>(hp + (size_t)row * gs.word_stride +
                                                        (wv < gs.word_stride ? wv : 0));
            }
#pragma unroll
            for (int u = 0; u < kBPer; ++u) {
                const int e = tid + kGThreads * u, r = e >> 4, v = e & 15;
                if (r < nr)
                    *reinterpret_cast<uint4 *>(&words[r][4 * v]) =
                        w0 + 4 * v < gs.word_stride ? x[u] : make_uint4(0u, 0u, 0u, 0u);
            }
        }
        __syncthreads();
        for (int c = c0; c < c1; ++c) {
            const int t = tc[c];
            if (t == 0) continue;
            const int o = off[c] - r0;
            const float sf = __half2float(sgrp[c][my_g]);
            float a[GP];
#pragma unroll
            for (int g = 0; g < GP; ++g) a[g] = qs[g][c] * sf;
            uint32_t b[kPlanes];
#pragma unroll
            for (int j = 0; j < kPlanes; ++j) {
                b[j] = 0u;
                if (j < t) b[j] = words[o + j][my_w] >> (8 * my_s);
            }
#pragma unroll
            for (int m = 0; m < 8; ++m) {
                uint32_t P = 0;
#pragma unroll
                for (int j = 0; j < kPlanes; ++j) P |= ((b[j] >> m) & 1u) << (3 - j);
                const float pf = (float)P;
#pragma unroll
                for (int g = 0; g < GP; ++g) acc[m][g] = fmaf(a[g], pf, acc[m][g]);
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
#pragma unroll
            for (int m = 0; m < 8; ++m)
                if (tok + m < n) row[tok + m] = acc[m][g];
        }
    }
}

template <int GP>
void launch_scan_gp(const fathom_gstore &gs, const float *q, const uint8_t *depth, int G,
                    float *scores, hipStream_t s) {
    const int W = (gs.n_tokens + 31) >> 5;
    const int tiles = (W + kGWords - 1) / kGWords;
    hipLaunchKernelGGL(k_scan_grouped<GP>, dim3(gs.n_heads * tiles), dim3(kGThreads), 0, s, gs,
                       q, depth, G, scores, tiles);
}

}  // namespace

hipError_t launch_quantize_groups(const float *keys, int64_t head_stride,
                                  const fathom_gstore &gs, int g0, int g1, hipStream_t s) {
    hipLaunchKernelGGL(k_quantize_groups, dim3(g1 - g0, gs.n_heads), dim3(kQThreads), 0, s,
                       keys, head_stride, gs, g0);
    hipLaunchKernelGGL(k_var_groups, dim3(gs.n_heads), dim3(kD), 0, s, gs, g0);
    return hipGetLastError();
}

hipError_t launch_scan_grouped(const fathom_gstore &gs, const float *q, const uint8_t *depth,
                               int G, float *scores, hipStream_t s) {
    if (G <= 1) launch_scan_gp<1>(gs, q, depth, G, scores, s);
    else if (G <= 2) launch_scan_gp<2>(gs, q, depth, G, scores, s);
    else if (G <= 4) launch_scan_gp<4>(gs, q, depth, G, scores, s);
    else launch_scan_gp<8>(gs, q, depth, G, scores, s);
    return hipGetLastError();
}

}  // namespace fathom
