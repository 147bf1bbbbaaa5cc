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
//   t-plane prefix times 2^(4-t), C_gG = sum_c q_gc (zf_cG + sf_cG h(t_c)) in fp64.  It
//   runs on the int8 matrix cores like the per-channel scan, with weights rebuilt for
//   every group and MFMA column blocks that never straddle two groups (below).
#include <hip/hip_fp16.h>

#include "common.h"
#include "scan_device.h"

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
        // rows past the group's tokens get the copies (they are never read: every read
        // below stays below the thread's own token count)
#pragma unroll
        for (int r = 0; r < kPer; ++r)
            reinterpret_cast<float4 *>(&tile[0][0])[tid + kQThreads * r] = v[r];
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
        const size_t tg = ((size_t)h * gs.group_stride + G) * kD + c;  // tables: group-major
        gs.scale16[tg] = __half_as_ushort(sh);
        gs.zero16[tg] = __half_as_ushort(zh);
        const size_t t = ((size_t)h * kD + c) * gs.group_stride + G;
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
        const size_t tg = ((size_t)h * gs.group_stride + G) * kD + c;
        const double zf = (double)__half2float(__ushort_as_half(gs.zero16[tg]));
        const double sf = (double)__half2float(__ushort_as_half(gs.scale16[tg]));
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
// scan on the matrix cores.  A score is C_gG + sum over the planes P = (c, j) the plan
// reads of bit_P * w_gGP, w_gGP = fl32(q_gc sf_cG) 2^(3-j): the per-channel scan's
// product of a token-by-plane bit matrix and a plane-by-query weight matrix, except
// that the weights change every 128-token group.  So each 16-column MFMA block must lie
// in one group: wave v of a workgroup scores words 8v .. 8v+7 (groups 2v and 2v+1 of a
// 64-word tile), and lane 16 q + 4 w + s reads word 8v + 4 pos + w of planes s and s+4
// of plane groups q and q+4 of the K-pair, so that pos picks the group.  The A operand
// (16 rows = 4 queries x 4 digits, K = 64 planes) of each (K-pair, group) is built in
// registers: each weight becomes an integer count of a per-(query, group) power-of-two
// unit (2^(e-30), e the binary exponent just above the group's largest weight of that
// query), split into 4 signed base-256 digits; the four lanes of a quad (one digit each)
// share the 16 weights of their K-slice, computing 4 each.  The int32 digit sums are
// exact; each score is C + S (D0 + 256 D1 + 65536 (D2 + 256 D3)) / 2^m in fp32 as in the
// per-channel scan, C_gG = sum_c q_gc (zf_cG + sf_cG h(t_c)) in fp64 rounded once.
// ---------------------------------------------------------------------------------
// A tile is TW words, 8 per wave.  From HBM TW = 32 (4 waves: less lock-step, 150 us
// against 185 us for 64 on the bench cache); from pinned host memory TW = 64, so that each
// plane row is read in 256-byte runs and a tile's fp16 scales and zeros (group-major) in
// 4 KiB runs -- the link loses most of its rate on shorter runs (1M-token layer: 0.96 of
// the link bound against 0.26 with 128-byte row runs and 16-byte table pieces).
constexpr int kMBatch = 128;                       // planes staged at once: two K-pairs

// Four waves per SIMD for one query set (five spill to scratch and run slower), two for
// two sets.
template <int QS, int TW>
__global__ __launch_bounds__(TW * 8)
__attribute__((amdgpu_waves_per_eu(QS == 1 ? 4 : 2))) void k_scan_grouped_mma(
    fathom_gstore gs, const float *__restrict__ q, const uint8_t *__restrict__ depth, int G,
    float *__restrict__ scores, int tiles_per_head) {
    constexpr int kMThreads = TW * 8;               // TW / 8 waves
    constexpr int kMWords = TW;                     // words per tile
    constexpr int kMGroups = kMWords / kGroupWords; // groups per tile, 2 per wave
    constexpr int kMRowPad = kMWords + 4;           // 16-byte aligned LDS rows
    constexpr int NQ = 4 * QS;
    __shared__ __align__(16) uint32_t words[kMBatch][kMRowPad];
    __shared__ float qs[NQ][kD];
    __shared__ __align__(8) __half sgrp[kMGroups][kD];  // group-major, as in the store
    __shared__ __align__(8) __half zgrp[kMGroups][kD];
    __shared__ float cg[kMGroups][NQ];
    __shared__ int tc[kD];
    __shared__ int off[kD + 1];
    __shared__ uint16_t pl[kMaxPlanesPerHead];
    const int h = blockIdx.x / tiles_per_head, tile = blockIdx.x - h * tiles_per_head;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n = gs.n_tokens, W = (n + 31) >> 5;
    const int ng = (n + kGroup - 1) / kGroup;
    const int w0 = tile * kMWords, gb = w0 / kGroupWords;  // first word, first group

    // inputs: every load unconditional (indices clamped into the head's tables) and
    // issued before any is used, so that they are all in flight together
    constexpr int kQPer = NQ * kD / kMThreads;       // 1 or 2
    static_assert(kD * kMGroups == 4 * kMThreads, "one 8-byte load per table a thread");
    const int tdep = depth[(size_t)h * kD + min(tid, kD - 1)];
    float qv[kQPer];
#pragma unroll
    for (int u = 0; u < kQPer; ++u) {
        const int e = tid + kMThreads * u, g = e / kD, c = e - g * kD;
        qv[u] = q[((size_t)h * G + min(g, G - 1)) * kD + c];
    }
    // the tile's scales and zeros: thread t takes channels 4 (t % 32) .. + 3 of group
    // t / 32 (groups past the head's last are its last group's)
    const int sgg = tid / (kD / 4), sc0 = 4 * (tid % (kD / 4));
    const size_t st0 = ((size_t)h * gs.group_stride + min(gb + sgg, ng - 1)) * kD + sc0;
    const uint2 sv = *reinterpret_cast<const uint2 *>(gs.scale16 + st0);
    const uint2 zv = *reinterpret_cast<const uint2 *>(gs.zero16 + st0);
    if (tid < kD) tc[tid] = min(tdep, kPlanes);
#pragma unroll
    for (int u = 0; u < kQPer; ++u) {
        const int e = tid + kMThreads * u, g = e / kD, c = e - g * kD;
        qs[g][c] = g < G ? qv[u] : 0.0f;
    }
    *reinterpret_cast<uint2 *>(&sgrp[sgg][sc0]) = sv;
    *reinterpret_cast<uint2 *>(&zgrp[sgg][sc0]) = zv;
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
    // C per (group, query) in fp64: eight adjacent threads take 16 channels each and
    // combine their sums with three lane exchanges (rounded once to fp32)
#pragma unroll
    for (int pr = tid >> 3; pr < kMGroups * NQ; pr += kMThreads / 8) {
        const int gg = pr / NQ, g = pr - gg * NQ, c0 = 16 * (tid & 7);
        double acc = 0.0;
#pragma unroll
        for (int c = c0; c < c0 + 16; ++c) {
            const double zf = (double)__half2float(zgrp[gg][c]);
            const double sf = (double)__half2float(sgrp[gg][c]);
            const double hm = (double)((16 >> tc[c]) - 1) * 0.5;
            acc += (double)qs[g][c] * (zf + sf * hm);
        }
#pragma unroll
        for (int o = 1; o < 8; o <<= 1) acc += __shfl_xor(acc, o, 64);
        if ((tid & 7) == 0) cg[gg][g] = (float)acc;
    }
    __syncthreads();
    if (tid < kD) {
        const int c = tid, t = tc[c];
        for (int j = 0; j < t; ++j) pl[off[c] + j] = (uint16_t)(c * kPlanes + j);
    }
    __syncthreads();
    const int nplanes = off[kD];
    const int ngr8 = (nplanes + kGroupBits - 1) / kGroupBits;
    const int nkb = max(1, (ngr8 + kKBlockGroups - 1) / kKBlockGroups);
    const int npr = (nkb + 1) >> 1;  // K-pairs
    const bool small = nkb < kMaxKBlocks;

    const int s = lane & 3, wq = (lane >> 2) & 3, jq = lane >> 4;
    // unit exponent of each (group pos of this wave, query): the group's largest weight
    // fl32(q sf) 8 over the channels read, from two channels a lane and a wave maximum
    int eu[2][NQ];
#pragma unroll
    for (int pos = 0; pos < 2; ++pos) {
        const int gr = 2 * wave + pos;
#pragma unroll
        for (int g = 0; g < NQ; ++g) {
            float mx = 0.0f;
#pragma unroll
            for (int cc = 0; cc < 2; ++cc) {
                const int c = lane + 64 * cc;
                if (tc[c] > 0) mx = fmaxf(mx, fabsf(qs[g][c] * __half2float(sgrp[gr][c])) * 8.0f);
            }
#pragma unroll
            for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
            int e = 0;
            frexpf(mx, &e);  // mx < 2^e
            eu[pos][g] = mx > 0.0f ? e : 0;
        }
    }

    const uint32_t *hp = gs.planes + (size_t)h * kMaxPlanesPerHead * gs.word_stride;
    v4i acc[2][8][QS];
    for (int kp0 = 0; kp0 < npr; kp0 += 2) {  // batches of two K-pairs
        const int p0 = 64 * kp0;
        const int np = max(0, min(kMBatch, nplanes - p0));
        if (kp0) __syncthreads();  // the previous batch's words are no longer read
        if (np > 0) {  // the plane list holds the batch's rows only when it has any
            // 16 bytes a load, all unconditional and in flight together (a slot past the
            // batch reads its last row, one past the row the row's first 16 bytes, and
            // is dropped); word_stride is a multiple of 4
            constexpr int kBPer = kMBatch * (kMWords / 4) / kMThreads;  // 4
            uint4 x[kBPer];
#pragma unroll
            for (int u = 0; u < kBPer; ++u) {
                const int e = tid + kMThreads * u, r = e / (kMWords / 4), v = e % (kMWords / 4);
                const int wv = w0 + 4 * v;
                const int row = pl[p0 + min(r, np - 1)];
                x[u] = *reinterpret_cast<const uint4 *>(hp + (size_t)row * gs.word_stride +
                                                        (wv < gs.word_stride ? wv : 0));
            }
#pragma unroll
            for (int u = 0; u < kBPer; ++u) {
                const int e = tid + kMThreads * u, r = e / (kMWords / 4), v = e % (kMWords / 4);
                if (r < np)
                    *reinterpret_cast<uint4 *>(&words[r][4 * v]) =
                        w0 + 4 * v < gs.word_stride ? x[u] : make_uint4(0u, 0u, 0u, 0u);
            }
        }
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            const int kp = kp0 + kk;
            if (kp >= npr) break;
#pragma unroll
            for (int pos = 0; pos < 2; ++pos) {
                const int gr = 2 * wave + pos;
                // A operand: this lane's row is (query 4 set + (lane & 15) / 4, digit s)
                // over planes 64 kp + 8 jq + i (i < 8) and 64 kp + 32 + 8 jq + i - 8
                v4i A[QS];
#pragma unroll
                for (int set = 0; set < QS; ++set) {
                    const int g = 4 * set + ((lane & 15) >> 2);
                    int mine[4];  // weights 4 s .. 4 s + 3 of the lane's 16, biased
#pragma unroll
                    for (int ii = 0; ii < 4; ++ii) {
                        const int i = 4 * s + ii;
                        const int P = 64 * kp + (i < 8 ? 8 * jq + i : 32 + 8 * jq + i - 8);
                        int M = 0;
                        if (P < nplanes) {
                            const int row = pl[P], c = row >> 2, j = row & 3;
                            const float w = qs[g][c] * __half2float(sgrp[gr][c]);
                            // w 2^(3-j) / 2^(e-30), an exact power-of-two scaling
                            M = (int)rintf(ldexpf(w, 33 - j - eu[pos][g]));
                        }
                        mine[ii] = M + (int)kDigitBias;  // |M| <= 2^30: no overflow
                    }
                    // dword src of the operand holds weights 4 src .. 4 src + 3 (lane src
                    // of the quad computed them): byte s of each biased weight, gathered
                    // with byte permutes, is digit s + 128 (s < 3, flipped back to a
                    // two's-complement byte) or the top digit (s = 3)
                    const uint32_t sel = (uint32_t)s | ((uint32_t)(4 + s) << 8) | 0x0C0C0000u;
                    const uint32_t flip = s < 3 ? 0x80808080u : 0u;
                    uint32_t bytes[4];
#pragma unroll
                    for (int src = 0; src < 4; ++src) {
                        uint32_t u[4];
#pragma unroll
                        for (int ii = 0; ii < 4; ++ii) {
                            if (src == 0) u[ii] = (uint32_t)__builtin_amdgcn_mov_dpp(mine[ii], 0x00, 0xF, 0xF, false);
                            else if (src == 1) u[ii] = (uint32_t)__builtin_amdgcn_mov_dpp(mine[ii], 0x55, 0xF, 0xF, false);
                            else if (src == 2) u[ii] = (uint32_t)__builtin_amdgcn_mov_dpp(mine[ii], 0xAA, 0xF, 0xF, false);
                            else u[ii] = (uint32_t)__builtin_amdgcn_mov_dpp(mine[ii], 0xFF, 0xF, 0xF, false);
                        }
                        const uint32_t lo = __builtin_amdgcn_perm(u[1], u[0], sel);
                        const uint32_t hi = __builtin_amdgcn_perm(u[3], u[2], sel);
                        bytes[src] = __builtin_amdgcn_perm(hi, lo, 0x05040100u) ^ flip;
                    }
                    A[set] = v4i{(int)bytes[0], (int)bytes[1], (int)bytes[2], (int)bytes[3]};
                }
                // B operand: byte s of word 8v + 4 pos + wq of the 8 planes of plane groups
                // jq and jq + 4, by the LDS transpose read (within each 16 lanes, lane i < 8
                // receives byte i of the 8 bytes each even lane read, lane 8 + i those of
                // the odd lanes): lane 16 jq + 2 j + p reads words 8v + 4 pos + 2p and the
                // next of plane j.  The rows' 144- or 272-byte stride puts each half-wave's
                // 32 reads on distinct banks.
                uint32_t x[2][2];
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    const int trj = (lane & 15) >> 1, trp = lane & 1;
                    const v2i r = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                        (__attribute__((address_space(3))) v2i *)&words[64 * kk + 8 * (jq + 4 * hh) + trj]
                                                                       [8 * wave + 4 * pos + 2 * trp]);
                    x[hh][0] = (uint32_t)r.x;
                    x[hh][1] = (uint32_t)r.y;
                }
#pragma unroll
                for (int m = 0; m < 8; ++m) {
                    const uint32_t mask = 0x01010101u << m;
                    const v4i b = {(int)(x[0][0] & mask), (int)(x[0][1] & mask),
                                   (int)(x[1][0] & mask), (int)(x[1][1] & mask)};
#pragma unroll
                    for (int set = 0; set < QS; ++set) {
                        const v4i c0 = kp == 0 ? v4i{0, 0, 0, 0} : acc[pos][m][set];
                        acc[pos][m][set] = __builtin_amdgcn_mfma_i32_16x16x64_i8(A[set], b, c0, 0, 0, 0);
                    }
                }
            }
        }
    }
    // scores: lane 16 j + 4 w + s holds query j's digit sums of byte s of word
    // 8v + 4 pos + w, bit m
#pragma unroll
    for (int pos = 0; pos < 2; ++pos) {
        const int gr = 2 * wave + pos;
        const int word = w0 + 8 * wave + 4 * pos + wq;
        if (word >= W) continue;
        const int tok = 32 * word + 8 * s;
#pragma unroll
        for (int set = 0; set < QS; ++set) {
            const int g = 4 * set + jq;
            if (g >= G) continue;
            const float C = cg[gr][g];
            const float S = ldexpf(1.0f, eu[pos][g] - 30);
            float v[8];
#pragma unroll
            for (int m = 0; m < 8; ++m) v[m] = combined_score<QS>(acc[pos][m][set], m, C, S, small);
            float *row = scores + ((size_t)h * G + g) * n;
            if ((n & 3) == 0 && tok + 8 <= n) {
                *reinterpret_cast<float4 *>(row + tok) = make_float4(v[0], v[1], v[2], v[3]);
                *reinterpret_cast<float4 *>(row + tok + 4) = make_float4(v[4], v[5], v[6], v[7]);
            } else {
#pragma unroll
                for (int m = 0; m < 8; ++m)
                    if (tok + m < n) row[tok + m] = v[m];
            }
        }
    }
}

template <int QS, int TW>
void launch_scan_mma(const fathom_gstore &gs, const float *q, const uint8_t *depth, int G,
                     float *scores, hipStream_t s) {
    const int W = (gs.n_tokens + 31) >> 5;
    const int tiles = (W + TW - 1) / TW;
    hipLaunchKernelGGL((k_scan_grouped_mma<QS, TW>), dim3(gs.n_heads * tiles), dim3(TW * 8), 0,
                       s, gs, q, depth, G, scores, tiles);
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
                               int G, float *scores, bool host_planes, hipStream_t s) {
    if (query_sets(G) == 1) {
        if (host_planes) launch_scan_mma<1, 64>(gs, q, depth, G, scores, s);
        else launch_scan_mma<1, 32>(gs, q, depth, G, scores, s);
    } else {
        if (host_planes) launch_scan_mma<2, 64>(gs, q, depth, G, scores, s);
        else launch_scan_mma<2, 32>(gs, q, depth, G, scores, s);
    }
    return hipGetLastError();
}

}  // namespace fathom
