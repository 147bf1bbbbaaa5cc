/*
 * fathom_oracle.c -- plain, slow CPU oracle for the Fathom bit-plane key scan.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU-baseline
 * leg of the benchmark load this library.  The product library (libfathom.so) never
 * links, calls or reads anything here, and this file shares no code, header, table or
 * constant with it.
 *
 * Sources.  "blog" is the author's post on vivekkalyanarangan.hashnode.dev (sections
 * named by their headings); "Glonce" is the editorial summary "Fathom speeds
 * long-context KV cache decoding 1.67x with per-query reads"; "Rootconf" is the talk
 * proposal "Decoding at a million tokens when the KV cache lives in host memory".
 *
 * Arithmetic.  Build with -O2 -ffp-contract=off (no fused multiply-add anywhere).
 * Where floating point decides an integer (the 4-bit code, the plan) the precision is
 * stated at the step: the quantizer runs in IEEE fp32 (the keys are fp32), the plan
 * compares fp64 keys exactly.  Everything else (scores, attention) is fp64.
 *
 * Every function works on ONE (layer, KV head) unless its name ends in _batch; the
 * _batch forms only loop the per-head function over heads (OpenMP over heads).
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_PLANES 4 /* 4-bit codes -> 4 bit planes (blog, "Bit planes") */

/* Threads the _batch forms use (OpenMP's default team size). */
int oracle_threads(void) { return omp_get_max_threads(); }
void oracle_set_threads(int n) { if (n > 0) omp_set_num_threads(n); }

/* ------------------------------------------------------------------------------ */
/* Quantize (blog, "How to read fewer bits per key": 4-bit storage; Glonce: "4-bit  */
/* K cache", per channel).  One (scale, zero) per channel over all n tokens:        */
/*   s = (max - min) / 15,  z = min            (both one fp32 operation each)       */
/*   code = clamp(floor((x - z) / s + 0.5), 0, 15), every step one fp32 operation.  */
/* A channel whose values are all equal (s == 0) gets code 0 everywhere.            */
/* ------------------------------------------------------------------------------ */
void oracle_quantize(const float *x, int n, int d, float *scale, float *zero,
                     uint8_t *codes)
{
    for (int c = 0; c < d; ++c) {
        float mn = x[c], mx = x[c];
        for (int i = 1; i < n; ++i) {
            float v = x[(size_t)i * d + c];
            if (v < mn) mn = v;
            if (v > mx) mx = v;
        }
        float range = mx - mn;
        float s = range / 15.0f;
        scale[c] = s;
        zero[c] = mn;
        for (int i = 0; i < n; ++i) {
            uint8_t code = 0;
            if (s != 0.0f) {
                float diff = x[(size_t)i * d + c] - mn;
                float u = diff / s;
                float r = u + 0.5f;
                float f = floorf(r);
                if (f < 0.0f) f = 0.0f;
                if (f > 15.0f) f = 15.0f;
                code = (uint8_t)f;
            }
            codes[(size_t)i * d + c] = code;
        }
    }
}

/* ------------------------------------------------------------------------------ */
/* Bit-plane packing (blog, "Bit planes": plane 0 holds the most significant bit    */
/* of every number, then the next bit, and so on; storage is channel-major).        */
/* Layout [c][j][w]: plane j of channel c, 32-token word w.  Token i sits in word   */
/* i/32 at bit i%32 (least significant bit = lowest token).  Bits of tokens >= n    */
/* are zero.                                                                        */
/* ------------------------------------------------------------------------------ */
void oracle_pack_planes(const uint8_t *codes, int n, int d, int W, uint32_t *planes)
{
    memset(planes, 0, sizeof(uint32_t) * (size_t)d * ORACLE_PLANES * W);
    for (int c = 0; c < d; ++c)
        for (int j = 0; j < ORACLE_PLANES; ++j)
            for (int i = 0; i < n; ++i) {
                uint32_t bit = (codes[(size_t)i * d + c] >> (3 - j)) & 1u;
                size_t word = ((size_t)c * ORACLE_PLANES + j) * W + (size_t)(i / 32);
                planes[word] |= bit << (i % 32);
            }
}

/* The ordinary layout the pages compare against (blog, "Where this does not work":  */
/* a plain 4-bit scan reads each 4-bit number whole).  Token-major, two channels a   */
/* byte: byte j of token i holds the code of channel 2j in its low four bits and     */
/* that of channel 2j+1 in its high four bits (the order within the byte is not      */
/* stated; this one is the plainest).  Layout [i][d/2], d even.                      */
void oracle_pack_nibbles(const uint8_t *codes, int n, int d, uint8_t *nib)
{
    for (int i = 0; i < n; ++i)
        for (int j = 0; j < d / 2; ++j) {
            const uint8_t lo = codes[(size_t)i * d + 2 * j] & 15u;
            const uint8_t hi = codes[(size_t)i * d + 2 * j + 1] & 15u;
            nib[(size_t)i * (d / 2) + j] = (uint8_t)(lo | (hi << 4));
        }
}

/* Inverse of the packing, for one channel at read depth t (0..4): the t-plane      */
/* prefix p of token i, i.e. the integer whose bits are planes 0..t-1 (blog, "Bit   */
/* planes": reading planes 0 and 1 gives every number rounded to 2 bits).           */
uint32_t oracle_plane_prefix(const uint32_t *planes, int W, int c, int t, int i)
{
    uint32_t p = 0;
    for (int j = 0; j < t; ++j) {
        size_t word = ((size_t)c * ORACLE_PLANES + j) * W + (size_t)(i / 32);
        p = (p << 1) | ((planes[word] >> (i % 32)) & 1u);
    }
    return p;
}

/* ------------------------------------------------------------------------------ */
/* Channel variance (blog, "How each query picks its own depth": importance is      */
/* roughly the share of score variance a channel carries; Glonce: variance-weighted */
/* importance).  Reading: the population variance of the DEQUANTIZED channel        */
/* z + s*code, from exact integer sums:                                             */
/*   var = s^2 * (n*S2 - S1^2) / n^2,  S1 = sum code, S2 = sum code^2 (int64),      */
/* evaluated in fp64 left to right and rounded once to fp32.                        */
/* ------------------------------------------------------------------------------ */
void oracle_var(const uint8_t *codes, const float *scale, int n, int d, float *var)
{
    for (int c = 0; c < d; ++c) {
        int64_t s1 = 0, s2 = 0;
        for (int i = 0; i < n; ++i) {
            int64_t v = codes[(size_t)i * d + c];
            s1 += v;
            s2 += v * v;
        }
        int64_t num = (int64_t)n * s2 - s1 * s1;
        double s = (double)scale[c];
        double v = (s * s) * (double)num / ((double)n * (double)n);
        var[c] = (float)v;
    }
}

/* ------------------------------------------------------------------------------ */
/* Plan (blog, "How each query picks its own depth": reverse water-filling; a bit   */
/* spent on a channel reduces the error in proportion to its importance divided by  */
/* four to the power of the bits it already has; 0..4 planes per channel).          */
/*   importance  w_c = var_c * sum_g q_gc^2   (G queries share one KV head's plan), */
/*   in fp64: each q^2 is exact, the sum runs over g ascending, then one product.   */
/* Greedy form: B times, give one more plane to the channel with the largest        */
/* w_c * 4^(-t_c) among channels with t_c < 4; on equal keys the lower channel      */
/* index wins.  Keys are compared exactly (4^-t is an exact power-of-two scaling).  */
/* Requires 0 <= B <= 4*d.                                                          */
/* ------------------------------------------------------------------------------ */
double oracle_importance(const float *q, int G, int d, const float *var, int c)
{
    double sq = 0.0;
    for (int g = 0; g < G; ++g) {
        double v = (double)q[(size_t)g * d + c];
        sq = sq + v * v;
    }
    return sq * (double)var[c];
}

int oracle_plan(const float *q, const float *var, int G, int d, int B, uint8_t *depth)
{
    if (B < 0 || B > ORACLE_PLANES * d) return -1;
    double *w = (double *)malloc(sizeof(double) * (size_t)d);
    if (!w) return -2;
    for (int c = 0; c < d; ++c) {
        w[c] = oracle_importance(q, G, d, var, c);
        depth[c] = 0;
    }
    for (int b = 0; b < B; ++b) {
        int best = -1;
        double best_key = 0.0;
        for (int c = 0; c < d; ++c) {
            if (depth[c] >= ORACLE_PLANES) continue;
            double key = ldexp(w[c], -2 * depth[c]);
            if (best < 0 || key > best_key) {
                best = c;
                best_key = key;
            }
        }
        depth[best] += 1;
    }
    free(w);
    return 0;
}

/* Query-independent comparator of the size the blog's "The catch" section gives for  */
/* the fixed 136-bit scans: all four planes of the n_channels channels with the      */
/* largest variance (equal variances: lower channel index first), nothing elsewhere. */
int oracle_plan_fixed(const float *var, int d, int n_channels, uint8_t *depth)
{
    if (n_channels < 0 || n_channels > d) return -1;
    for (int c = 0; c < d; ++c) depth[c] = 0;
    for (int taken = 0; taken < n_channels; ++taken) {
        int best = -1;
        for (int c = 0; c < d; ++c) {
            if (depth[c] != 0) continue;
            if (best < 0 || var[c] > var[best]) best = c;
        }
        depth[best] = ORACLE_PLANES;
    }
    return 0;
}

/* ------------------------------------------------------------------------------ */
/* IEEE 754 binary16 (fp16), round to nearest, ties to even, from the format's       */
/* definition: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits; values below */
/* 2^-14 are multiples of 2^-24; at or above 65520 the value rounds to infinity.     */
/* ------------------------------------------------------------------------------ */
uint16_t oracle_f32_to_f16(float x)
{
    uint32_t u;
    memcpy(&u, &x, sizeof u);
    const uint16_t sign = (uint16_t)((u >> 16) & 0x8000u);
    const uint32_t a = u & 0x7FFFFFFFu;
    if (a >= 0x7F800000u) return sign | (a > 0x7F800000u ? 0x7E00u : 0x7C00u);
    const double v = fabs((double)x);
    if (v >= 65520.0) return sign | 0x7C00u;
    if (v < 6.103515625e-05) {               /* below 2^-14: steps of 2^-24 */
        const double r = nearbyint(v * 16777216.0);
        return sign | (uint16_t)r;           /* r = 1024 is the smallest normal */
    }
    int e;
    const double f = frexp(v, &e);           /* v = f 2^e, f in [0.5, 1) */
    double r = nearbyint(ldexp(f, 11));      /* 11 significant bits */
    if (r == 2048.0) {
        r = 1024.0;
        e += 1;
    }
    const int E = e - 1 + 15;
    if (E >= 31) return sign | 0x7C00u;
    return sign | (uint16_t)((E << 10) | ((uint32_t)r - 1024u));
}

float oracle_f16_to_f32(uint16_t h)
{
    const int E = (h >> 10) & 31, F = h & 1023;
    double v;
    if (E == 31) v = F ? NAN : INFINITY;
    else if (E == 0) v = ldexp((double)F, -24);
    else v = ldexp((double)(1024 + F), E - 25);
    return (float)((h & 0x8000u) ? -v : v);
}

/* ------------------------------------------------------------------------------ */
/* Grouped scale and zero.  A reading of the blog's "Where this does not work": the  */
/* index costs 68 bytes per token per KV head, 4 more than 128 channels of 4-bit     */
/* codes; one fp16 scale and one fp16 zero per channel per group of 128 tokens are   */
/* exactly those 4 bytes.  Per channel, per group of `group` consecutive tokens (the */
/* last may be shorter): s = (max - min)/15 and z = min in fp32 as in               */
/* oracle_quantize, each rounded to fp16; the codes use the fp16 values:            */
/*   code = clamp(floor((x - zf)/sf + 0.5), 0, 15), every step one fp32 operation,   */
/* sf == 0 gives code 0.  s16, z16: fp16 bits [d][ceil(n/group)].                   */
/* ------------------------------------------------------------------------------ */
void oracle_quantize_grouped(const float *x, int n, int d, int group, uint16_t *s16,
                             uint16_t *z16, uint8_t *codes)
{
    const int ng = (n + group - 1) / group;
    for (int c = 0; c < d; ++c)
        for (int gi = 0; gi < ng; ++gi) {
            const int i0 = gi * group, i1 = i0 + group < n ? i0 + group : n;
            float mn = x[(size_t)i0 * d + c], mx = mn;
            for (int i = i0 + 1; i < i1; ++i) {
                const float v = x[(size_t)i * d + c];
                if (v < mn) mn = v;
                if (v > mx) mx = v;
            }
            const float range = mx - mn;
            const uint16_t sh = oracle_f32_to_f16(range / 15.0f);
            const uint16_t zh = oracle_f32_to_f16(mn);
            s16[(size_t)c * ng + gi] = sh;
            z16[(size_t)c * ng + gi] = zh;
            const float sf = oracle_f16_to_f32(sh), zf = oracle_f16_to_f32(zh);
            for (int i = i0; i < i1; ++i) {
                uint8_t code = 0;
                if (sf != 0.0f) {
                    float diff = x[(size_t)i * d + c] - zf;
                    float u = diff / sf;
                    float r = u + 0.5f;
                    float f = floorf(r);
                    if (f < 0.0f) f = 0.0f;
                    if (f > 15.0f) f = 15.0f;
                    code = (uint8_t)f;
                }
                codes[(size_t)i * d + c] = code;
            }
        }
}

/* Variance of the dequantized channel zf + sf*code over all n tokens (the importance  */
/* of "How each query picks its own depth"), from per-group integer code sums S1, S2: */
/*   S = sum_G (n_G zf + sf S1),  Q = sum_G (n_G zf^2 + 2 zf sf S1 + sf^2 S2),         */
/* each product exact in fp64, each term added in that order, groups ascending; then  */
/* var = (n Q - S^2) / n^2 in fp64, rounded once to fp32.                            */
void oracle_var_grouped(const uint8_t *codes, const uint16_t *s16, const uint16_t *z16,
                        int n, int d, int group, float *var)
{
    const int ng = (n + group - 1) / group;
    for (int c = 0; c < d; ++c) {
        double S = 0.0, Q = 0.0;
        for (int gi = 0; gi < ng; ++gi) {
            const int i0 = gi * group, i1 = i0 + group < n ? i0 + group : n;
            int64_t s1 = 0, s2 = 0;
            for (int i = i0; i < i1; ++i) {
                const int64_t k = codes[(size_t)i * d + c];
                s1 += k;
                s2 += k * k;
            }
            const double zf = oracle_f16_to_f32(z16[(size_t)c * ng + gi]);
            const double sf = oracle_f16_to_f32(s16[(size_t)c * ng + gi]);
            const double nG = (double)(i1 - i0);
            S = S + nG * zf;
            S = S + sf * (double)s1;
            Q = Q + nG * (zf * zf);
            Q = Q + 2.0 * zf * sf * (double)s1;
            Q = Q + (sf * sf) * (double)s2;
        }
        const double nn = (double)n;
        var[c] = (float)((nn * Q - S * S) / (nn * nn));
    }
}

/* Approximate scores over a grouped store: as oracle_scores, each token dequantized */
/* with its group's fp16 scale and zero.  fp64.                                       */
void oracle_scores_grouped(const uint8_t *codes, const uint16_t *s16, const uint16_t *z16,
                           const uint8_t *depth, const float *q, int n, int d, int G,
                           int group, double *scores);

/* ------------------------------------------------------------------------------ */
/* Reconstruction at the bin midpoint.  A t-plane prefix p pins the 4-bit code to   */
/* the 2^(4-t) codes p*2^(4-t) .. p*2^(4-t) + 2^(4-t) - 1; the channel is            */
/* reconstructed at the middle of that run: m = p*2^(4-t) + (2^(4-t) - 1)/2,         */
/* so k_hat = z + s*m.  t = 0 reads nothing and gives the midpoint 7.5 of the whole  */
/* range.  (blog, "Bit planes": a prefix read is exactly the lower-precision copy.)  */
/* ------------------------------------------------------------------------------ */
double oracle_midpoint_level(int code, int t)
{
    if (t <= 0) return 7.5;
    int shift = ORACLE_PLANES - t;
    int p = code >> shift;
    double width = (double)(1 << shift);
    return (double)p * width + (width - 1.0) / 2.0;
}

/* ------------------------------------------------------------------------------ */
/* Approximate scores (blog, "The first fix": score every key; "How each query      */
/* picks its own depth": each channel read to its own depth).  Definition, in fp64: */
/*   score[g][i] = sum over c ascending of q_gc * (z_c + s_c * m(code_ic, t_c)).     */
/* The oracle works from its own integer codes, not from the planes.                */
/* ------------------------------------------------------------------------------ */
void oracle_scores(const uint8_t *codes, const float *scale, const float *zero,
                   const uint8_t *depth, const float *q, int n, int d, int G,
                   double *scores)
{
    for (int g = 0; g < G; ++g)
        for (int i = 0; i < n; ++i) {
            double acc = 0.0;
            for (int c = 0; c < d; ++c) {
                double m = oracle_midpoint_level(codes[(size_t)i * d + c], depth[c]);
                double khat = (double)zero[c] + (double)scale[c] * m;
                acc += (double)q[(size_t)g * d + c] * khat;
            }
            scores[(size_t)g * n + i] = acc;
        }
}

void oracle_scores_grouped(const uint8_t *codes, const uint16_t *s16, const uint16_t *z16,
                           const uint8_t *depth, const float *q, int n, int d, int G,
                           int group, double *scores)
{
    const int ng = (n + group - 1) / group;
    for (int g = 0; g < G; ++g)
        for (int i = 0; i < n; ++i) {
            const int gi = i / group;
            double acc = 0.0;
            for (int c = 0; c < d; ++c) {
                const double m = oracle_midpoint_level(codes[(size_t)i * d + c], depth[c]);
                const double zf = oracle_f16_to_f32(z16[(size_t)c * ng + gi]);
                const double sf = oracle_f16_to_f32(s16[(size_t)c * ng + gi]);
                acc += (double)q[(size_t)g * d + c] * (zf + sf * m);
            }
            scores[(size_t)g * n + i] = acc;
        }
}

/* Dequantized keys z + s*code in fp64 (the 4-bit value every plane prefix refines). */
void oracle_dequantize(const uint8_t *codes, const float *scale, const float *zero,
                       int n, int d, double *out)
{
    for (int i = 0; i < n; ++i)
        for (int c = 0; c < d; ++c)
            out[(size_t)i * d + c] =
                (double)zero[c] + (double)scale[c] * (double)codes[(size_t)i * d + c];
}

/* ------------------------------------------------------------------------------ */
/* Top-k (blog, "The first fix": take the top k).  Order all n entries by score     */
/* descending, then token index ascending (so equal scores go to the lower index;   */
/* -0 and +0 compare equal), keep the first k, return them ascending by index.      */
/* Scores must be finite.  Requires 1 <= k <= n.                                    */
/* ------------------------------------------------------------------------------ */
typedef struct {
    float s;
    int32_t i;
} oracle_entry;

static int oracle_entry_cmp(const void *a, const void *b)
{
    const oracle_entry *x = (const oracle_entry *)a, *y = (const oracle_entry *)b;
    if (x->s > y->s) return -1;
    if (x->s < y->s) return 1;
    return (x->i < y->i) ? -1 : (x->i > y->i);
}

static int oracle_int_cmp(const void *a, const void *b)
{
    int32_t x = *(const int32_t *)a, y = *(const int32_t *)b;
    return (x > y) - (x < y);
}

int oracle_topk(const float *scores, int n, int k, int32_t *idx)
{
    if (k < 1 || k > n) return -1;
    oracle_entry *e = (oracle_entry *)malloc(sizeof(oracle_entry) * (size_t)n);
    if (!e) return -2;
    for (int i = 0; i < n; ++i) {
        e[i].s = scores[i];
        e[i].i = i;
    }
    qsort(e, (size_t)n, sizeof(oracle_entry), oracle_entry_cmp);
    for (int r = 0; r < k; ++r) idx[r] = e[r].i;
    free(e);
    qsort(idx, (size_t)k, sizeof(int32_t), oracle_int_cmp);
    return 0;
}

/* The same order over fp64 values (the exact attention logits of every token, whose */
/* k largest are the exact top-k the approximate scan is measured against).          */
typedef struct {
    double s;
    int32_t i;
} oracle_entry64;

static int oracle_entry64_cmp(const void *a, const void *b)
{
    const oracle_entry64 *x = (const oracle_entry64 *)a, *y = (const oracle_entry64 *)b;
    if (x->s > y->s) return -1;
    if (x->s < y->s) return 1;
    return (x->i < y->i) ? -1 : (x->i > y->i);
}

int oracle_topk_f64(const double *scores, int n, int k, int32_t *idx)
{
    if (k < 1 || k > n) return -1;
    oracle_entry64 *e = (oracle_entry64 *)malloc(sizeof(oracle_entry64) * (size_t)n);
    if (!e) return -2;
    for (int i = 0; i < n; ++i) {
        e[i].s = scores[i] == 0.0 ? 0.0 : scores[i]; /* -0 ranks as +0 */
        e[i].i = i;
    }
    qsort(e, (size_t)n, sizeof(oracle_entry64), oracle_entry64_cmp);
    for (int r = 0; r < k; ++r) idx[r] = e[r].i;
    free(e);
    qsort(idx, (size_t)k, sizeof(int32_t), oracle_int_cmp);
    return 0;
}

/* ------------------------------------------------------------------------------ */
/* bf16 <-> fp32.  A bf16 value is the upper 16 bits of an fp32 value; the widening  */
/* is exact.  The narrowing rounds to nearest, ties to even (NaN kept quiet).        */
/* ------------------------------------------------------------------------------ */
float oracle_bf16_to_f32(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

uint16_t oracle_f32_to_bf16(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu))
        return (uint16_t)((u >> 16) | 0x0040u);
    uint32_t lower = u & 0xffffu;
    uint32_t upper = u >> 16;
    if (lower > 0x8000u || (lower == 0x8000u && (upper & 1u))) upper += 1u;
    return (uint16_t)upper;
}

void oracle_f32_to_bf16_array(const float *x, size_t count, uint16_t *out)
{
    for (size_t i = 0; i < count; ++i) out[i] = oracle_f32_to_bf16(x[i]);
}

/* ------------------------------------------------------------------------------ */
/* Exact attention over the selected rows (blog, "The first fix": compute attention */
/* over just those k tokens).  For one query q (fp32, d channels) and index set idx */
/* (k rows of bf16 K and V, each row d values):                                     */
/*   l_r = sm_scale * sum_c q_c * K[idx_r][c]         (fp64)                         */
/*   p   = softmax(l) with the maximum subtracted     (fp64)                         */
/*   out = sum_r p_r * V[idx_r]                       (fp64, d values)               */
/* ------------------------------------------------------------------------------ */
void oracle_attention(const float *q, const uint16_t *K, const uint16_t *V, int d,
                      const int32_t *idx, int k, double sm_scale, double *out)
{
    double *l = (double *)malloc(sizeof(double) * (size_t)k);
    double mx = -INFINITY;
    for (int r = 0; r < k; ++r) {
        const uint16_t *row = K + (size_t)idx[r] * d;
        double dot = 0.0;
        for (int c = 0; c < d; ++c)
            dot += (double)q[c] * (double)oracle_bf16_to_f32(row[c]);
        l[r] = dot * sm_scale;
        if (l[r] > mx) mx = l[r];
    }
    double sum = 0.0;
    for (int r = 0; r < k; ++r) {
        l[r] = exp(l[r] - mx);
        sum += l[r];
    }
    for (int c = 0; c < d; ++c) out[c] = 0.0;
    for (int r = 0; r < k; ++r) {
        const uint16_t *row = V + (size_t)idx[r] * d;
        double p = l[r] / sum;
        for (int c = 0; c < d; ++c) out[c] += p * (double)oracle_bf16_to_f32(row[c]);
    }
    free(l);
}

/* Exact attention logits of every one of the n rows (the first step of the         */
/* attention above, over all tokens):  l_i = sm_scale * sum_c q_c * K[i][c]  (fp64). */
void oracle_logits(const float *q, const uint16_t *K, int n, int d, double sm_scale,
                   double *out)
{
    for (int i = 0; i < n; ++i) {
        const uint16_t *row = K + (size_t)i * d;
        double dot = 0.0;
        for (int c = 0; c < d; ++c)
            dot += (double)q[c] * (double)oracle_bf16_to_f32(row[c]);
        out[i] = dot * sm_scale;
    }
}

/* ============================================================================== */
/* Batched forms: the per-head functions above, looped over heads.                 */
/* Shapes: x [H][n][d]; scale/zero/var [H][d]; codes [H][n][d]; planes [H][d][4][W]; */
/* q [H][G][d]; depth [H][d]; scores [H][G][n]; idx [R][k] over R rows of n.        */
/* ============================================================================== */
void oracle_quantize_batch(const float *x, int H, int n, int d, float *scale,
                           float *zero, uint8_t *codes)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int h = 0; h < H; ++h)
        oracle_quantize(x + (size_t)h * n * d, n, d, scale + (size_t)h * d,
                        zero + (size_t)h * d, codes + (size_t)h * n * d);
}

void oracle_pack_planes_batch(const uint8_t *codes, int H, int n, int d, int W,
                              uint32_t *planes)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int h = 0; h < H; ++h)
        oracle_pack_planes(codes + (size_t)h * n * d, n, d, W,
                           planes + (size_t)h * d * ORACLE_PLANES * W);
}

void oracle_pack_nibbles_batch(const uint8_t *codes, int H, int n, int d, uint8_t *nib)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int h = 0; h < H; ++h)
        oracle_pack_nibbles(codes + (size_t)h * n * d, n, d, nib + (size_t)h * n * (d / 2));
}

void oracle_quantize_grouped_batch(const float *x, int H, int n, int d, int group,
                                   uint16_t *s16, uint16_t *z16, uint8_t *codes)
{
    const int ng = (n + group - 1) / group;
#pragma omp parallel for schedule(dynamic, 1)
    for (int h = 0; h < H; ++h)
        oracle_quantize_grouped(x + (size_t)h * n * d, n, d, group, s16 + (size_t)h * d * ng,
                                z16 + (size_t)h * d * ng, codes + (size_t)h * n * d);
}

void oracle_var_grouped_batch(const uint8_t *codes, const uint16_t *s16, const uint16_t *z16,
                              int H, int n, int d, int group, float *var)
{
    const int ng = (n + group - 1) / group;
#pragma omp parallel for schedule(dynamic, 1)
    for (int h = 0; h < H; ++h)
        oracle_var_grouped(codes + (size_t)h * n * d, s16 + (size_t)h * d * ng,
                           z16 + (size_t)h * d * ng, n, d, group, var + (size_t)h * d);
}

void oracle_scores_grouped_batch(const uint8_t *codes, const uint16_t *s16,
                                 const uint16_t *z16, const uint8_t *depth, const float *q,
                                 int H, int n, int d, int G, int group, double *scores)
{
    const int ng = (n + group - 1) / group;
#pragma omp parallel for schedule(dynamic, 1)
    for (int h = 0; h < H; ++h)
        oracle_scores_grouped(codes + (size_t)h * n * d, s16 + (size_t)h * d * ng,
                              z16 + (size_t)h * d * ng, depth + (size_t)h * d,
                              q + (size_t)h * G * d, n, d, G, group,
                              scores + (size_t)h * G * n);
}

void oracle_var_batch(const uint8_t *codes, const float *scale, int H, int n, int d,
                      float *var)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int h = 0; h < H; ++h)
        oracle_var(codes + (size_t)h * n * d, scale + (size_t)h * d, n, d,
                   var + (size_t)h * d);
}

int oracle_plan_batch(const float *q, const float *var, int H, int G, int d, int B,
                      uint8_t *depth)
{
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
    for (int h = 0; h < H; ++h)
        bad |= oracle_plan(q + (size_t)h * G * d, var + (size_t)h * d, G, d, B,
                           depth + (size_t)h * d) != 0;
    return bad ? -1 : 0;
}

void oracle_scores_batch(const uint8_t *codes, const float *scale, const float *zero,
                         const uint8_t *depth, const float *q, int H, int n, int d,
                         int G, double *scores)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int h = 0; h < H; ++h)
        oracle_scores(codes + (size_t)h * n * d, scale + (size_t)h * d,
                      zero + (size_t)h * d, depth + (size_t)h * d,
                      q + (size_t)h * G * d, n, d, G, scores + (size_t)h * G * n);
}

int oracle_topk_batch(const float *scores, int R, int n, int k, int32_t *idx)
{
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
    for (int r = 0; r < R; ++r)
        bad |= oracle_topk(scores + (size_t)r * n, n, k, idx + (size_t)r * k) != 0;
    return bad ? -1 : 0;
}

/* q [H][G][d]; K, V [H][n][d]; idx [H][G][k]; out [H][G][d]. */
void oracle_attention_batch(const float *q, const uint16_t *K, const uint16_t *V, int H,
                            int G, int n, int d, const int32_t *idx, int k,
                            double sm_scale, double *out)
{
#pragma omp parallel for collapse(2) schedule(dynamic, 1)
    for (int h = 0; h < H; ++h)
        for (int g = 0; g < G; ++g)
            oracle_attention(q + ((size_t)h * G + g) * d, K + (size_t)h * n * d,
                             V + (size_t)h * n * d, d,
                             idx + ((size_t)h * G + g) * k, k, sm_scale,
                             out + ((size_t)h * G + g) * d);
}

int oracle_topk_f64_batch(const double *scores, int R, int n, int k, int32_t *idx)
{
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
    for (int r = 0; r < R; ++r)
        bad |= oracle_topk_f64(scores + (size_t)r * n, n, k, idx + (size_t)r * k) != 0;
    return bad ? -1 : 0;
}

/* q [H][G][d]; K [H][n][d]; out [H][G][n]. */
void oracle_logits_batch(const float *q, const uint16_t *K, int H, int G, int n, int d,
                         double sm_scale, double *out)
{
#pragma omp parallel for collapse(2) schedule(dynamic, 1)
    for (int h = 0; h < H; ++h)
        for (int g = 0; g < G; ++g)
            oracle_logits(q + ((size_t)h * G + g) * d, K + (size_t)h * n * d, n, d,
                          sm_scale, out + ((size_t)h * G + g) * n);
}
