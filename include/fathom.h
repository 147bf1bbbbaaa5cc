/*
 * fathom.h -- C-ABI of libfathom.so, the MI355X (gfx950) Fathom bit-plane key scan.
 *
 * The method (sources: the author's blog post on vivekkalyanarangan.hashnode.dev, by
 * section heading; the Glonce summary "Fathom speeds long-context KV cache decoding
 * 1.67x with per-query reads"; the Rootconf proposal "Decoding at a million tokens when
 * the KV cache lives in host memory"):
 *   score every cached key cheaply, take the top k, attend exactly over those k
 *   (blog, "The first fix: stop attending to everything"); the cheap scores come from a
 *   4-bit per-channel copy of K stored channel-major as bit planes, most significant
 *   plane first, so that a prefix of t planes is that channel's t-bit quantizer (blog,
 *   "Bit planes: how a partial read becomes a valid read"); each query spends a budget
 *   of B planes over the channels by reverse water-filling on the importance
 *   var_c * q_c^2 (blog, "How each query picks its own depth"; Glonce).
 *
 * Conventions for every call below.
 *   - Status: every call returns FATHOM_OK (0) or one of the FATHOM_ERR_* codes.
 *     Argument errors are found on the host before anything is enqueued; then nothing
 *     is enqueued.  A failed launch returns FATHOM_ERR_HIP and the HIP error code is
 *     available from fathom_last_hip_error() on the calling thread.
 *   - Execution: every call is asynchronous on `stream` (a hipStream_t; NULL means the
 *     default stream) and returns once its kernels are enqueued.  No call synchronizes,
 *     allocates device memory, prints, or keeps a pointer after it returns.
 *   - Memory: the caller owns every buffer, including the workspace `ws`.  Pointers are
 *     device-visible addresses: HBM, or pinned host memory the GPU can read (for the
 *     store's planes and the K/V rows, which may live in host memory).  A pointer the
 *     GPU cannot access is rejected with FATHOM_ERR_NOT_MAPPED.  Large buffers (keys,
 *     planes, scores, K, V, ws) must be 16-byte aligned; everything else 4-byte aligned
 *     (depth: 1-byte).
 *   - Shapes: H = (layer, KV head) pairs in the call, G = queries per KV head (1..8),
 *     d = channels per head (must be 128), n = tokens, B = planes per head (0..4d),
 *     k = winners per query.  All arrays are dense row-major in the order given.
 *   - Thread safety: calls may be made from several threads; the library has no state
 *     besides the per-thread last HIP error.
 */
#ifndef FATHOM_H
#define FATHOM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FATHOM_VERSION 100 /* 1.0.0 */

enum fathom_status {
    FATHOM_OK = 0,
    FATHOM_ERR_INVALID_ARG = 1, /* null pointer, bad size or misaligned buffer */
    FATHOM_ERR_BUDGET = 2,      /* B outside [0, 4d] */
    FATHOM_ERR_UNSUPPORTED = 3, /* d != 128, G > 8, or k beyond the top-k limits */
    FATHOM_ERR_WORKSPACE = 4,   /* ws too small (see fathom_workspace_size) */
    FATHOM_ERR_NOT_MAPPED = 5,  /* a pointer the GPU cannot read or write */
    FATHOM_ERR_HIP = 6,         /* a HIP runtime call or launch failed */
    FATHOM_ERR_SCRATCH = 7      /* needs more than the static scratch of fathom_step_noalloc */
};

#define FATHOM_D 128          /* channels per head this build supports */
#define FATHOM_PLANES 4       /* 4-bit codes: planes 0 (MSB) .. 3 (LSB) */
#define FATHOM_MAX_G 8        /* queries per KV head */
#define FATHOM_TOPK_CHUNK 32768 /* elements one top-k workgroup ranks at once */

/*
 * The bit-plane store of H heads (blog, "Bit planes"; Glonce: "stored channel-major as
 * bit planes").  A plain descriptor of caller-owned buffers:
 *   planes [H][d][4][word_stride] uint32: plane j of channel c of head h; plane 0 holds
 *          the most significant bit of every 4-bit code.  Word w holds tokens
 *          32w .. 32w+31, token 32w+i at bit i (least significant bit first).  Bits of
 *          tokens >= n_tokens are zero.  HBM or pinned host memory.
 *   scale, zero, var [H][d] fp32: per channel s, z and the variance of the dequantized
 *          channel z + s*code (see fathom_quantize_store).  Device memory.
 */
typedef struct fathom_store {
    int32_t n_heads;     /* H */
    int32_t n_tokens;    /* n, >= 1 */
    int32_t d;           /* channels, must be FATHOM_D */
    int32_t word_stride; /* uint32 words per plane row: >= ceil(n/32) and a multiple
                            of 4 (rows start on 16-byte boundaries) */
    uint32_t *planes;
    float *scale;
    float *zero;
    float *var;
} fathom_store;

#define FATHOM_GROUP 128      /* tokens per scale/zero group of the grouped store */

/*
 * The grouped store (a reading of the blog's "Where this does not work": the index is
 * 68 bytes per token per KV head, i.e. 4-bit codes plus 4 bytes, which one fp16 scale
 * and one fp16 zero per channel per 128-token group give).  Caller-owned buffers:
 *   planes [H][d][4][word_stride] uint32, as in fathom_store; word_stride >=
 *          4*ceil(n/128) and a multiple of 4 (whole groups of 4 words).
 *   scale16, zero16 [H][group_stride][d] fp16 bits: group G of channel c of head h
 *          (group-major, so that one group's 128 channels are 256 contiguous bytes);
 *          8-byte aligned.
 *   sums [H][d][group_stride][2] int32: the group's sum of codes and of squared codes.
 *   var [H][d] fp32: variance of the group-dequantized channel over all n tokens.
 *   prefix [H][d][2] fp64 and prefix_groups [H][d] int32: the variance's running sums
 *          (S, Q below) over the first prefix_groups groups, kept so that an append
 *          adds only the groups it changed.  Zero them before the first call.
 * group_stride >= ceil(n/128).  All device memory except planes, scale16 and zero16
 * (HBM or pinned host).
 */
typedef struct fathom_gstore {
    int32_t n_heads;      /* H */
    int32_t n_tokens;     /* n, >= 1 */
    int32_t d;            /* must be FATHOM_D */
    int32_t word_stride;  /* see above */
    int32_t group_stride; /* see above */
    int32_t pad;          /* 0 */
    uint32_t *planes;
    uint16_t *scale16;
    uint16_t *zero16;
    int32_t *sums;
    float *var;
    double *prefix;
    int32_t *prefix_groups;
} fathom_gstore;

/* Operations for fathom_workspace_size. */
enum fathom_op {
    FATHOM_OP_QUANTIZE = 0, /* fathom_quantize_store: uses H, n */
    FATHOM_OP_SCAN = 1,     /* fathom_scan / fathom_scan_prepare(d): uses H, G */
    FATHOM_OP_TOPK = 2,     /* fathom_topk: uses H as the row count R, n, k */
    FATHOM_OP_STEP = 3,     /* fathom_step: uses H, G, n, k */
    FATHOM_OP_SCAN_TOPK = 4, /* fathom_scan_topk: uses H, G, n, k */
    FATHOM_OP_STEP_GROUPED = 5 /* fathom_step_grouped: uses H, G, n, k */
};

/* Bytes of workspace `op` needs for the given sizes (0 is possible).  Status only. */
int fathom_workspace_size(int op, int H, int G, int n, int k, size_t *bytes);

/* Text for a status code (static storage). */
const char *fathom_status_string(int status);

/* The HIP error code behind the last FATHOM_ERR_HIP on the calling thread (0 if none). */
int fathom_last_hip_error(void);

/* FATHOM_VERSION of the built library. */
int fathom_version(void);

/*
 * A plane-row stride (uint32 words) for a store of n_tokens tokens, for callers that
 * allocate one (either store): ceil(n/32) rounded up to a multiple of 4; once a row is
 * 16 pages of 4 KiB or more (n >= 524288), whole 4 KiB pages, an odd number of them.
 * Host-resident scans read a few hundred bytes of each planned row at a time, and with the
 * index in pinned host memory (blog, "Where the memory lives changes the answer": there
 * bytes are time) rows a large power of two apart read slower over the link: at n = 1M
 * (32-page rows) a plan reading one plane of each of 92 channels ran at 75% of the link
 * rate, at 94% with 33-page rows; strides that leave rows unaligned to pages were slower
 * still.  Returns 4 for n < 1 (no error is reported).
 */
int32_t fathom_word_stride(int32_t n_tokens);

/*
 * Build the store from fp32 keys (blog, "How to read fewer bits per key": 4-bit
 * storage; "Bit planes": the plane layout; Glonce: 4-bit per-channel K cache).
 *   keys [H][n][d] fp32, device-visible, finite.
 * Per channel over all n tokens: s = (max - min)/15 and z = min, each one fp32
 * operation; code = clamp(floor((x - z)/s + 0.5), 0, 15) with every step an fp32
 * operation (a constant channel, s == 0, gets code 0).  The codes are packed into
 * st->planes (words from ceil(n/32) to word_stride are zeroed), and
 * var = s^2 (n*S2 - S1^2) / n^2 from the exact integer sums S1 = sum code and
 * S2 = sum code^2, evaluated in fp64 and rounded once to fp32.
 * st->n_heads == H and st->n_tokens == n are required.  ws: FATHOM_OP_QUANTIZE bytes.
 */
int fathom_quantize_store(const float *keys, int H, int n, int d, const fathom_store *st,
                          void *ws, size_t ws_bytes, void *stream);

/*
 * Per-head plan (blog, "How each query picks its own depth": reverse water-filling).
 *   q [H][G][d] fp32: the G queries that share each KV head.
 *   depth [H][d] uint8 out: planes read per channel, 0..4, summing to B per head.
 * Importance w_c = var_c * sum_g q_gc^2 in fp64 (each square exact, sum over g in
 * ascending order, then one product).  The B planes go, one at a time, to the channel
 * with the largest w_c * 4^-t_c among channels with t_c < 4 (each plane cuts a
 * channel's error by four); equal values go to the lower channel index.  Exact.
 */
int fathom_plan(const fathom_store *st, const float *q, int G, int B, uint8_t *depth,
                void *stream);

/*
 * A query-independent comparator plan: depth 4 on the `n_channels` channels with the
 * largest var (equal var: lower channel index), 0 elsewhere, i.e. 4*n_channels planes
 * per head -- the fixed-depth index of the size the blog's "The catch" section gives
 * for the 136-bit scans (n_channels = 34).  0 <= n_channels <= d.
 */
int fathom_plan_fixed(const fathom_store *st, int n_channels, uint8_t *depth,
                      void *stream);

/*
 * Approximate scores of every key from the planes each channel reads (blog, "The first
 * fix": score every key; "Bit planes": a t-plane prefix is the t-bit quantizer).
 *   q [H][G][d] fp32; depth [H][d] (any values 0..4, e.g. from fathom_plan or
 *   fathom_plan_fixed); scores [H][G][n] fp32 out.
 * For token i and query g:  score = sum_c q_gc * (z_c + s_c * m_ic), where m_ic is the
 * middle of the 4-bit codes the t_c planes read allow: p * 2^(4-t) + (2^(4-t) - 1)/2
 * with p the t-plane prefix (t = 0 reads nothing: m = 7.5).  fp32 result: the sum over
 * planes is taken exactly in integers, with each plane's weight q_gc s_c 2^(3-j) held to
 * 2^-31 of the head's largest weight, then combined with the constant term in fp32.
 * ws: FATHOM_OP_SCAN bytes.  fathom_scan = fathom_scan_prepare + fathom_scan_prepared.
 */
int fathom_scan(const fathom_store *st, const float *q, int G, const uint8_t *depth,
                float *scores, void *ws, size_t ws_bytes, void *stream);

/* First half of fathom_scan: per-head plane list, constant terms and the weights of the
 * planes in matrix-core operand form, into ws (one small kernel). */
int fathom_scan_prepare(const fathom_store *st, const float *q, int G,
                        const uint8_t *depth, void *ws, size_t ws_bytes, void *stream);

/* Second half of fathom_scan: the plane-reading kernel, using what fathom_scan_prepare
 * left in ws for the same store and G. */
int fathom_scan_prepared(const fathom_store *st, int G, float *scores, void *ws,
                         size_t ws_bytes, void *stream);

/*
 * Comparator for measurement: the same scores as fathom_scan, computed the way the blog's
 * "Where this does not work" section costs the bit-plane scan -- each bit extracted on
 * the integer units (about 2 operations per bit) to rebuild every channel's t-plane
 * prefix p, then score = C_g + sum_c A_gc p_c with A_gc = fl32(q_gc s_c) 2^(4 - t_c),
 * accumulated in fp32 over channels in ascending order.  Same arguments and layouts as
 * fathom_scan, no workspace.  Slower than fathom_scan by design.
 */
int fathom_scan_extract(const fathom_store *st, const float *q, int G, const uint8_t *depth,
                        float *scores, void *stream);

/*
 * Build and decode-time append of the grouped store (the 68-byte index the pages count,
 * read as fp16 scale and zero per 128-token group; blog, "Bit planes" for the layout):
 * (re)quantize groups g0 .. g1-1 of every head from keys, then recompute var from all
 * groups' sums.
 *   keys: fp32, head h's tokens 128*g0 .. min(n, 128*g1) - 1 at keys + h*keys_head_stride,
 *         d floats per token (keys 16-byte aligned; keys_head_stride in floats, a
 *         multiple of 4, >= (min(n,128*g1) - 128*g0)*d).
 * Per group and channel: s = (max - min)/15 and z = min in fp32, each rounded to fp16
 * (nearest, ties to even); code = clamp(floor((x - zf)/sf + 0.5), 0, 15) with zf, sf the
 * fp16 values as fp32, every step one fp32 operation (sf = 0: code 0).  A group's 4 words
 * per plane are rewritten whole (bits of tokens >= n zero).  var is recomputed as
 * (n Q - S^2)/n^2 in fp64 from S = sum_G (n_G zf + sf S1_G) and Q = sum_G (n_G zf^2 +
 * 2 zf sf S1_G + sf^2 S2_G), term by term, groups ascending, rounded once; the running
 * sums over the groups before g0 are reused from prefix when it covers no group >= g0,
 * which gives the same fp64 values as summing from group 0.
 * Build: g0 = 0, g1 = ceil(n/128).  Append one token: set n to the new count, g0 = g1 - 1
 * = (n-1)/128, keys = that group's tokens.  0 <= g0 < g1 <= ceil(n/128).
 */
int fathom_quantize_groups(const float *keys, int64_t keys_head_stride,
                           const fathom_gstore *gs, int g0, int g1, void *stream);

/*
 * Plan for the grouped store: fathom_plan with gs->var (same rule and arithmetic).
 */
int fathom_plan_grouped(const fathom_gstore *gs, const float *q, int G, int B,
                        uint8_t *depth, void *stream);

/*
 * Scan of the grouped store (blog, "Bit planes"; "How each query picks its own depth"):
 * each channel read to its depth, reconstructed at the bin midpoint with its token's
 * group scale and zero:  score_g(i) = C_gG + sum_c fl32(q_gc sf_cG) * P_c(i), P the
 * t-plane prefix times 2^(4-t), C_gG = sum_c q_gc (zf_cG + sf_cG h(t_c)) in fp64 rounded
 * once.  The sum over the planes runs on the int8 matrix cores as in fathom_scan, with
 * each weight an integer count of a power-of-two unit of its (query, group), so scores
 * are within a few fp32 ulps of that sum (1e-5 of the row's largest score).
 * q [H][G][d] fp32, depth [H][d], scores [H][G][n] fp32 out.
 */
int fathom_scan_grouped(const fathom_gstore *gs, const float *q, int G, const uint8_t *depth,
                        float *scores, void *stream);

/*
 * One decode step over the grouped store (blog, "That is the whole method", on the index
 * of "Where this does not work"): fathom_plan_grouped -> fathom_scan_grouped (every
 * score) -> fathom_topk -> fathom_sparse_attn, enqueued on `stream` with no host
 * synchronization; the same results as those four calls made in turn.
 *   q [H][G][d] fp32; K, V [H][n][d] bf16 bits (HBM or pinned host); out [H][G][d] bf16.
 *   depth_out [H][d], scores_out [H][G][n] fp32 (16-byte aligned) and idx_out [H][G][k]
 *   are optional (NULL: the intermediate lives in ws).
 *   0 <= B <= d*4 (else FATHOM_ERR_BUDGET); k as for fathom_topk.
 *   ws: FATHOM_OP_STEP_GROUPED bytes, 16-byte aligned (FATHOM_ERR_WORKSPACE if smaller).
 */
int fathom_step_grouped(const fathom_gstore *gs, const float *q, const uint16_t *K,
                        const uint16_t *V, int G, int B, int k, float sm_scale, uint16_t *out,
                        uint8_t *depth_out, float *scores_out, int32_t *idx_out, void *ws,
                        size_t ws_bytes, void *stream);

/*
 * The ordinary 4-bit layout the pages compare the bit planes against (blog, "Where this
 * does not work": a plain 4-bit scan reads each number whole).  Writes the store's codes
 * token-major, two channels a byte: nib [H][n][d/2] uint8, byte j of token i = code of
 * channel 2j | code of channel 2j+1 << 4 (64 bytes per token at d = 128).  The codes are
 * read from st->planes (all four planes), so both layouts hold the same numbers.
 * nib: device memory, 16-byte aligned, caller-owned.
 */
int fathom_pack_nibbles(const fathom_store *st, uint8_t *nib, void *stream);

/*
 * The plain 4-bit scan over that layout (the comparator of "Where this does not work"):
 * every channel read in full, score_g(i) = C_g + sum_c fl32(q_gc s_c) code_c(i), with
 * C_g = sum_c q_gc z_c in fp64 (fixed tree order, rounded once) and the channel sum in
 * fp32, ascending.  The same numbers as fathom_scan at depth 4 on every channel, up to
 * fp32 rounding.  nib [H][n][d/2] as written by fathom_pack_nibbles (16-byte aligned);
 * scale, zero [H][d] fp32 (the store's); q [H][G][d] fp32; scores [H][G][n] fp32 out.
 */
int fathom_scan_nibble(const uint8_t *nib, const float *scale, const float *zero, int H,
                       int n, const float *q, int G, float *scores, void *stream);

/*
 * Scan and top-k in one call, without writing every score (blog, "The first fix":
 * score every key, keep the top k; "That is the whole method": the scan feeds the
 * select).  Same inputs as fathom_scan; idx [H][G][k] int32 out, exactly what
 * fathom_scan followed by fathom_topk gives (same order and tie rule).
 * How: the prepare step guesses, per query, a score threshold from a sample of the
 * head's tokens; the scan writes only the scores whose key clears it, compacted, with a
 * bit mask of the kept tokens and a per-query count; the select reads only those.  A
 * threshold is safe whenever at least k tokens of the row clear it (every winner then
 * clears it); a row that kept fewer is rescored in full inside the select, from the
 * store, with the scan's own integer arithmetic, so the result never depends on the
 * guess.  1 <= k <= n, with fathom_topk's limits.  ws: FATHOM_OP_SCAN_TOPK bytes (the
 * prepared scan workspace comes first).
 */
int fathom_scan_topk(const fathom_store *st, const float *q, int G, const uint8_t *depth,
                     int k, int32_t *idx, void *ws, size_t ws_bytes, void *stream);

/*
 * Top k of each row (blog, "The first fix": take the top k).
 *   scores [R][n] fp32, finite; idx [R][k] int32 out, ascending by token index.
 * Order: score descending, then token index ascending (equal scores go to the lower
 * index; -0 equals +0).  1 <= k <= n; when n > FATHOM_TOPK_CHUNK, k must be at most
 * FATHOM_TOPK_CHUNK/2 (else FATHOM_ERR_UNSUPPORTED).  ws: FATHOM_OP_TOPK bytes.
 */
int fathom_topk(const float *scores, int R, int n, int k, int32_t *idx, void *ws,
                size_t ws_bytes, void *stream);

/*
 * Exact attention over the winners (blog, "The first fix": attention over just those k
 * tokens, reading the values for k tokens).
 *   q [H][G][d] fp32; K, V [H][n][d] bf16 bits (HBM or pinned host); idx [H][G][k]
 *   int32 in [0, n); out [H][G][d] bf16 bits.
 * l_r = sm_scale * (q_g . K[idx_r]), p = softmax(l), out = sum_r p_r V[idx_r];
 * fp32 arithmetic, output rounded to nearest-even bf16.  Rows are not deduplicated.
 */
int fathom_sparse_attn(const float *q, const uint16_t *K, const uint16_t *V, int H, int G,
                       int n, int d, const int32_t *idx, int k, float sm_scale,
                       uint16_t *out, void *stream);

/*
 * One decode step for the H heads of the store: plan -> scan -> top-k -> attention,
 * all enqueued on `stream` with no host synchronization (blog, "That is the whole
 * method"; Rootconf: sync-free accounting).  Same arguments as the calls above.
 * depth_out [H][d], scores_out [H][G][n] and idx_out [H][G][k] are optional (NULL: the
 * intermediate lives in ws).  Without scores_out the scan and the select run as in
 * fathom_scan_topk (only candidate scores are written); with it every score is written
 * and selected from.  The winners are the same either way.  ws: FATHOM_OP_STEP bytes.
 */
int fathom_step(const fathom_store *st, const float *q, const uint16_t *K,
                const uint16_t *V, int G, int B, int k, float sm_scale, uint16_t *out,
                uint8_t *depth_out, float *scores_out, int32_t *idx_out, void *ws,
                size_t ws_bytes, void *stream);

/*
 * fathom_step with its phases timed on the stream, for measuring each kernel inside a
 * running sequence of steps (blog, "The catch": what a decode step waits on is the index
 * scan, not the winner rows).  Same arguments, preconditions and results as fathom_step,
 * plus
 *   events  FATHOM_STEP_PHASES + 1 hipEvent_t handles created by the caller; events[0] is
 *           recorded before the plan, events[1] after the plan and scan preparation,
 *           events[2] after the scan, events[3] after the select, events[4] after the
 *           attention, each on `stream`, so hipEventElapsedTime(events[i], events[i+1])
 *           is phase i.  The library keeps no handle past the call.
 *   n_events must be FATHOM_STEP_PHASES + 1 (else FATHOM_ERR_INVALID_ARG; a NULL handle
 *           too).  A failed record returns FATHOM_ERR_HIP.
 */
#define FATHOM_STEP_PHASES 4
int fathom_step_timed(const fathom_store *st, const float *q, const uint16_t *K,
                      const uint16_t *V, int G, int B, int k, float sm_scale, uint16_t *out,
                      uint8_t *depth_out, float *scores_out, int32_t *idx_out, void *ws,
                      size_t ws_bytes, void *stream, void *const *events, int n_events);

/*
 * fathom_step for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation.  Same arguments,
 * preconditions and results as fathom_step, without ws / ws_bytes: the intermediates
 * live in a static device array of the library, FATHOM_STATIC_SCRATCH_BYTES (64 MiB)
 * on each GPU the library runs on, held until the process ends.  The array of the
 * current device is used (the stream must belong to it).  A problem whose
 * FATHOM_OP_STEP workspace exceeds it is refused on the host with FATHOM_ERR_SCRATCH
 * (one layer of 8 KV heads x 4 queries fits up to about 480k tokens; 288 heads x 4
 * queries up to about 12k).  The call allocates nothing and frees nothing; every value
 * its kernels need to start from zero is cleared by them.  Calls share the array:
 * calls that overlap on one GPU (other streams, other threads) race and must be
 * ordered by the caller.
 */
#define FATHOM_STATIC_SCRATCH_BYTES ((size_t)64 << 20)
int fathom_step_noalloc(const fathom_store *st, const float *q, const uint16_t *K,
                        const uint16_t *V, int G, int B, int k, float sm_scale, uint16_t *out,
                        uint8_t *depth_out, float *scores_out, int32_t *idx_out, void *stream);

/*
 * Measurement helper for the roofline denominators (blog, "One measurement worth
 * carrying around": contiguous reads from pinned host memory): streams `bytes`
 * (multiple of 16) from the device-visible address `src` (HBM or pinned host) with
 * coalesced 16-byte loads and writes a checksum to *sink (device memory, 16 bytes).
 */
int fathom_stream_read(const void *src, size_t bytes, uint64_t *sink, void *stream);

/*
 * Run-length sweep of the same measurement (blog, "One measurement worth carrying
 * around": the link rate depends on the length of the contiguous runs): reads n_runs
 * runs of run_bytes bytes, the r-th starting at src + r * stride_bytes, with 16-byte
 * loads, and writes a checksum to *sink.  run_bytes and stride_bytes are multiples of
 * 16, stride_bytes >= run_bytes, run_bytes/16 * n_runs < 2^32 (else
 * FATHOM_ERR_UNSUPPORTED).  Every byte read must lie inside the allocation holding src
 * (checked with hipMemGetAddressRange; FATHOM_ERR_INVALID_ARG otherwise).
 */
int fathom_stream_read_runs(const void *src, size_t run_bytes, size_t stride_bytes,
                            size_t n_runs, uint64_t *sink, void *stream);

/*
 * Pinned host memory the GPU can read directly (hipHostMalloc).  flags: 0 = coherent
 * (fine-grained), 1 = non-coherent (coarse-grained).  fathom_host_free releases it.
 * These are the only calls that allocate; they exist so that callers can place the
 * store or the K/V rows in host memory.
 */
int fathom_host_alloc(size_t bytes, int flags, void **ptr);
int fathom_host_free(void *ptr);

#ifdef __cplusplus
}
#endif

#endif /* FATHOM_H */
