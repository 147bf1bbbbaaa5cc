// C-ABI entry points of libfathom.so: argument checks on the host (nothing is enqueued
// when they fail), device-visibility checks of the pointers, then the launches.
#include <cstddef>
#include <algorithm>
#include <cstring>
#include <mutex>

#include "common.h"

using namespace fathom;

namespace {

thread_local int g_last_hip = 0;

int hip_status(hipError_t e) {
    if (e == hipSuccess) return FATHOM_OK;
    g_last_hip = (int)e;
    return FATHOM_ERR_HIP;
}

bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

size_t round256(size_t x) { return (x + 255) / 256 * 256; }

// The GPU must be able to dereference p: device memory, or host memory that HIP has
// pinned and mapped (hipHostMalloc / torch pinned tensors).
int check_visible(const void *p) {
    if (!p) return FATHOM_ERR_INVALID_ARG;
    hipPointerAttribute_t attr;
    std::memset(&attr, 0, sizeof attr);
    const hipError_t e = hipPointerGetAttributes(&attr, p);
    if (e != hipSuccess) {
        (void)hipGetLastError();  // clear the sticky error of an unknown pointer
        return FATHOM_ERR_NOT_MAPPED;
    }
    if (attr.type == hipMemoryTypeDevice || attr.type == hipMemoryTypeManaged ||
        attr.type == hipMemoryTypeArray)
        return FATHOM_OK;
    if (attr.type == hipMemoryTypeHost && attr.devicePointer == p) return FATHOM_OK;
    return FATHOM_ERR_NOT_MAPPED;
}

// p is pinned host memory mapped for the GPU (read over the host link).
bool is_pinned_host(const void *p) {
    hipPointerAttribute_t attr;
    std::memset(&attr, 0, sizeof attr);
    if (hipPointerGetAttributes(&attr, p) != hipSuccess) {
        (void)hipGetLastError();
        return false;
    }
    return attr.type == hipMemoryTypeHost;
}

int check_all(std::initializer_list<const void *> ptrs) {
    for (const void *p : ptrs) {
        if (!p) continue;
        const int rc = check_visible(p);
        if (rc != FATHOM_OK) return rc;
    }
    return FATHOM_OK;
}

int check_store(const fathom_store *st) {
    if (!st) return FATHOM_ERR_INVALID_ARG;
    if (st->n_heads < 1 || st->n_heads > 65535 || st->n_tokens < 1)
        return FATHOM_ERR_INVALID_ARG;
    if (st->word_stride < (st->n_tokens + 31) / 32 || (st->word_stride & 3) != 0)
        return FATHOM_ERR_INVALID_ARG;
    if (!st->planes || !st->scale || !st->zero || !st->var) return FATHOM_ERR_INVALID_ARG;
    if (!aligned(st->planes, 16) || !aligned(st->scale, 4) || !aligned(st->zero, 4) ||
        !aligned(st->var, 4))
        return FATHOM_ERR_INVALID_ARG;
    if (st->d != FATHOM_D) return FATHOM_ERR_UNSUPPORTED;
    return FATHOM_OK;
}

int check_g(int G) {
    if (G < 1) return FATHOM_ERR_INVALID_ARG;
    if (G > FATHOM_MAX_G) return FATHOM_ERR_UNSUPPORTED;
    return FATHOM_OK;
}

int check_topk_k(int n, int k) {
    if (n < 1 || k < 1 || k > n) return FATHOM_ERR_INVALID_ARG;
    if (n > FATHOM_TOPK_CHUNK && k > FATHOM_TOPK_CHUNK / 2) return FATHOM_ERR_UNSUPPORTED;
    return FATHOM_OK;
}

size_t step_ws_bytes(int H, int G, int n, int k) {
    // the score area holds every score (full path) or the candidate records (filtering
    // path), whose rows are rounded up to whole 256-token blocks
    return round256(scan_ws_bytes(H, G)) + round256(cand_bytes(H, G, n)) +
           round256(topk_ws_bytes(H * G, n, k)) + round256((size_t)H * G * k * sizeof(int32_t)) +
           round256((size_t)H * FATHOM_D) + round256(filter_mask_bytes(H, G, n)) +
           round256(filter_redo_bytes(H, G, n)) + round256(attn_part_bytes(H * G));
}

// the grouped step: every score, the top-k levels, the winners, the depths, then the split
// attention's parts and per-row counters
size_t step_grouped_ws_bytes(int H, int G, int n, int k) {
    return round256((size_t)H * G * n * sizeof(float)) + round256(topk_ws_bytes(H * G, n, k)) +
           round256((size_t)H * G * k * sizeof(int32_t)) + round256((size_t)H * FATHOM_D) +
           round256(attn_part_bytes(H * G)) + round256((size_t)H * G * sizeof(uint32_t));
}

size_t scan_topk_ws_bytes(int H, int G, int n, int k) {
    return round256(scan_ws_bytes(H, G)) + round256(cand_bytes(H, G, n)) +
           round256(filter_mask_bytes(H, G, n)) + round256(topk_ws_bytes(H * G, n, k)) +
           round256(filter_redo_bytes(H, G, n));
}

hipStream_t as_stream(void *s) { return static_cast<hipStream_t>(s); }

// The workspace of fathom_step_noalloc: device memory the library owns, one copy on
// each GPU that loads it.  In host code this name stands for a host-side shadow, not a
// device address; the device address comes from hipGetSymbolAddress (scratch_address)
// and only that address is ever passed to kernels.
static __device__ __align__(256) unsigned char scratch[FATHOM_STATIC_SCRATCH_BYTES];

// Device address of the current device's scratch array, looked up once per device.
int scratch_address(void **out) {
    static std::mutex mu;
    static void *addr[64] = {};
    int dev = -1;
    const hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_status(e);
    if (dev < 0 || dev >= 64) return FATHOM_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void *p = nullptr;
        const hipError_t g = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (g != hipSuccess) return hip_status(g);
        if (!p) return hip_status(hipErrorInvalidSymbol);
        addr[dev] = p;
    }
    *out = addr[dev];
    return FATHOM_OK;
}

#define FATHOM_TRY(expr)                                                                 \
    do {                                                                                 \
        const int rc__ = (expr);                                                         \
        if (rc__ != FATHOM_OK) return rc__;                                              \
    } while (0)

}  // namespace

extern "C" {

int fathom_version(void) { return FATHOM_VERSION; }

int32_t fathom_word_stride(int32_t n_tokens) {
    constexpr int64_t kPageWords = 1024;  // 4 KiB
    const int64_t W = ((int64_t)std::max<int32_t>(n_tokens, 1) + 31) / 32;
    if (W < 16 * kPageWords) return (int32_t)((W + 3) / 4 * 4);
    const int64_t pages = ((W + kPageWords - 1) / kPageWords) | 1;  // odd
    return (int32_t)(pages * kPageWords);
}

int fathom_last_hip_error(void) { return g_last_hip; }

const char *fathom_status_string(int status) {
    switch (status) {
    case FATHOM_OK: return "ok";
    case FATHOM_ERR_INVALID_ARG: return "invalid argument (null pointer, size or alignment)";
    case FATHOM_ERR_BUDGET: return "bit budget outside [0, 4d]";
    case FATHOM_ERR_UNSUPPORTED: return "unsupported shape (d != 128, G > 8 or k too large)";
    case FATHOM_ERR_WORKSPACE: return "workspace too small";
    case FATHOM_ERR_NOT_MAPPED: return "pointer not accessible by the GPU";
    case FATHOM_ERR_HIP: return "HIP runtime error";
    case FATHOM_ERR_SCRATCH: return "problem needs more than the 64 MiB static scratch";
    default: return "unknown status";
    }
}

int fathom_workspace_size(int op, int H, int G, int n, int k, size_t *bytes) {
    if (!bytes) return FATHOM_ERR_INVALID_ARG;
    *bytes = 0;
    switch (op) {
    case FATHOM_OP_QUANTIZE:
        if (H < 1 || n < 1) return FATHOM_ERR_INVALID_ARG;
        *bytes = quantize_ws_bytes(H, n);
        return FATHOM_OK;
    case FATHOM_OP_SCAN:
        if (H < 1) return FATHOM_ERR_INVALID_ARG;
        FATHOM_TRY(check_g(G));
        *bytes = scan_ws_bytes(H, G);
        return FATHOM_OK;
    case FATHOM_OP_TOPK:
        if (H < 1) return FATHOM_ERR_INVALID_ARG;
        FATHOM_TRY(check_topk_k(n, k));
        *bytes = topk_ws_bytes(H, n, k);
        return FATHOM_OK;
    case FATHOM_OP_STEP:
        if (H < 1) return FATHOM_ERR_INVALID_ARG;
        FATHOM_TRY(check_g(G));
        FATHOM_TRY(check_topk_k(n, k));
        *bytes = step_ws_bytes(H, G, n, k);
        return FATHOM_OK;
    case FATHOM_OP_SCAN_TOPK:
        if (H < 1) return FATHOM_ERR_INVALID_ARG;
        FATHOM_TRY(check_g(G));
        FATHOM_TRY(check_topk_k(n, k));
        *bytes = scan_topk_ws_bytes(H, G, n, k);
        return FATHOM_OK;
    case FATHOM_OP_STEP_GROUPED:
        if (H < 1) return FATHOM_ERR_INVALID_ARG;
        FATHOM_TRY(check_g(G));
        FATHOM_TRY(check_topk_k(n, k));
        *bytes = step_grouped_ws_bytes(H, G, n, k);
        return FATHOM_OK;
    default: return FATHOM_ERR_INVALID_ARG;
    }
}

int fathom_quantize_store(const float *keys, int H, int n, int d, const fathom_store *st,
                          void *ws, size_t ws_bytes, void *stream) {
    if (!keys || !aligned(keys, 16)) return FATHOM_ERR_INVALID_ARG;
    FATHOM_TRY(check_store(st));
    if (H != st->n_heads || n != st->n_tokens) return FATHOM_ERR_INVALID_ARG;
    if (d != FATHOM_D) return FATHOM_ERR_UNSUPPORTED;
    if (!ws || !aligned(ws, 16)) return FATHOM_ERR_INVALID_ARG;
    if (ws_bytes < quantize_ws_bytes(H, n)) return FATHOM_ERR_WORKSPACE;
    FATHOM_TRY(check_all({keys, st->planes, st->scale, st->zero, st->var, ws}));
    return hip_status(launch_quantize_store(keys, H, n, *st, ws, as_stream(stream)));
}

int fathom_plan(const fathom_store *st, const float *q, int G, int B, uint8_t *depth,
                void *stream) {
    FATHOM_TRY(check_store(st));
    if (!q || !depth || !aligned(q, 16)) return FATHOM_ERR_INVALID_ARG;
    FATHOM_TRY(check_g(G));
    if (B < 0 || B > FATHOM_D * FATHOM_PLANES) return FATHOM_ERR_BUDGET;
    FATHOM_TRY(check_all({st->var, q, depth}));
    return hip_status(launch_plan(*st, q, G, B, depth, as_stream(stream)));
}

int fathom_plan_fixed(const fathom_store *st, int n_channels, uint8_t *depth, void *stream) {
    FATHOM_TRY(check_store(st));
    if (!depth) return FATHOM_ERR_INVALID_ARG;
    if (n_channels < 0 || n_channels > FATHOM_D) return FATHOM_ERR_BUDGET;
    FATHOM_TRY(check_all({st->var, depth}));
    return hip_status(launch_plan_fixed(*st, n_channels, depth, as_stream(stream)));
}

static int scan_common(const fathom_store *st, int G, void *ws, size_t ws_bytes) {
    FATHOM_TRY(check_store(st));
    FATHOM_TRY(check_g(G));
    if (!ws || !aligned(ws, 16)) return FATHOM_ERR_INVALID_ARG;
    if (ws_bytes < scan_ws_bytes(st->n_heads, G)) return FATHOM_ERR_WORKSPACE;
    return FATHOM_OK;
}

int fathom_scan_prepare(const fathom_store *st, const float *q, int G, const uint8_t *depth,
                        void *ws, size_t ws_bytes, void *stream) {
    FATHOM_TRY(scan_common(st, G, ws, ws_bytes));
    if (!q || !depth || !aligned(q, 16)) return FATHOM_ERR_INVALID_ARG;
    FATHOM_TRY(check_all({q, depth, st->scale, st->zero, ws}));
    return hip_status(launch_scan_prepare(*st, q, G, depth, 0, ws, as_stream(stream)));
}

int fathom_scan_prepared(const fathom_store *st, int G, float *scores, void *ws,
                         size_t ws_bytes, void *stream) {
    FATHOM_TRY(scan_common(st, G, ws, ws_bytes));
    if (!scores || !aligned(scores, 16)) return FATHOM_ERR_INVALID_ARG;
    FATHOM_TRY(check_all({st->planes, scores, ws}));
    return hip_status(launch_scan_main(*st, G, scores, ws, as_stream(stream)));
}

int fathom_scan_extract(const fathom_store *st, const float *q, int G, const uint8_t *depth,
                        float *scores, void *stream) {
    FATHOM_TRY(check_store(st));
    FATHOM_TRY(check_g(G));
    if (!q || !depth || !scores || !aligned(q, 4) || !aligned(scores, 4))
        return FATHOM_ERR_INVALID_ARG;
    FATHOM_TRY(check_all({q, depth, st->planes, st->scale, st->zero, scores}));
    return hip_status(launch_scan_extract(*st, q, G, depth, scores, as_stream(stream)));
}

static int check_gstore(const fathom_gstore *gs) {
    if (!gs || gs->n_heads < 1 || gs->n_tokens < 1 || !gs->planes || !gs->scale16 ||
        !gs->zero16 || !gs->sums || !gs->var || !gs->prefix || !gs->prefix_groups ||
        gs->pad != 0)
        return FATHOM_ERR_INVALID_ARG;
    if (gs->d != FATHOM_D) return FATHOM_ERR_UNSUPPORTED;
    const int ng = (gs->n_tokens + FATHOM_GROUP - 1) / FATHOM_GROUP;
    if (gs->word_stride < 4 * ng || (gs->word_stride & 3) || gs->group_stride < ng)
        return FATHOM_ERR_INVALID_ARG;
    if (!aligned(gs->planes, 16) || !aligned(gs->scale16, 8) || !aligned(gs->zero16, 8) ||
        !aligned(gs->sums, 8) || !aligned(gs->var, 4) || !aligned(gs->prefix, 16) ||
        !aligned(gs->prefix_groups, 4))
        return FATHOM_ERR_INVALID_ARG;
    return check_all({gs->planes, gs->scale16, gs->zero16, gs->sums, gs->var, gs->prefix,
                      gs->prefix_groups});
}

int fathom_quantize_groups(const float *keys, int64_t keys_head_stride, const fathom_gstore *gs,
                           int g0, int g1, void *stream) {
    FATHOM_TRY(check_gstore(gs));
    const int n = gs->n_tokens, ng = (n + FATHOM_GROUP - 1) / FATHOM_GROUP;
    if (!keys || !aligned(keys, 16) || g0 < 0 || g1 <= g0 || g1 > ng)
        return FATHOM_ERR_INVALID_ARG;
    const int64_t m = (int64_t)std::min(n, FATHOM_GROUP * g1) - (int64_t)FATHOM_GROUP * g0;
    if (keys_head_stride % 4 != 0 || (gs->n_heads > 1 && keys_head_stride < m * FATHOM_D))
        return FATHOM_ERR_INVALID_ARG;
    FATHOM_TRY(check_all({keys}));
    return hip_status(launch_quantize_groups(keys, keys_head_stride, *gs, g0, g1,
                                             as_stream(stream)));
}

int fathom_plan_grouped(const fathom_gstore *gs, const float *q, int G, int B, uint8_t *depth,
                        void *stream) {
    FATHOM_TRY(check_gstore(gs));
    FATHOM_TRY(check_g(G));
    if (!q || !depth || !aligned(q, 4)) return FATHOM_ERR_INVALID_ARG;
    if (B < 0 || B > FATHOM_D * FATHOM_PLANES) return FATHOM_ERR_BUDGET;
    FATHOM_TRY(check_all({q, depth}));
    fathom_store view{};
    view.n_heads = gs->n_heads;
    view.n_tokens = gs->n_tokens;
    view.d = gs->d;
    view.word_stride = gs->word_stride;
    view.planes = gs->planes;
    view.var = gs->var;
    return hip_status(launch_plan(view, q, G, B, depth, as_stream(stream)));
}

int fathom_scan_grouped(const fathom_gstore *gs, const float *q, int G, const uint8_t *depth,
                        float *scores, void *stream) {
    FATHOM_TRY(check_gstore(gs));
    FATHOM_TRY(check_g(G));
    if (!q || !depth || !scores || !aligned(q, 4) || !aligned(scores, 4))
        return FATHOM_ERR_INVALID_ARG;
    FATHOM_TRY(check_all({q, depth, scores}));
    return hip_status(launch_scan_grouped(*gs, q, depth, G, scores, is_pinned_host(gs->planes),
                                          as_stream(stream)));
}

int fathom_step_grouped(const fathom_gstore *gs, const float *q, const uint16_t *K,
                        const uint16_t *V, int G, int B, int k, float sm_scale, uint16_t *out,
                        uint8_t *depth_out, float *scores_out, int32_t *idx_out, void *ws,
                        size_t ws_bytes, void *stream) {
    FATHOM_TRY(check_gstore(gs));
    if (!q || !K || !V || !out || !ws) return FATHOM_ERR_INVALID_ARG;
    if (!aligned(q, 16) || !aligned(K, 16) || !aligned(V, 16) || !aligned(out, 2) ||
        !aligned(ws, 16) || (scores_out && !aligned(scores_out, 16)) ||
        (idx_out && !aligned(idx_out, 4)))
        return FATHOM_ERR_INVALID_ARG;
    FATHOM_TRY(check_g(G));
    if (B < 0 || B > FATHOM_D * FATHOM_PLANES) return FATHOM_ERR_BUDGET;
    const int H = gs->n_heads, n = gs->n_tokens;
    FATHOM_TRY(check_topk_k(n, k));
    if (ws_bytes < step_grouped_ws_bytes(H, G, n, k)) return FATHOM_ERR_WORKSPACE;
    FATHOM_TRY(check_all({q, K, V, out, depth_out, scores_out, idx_out, ws}));

    char *w = static_cast<char *>(ws);
    float *scores = scores_out ? scores_out : reinterpret_cast<float *>(w);
    w += round256((size_t)H * G * n * sizeof(float));
    void *topk_ws = w;
    w += round256(topk_ws_bytes(H * G, n, k));
    int32_t *idx = idx_out ? idx_out : reinterpret_cast<int32_t *>(w);
    w += round256((size_t)H * G * k * sizeof(int32_t));
    uint8_t *depth = depth_out ? depth_out : reinterpret_cast<uint8_t *>(w);
    w += round256((size_t)H * FATHOM_D);
    float *part = reinterpret_cast<float *>(w);
    w += round256(attn_part_bytes(H * G));
    uint32_t *count = reinterpret_cast<uint32_t *>(w);  // cleared by the plan

    fathom_store view{};  // the plan reads planes' shape and var only
    view.n_heads = H;
    view.n_tokens = n;
    view.d = gs->d;
    view.word_stride = gs->word_stride;
    view.planes = gs->planes;
    view.var = gs->var;
    const hipStream_t s = as_stream(stream);
    FATHOM_TRY(hip_status(launch_plan(view, q, G, B, depth, s, count)));
    FATHOM_TRY(hip_status(
        launch_scan_grouped(*gs, q, depth, G, scores, is_pinned_host(gs->planes), s)));
    FATHOM_TRY(hip_status(launch_topk(scores, H * G, n, k, idx, topk_ws, s)));
    // few rows from device memory: each row's attention split over several workgroups (the
    // same output bits as one workgroup a row)
    if (is_pinned_host(K) || is_pinned_host(V))
        return hip_status(launch_sparse_attn(q, K, V, H, G, n, idx, k, sm_scale, out, s));
    return hip_status(
        launch_sparse_attn_split(q, K, V, H, G, n, idx, k, sm_scale, out, part, count, G, s));
}

int fathom_pack_nibbles(const fathom_store *st, uint8_t *nib, void *stream) {
    FATHOM_TRY(check_store(st));
    if (!nib || !aligned(nib, 16)) return FATHOM_ERR_INVALID_ARG;
    FATHOM_TRY(check_all({st->planes, nib}));
    return hip_status(launch_pack_nibbles(*st, nib, as_stream(stream)));
}

int fathom_scan_nibble(const uint8_t *nib, const float *scale, const float *zero, int H, int n,
                       const float *q, int G, float *scores, void *stream) {
    if (!nib || !scale || !zero || !q || !scores || H < 1 || n < 1) return FATHOM_ERR_INVALID_ARG;
    FATHOM_TRY(check_g(G));
    if (!aligned(nib, 16) || !aligned(q, 4) || !aligned(scores, 4) || !aligned(scale, 4) ||
        !aligned(zero, 4))
        return FATHOM_ERR_INVALID_ARG;
    FATHOM_TRY(check_all({nib, scale, zero, q, scores}));
    return hip_status(launch_scan_nibble(nib, scale, zero, H, n, q, G, scores, as_stream(stream)));
}

int fathom_scan(const fathom_store *st, const float *q, int G, const uint8_t *depth,
                float *scores, void *ws, size_t ws_bytes, void *stream) {
    FATHOM_TRY(scan_common(st, G, ws, ws_bytes));
    if (!q || !depth || !scores || !aligned(q, 16) || !aligned(scores, 16))
        return FATHOM_ERR_INVALID_ARG;
    FATHOM_TRY(check_all({q, depth, st->planes, st->scale, st->zero, scores, ws}));
    const hipStream_t s = as_stream(stream);
    FATHOM_TRY(hip_status(launch_scan_prepare(*st, q, G, depth, 0, ws, s)));
    return hip_status(launch_scan_main(*st, G, scores, ws, s));
}

int fathom_scan_topk(const fathom_store *st, const float *q, int G, const uint8_t *depth,
                     int k, int32_t *idx, void *ws, size_t ws_bytes, void *stream) {
    FATHOM_TRY(check_store(st));
    FATHOM_TRY(check_g(G));
    if (!q || !depth || !idx || !ws || !aligned(q, 16) || !aligned(idx, 4) || !aligned(ws, 16))
        return FATHOM_ERR_INVALID_ARG;
    const int H = st->n_heads, n = st->n_tokens;
    FATHOM_TRY(check_topk_k(n, k));
    if (ws_bytes < scan_topk_ws_bytes(H, G, n, k)) return FATHOM_ERR_WORKSPACE;
    FATHOM_TRY(check_all({q, depth, st->planes, st->scale, st->zero, idx, ws}));
    char *w = static_cast<char *>(ws);
    void *scan_ws = w;
    w += round256(scan_ws_bytes(H, G));
    float *cand = reinterpret_cast<float *>(w);
    w += round256(cand_bytes(H, G, n));
    uint32_t *masks = reinterpret_cast<uint32_t *>(w);
    w += round256(filter_mask_bytes(H, G, n));
    void *topk_ws = w;
    w += round256(topk_ws_bytes(H * G, n, k));
    uint32_t *redo = reinterpret_cast<uint32_t *>(w);
    const hipStream_t s = as_stream(stream);
    if (sample_rank(n, k) == 0) {  // no threshold possible (k too close to n): scan all
        FATHOM_TRY(hip_status(launch_scan_prepare(*st, q, G, depth, 0, scan_ws, s)));
        FATHOM_TRY(hip_status(launch_scan_main(*st, G, cand, scan_ws, s)));
        return hip_status(launch_topk(cand, H * G, n, k, idx, topk_ws, s));
    }
    FATHOM_TRY(hip_status(launch_scan_prepare(*st, q, G, depth, k, scan_ws, s)));
    FATHOM_TRY(hip_status(launch_scan_main(*st, G, cand, scan_ws, s, masks)));
    return hip_status(
        launch_topk_filtered(*st, G, cand, masks, scan_ws, redo, k, idx, topk_ws, s));
}

int fathom_topk(const float *scores, int R, int n, int k, int32_t *idx, void *ws,
                size_t ws_bytes, void *stream) {
    if (!scores || !idx || !aligned(scores, 16) || !aligned(idx, 4) || R < 1)
        return FATHOM_ERR_INVALID_ARG;
    FATHOM_TRY(check_topk_k(n, k));
    const size_t need = topk_ws_bytes(R, n, k);
    if (need > 0 && (!ws || !aligned(ws, 16))) return FATHOM_ERR_INVALID_ARG;
    if (ws_bytes < need) return FATHOM_ERR_WORKSPACE;
    FATHOM_TRY(check_all({scores, idx, need > 0 ? ws : nullptr}));
    return hip_status(launch_topk(scores, R, n, k, idx, ws, as_stream(stream)));
}

int fathom_sparse_attn(const float *q, const uint16_t *K, const uint16_t *V, int H, int G,
                       int n, int d, const int32_t *idx, int k, float sm_scale,
                       uint16_t *out, void *stream) {
    if (!q || !K || !V || !idx || !out) return FATHOM_ERR_INVALID_ARG;
    if (!aligned(q, 16) || !aligned(K, 16) || !aligned(V, 16) || !aligned(idx, 4) ||
        !aligned(out, 2))
        return FATHOM_ERR_INVALID_ARG;
    if (H < 1 || n < 1 || k < 1 || k > n) return FATHOM_ERR_INVALID_ARG;
    FATHOM_TRY(check_g(G));
    if (d != FATHOM_D) return FATHOM_ERR_UNSUPPORTED;
    FATHOM_TRY(check_all({q, K, V, idx, out}));
    return hip_status(
        launch_sparse_attn(q, K, V, H, G, n, idx, k, sm_scale, out, as_stream(stream)));
}

// The step; with ev non-null, ev[0..FATHOM_STEP_PHASES] are recorded on the stream at
// the phase boundaries (before the plan, after the plan and scan preparation, after the
// scan, after the select, after the attention).
static int step_impl(const fathom_store *st, const float *q, const uint16_t *K,
                     const uint16_t *V, int G, int B, int k, float sm_scale, uint16_t *out,
                     uint8_t *depth_out, float *scores_out, int32_t *idx_out, void *ws,
                     size_t ws_bytes, void *stream, const hipEvent_t *ev) {
    FATHOM_TRY(check_store(st));
    if (!q || !K || !V || !out || !ws) return FATHOM_ERR_INVALID_ARG;
    if (!aligned(q, 16) || !aligned(K, 16) || !aligned(V, 16) || !aligned(out, 2) ||
        !aligned(ws, 16) || (scores_out && !aligned(scores_out, 16)) ||
        (idx_out && !aligned(idx_out, 4)))
        return FATHOM_ERR_INVALID_ARG;
    FATHOM_TRY(check_g(G));
    if (B < 0 || B > FATHOM_D * FATHOM_PLANES) return FATHOM_ERR_BUDGET;
    const int H = st->n_heads, n = st->n_tokens;
    FATHOM_TRY(check_topk_k(n, k));
    if (ws_bytes < step_ws_bytes(H, G, n, k)) return FATHOM_ERR_WORKSPACE;
    FATHOM_TRY(check_all({st->planes, st->scale, st->zero, st->var, q, K, V, out, depth_out,
                          scores_out, idx_out, ws}));

    char *w = static_cast<char *>(ws);
    void *scan_ws = w;
    w += round256(scan_ws_bytes(H, G));
    float *scores = reinterpret_cast<float *>(w);  // every score, or candidate records
    w += round256(cand_bytes(H, G, n));
    void *topk_ws = w;
    w += round256(topk_ws_bytes(H * G, n, k));
    int32_t *idx = idx_out ? idx_out : reinterpret_cast<int32_t *>(w);
    w += round256((size_t)H * G * k * sizeof(int32_t));
    uint8_t *depth = depth_out ? depth_out : reinterpret_cast<uint8_t *>(w);
    w += round256((size_t)H * FATHOM_D);
    uint32_t *masks = reinterpret_cast<uint32_t *>(w);
    w += round256(filter_mask_bytes(H, G, n));
    uint32_t *redo = reinterpret_cast<uint32_t *>(w);
    w += round256(filter_redo_bytes(H, G, n));
    float *part = reinterpret_cast<float *>(w);  // the split attention's partial results

    const hipStream_t s = as_stream(stream);
    auto mark = [&](int i) { return ev ? hip_status(hipEventRecord(ev[i], s)) : FATHOM_OK; };
    // every score is asked for, or no threshold can help (k too close to n for the
    // sample, or B = 0: every score of a row is the same), or the heads read more than
    // 480 planes (the filter keeps no records for them): scan all, then select
    const bool full = scores_out || sample_rank(n, k) == 0 || B == 0 || B > 480;
    // K/V rows read from pinned host memory: one attention workgroup a row, which the link
    // serves better than a row split over several (8.4 MB of a 1M-token layer's rows: 154
    // against 171 us split), so select and attention stay separate launches
    const bool host_kv = is_pinned_host(K) || is_pinned_host(V);
    FATHOM_TRY(mark(0));
    const bool fused_front = !full && filtered_direct_applies(H * G, n, k) &&
                             front_fused_applies(*st, G);
    if (fused_front) {
        // few heads of one-chunk rows (a layer of a decode step): plan, prepare and the
        // filtering scan in one kernel; the plan-prepare phase holds it, the scan phase is
        // empty
        FATHOM_TRY(hip_status(
            launch_front_fused(*st, q, G, B, k, depth, scan_ws, scores, masks, s)));
        FATHOM_TRY(mark(1));
        FATHOM_TRY(mark(2));
    } else {
        FATHOM_TRY(
            hip_status(launch_plan_prepare(*st, q, G, B, full ? 0 : k, depth, scan_ws, s)));
        FATHOM_TRY(mark(1));
        if (full) {
            float *all = scores_out ? scores_out : scores;
            FATHOM_TRY(hip_status(launch_scan_main(*st, G, all, scan_ws, s)));
            FATHOM_TRY(mark(2));
            FATHOM_TRY(hip_status(launch_topk(all, H * G, n, k, idx, topk_ws, s)));
        } else {  // the filtering scan keeps the candidates only
            FATHOM_TRY(hip_status(launch_scan_main(*st, G, scores, scan_ws, s, masks)));
            FATHOM_TRY(mark(2));
        }
    }
    if (!full) {
        if (filtered_attend_applies(H * G, n, k) && !host_kv) {
            // as many rows as fill the CUs once (a layer of a decode step): select and
            // attention in one kernel; its time falls in the select phase, the attention
            // phase is empty
            FATHOM_TRY(hip_status(launch_topk_filtered_attend(
                *st, G, scores, masks, scan_ws, k, idx, q, K, V, sm_scale, out, part, s)));
            FATHOM_TRY(mark(3));
            return mark(4);
        }
        FATHOM_TRY(hip_status(
            launch_topk_filtered(*st, G, scores, masks, scan_ws, redo, k, idx, topk_ws, s)));
    }
    FATHOM_TRY(mark(3));
    // few rows from device memory: each row's attention split over several workgroups
    if (host_kv)
        FATHOM_TRY(hip_status(launch_sparse_attn(q, K, V, H, G, n, idx, k, sm_scale, out, s)));
    else
        FATHOM_TRY(hip_status(launch_sparse_attn_split(
            q, K, V, H, G, n, idx, k, sm_scale, out, part,
            reinterpret_cast<uint32_t *>(static_cast<char *>(scan_ws) +
                                         offsetof(ScanMeta, attn_done)),
            (int)(kMetaBytes / sizeof(uint32_t)), s)));
    return mark(4);
}

int fathom_step(const fathom_store *st, const float *q, const uint16_t *K, const uint16_t *V,
                int G, int B, int k, float sm_scale, uint16_t *out, uint8_t *depth_out,
                float *scores_out, int32_t *idx_out, void *ws, size_t ws_bytes,
                void *stream) {
    return step_impl(st, q, K, V, G, B, k, sm_scale, out, depth_out, scores_out, idx_out, ws,
                     ws_bytes, stream, nullptr);
}

int fathom_step_noalloc(const fathom_store *st, const float *q, const uint16_t *K,
                        const uint16_t *V, int G, int B, int k, float sm_scale, uint16_t *out,
                        uint8_t *depth_out, float *scores_out, int32_t *idx_out,
                        void *stream) {
    FATHOM_TRY(check_store(st));
    FATHOM_TRY(check_g(G));
    FATHOM_TRY(check_topk_k(st->n_tokens, k));
    if (B < 0 || B > FATHOM_D * FATHOM_PLANES) return FATHOM_ERR_BUDGET;
    if (step_ws_bytes(st->n_heads, G, st->n_tokens, k) > FATHOM_STATIC_SCRATCH_BYTES)
        return FATHOM_ERR_SCRATCH;
    if (!q || !K || !V || !out) return FATHOM_ERR_INVALID_ARG;
    void *ws = nullptr;
    FATHOM_TRY(scratch_address(&ws));
    return step_impl(st, q, K, V, G, B, k, sm_scale, out, depth_out, scores_out, idx_out, ws,
                     FATHOM_STATIC_SCRATCH_BYTES, stream, nullptr);
}

int fathom_step_timed(const fathom_store *st, const float *q, const uint16_t *K,
                      const uint16_t *V, int G, int B, int k, float sm_scale, uint16_t *out,
                      uint8_t *depth_out, float *scores_out, int32_t *idx_out, void *ws,
                      size_t ws_bytes, void *stream, void *const *events, int n_events) {
    if (!events || n_events != FATHOM_STEP_PHASES + 1) return FATHOM_ERR_INVALID_ARG;
    hipEvent_t ev[FATHOM_STEP_PHASES + 1];
    for (int i = 0; i <= FATHOM_STEP_PHASES; ++i) {
        if (!events[i]) return FATHOM_ERR_INVALID_ARG;
        ev[i] = static_cast<hipEvent_t>(events[i]);
    }
    return step_impl(st, q, K, V, G, B, k, sm_scale, out, depth_out, scores_out, idx_out, ws,
                     ws_bytes, stream, ev);
}

int fathom_stream_read(const void *src, size_t bytes, uint64_t *sink, void *stream) {
    if (!src || !sink || bytes == 0 || bytes % 16 != 0 || !aligned(src, 16) ||
        !aligned(sink, 8))
        return FATHOM_ERR_INVALID_ARG;
    FATHOM_TRY(check_all({src, sink}));
    return hip_status(launch_stream_read(src, bytes, sink, as_stream(stream)));
}

int fathom_stream_read_runs(const void *src, size_t run_bytes, size_t stride_bytes,
                            size_t n_runs, uint64_t *sink, void *stream) {
    if (!src || !sink || run_bytes == 0 || run_bytes % 16 != 0 || n_runs == 0 ||
        stride_bytes < run_bytes || stride_bytes % 16 != 0 || !aligned(src, 16) ||
        !aligned(sink, 8))
        return FATHOM_ERR_INVALID_ARG;
    if ((run_bytes / 16) * (unsigned __int128)n_runs >= ((unsigned __int128)1 << 32))
        return FATHOM_ERR_UNSUPPORTED;
    FATHOM_TRY(check_all({src, sink}));
    // every byte read must lie inside src's allocation
    const size_t last = (n_runs - 1) * stride_bytes + run_bytes;  // one past the last byte
    void *base = nullptr;
    size_t size = 0;
    if (hipMemGetAddressRange(&base, &size, const_cast<void *>(src)) != hipSuccess || !base)
        return FATHOM_ERR_INVALID_ARG;
    const size_t off = (size_t)((const char *)src - (const char *)base);
    if (off > size || last > size - off) return FATHOM_ERR_INVALID_ARG;
    return hip_status(launch_stream_runs(src, run_bytes, stride_bytes, n_runs, sink,
                                         as_stream(stream)));
}

int fathom_host_alloc(size_t bytes, int flags, void **ptr) {
    if (!ptr || bytes == 0 || (flags != 0 && flags != 1)) return FATHOM_ERR_INVALID_ARG;
    *ptr = nullptr;
    const unsigned f = flags == 1 ? (hipHostMallocMapped | hipHostMallocNonCoherent)
                                  : (hipHostMallocMapped | hipHostMallocCoherent);
    return hip_status(hipHostMalloc(ptr, bytes, f));
}

int fathom_host_free(void *ptr) {
    if (!ptr) return FATHOM_ERR_INVALID_ARG;
    return hip_status(hipHostFree(ptr));
}

}  // extern "C"
