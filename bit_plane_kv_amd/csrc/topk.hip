// Top-k select: the k largest scores of each row, equal scores to the lower token index,
// output ascending by index (blog, "The first fix": score every key, take the top k).
//
// One 1024-thread workgroup ranks one chunk of up to 32768 entries held in registers
// (32 consecutive positions per thread).  Radix select on order-preserving 32-bit keys
// (12-bit digits from just below the bits every key shares, LDS histograms; a winning bin
// of at most 64 keys ranked directly) finds the k-th largest key T and how many
// entries equal to T are needed; a block-wide scan of (greater, equal) counts in
// position order then writes the winners in index order, taking the equal entries with
// the lowest positions.  Rows longer than a chunk are cut into chunks whose top
// min(k, chunk) survive as (value, index) candidates, in index order, for the next
// level, until one chunk remains.
#include <mutex>

#include "attn_device.h"
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
    uint32_t c4[4] = {0u, 0u, 0u, 0u};
    // thread t owns bins nb-1-4t .. nb-4-4t, highest first: one aligned 16-byte piece
    // (word by word, lanes 16 bytes apart conflict 4-way on the banks)
    const int lo = nb - 4 - 4 * tid;
    if (lo >= 0) {
        const uint4 x = *reinterpret_cast<const uint4 *>(&hist[lo]);
        c4[0] = x.w;
        c4[1] = x.z;
        c4[2] = x.y;
        c4[3] = x.x;
    }
    const uint32_t local = c4[0] + c4[1] + c4[2] + c4[3];
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

// A radix pass that leaves at most this many keys in the winning bin is the last: they
// are ranked directly (each counts the larger and the equal ones).
constexpr int kFewKeys = 64;

// What the first level of a filtered select reads besides the candidates.
struct FilterArgs {
    const uint32_t *masks;    // [R][W] kept-token masks
    const char *scan_ws;      // the prepared scan workspace (meta blocks, records)
    const uint32_t *planes;   // the store, for rows that are rescored
    int64_t cstride;          // 4-byte words per row of the candidate record area
    int word_stride, W, G, H, qs;
};

// The scan's fp32 score of a candidate from its record (the candidate filter in
// common.h): the same operations, in the same order, as the scan's combine of the
// digit sums, for the token at bit m of its byte (S 2^-m by ldexp: the same exact
// power-of-two scaling the scan applies).  Records exist only for heads of at most
// 480 planes, whose low part R is an int32 sum.
__device__ __forceinline__ float record_score(int2 rec, int m, float C, float S) {
    const float f = fmaf((float)rec.x, 65536.0f, (float)rec.y);
    const float mult = m < 7 ? ldexpf(S, -m) : -ldexpf(S, -7);
    return fmaf(f, mult, C);
}

// A row whose candidates may miss a winner: it kept fewer than k tokens, a block of it
// overflowed its record area, or fewer than k of its candidates (as counted by the
// select) clear its threshold exactly.  Such rows are rescored from the store.
__device__ __forceinline__ bool needs_rescore(const ScanMeta *meta, int g, int k) {
    return meta->cnt[g] < (uint32_t)k || ((meta->ovf >> g) & 1u) ||
           meta->cnt_exact[g] < (uint32_t)k;
}

// Filler candidates for slots [from, to) of a chunk's output: value with key 0 (below
// every score) and an index past any row.  They fill the slots of a chunk that kept
// fewer than k candidates; the rows they belong to kept at least k in total, so the
// later levels never select them.
__device__ __forceinline__ void fill_slots(float *out_val, int32_t *out_idx, int64_t base,
                                           int from, int to) {
    for (int o = from + (int)threadIdx.x; o < to; o += (int)blockDim.x) {
        out_val[base + o] = __uint_as_float(0xFFFFFFFFu);
        out_idx[base + o] = 0x7FFFFFFF;
    }
}

// Kept-candidate keys of this thread's word (tokens 32*word .. +31): the block's
// records lie at the front of its 256-token region in token order.  Returns the mask.
__device__ __forceinline__ uint32_t load_kept(const int2 *row_rec, const uint32_t *row_mask,
                                              int word, int W, uint32_t lenmask, float C,
                                              float S, uint32_t (&key)[kEPT]) {
    const uint32_t mk = (word < W ? row_mask[word] : 0u) & lenmask;
    const uint32_t c = (uint32_t)__popc(mk);
    const int j = threadIdx.x & 7;  // word within the block (blocks are 8 threads)
    uint32_t pre = 0u;
#pragma unroll
    for (int o = 0; o < 7; ++o) {  // words stored before this one
        const uint32_t co = (uint32_t)__shfl((int)c, o, 8);
        if (o < j) pre += co;
    }
    const int2 *src = row_rec + (size_t)(word & ~7) * 16 + pre;
    uint32_t r = 0u;
#pragma unroll
    for (int e = 0; e < kEPT; ++e) {
        key[e] = 0u;
        if ((mk >> e) & 1u) key[e] = order_key(record_score(src[r++], e & 7, C, S));
    }
    return mk;
}

// Scores of this thread's word of row (h, g), recomputed from the store and the
// prepared records with the scan's own arithmetic, so they equal its scores bit for
// bit: per token the exact integer sums L = sum bit * (d0 + 256 d1) and
// Hs = sum bit * (d2 + 256 d3) over the head's planes (d the weight's base-256 digits),
// f = fl(fl(Hs) 65536 + fl(L)), and with m the token's bit within its byte the scan's
// final step fl(f 2^m * fl(S 2^-m) + C) (-128 in place of 2^7).  tab: 3*512 words of LDS.
// It runs only for rows whose threshold guess failed.  Inlined into the final select
// (rows of one chunk), which then needs no scratch memory: a kernel that uses scratch
// cost ~3 us more a launch in the decode step, even with an empty redo list.  Called out
// of line from the candidate level, where inlined it makes the compiler duplicate the
// select around it and spill.
__device__ __forceinline__ void rescore_word(const FilterArgs &fa, int h, int g, int word,
                                             uint32_t lenmask, uint32_t *tab,
                                             uint32_t (&key)[kEPT]) {
    const ScanMeta *meta = reinterpret_cast<const ScanMeta *>(fa.scan_ws + (size_t)h * kMetaBytes);
    const int np = min(max(meta->n_planes, 0), kMaxPlanesPerHead);
    const uint32_t *rec = reinterpret_cast<const uint32_t *>(
        fa.scan_ws + (size_t)fa.H * kMetaBytes + (size_t)h * kMaxKBlocks * 64 * 16 * fa.qs);
    int *tl = reinterpret_cast<int *>(tab), *th = tl + kMaxPlanesPerHead;
    uint32_t *tp = tab + 2 * kMaxPlanesPerHead;
    for (int p = threadIdx.x; p < np; p += kThreads) {
        const int grp = p >> 3, i = p & 7, kbl = grp >> 2;
        int dg[kDigits];
#pragma unroll
        for (int d = 0; d < kDigits; ++d) {
            const int ln = 16 * (grp & 3) + 4 * (g & 3) + d;
            const uint32_t wv =
                rec[(size_t)(kbl * 64 + ln) * 4 * fa.qs + 2 + 2 * (g >> 2) + (i >> 2)];
            dg[d] = (int)(int8_t)(uint8_t)(wv >> (8 * (i & 3)));
        }
        tl[p] = dg[0] + 256 * dg[1];
        th[p] = dg[2] + 256 * dg[3];
        tp[p] = meta->plane[p];
    }
    __syncthreads();
    const float C = meta->C[g], S = meta->S[g];
    const uint32_t *hp = fa.planes + (size_t)h * kMaxPlanesPerHead * fa.word_stride + word;
    const bool inrow = word < fa.W;
#pragma unroll
    for (int b = 0; b < 8; ++b) {  // 4 tokens a pass: 8*(b/2) + 4*(b%2) + m4
        int la[4], ha[4];
#pragma unroll
        for (int m4 = 0; m4 < 4; ++m4) la[m4] = ha[m4] = 0;
        if (inrow) {
            for (int p = 0; p < np; ++p) {
                const uint32_t x = hp[(size_t)tp[p] * fa.word_stride] >> (4 * b);
                const int l = tl[p], hh = th[p];
#pragma unroll
                for (int m4 = 0; m4 < 4; ++m4) {
                    const int on = -(int)((x >> m4) & 1u);
                    la[m4] += l & on;
                    ha[m4] += hh & on;
                }
            }
        }
#pragma unroll
        for (int m4 = 0; m4 < 4; ++m4) {
            const int m = 4 * (b & 1) + m4;  // bit within the byte
            const float f = fmaf((float)ha[m4], 65536.0f, (float)la[m4]);
            const float fm = m < 7 ? f * (float)(1 << m) : f * -128.0f;
            const float mult = m < 7 ? S * (1.0f / (float)(1 << m)) : S * (-1.0f / 128.0f);
            const int e = 4 * b + m4;
            key[e] = ((lenmask >> e) & 1u) ? order_key(fmaf(fm, mult, C)) : 0u;
        }
    }
    __syncthreads();  // the tables are no longer read
}

__device__ __noinline__ void rescore_word_call(const FilterArgs &fa, int h, int g, int word,
                                               uint32_t lenmask, uint32_t *tab,
                                               uint32_t (&key)[kEPT]) {
    rescore_word(fa, h, g, word, lenmask, tab, key);
}


// kExplicit: input entries carry their own int32 index (candidate levels); otherwise
// the index is the position in the row.  kCandOut: write (value, index) candidates
// (at column chunk*kk of the output row) instead of final indices.  kDirect (with
// kMasked, a row of one chunk): the select runs alone, without the lean select.
template <bool kExplicit, bool kCandOut, bool kMasked, bool kDirect = false>
__device__ __forceinline__ void select_chunk(
    int64_t row, int chunk, const float *__restrict__ vals, const int32_t *__restrict__ in_idx,
    int64_t row_len, int64_t in_stride, int k, float *__restrict__ out_val,
    int32_t *__restrict__ out_idx, int64_t out_stride, const FilterArgs &fa,
    int32_t *lds_idx = nullptr, bool direct_rescore = false) {
    __shared__ __align__(16) uint32_t hist[4096];
    __shared__ uint32_t scan_sh[17];
    __shared__ uint32_t pick[3];
    __shared__ uint32_t kmm[2][kThreads / 64];  // per-wave least and largest valid key
    __shared__ uint32_t few[kFewKeys], nfew, few_key, few_above;
    const int tid = threadIdx.x;
    const int64_t start = (int64_t)chunk * kTopkChunk;
    const int len = (int)min((int64_t)kTopkChunk, row_len - start);
    const float *v = vals + row * in_stride + start;
    const int p0 = tid * kEPT;  // this thread's positions p0 .. p0+31
    const int nvalid = max(0, min(kEPT, len - p0));
    uint32_t vmask = nvalid >= 32 ? 0xFFFFFFFFu : ((1u << nvalid) - 1u);

    uint32_t key[kEPT];
    int kr = min(k, len);
    if constexpr (kMasked) {
        // Candidates of the filtering scan.  A row that kept fewer than k tokens is
        // rescored in full here (its threshold guess was too high).
        const int h = (int)(row / fa.G), g = (int)(row - (int64_t)h * fa.G);
        const ScanMeta *meta =
            reinterpret_cast<const ScanMeta *>(fa.scan_ws + (size_t)h * kMetaBytes);
        const int word = chunk * kThreads + tid;
        if constexpr (!kCandOut && kDirect) {
            // Run alone (a row of one chunk), the select itself counts the kept keys
            // that clear the row's threshold exactly (otherwise the lean select did);
            // whether the candidates are complete its caller found from the masks (the
            // scan's overflow bit, when it set one, says the same).
            bool rescore = direct_rescore || ((meta->ovf >> g) & 1u);
            if (!rescore) {
                const uint32_t lenmask = vmask;
                vmask = load_kept(reinterpret_cast<const int2 *>(vals + row * fa.cstride),
                                  fa.masks + row * fa.W, word, fa.W, vmask, meta->C[g],
                                  meta->S[g], key);
                const uint32_t tkey = meta->tkey[g];
                uint32_t nex = 0u;
#pragma unroll
                for (int e = 0; e < kEPT; ++e) nex += ((vmask >> e) & 1u) && key[e] >= tkey;
                uint32_t total;
                block_excl_scan(nex, scan_sh, &total);
                rescore = total < (uint32_t)k;  // a winner may be missing
                if (rescore) vmask = lenmask;
            }
            if (rescore) rescore_word(fa, h, g, word, vmask, hist, key);
        } else if (needs_rescore(meta, g, k)) {
            if constexpr (kCandOut)
                rescore_word_call(fa, h, g, word, vmask, hist, key);
            else
                rescore_word(fa, h, g, word, vmask, hist, key);
        } else {
            vmask = load_kept(reinterpret_cast<const int2 *>(vals + row * fa.cstride),
                              fa.masks + row * fa.W, word, fa.W, vmask, meta->C[g], meta->S[g],
                              key);
            if (kCandOut) {  // this chunk may hold fewer than k candidates
                uint32_t total;
                block_excl_scan((uint32_t)__popc(vmask), scan_sh, &total);
                kr = min(kr, (int)total);
            }
        }
    } else if (((((uintptr_t)(v + p0)) & 15u) == 0) && nvalid == kEPT) {
#pragma unroll
        for (int e = 0; e < kEPT; e += 4) {
            const float4 f = *reinterpret_cast<const float4 *>(v + p0 + e);
            key[e] = order_key(f.x);
            key[e + 1] = order_key(f.y);
            key[e + 2] = order_key(f.z);
            key[e + 3] = order_key(f.w);
        }
    } else {
        // unconditional loads (positions past the chunk read its last entry, then are
        // dropped), so that all of them are in flight together
        float x[kEPT];
#pragma unroll
        for (int e = 0; e < kEPT; ++e) x[e] = v[min(p0 + e, len - 1)];
#pragma unroll
        for (int e = 0; e < kEPT; ++e) key[e] = e < nvalid ? order_key(x[e]) : 0u;
    }

    // ---- radix select, 12 bits a pass, starting below the bits every valid key shares
    //      (from their least and largest); a pass that leaves at most kFewKeys keys in the
    //      winning bin is the last, those keys ranked directly
    uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
#pragma unroll
    for (int e = 0; e < kEPT; ++e) {
        if ((vmask >> e) & 1u) {
            kmin = min(kmin, key[e]);
            kmax = max(kmax, key[e]);
        }
    }
    kmin = __ockl_wfred_min_u32(kmin);
    kmax = __ockl_wfred_max_u32(kmax);
    for (int b = tid; b < 4096; b += kThreads) hist[b] = 0u;
    if (tid == 0) nfew = 0u;
    if ((tid & 63) == 0) {
        kmm[0][tid >> 6] = kmin;
        kmm[1][tid >> 6] = kmax;
    }
    __syncthreads();
    if (kCandOut && kMasked && kr == 0) {  // a chunk without candidates: all filler
        fill_slots(out_val, out_idx, row * out_stride + (int64_t)chunk * min(k, kTopkChunk), 0,
                   min(k, len));
        return;
    }
#pragma unroll
    for (int w = 0; w < kThreads / 64; ++w) {
        kmin = min(kmin, kmm[0][w]);
        kmax = max(kmax, kmm[1][w]);
    }
    // the bits >= shift are the same in every valid key; pbits holds the settled high
    // bits in place, hmask selects them
    const uint32_t diff = kmin ^ kmax;
    int shift = diff == 0u ? 0 : 32 - (int)__clz(diff);
    uint32_t hmask = shift >= 32 ? 0u : 0xFFFFFFFFu << shift;
    uint32_t pbits = kmin & hmask;
    uint32_t need = (uint32_t)kr;
    for (int pass = 0; shift > 0; ++pass) {
        const int sd = max(0, shift - 12);
        const uint32_t dmask = (1u << (shift - sd)) - 1u;
        if (pass > 0) {  // find_bin ended with a barrier: every read of hist is done
            for (int b = tid; b < 4096; b += kThreads) hist[b] = 0u;
            __syncthreads();
        }
#pragma unroll
        for (int e = 0; e < kEPT; ++e) {
            if (((vmask >> e) & 1u) && (key[e] & hmask) == pbits)
                atomicAdd(&hist[(key[e] >> sd) & dmask], 1u);
        }
        __syncthreads();
        // find_bin reads bins four at a time: at least 4 (the ones past the digit are 0)
        find_bin(hist, scan_sh, pick, max(4, (int)dmask + 1), need);
        pbits |= pick[0] << sd;
        need -= pick[1];
        const uint32_t in_bin = pick[2];
        shift = sd;
        hmask = 0xFFFFFFFFu << sd;
        if (in_bin == need) break;  // every entry of the bin is a winner
        if (shift > 0 && in_bin <= (uint32_t)kFewKeys) {
            // the need-th largest of the bin's keys is the last winning key; the keys
            // equal to it are then taken in position order as after a last pass
#pragma unroll
            for (int e = 0; e < kEPT; ++e) {
                if (((vmask >> e) & 1u) && (key[e] & hmask) == pbits)
                    few[atomicAdd(&nfew, 1u)] = key[e];
            }
            __syncthreads();
            if (tid < (int)in_bin) {
                const uint32_t kv = few[tid];
                uint32_t gt = 0u, eq = 0u;
                for (uint32_t jj = 0; jj < in_bin; ++jj) {
                    gt += few[jj] > kv;
                    eq += few[jj] == kv;
                }
                if (gt < need && need <= gt + eq) {  // the same for equal keys
                    few_key = kv;
                    few_above = gt;
                }
            }
            __syncthreads();
            pbits = few_key;
            need -= few_above;
            shift = 0;
            break;
        }
    }
    const uint32_t prefix = pbits >> shift;  // shift <= 20 here

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
                if (lds_idx) lds_idx[slot] = index;  // the winners, also for this workgroup
            }
        }
        ++slot;
    }
    if (kCandOut && kMasked)  // slots past this chunk's candidates: filler
        fill_slots(out_val, out_idx, row * out_stride + (int64_t)chunk * min(k, kTopkChunk), kr,
                   min(k, len));
}

template <bool kExplicit, bool kCandOut, bool kMasked>
__global__ __launch_bounds__(kThreads, 8) void k_topk_chunk(
    const float *__restrict__ vals, const int32_t *__restrict__ in_idx, int64_t row_len,
    int64_t in_stride, int row0, int k, float *__restrict__ out_val,
    int32_t *__restrict__ out_idx, int64_t out_stride, FilterArgs fa) {
    select_chunk<kExplicit, kCandOut, kMasked>((int64_t)row0 + blockIdx.y, blockIdx.x, vals,
                                               in_idx, row_len, in_stride, k, out_val, out_idx,
                                               out_stride, fa);
}

// The row chunks the filtered select handed over, and every chunk of a row of several
// chunks whose exact count fell short of k (listed as row * nch + chunk; their count is the
// head-0 meta block's redo field; a chunk may be listed twice, which gives the same
// output twice), a grid-stride loop over the list: a small grid, as the list is usually
// empty.
constexpr int kRedoGrid = 16;
// The final select (!kCandOut) may use 128 VGPRs, so that it needs no scratch.
template <bool kCandOut>
__global__ __launch_bounds__(kThreads, kCandOut ? 8 : 1) void k_topk_redo(
    const float *__restrict__ vals, int64_t row_len, int k, float *__restrict__ out_val,
    int32_t *__restrict__ out_idx, int64_t out_stride, FilterArgs fa,
    const uint32_t *__restrict__ list, int nch) {
    const uint32_t total = reinterpret_cast<const ScanMeta *>(fa.scan_ws)->redo;
    for (uint32_t it = blockIdx.x; it < total; it += gridDim.x) {
        const uint32_t item = list[it];
        select_chunk<false, kCandOut, true>((int64_t)(item / (uint32_t)nch),
                                            (int)(item % (uint32_t)nch), vals, nullptr, row_len,
                                            row_len, k, out_val, out_idx, out_stride, fa);
        __syncthreads();  // LDS is reused by the next item
    }
}

// ---------------------------------------------------------------------------------
// Filtered select: one workgroup per row chunk ranks the chunk's kept candidates in
// LDS (up to kSelCap of them).  With many rows (a batched step) a workgroup has 256
// threads, so that every row runs at once, and a chunk with more candidates, of a row
// that kept fewer than k tokens, or of a one-chunk row of which fewer than k candidates
// clear the threshold exactly, is appended to the redo list for the full select above.
// With few rows of one chunk (one layer of a decode step: kDirect) a workgroup has 1024
// threads and finishes such a row itself with the full select, so that no second
// launch follows.
// ---------------------------------------------------------------------------------
constexpr int kSelCap = 3840;   // with 8 KB of histogram: 5 workgroups of 256 a CU
constexpr int kSelBins = 2048;  // 11-bit digits: passes over bits 31-21, 20-10, 9-0

// Exclusive prefix over the NT threads with one barrier: each thread adds the totals
// of the waves before its own.  sh (NT / 64 words) must not be rewritten before every
// thread has read it: callers alternate between two.
template <int NT>
__device__ __forceinline__ uint32_t block_prefix1(uint32_t v, uint32_t *sh, uint32_t *total) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const uint32_t inc = wave_incl_scan(v, lane);
    if (lane == 63) sh[wave] = inc;
    __syncthreads();
    uint32_t before = 0u, all = 0u;
#pragma unroll
    for (int w = 0; w < NT / 64; ++w) {
        const uint32_t t = sh[w];
        before += w < wave ? t : 0u;
        all += t;
    }
    *total = all;
    return inc - v + before;
}

// The lean select's body for NT threads (256, or 1024 with kDirect).
template <bool kCandOut, bool kDirect, int NT>
__device__ __forceinline__ void select_kept(
    const float *__restrict__ cand, int64_t n, int row0, int k, const FilterArgs &fa,
    uint32_t *__restrict__ list, float *__restrict__ out_val, int32_t *__restrict__ out_idx,
    int64_t out_stride, int32_t *lds_idx = nullptr) {
    constexpr int NW = NT / 64;                 // waves
    constexpr int WPT = kTopkChunk / 32 / NT;   // mask words a thread: 4 or 1
    constexpr int BPT = kSelBins / NT;          // histogram bins a thread: 8 or 2
    constexpr int kPer = (kSelCap + NT - 1) / NT;
    static_assert(WPT == 4 || WPT == 1, "two threads, or eight, per 8-word block");
    static_assert(!kDirect || (NT == kThreads && !kCandOut), "the direct select: one chunk");
    __shared__ uint32_t skey[kSelCap];
    __shared__ uint16_t soff[kSelCap];
    __shared__ __align__(16) uint32_t hist[kSelBins];
    __shared__ uint32_t sh[2][NW];
    __shared__ uint32_t pick[2][3];
    __shared__ uint32_t smm[3][NW];  // per-wave min and max key, count clearing the threshold
    __shared__ uint32_t few[kFewKeys], nfew, few_key, few_above;  // a small pivot bin's keys
    const int tid = threadIdx.x, chunk = blockIdx.x, nch = gridDim.x;
    const int64_t row = (int64_t)row0 + blockIdx.y;
    const int64_t start = (int64_t)chunk * kTopkChunk;
    const int len = (int)min((int64_t)kTopkChunk, n - start);
    const int h = (int)(row / fa.G), g = (int)(row - (int64_t)h * fa.G);
    ScanMeta *meta0 = reinterpret_cast<ScanMeta *>(const_cast<char *>(fa.scan_ws));
    ScanMeta *meta =
        reinterpret_cast<ScanMeta *>(const_cast<char *>(fa.scan_ws) + (size_t)h * kMetaBytes);
    // a row chunk that needs the full select: listed for the redo kernel, or (kDirect)
    // finished here by all NT threads (the condition is the same for every thread), with
    // every token rescored when `full` (its candidates may miss a winner)
    bool full = false;
    auto hand_over = [&]() {
        if constexpr (kDirect)
            select_chunk<false, false, true, true>(row, 0, cand, nullptr, n, n, k, nullptr,
                                                   out_idx, 0, fa, lds_idx, full);
        else if (tid == 0)
            list[atomicAdd(&meta0->redo, 1u)] = (uint32_t)(row * nch + chunk);
    };
    // this thread's WPT mask words: chunk words WPT tid .. WPT tid + WPT - 1
    const int wl = WPT * tid;
    const int64_t wg = (int64_t)chunk * (kTopkChunk / 32) + wl;
    uint32_t mk[WPT], c[WPT];
    // every load unconditional (a word past the row reads the row's last word, then
    // masked off), so that they are all in flight together
#pragma unroll
    for (int j = 0; j < WPT; ++j)
        mk[j] = fa.masks[row * fa.W + min(wg + j, (int64_t)fa.W - 1)];
    // the direct select's rows are one chunk: their kept count is the masks' and a block
    // overflowed its records exactly when it kept more than it holds, so both come from
    // the masks (the scan need not have counted them); else from the scan's counts
    const uint32_t kept = kDirect ? 0u : meta->cnt[g];
    const bool no_records = kDirect && meta->n_planes > 480;
#pragma unroll
    for (int j = 0; j < WPT; ++j) {
        const int t0 = 32 * (wl + j);  // first chunk token of the word
        const uint32_t lm = t0 >= len ? 0u : (len - t0 >= 32 ? 0xFFFFFFFFu : (1u << (len - t0)) - 1u);
        mk[j] = wg + j < fa.W ? mk[j] & lm : 0u;
    }
    // the row is rescored by the full select
    full = kDirect ? no_records : kept < (uint32_t)k || ((meta->ovf >> g) & 1u);
    uint32_t csum = 0u;
#pragma unroll
    for (int j = 0; j < WPT; ++j) {
        if (full) mk[j] = 0u;
        c[j] = (uint32_t)__popc(mk[j]);
        csum += c[j];
    }
    if constexpr (kDirect) {  // thread 8b + j holds word j of block b: the block's count
        uint32_t bc = csum;
        bc += (uint32_t)__shfl_xor((int)bc, 1, 64);
        bc += (uint32_t)__shfl_xor((int)bc, 2, 64);
        bc += (uint32_t)__shfl_xor((int)bc, 4, 64);
        const uint32_t cap = fa.qs == 1 ? 64u : (uint32_t)kBlockRecords;
        // flag it in bits 20 and up of the first word's count: the prefix's total then
        // carries the overflowing blocks (C <= 32768 < 2^20)
        if ((tid & 7) == 0 && bc > cap) csum += 1u << 20;
    }
    for (int b = tid; b < kSelBins; b += NT) hist[b] = 0u;
    if (tid == 0) nfew = 0u;
    uint32_t C;
    uint32_t pos0 = block_prefix1<NT>(csum, sh[0], &C);
    if constexpr (kDirect) {
        full = full || (C >> 20) != 0 || (C & 0xFFFFFu) < (uint32_t)k;
        C &= 0xFFFFFu;
        pos0 &= 0xFFFFFu;
    }
    if (full || C > (uint32_t)kSelCap) {
        hand_over();
        return;
    }
    // A block's kept scores are stored in token order; off[j]: the kept tokens of the
    // block stored before those of word wl + j.
    uint32_t off[WPT];
    if constexpr (WPT == 4) {  // thread 2b: words 0-3 of block b, thread 2b+1 words 4-7
        const uint32_t E = c[0] + c[1] + c[2] + c[3];
        const uint32_t pE = (uint32_t)__shfl_xor((int)E, 1, 64);
        off[0] = (tid & 1) ? pE : 0u;
        off[1] = off[0] + c[0];
        off[2] = off[1] + c[1];
        off[3] = off[2] + c[2];
    } else {  // thread 8b + j: word j of block b
        const int j = tid & 7;
        uint32_t pre = 0u;
#pragma unroll
        for (int o = 0; o < 7; ++o) {
            const uint32_t co = (uint32_t)__shfl((int)c[0], o, 8);
            if (o < j) pre += co;
        }
        off[0] = pre;
    }
    {   // first the record index of each kept token in the row, in token order ...
        const uint32_t blk = (uint32_t)((start + 32 * (int64_t)(wl & ~7)) / 2);
        uint32_t pos = pos0;
#pragma unroll
        for (int j = 0; j < WPT; ++j) {
            uint32_t m = mk[j], r = blk + off[j];
            while (m) {
                const int b = __ffs(m) - 1;
                m &= m - 1u;
                skey[pos] = r++;
                soff[pos] = (uint16_t)(32 * (wl + j) + b);
                ++pos;
            }
        }
    }
    __syncthreads();
    {   // ... then all the loads at once, each thread up to kSelCap / NT of them; each
        // record becomes the scan's exact score and its order key
        const int2 *crow = reinterpret_cast<const int2 *>(cand + row * fa.cstride);
        int2 v[kPer];
#pragma unroll
        for (int u = 0; u < kPer; ++u) {
            const int e = tid + NT * u;
            v[u] = e < (int)C ? crow[skey[e]] : make_int2(0, 0);
        }
        const float Cg = meta->C[g], Sg = meta->S[g];
        const uint32_t tkey = meta->tkey[g];
        // the keys' minimum and maximum on the way (for the radix start below), and how
        // many clear the row's threshold
        uint32_t kmin = 0xFFFFFFFFu, kmax = 0u, nex = 0u;
#pragma unroll
        for (int u = 0; u < kPer; ++u) {
            const int e = tid + NT * u;
            if (e < (int)C) {
                const uint32_t key = order_key(record_score(v[u], soff[e] & 7, Cg, Sg));
                skey[e] = key;
                kmin = min(kmin, key);
                kmax = max(kmax, key);
                nex += key >= tkey;
            }
        }
        kmin = __ockl_wfred_min_u32(kmin);
        kmax = __ockl_wfred_max_u32(kmax);
        nex = __ockl_wfred_add_u32(nex);
        if ((tid & 63) == 0) {
            smm[0][tid >> 6] = kmin;
            smm[1][tid >> 6] = kmax;
            smm[2][tid >> 6] = nex;
        }
    }
    __syncthreads();
    uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
    {   // the candidates clearing the threshold exactly: with fewer than k a winner may be
        // missing (rows of one chunk go to the full select; a row of several chunks is
        // judged on its sum over chunks by the redo kernel)
        uint32_t nex = 0u;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            kmin = min(kmin, smm[0][w]);
            kmax = max(kmax, smm[1][w]);
            nex += smm[2][w];
        }
        if (!kDirect && tid == 0) atomicAdd(&meta->cnt_exact[g], nex);
        if (!kCandOut && nex < (uint32_t)k) {
            hand_over();
            return;
        }
    }
    const int kk = min(k, kTopkChunk);
    const int64_t obase = row * out_stride + (int64_t)chunk * kk;
    const int kr = min(min(k, len), (int)C);
    if (kCandOut && kr == 0) {
        fill_slots(out_val, out_idx, obase, 0, min(k, len));
        return;
    }
    // The kept keys are the top few percent of the row and share their top bits; the
    // radix select starts below the bits all of them share (from their min and max), so
    // that its first histogram spreads them over many bins instead of a few contended
    // ones.  Digits of up to 11 bits.
    const uint32_t diff = kmin ^ kmax;
    int shift = diff == 0u ? 0 : 32 - __clz(diff);  // bits >= shift: the same in every key
    uint32_t prefix = (uint32_t)((uint64_t)kmin >> shift), need = (uint32_t)kr;
    for (int pass = 0; shift > 0; ++pass) {
        const int sd = max(0, shift - 11), width = shift - sd, nb = 1 << width;
        for (int i = tid; i < (int)C; i += NT) {
            const uint32_t key = skey[i];
            if (((uint64_t)key >> shift) == prefix) atomicAdd(&hist[(key >> sd) & (nb - 1)], 1u);
        }
        __syncthreads();
        // thread t owns bins nb-1-BPT t .. nb-BPT-BPT t (largest first); when all of
        // them exist they are one aligned run, read as 16-byte pieces (lanes 4 BPT bytes
        // apart: word by word that is a BPT-way bank conflict)
        uint32_t cb[BPT], local = 0u;
        const int lo = nb - BPT - BPT * tid;  // the thread's lowest bin
        if constexpr (BPT % 4 == 0) {
            if (lo >= 0) {
#pragma unroll
                for (int v = 0; v < BPT / 4; ++v) {
                    const uint4 x = *reinterpret_cast<const uint4 *>(&hist[lo + 4 * v]);
                    cb[BPT - 1 - 4 * v] = x.x;
                    cb[BPT - 2 - 4 * v] = x.y;
                    cb[BPT - 3 - 4 * v] = x.z;
                    cb[BPT - 4 - 4 * v] = x.w;
                }
            } else {
#pragma unroll
                for (int e = 0; e < BPT; ++e) {
                    const int bin = nb - 1 - (BPT * tid + e);
                    cb[e] = bin >= 0 ? hist[bin] : 0u;
                }
            }
        } else {
#pragma unroll
            for (int e = 0; e < BPT; ++e) {
                const int bin = nb - 1 - (BPT * tid + e);
                cb[e] = bin >= 0 ? hist[bin] : 0u;
            }
        }
#pragma unroll
        for (int e = 0; e < BPT; ++e) local += cb[e];
        uint32_t tot;
        const uint32_t above = block_prefix1<NT>(local, sh[(pass + 1) & 1], &tot);
        if (above < need && need <= above + local) {
            uint32_t cum = above;
#pragma unroll
            for (int e = 0; e < BPT; ++e) {
                if (cum < need && need <= cum + cb[e]) {
                    pick[pass & 1][0] = (uint32_t)(nb - 1 - (BPT * tid + e));
                    pick[pass & 1][1] = cum;
                    pick[pass & 1][2] = cb[e];
                }
                cum += cb[e];
            }
        }
        // every thread has read hist: clear it for the next pass
        if (BPT % 4 == 0 && lo >= 0) {
#pragma unroll
            for (int v = 0; v < BPT / 4; ++v)
                *reinterpret_cast<uint4 *>(&hist[lo + 4 * v]) = make_uint4(0u, 0u, 0u, 0u);
        } else {
#pragma unroll
            for (int e = 0; e < BPT; ++e) {
                const int bin = nb - 1 - (BPT * tid + e);
                if (bin >= 0) hist[bin] = 0u;
            }
        }
        __syncthreads();
        prefix = (prefix << width) | pick[pass & 1][0];
        need -= pick[pass & 1][1];
        const uint32_t in_bin = pick[pass & 1][2];
        shift = sd;
        if (in_bin == need) break;
        if (shift > 0 && in_bin <= (uint32_t)kFewKeys) {
            // A few keys left in the bin: rank them directly instead of another
            // histogram pass.  The need-th largest of them is the last winning key; the
            // keys equal to it are then taken in token order as after a last pass.
            for (int i = tid; i < (int)C; i += NT) {
                const uint32_t key = skey[i];
                if (((uint64_t)key >> shift) == prefix) few[atomicAdd(&nfew, 1u)] = key;
            }
            __syncthreads();
            if (tid < (int)in_bin) {
                const uint32_t kv = few[tid];
                uint32_t gt = 0u, eq = 0u;
                for (uint32_t j = 0; j < in_bin; ++j) {
                    gt += few[j] > kv;
                    eq += few[j] == kv;
                }
                if (gt < need && need <= gt + eq) {  // the same for equal keys
                    few_key = kv;
                    few_above = gt;
                }
            }
            __syncthreads();
            prefix = few_key;
            need -= few_above;
            shift = 0;
            break;
        }
    }
    // ordered output: greater keys all win; of the keys equal to the prefix, the `need`
    // first in token order
    const int seg = ((int)C + NT - 1) / NT;
    const int b0 = min((int)C, tid * seg), b1 = min((int)C, b0 + seg);
    uint32_t gt = 0u, eq = 0u;
    for (int i = b0; i < b1; ++i) {
        const uint32_t kv = (uint32_t)((uint64_t)skey[i] >> shift);
        gt += kv > prefix;
        eq += kv == prefix;
    }
    uint32_t tot;
    const uint32_t before = block_prefix1<NT>(gt | (eq << 16), sh[1], &tot);
    const uint32_t gtb = before & 0xFFFFu, eqb = before >> 16;
    const uint32_t eq_won_before = min(eqb, need);
    uint32_t take = min(need - eq_won_before, eq);
    int slot = (int)(gtb + eq_won_before);
    for (int i = b0; i < b1; ++i) {
        const uint32_t kv = (uint32_t)((uint64_t)skey[i] >> shift);
        bool win = kv > prefix;
        if (kv == prefix && take > 0u) {
            win = true;
            --take;
        }
        if (win) {
            if (slot < kr) {
                const int32_t index = (int32_t)(start + soff[i]);
                if (kCandOut) {
                    out_val[obase + slot] = key_value(skey[i]);
                    out_idx[obase + slot] = index;
                } else {
                    out_idx[row * (int64_t)k + slot] = index;
                    if (lds_idx) lds_idx[slot] = index;
                }
            }
            ++slot;
        }
    }
    if (kCandOut) fill_slots(out_val, out_idx, obase, kr, min(k, len));
}

// kCandOut (rows of several chunks): the row's chunk selects count themselves done, and
// the last lists all of the row's chunks for the full select when the row's exact count,
// summed by its chunk selects, fell short of k although its candidates were complete (the
// chunks of a row that kept fewer than k, or overflowed, were listed by their selects).
// Each count waits for the workgroup's own exact-count atomic (thread 0's) to be done, and
// the last reads the sum with an atomic after its own count.
template <bool kCandOut>
__global__ __launch_bounds__(256) void k_select_kept(
    const float *__restrict__ cand, int64_t n, int row0, int k, FilterArgs fa,
    uint32_t *__restrict__ list, float *__restrict__ out_val, int32_t *__restrict__ out_idx,
    int64_t out_stride) {
    select_kept<kCandOut, false, 256>(cand, n, row0, k, fa, list, out_val, out_idx, out_stride);
    if constexpr (kCandOut) {
        __shared__ bool last;
        const int64_t row = (int64_t)row0 + blockIdx.y;
        const int h = (int)(row / fa.G), g = (int)(row - (int64_t)h * fa.G);
        ScanMeta *meta0 = reinterpret_cast<ScanMeta *>(const_cast<char *>(fa.scan_ws));
        ScanMeta *meta = reinterpret_cast<ScanMeta *>(const_cast<char *>(fa.scan_ws) +
                                                      (size_t)h * kMetaBytes);
        __syncthreads();
        if (threadIdx.x == 0) {
            __builtin_amdgcn_s_waitcnt(0);  // this workgroup's atomics are done
            last = atomicAdd(&meta->sel_done[g], 1u) == gridDim.x - 1;
        }
        __syncthreads();
        // the sum is read by an atomic add of 0, performed where the chunk selects' adds
        // are: a load can be served by a copy of its line in this CU's caches, filled by
        // the select's earlier load of the overflow word beside it
        __shared__ uint32_t exact;
        if (last && threadIdx.x == 0) exact = atomicAdd(&meta->cnt_exact[g], 0u);
        __syncthreads();
        if (last && meta->cnt[g] >= (uint32_t)k && !((meta->ovf >> g) & 1u) &&
            exact < (uint32_t)k) {
            const uint32_t nch = gridDim.x;
            for (uint32_t c = threadIdx.x; c < nch; c += 256)
                list[atomicAdd(&meta0->redo, 1u)] = (uint32_t)row * nch + c;
        }
    }
}

// Like the final select it may use 128 VGPRs, so that it needs no scratch.
__global__ __launch_bounds__(kThreads, 1) void k_select_direct(
    const float *__restrict__ cand, int64_t n, int row0, int k, FilterArgs fa,
    int32_t *__restrict__ out_idx) {
    select_kept<false, true, kThreads>(cand, n, row0, k, fa, nullptr, nullptr, out_idx, 0);
}

// The direct select and the attention of its row (one layer of a decode step): the
// winners pass to the attention in LDS, so no index round trip through memory and no
// second launch.  A row runs as kShareGroups workgroups (blockIdx.z = the group): each
// makes the same select (it is deterministic) and attends its group's shares of the
// winners (attend_group_split: the last of the row to finish, by a counter in the head's
// meta block cleared by the scan's prepare, merges the groups' parts).  k <= kFusedMaxK.
constexpr int kFusedMaxK = 1024;
__global__ __launch_bounds__(kThreads, 1) void k_select_attend(
    const float *__restrict__ cand, int64_t n, int row0, int k, FilterArgs fa,
    int32_t *__restrict__ out_idx, const float *__restrict__ q, const uint16_t *__restrict__ K,
    const uint16_t *__restrict__ V, float sm_scale, uint16_t *__restrict__ out,
    float *__restrict__ part) {
    static_assert(kThreads >= kSharesPerGroup * 64, "a wave a share of the group");
    __shared__ int32_t widx[kFusedMaxK];
    select_kept<false, true, kThreads>(cand, n, row0, k, fa, nullptr, nullptr, out_idx, 0,
                                       widx);
    __syncthreads();  // every winner is in widx
    const int row = row0 + (int)blockIdx.y, grp = (int)blockIdx.z;
    const int h = row / fa.G, g = row - h * fa.G;
    ScanMeta *meta =
        reinterpret_cast<ScanMeta *>(const_cast<char *>(fa.scan_ws) + (size_t)h * kMetaBytes);
    attend_group_split(q, K, V, fa.G, (int)n, [](int r) { return widx[r]; }, k, grp, sm_scale,
                       row, part + (size_t)row * kShareGroups * kPartFloats,
                       &meta->attn_done[g], out);
}

template <bool kExplicit, bool kCandOut>
void launch_level(const float *vals, const int32_t *in_idx, int64_t len, int64_t in_stride,
                  int R, int k, float *out_val, int32_t *out_idx, int64_t out_stride,
                  hipStream_t s) {
    const int nch = (int)((len + kTopkChunk - 1) / kTopkChunk);
    for (int r0 = 0; r0 < R; r0 += 65535) {
        const int rows = std::min(65535, R - r0);
        hipLaunchKernelGGL((k_topk_chunk<kExplicit, kCandOut, false>), dim3(nch, rows),
                           dim3(kThreads), 0, s, vals, in_idx, len, in_stride, r0, k,
                           out_val, out_idx, out_stride, FilterArgs{});
    }
}

// Level 0 of the filtered select: the lean select over every row chunk, then the full
// select over the chunks it handed over.
template <bool kCandOut>
void launch_filtered_level(const float *cand, int64_t n, int R, int k, const FilterArgs &fa,
                           uint32_t *list, float *out_val, int32_t *out_idx, int64_t out_stride,
                           hipStream_t s) {
    const int nch = (int)((n + kTopkChunk - 1) / kTopkChunk);
    for (int r0 = 0; r0 < R; r0 += 65535) {
        const int rows = std::min(65535, R - r0);
        hipLaunchKernelGGL(k_select_kept<kCandOut>, dim3(nch, rows), dim3(256), 0, s,
                           cand, n, r0, k, fa, list, out_val, out_idx, out_stride);
    }
    const int grid = (int)std::min<int64_t>((int64_t)R * nch, kRedoGrid);
    hipLaunchKernelGGL(k_topk_redo<kCandOut>, dim3(grid), dim3(kThreads), 0, s, cand, n, k,
                       out_val, out_idx, out_stride, fa, list, nch);
}

// Rows of one chunk of a filtered select run k_select_direct when there are at most this
// many (one row a CU); more rows run the lean 256-thread select, then the full select
// over the chunks it hands over.
constexpr int kDirectRows = 256;

// Levels over R rows of n entries; the first reads either plain scores or (with a redo
// list) the filtering scan's candidates.
hipError_t run_levels(const float *scores, int R, int n, int k, int32_t *idx, void *ws,
                      hipStream_t s, const FilterArgs &fa, uint32_t *list) {
    const TopkLevels L = topk_levels(n, k);
    if (L.n_levels == 0) {
        if (list && R <= kDirectRows) {
            for (int r0 = 0; r0 < R; r0 += 65535)
                hipLaunchKernelGGL(k_select_direct, dim3(1, std::min(65535, R - r0)),
                                   dim3(kThreads), 0, s, scores, (int64_t)n, r0, k, fa, idx);
        } else if (list)
            launch_filtered_level<false>(scores, n, R, k, fa, list, nullptr, idx, 0, s);
        else
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
        if (l == 0 && list)
            launch_filtered_level<true>(in_val, cin, R, k, fa, list, ov, oi, os, s);
        else if (l == 0)
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

}  // namespace

hipError_t launch_topk(const float *scores, int R, int n, int k, int32_t *idx, void *ws,
                       hipStream_t s) {
    return run_levels(scores, R, n, k, idx, ws, s, FilterArgs{}, nullptr);
}

bool filtered_direct_applies(int R, int n, int k) {
    return topk_levels(n, k).n_levels == 0 && R <= kDirectRows && k <= kFusedMaxK;
}

// Compute units of the current device (asked once per device; 256 if it cannot be asked).
static int device_cus() {
    static std::mutex mu;
    static int cus[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    std::lock_guard<std::mutex> lock(mu);
    if (!cus[dev]) {
        int c = 0;
        if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            c <= 0)
            c = 256;
        cus[dev] = c;
    }
    return cus[dev];
}

// The fused select and attention launches kShareGroups 1024-thread workgroups a row, each
// repeating the row's select, one a CU: it pays only while they all run in one round.
// Beyond that the one-workgroup select and the split attention are far cheaper (at 256 rows
// on 256 CUs: eight rounds of ~12 us against one select and one gather).
bool filtered_attend_applies(int R, int n, int k) {
    return filtered_direct_applies(R, n, k) && (long)R * kShareGroups <= (long)device_cus();
}

hipError_t launch_topk_filtered_attend(const fathom_store &st, int G, const float *cand,
                                       const uint32_t *masks, void *scan_ws, int k,
                                       int32_t *idx, const float *q, const uint16_t *K,
                                       const uint16_t *V, float sm_scale, uint16_t *out,
                                       float *part, hipStream_t s) {
    FilterArgs fa;
    fa.masks = masks;
    fa.scan_ws = static_cast<const char *>(scan_ws);
    fa.planes = st.planes;
    fa.word_stride = st.word_stride;
    fa.W = (st.n_tokens + 31) / 32;
    fa.cstride = cand_stride(st.n_tokens);
    fa.G = G;
    fa.H = st.n_heads;
    fa.qs = query_sets(G);
    const int R = st.n_heads * G;
    hipLaunchKernelGGL(k_select_attend, dim3(1, R, kShareGroups), dim3(kThreads), 0, s, cand,
                       (int64_t)st.n_tokens, 0, k, fa, idx, q, K, V, sm_scale, out, part);
    return hipGetLastError();
}

hipError_t launch_topk_filtered(const fathom_store &st, int G, const float *cand,
                                const uint32_t *masks, void *scan_ws, uint32_t *redo_list,
                                int k, int32_t *idx, void *ws, hipStream_t s) {
    FilterArgs fa;
    fa.masks = masks;
    fa.scan_ws = static_cast<const char *>(scan_ws);
    fa.planes = st.planes;
    fa.word_stride = st.word_stride;
    fa.W = (st.n_tokens + 31) / 32;
    fa.cstride = cand_stride(st.n_tokens);
    fa.G = G;
    fa.H = st.n_heads;
    fa.qs = query_sets(G);
    return run_levels(cand, st.n_heads * G, st.n_tokens, k, idx, ws, s, fa, redo_list);
}

}  // namespace fathom
