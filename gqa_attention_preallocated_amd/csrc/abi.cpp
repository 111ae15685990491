// C ABI of the preallocated-KV-cache GQA library: validation, host lengths,
// work planning and kernel launches. Declarations and contracts live in
// include/gqa_kv.h.
//
// Pages cited: [GQA] "Implement grouped-query attention over a preallocated KV
// cache, with no torch.cat, for both prefill chunks and decode"; [CH16]
// "16. Prefill, decode and the KV cache".

#include "gqa_kv.h"

#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <array>
#include <chrono>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <functional>
#include <new>
#include <numeric>
#include <queue>
#include <string>
#include <vector>

#include "indexing.h"
#include "internal.h"

using namespace gqakv;

struct kv_cache {
    int32_t batch, kv_heads, max_len, head_dim;
    kv_dtype dtype;
    int32_t elem_bytes;          // bytes of one cached K or V element
    int32_t io_bytes;            // bytes of one q / out / k_new / v_new element
    std::vector<float> k_scale, v_scale;   // E4M3 caches: per KV head
    std::vector<float> k_inv, v_inv;       // float32 1 / scale, used by the append
    void *k, *v;
    int32_t *lens_dev;
    std::vector<int32_t> lens;   // host copy, authoritative, updated at enqueue
    int32_t path_policy = 0;     // 0 auto, 1 split-K decode kernel, 2 prefill kernel
    int32_t keys_per_split = 0;  // 0 auto
    bool ring = false;           // token p in slot p mod max_len; lens are absolute positions
    int32_t window = kNoWindow;  // a query at p sees keys p - window < j <= p
    // paged: k and v are a pool [num_pages, Hkv, page_size, d]; logical block
    // i of row b is page table[b * max_blocks + i]; max_len = max_blocks * page_size
    bool paged = false;
    int32_t num_pages = 0, page_size = 0, page_shift = 0, max_blocks = 0;
    int32_t *table_dev = nullptr;                 // caller's device copy, kept in stream order
    std::vector<int32_t> table;                   // host copy, authoritative (-1: no page)
    std::priority_queue<int32_t, std::vector<int32_t>, std::greater<int32_t>> free_pages;
    SideStream side;             // created on the first mixed decode + prefill call
};

namespace {

thread_local std::string g_err;

kv_status fail(kv_status s, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return s;
}

kv_status ok() {
    g_err.clear();
    return KV_OK;
}

kv_status device_fail(hipError_t e, const char *what) {
    return fail(KV_ERR_DEVICE, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// ---------------------------------------------------------------------------
// attention plan
// ---------------------------------------------------------------------------
struct RowPlan {
    int32_t b, len, nnew;
    int32_t nq, nsplit, lsplit;
    int64_t pbase;     // -1: direct write
    int64_t work;      // key tiles x query tiles x kv heads (ordering key)
};

struct Plan {
    int group = 0;
    int nsub = 1;                      // decode subtiles (16 columns each)
    int dec_cols = 16;
    std::vector<RowPlan> dec, pre;     // rows per kernel
    std::vector<int32_t> zero_rows;    // rows with no new tokens (all slots zero)
    int64_t records = 0;               // partial records (d + 2 floats each)
    int64_t dec_records = 0;           // those of decode rows (the first dec_records)
    std::vector<int32_t> pad_rows;     // rows with padded slots (n_new < T), zero-filled
};

// Keys of query tile qt of a row (len keys after the append, n new queries,
// tq queries per tile): from the window's start for the tile's first query
// (range_start) to the tile's last query. Without a window, base + t_end.
int64_t tile_span(int32_t len, int32_t n, int tq, int qt, int32_t window) {
    const int base = len - n, t0 = qt * tq;
    const int hi = base + std::min(t0 + tq, (int)n);
    return hi - range_start(base + t0, window);
}

// Automatic kernel choice: rows of up to 32 columns (G * n_new, one or two
// 16-column subtiles) stream faster on the split-K decode kernel; wider rows
// measured 1.5-1.7x faster on the chunked-prefill kernel (both at 4,096 keys).
constexpr int64_t kDecodeAutoCols = 32;
// Decode work groups (kDecodeWaves waves each) the chip runs at once: one per
// CU. Rows are split across work groups only as far as needed to fill them.
constexpr int64_t kDecodeSlots = 256;
// Prefill work-group slots on the chip: 256 CUs x one resident work group
// (8 waves, or 4 at one wave per SIMD; prefill_waves).
constexpr int64_t kPrefillSlots = 256;

// A split length fixed by the policy: keys_per_split rounded up to the key
// tile, but never past the row's own key range rounded up to the tile (one
// split then covers the row), so every row gets at least one split. Computed
// in 64 bits: a policy near INT32_MAX must not wrap.
void fixed_split(int64_t keys_per_split, int64_t span, int tile, RowPlan &r) {
    const int64_t whole = std::max<int64_t>(tile, ceil_div(span, tile) * tile);
    const int64_t ls = std::min(whole, ceil_div(keys_per_split, tile) * tile);
    r.lsplit = (int32_t)ls;
    r.nsplit = (int32_t)std::max<int64_t>(1, ceil_div(span, ls));
}

// `lens`: the row lengths the call sees (the host lengths, or those after a
// fused append)
void plan_attention(const kv_cache *c, const int32_t *lens, int32_t q_heads, int32_t T, const int32_t *n_new,
                    Plan &p, bool all_decode) {
    const int G = q_heads / c->kv_heads;
    p.group = G;
    std::vector<int> dec_rows, pre_rows;
    int max_dec_cols = 0;
    for (int b = 0; b < c->batch; ++b) {
        const int n = n_new[b];
        if (n == 0) {
            p.zero_rows.push_back(b);
            continue;
        }
        bool use_dec;
        if (c->path_policy == 1 || all_decode) use_dec = G <= 64;
        else if (c->path_policy == 2) use_dec = false;
        else use_dec = (int64_t)G * n <= kDecodeAutoCols;
        if (use_dec) {
            dec_rows.push_back(b);
            max_dec_cols = std::max<int>(max_dec_cols, (int)std::min<int64_t>((int64_t)G * n, 64));
        } else {
            pre_rows.push_back(b);
        }
    }
    // decode: one column width for the launch, at least G so a tile holds a query.
    // A float32 cache at d = 128 takes at most two subtiles (32 columns) when G
    // allows: its four-subtile instance runs out of registers and spills, so
    // wider rows get more query tiles instead (their keys are read once per tile)
    int need = std::max(max_dec_cols, G);
    if (c->dtype == KV_DTYPE_F32 && c->head_dim == 128 && G <= 32) need = std::min(need, 32);
    p.nsub = need <= 16 ? 1 : (need <= 32 ? 2 : 4);
    p.dec_cols = 16 * p.nsub;

    // ---- decode rows: a work group streams at least kDecodeWaves tiles per
    //      split; keep splitting the longest rows while the chip is not full
    {
        const int tq = p.dec_cols / G;
        int64_t total = 0;
        for (int b : dec_rows)
            for (int qt = 0; qt < ceil_div(n_new[b], tq); ++qt)
                total += (int64_t)c->kv_heads * ceil_div(tile_span(lens[b], n_new[b], tq, qt, c->window),
                                                         kDecodeKeyTile);
        // tiles per work group: the whole job spread over the slots, never
        // fewer than one tile per wave
        const int64_t tpw = std::max<int64_t>(kDecodeWaves, ceil_div(total, kDecodeSlots));
        for (int b : dec_rows) {
            RowPlan r{};
            r.b = b;
            r.len = lens[b];
            r.nnew = n_new[b];
            r.nq = (int)ceil_div(r.nnew, tq);
            int64_t span = 0;                      // the longest query tile's key range
            for (int qt = 0; qt < r.nq; ++qt) span = std::max(span, tile_span(r.len, r.nnew, tq, qt, c->window));
            const int64_t tiles = ceil_div(span, kDecodeKeyTile);
            if (c->keys_per_split > 0) {
                fixed_split(c->keys_per_split, span, kDecodeKeyTile, r);
            } else {
                r.nsplit = (int)ceil_div(tiles, tpw);
                r.lsplit = (int)(ceil_div(tiles, r.nsplit) * kDecodeKeyTile);
                // A work group's waves take its tiles in rounds of kDecodeWaves.
                // When whole rounds per split leave at most one more round of
                // tiles (a decode step: a cached length of whole rounds plus
                // the new token), only the last split runs that round, and its
                // tiles there are the row's last (the new token's tile holds
                // one key), instead of every split running one more round.
                const int64_t whole = tiles / (r.nsplit * kDecodeWaves) * kDecodeWaves;
                if (r.nsplit > 1 && whole > 0 && tiles - r.nsplit * whole <= kDecodeWaves)
                    r.lsplit = (int)(whole * kDecodeKeyTile);
            }
            r.work = tiles * r.nq;
            p.dec.push_back(r);
        }
    }
    // ---- prefill rows: split only rows whose longest item would dominate
    {
        const int tq = prefill_cols(c->dtype, c->head_dim) / G;
        int64_t total = 0;
        for (int b : pre_rows)
            for (int qt = 0; qt < ceil_div(n_new[b], tq); ++qt)
                total += (int64_t)c->kv_heads * ceil_div(tile_span(lens[b], n_new[b], tq, qt, c->window),
                                                         kPrefillKeyTile);
        // a row is split only when its longest item would run well past the
        // per-slot share of the whole launch (the launch lasts as long as its
        // longest item)
        const int64_t cap = std::max<int64_t>(8, ceil_div(total, kPrefillSlots));    // tiles per item
        for (int b : pre_rows) {
            RowPlan r{};
            r.b = b;
            r.len = lens[b];
            r.nnew = n_new[b];
            r.nq = (int)ceil_div(r.nnew, tq);
            int64_t span = 0;
            for (int qt = 0; qt < r.nq; ++qt) span = std::max(span, tile_span(r.len, r.nnew, tq, qt, c->window));
            const int64_t tiles = ceil_div(span, kPrefillKeyTile);
            if (c->keys_per_split > 0) {
                fixed_split(c->keys_per_split, span, kPrefillKeyTile, r);
            } else {
                r.nsplit = 2 * tiles > 3 * cap ? (int)ceil_div(tiles, cap) : 1;
                r.lsplit = (int)(ceil_div(tiles, r.nsplit) * kPrefillKeyTile);
            }
            r.work = tiles * r.nq;
            p.pre.push_back(r);
        }
    }
    // heaviest rows first so long items start early
    auto heavier = [](const RowPlan &x, const RowPlan &y) { return x.work > y.work; };
    std::stable_sort(p.dec.begin(), p.dec.end(), heavier);
    std::stable_sort(p.pre.begin(), p.pre.end(), heavier);

    // ---- partial records for rows split across work groups
    p.records = 0;
    auto assign = [&](RowPlan &r, int cols) {
        if (r.nsplit > 1) {
            r.pbase = p.records;
            p.records += (int64_t)c->kv_heads * r.nq * r.nsplit * cols;
        } else {
            r.pbase = -1;
        }
    };
    for (auto &r : p.dec) assign(r, p.dec_cols);
    p.dec_records = p.records;
    for (auto &r : p.pre) assign(r, prefill_cols(c->dtype, c->head_dim));
    for (int b = 0; b < c->batch; ++b)
        if (n_new[b] < T) p.pad_rows.push_back(b);
}

// workspace: [partial acc: records x d floats][partial (m, l): records x 2 floats]
// [arrival counters of the decode kernel's merge: one 64-bit word per dec_cols
// decode records], each region 256-byte aligned
struct WsLayout {
    size_t acc = 0, ml = 0, cnt = 0, total = 0;
};

WsLayout ws_layout(const kv_cache *c, const Plan &p) {
    auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
    WsLayout w;
    if (p.records == 0) return w;
    w.acc = 0;
    w.ml = up((size_t)p.records * c->head_dim * sizeof(float));
    w.cnt = up(w.ml + (size_t)p.records * 2 * sizeof(float));
    w.total = w.cnt + (size_t)(p.dec_records / p.dec_cols) * sizeof(unsigned long long);
    return w;
}

// The tag of the decode kernel's arrival counters in this process: splitmix64
// (Steele, Lea and Flood, "Fast splittable pseudorandom number generators",
// 2014) of the clock at first use, cut to 64 - kMergeCountBits bits, never
// zero. Every completed call leaves its counter words at (tag, 0); a word the
// process has not used yet matches the tag only by chance (2^-56), so the
// workspace needs no clearing.
unsigned long long merge_tag() {
    static const unsigned long long tag = [] {
        uint64_t z = (uint64_t)std::chrono::steady_clock::now().time_since_epoch().count() + 0x9E3779B97F4A7C15ull;
        z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
        z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
        z ^= z >> 31;
        z >>= kMergeCountBits;
        return z == 0 ? 1ull : (unsigned long long)z;
    }();
    return tag;
}

size_t workspace_bytes_for(const kv_cache *c, const Plan &p) { return ws_layout(c, p).total; }

kv_status check_attention_args(const kv_cache *c, const int32_t *lens, int32_t q_heads, int32_t T,
                               const int32_t *n_new) {
    if (c == nullptr) return fail(KV_ERR_INVALID_ARG, "null cache handle");
    if (q_heads <= 0 || q_heads % c->kv_heads != 0)
        return fail(KV_ERR_INVALID_ARG, "q_heads %d is not a positive multiple of kv_heads %d", q_heads,
                    c->kv_heads);
    if (q_heads / c->kv_heads > 128)
        return fail(KV_ERR_UNSUPPORTED, "group size %d > 128", q_heads / c->kv_heads);
    if (T < 0) return fail(KV_ERR_INVALID_ARG, "T %d < 0", T);
    if (c->batch > 0 && n_new == nullptr) return fail(KV_ERR_INVALID_ARG, "n_new is null");
    for (int b = 0; b < c->batch; ++b) {
        if (n_new[b] < 0 || n_new[b] > T)
            return fail(KV_ERR_INVALID_ARG, "row %d: n_new %d outside 0..%d", b, n_new[b], T);
        if (n_new[b] > lens[b])
            return fail(KV_ERR_INVALID_ARG, "row %d: n_new %d > length %d (append before attention)", b,
                        n_new[b], lens[b]);
    }
    return KV_OK;
}

// Workspace for a call with these rows: the larger of the automatic plan and
// the all-decode plan that a tree-verify call makes (the size queries do not
// know whether the call will pass parents).
size_t workspace_need(const kv_cache *c, const int32_t *lens, int32_t q_heads, int32_t T, const int32_t *n_new) {
    Plan p;
    plan_attention(c, lens, q_heads, T, n_new, p, false);
    size_t need = workspace_bytes_for(c, p);
    if ((int64_t)(q_heads / c->kv_heads) * T <= 64) {
        Plan t;
        plan_attention(c, lens, q_heads, T, n_new, t, true);
        need = std::max(need, workspace_bytes_for(c, t));
    }
    return need;
}

void fill_attn_rows(const std::vector<RowPlan> &rows, size_t lo, size_t hi, int hkv, AttnRows &t) {
    std::memset(&t, 0, sizeof t);
    t.n_rows = (int32_t)(hi - lo);
    int32_t item = 0;
    for (size_t i = lo; i < hi; ++i) {
        const RowPlan &r = rows[i];
        const int j = (int)(i - lo);
        t.b[j] = r.b;
        t.len[j] = r.len;
        t.nnew[j] = r.nnew;
        t.nsplit[j] = r.nsplit;
        t.lsplit[j] = r.lsplit;
        t.pbase[j] = (int32_t)r.pbase;
        t.item0[j] = item;
        item += hkv * r.nq * r.nsplit;
    }
    t.item0[t.n_rows] = item;
    t.total_items = item;
}

struct PagedSpec {
    int32_t num_pages, page_size, max_blocks;
    int32_t *table_dev;
};

kv_status create_cache(int32_t batch, int32_t kv_heads, int32_t max_len, int32_t head_dim, kv_dtype dtype,
                       void *k_buf, void *v_buf, int32_t *lens_dev, void *stream, bool ring, int32_t window,
                       const float *k_scale, const float *v_scale, const PagedSpec *pg, kv_cache **out);

// Paged caches: blocks a row of `len` tokens occupies.
int64_t blocks_of(const kv_cache *c, int64_t len) { return ceil_div(len, c->page_size); }

// Enqueue device block-table updates (index, page) in chunks that fit the
// kernel arguments.
kv_status push_table_updates(kv_cache *c, const std::vector<std::pair<int32_t, int32_t>> &upd, hipStream_t st,
                             const char *what) {
    for (size_t lo = 0; lo < upd.size(); lo += kMaxTableUpdates) {
        TableArgs t{};
        t.table = c->table_dev;
        const size_t hi = std::min(upd.size(), lo + kMaxTableUpdates);
        t.n = (int32_t)(hi - lo);
        for (size_t i = lo; i < hi; ++i) {
            t.idx[i - lo] = upd[i].first;
            t.page[i - lo] = upd[i].second;
        }
        hipError_t e = launch_table_set(t, st);
        if (e != hipSuccess) return device_fail(e, what);
    }
    return KV_OK;
}

kv_status attention_call(kv_cache *c, const void *q, int32_t q_heads, int32_t T, const int32_t *n_new,
                         const int32_t *parents, void *out, void *workspace, size_t workspace_bytes, void *stream);

// An attention call's checks and plan, against `lens`, before anything is enqueued.
kv_status attention_prepare(const kv_cache *c, const int32_t *lens, const void *q, int32_t q_heads, int32_t T,
                            const int32_t *n_new, void *out, void *workspace, size_t workspace_bytes, Plan &p,
                            bool all_decode);
// New tokens a decode kernel appends itself (kv_append_attention): read from
// k_new / v_new [B, Hkv, T, d] and written to the cache by the kernel.
kv_status check_tree(const kv_cache *c, int32_t q_heads, int32_t T, const int32_t *n_new, const int32_t *parents);
// one_stream: every kernel of the call on `stream` (no side stream is created
// or used, so the call creates no stream or event)
kv_status append_attention_call(kv_cache *c, const void *k_new, const void *v_new, const void *q, int32_t q_heads,
                                int32_t T, const int32_t *n_new, const int32_t *parents, void *out,
                                void *workspace, size_t workspace_bytes, void *stream, bool one_stream = false);
struct Fused {
    const void *k_new = nullptr, *v_new = nullptr;
};
kv_status attention_launch(kv_cache *c, const Plan &p, const void *q, int32_t q_heads, int32_t T,
                           const int32_t *n_new, const int32_t *parents, void *out, void *workspace,
                           const Fused *fused, void *stream, bool one_stream = false);
// An append's checks (all rows, the pool), before anything is enqueued.
kv_status append_check(const kv_cache *c, const void *k_new, const void *v_new, int32_t T, const int32_t *n_new,
                       int64_t *pages_needed, bool check_pointers = true);
// Enqueue an append that append_check accepted: pages, the copy kernel for
// every row with skip[b] == 0 (all rows when skip is null), then the lengths.
kv_status append_commit(kv_cache *c, const void *k_new, const void *v_new, int32_t T, const int32_t *n_new,
                        int64_t pages_needed, const std::vector<char> *skip, void *stream);

// Ring caches: the lowest position a row of this length still holds, and the
// lowest key a query at position pos sees ([MASK] "A strong answer", reversal).
int64_t oldest_kept(const kv_cache *c, int64_t len) { return c->ring ? std::max<int64_t>(0, len - c->max_len) : 0; }
int64_t lowest_needed(const kv_cache *c, int64_t pos) { return std::max<int64_t>(0, pos - c->window + 1); }

}  // namespace

// ===========================================================================
extern "C" {

kv_status kv_cache_create(int32_t batch, int32_t kv_heads, int32_t max_len, int32_t head_dim,
                          kv_dtype dtype, void *k_buf, void *v_buf, int32_t *lens_dev, void *stream,
                          kv_cache **out) {
    if (dtype == KV_DTYPE_FP8_E4M3)
        return fail(KV_ERR_UNSUPPORTED, "an E4M3 cache needs its scales: use kv_cache_create_fp8");
    return create_cache(batch, kv_heads, max_len, head_dim, dtype, k_buf, v_buf, lens_dev, stream, false,
                        kNoWindow, nullptr, nullptr, nullptr, out);
}

kv_status kv_cache_create_fp8(int32_t batch, int32_t kv_heads, int32_t max_len, int32_t head_dim,
                              const float *k_scale, const float *v_scale, void *k_buf, void *v_buf,
                              int32_t *lens_dev, void *stream, kv_cache **out) {
    if (out == nullptr) return fail(KV_ERR_INVALID_ARG, "out is null");
    *out = nullptr;
    if (kv_heads > kMaxScaleHeads)
        return fail(KV_ERR_UNSUPPORTED, "an E4M3 cache supports at most %d kv heads", kMaxScaleHeads);
    if (kv_heads > 0 && (k_scale == nullptr || v_scale == nullptr))
        return fail(KV_ERR_INVALID_ARG, "k_scale/v_scale is null");
    for (int h = 0; h < kv_heads; ++h)
        if (!(std::isfinite(k_scale[h]) && k_scale[h] > 0.f && std::isfinite(v_scale[h]) && v_scale[h] > 0.f))
            return fail(KV_ERR_INVALID_ARG, "kv head %d: scales must be finite and positive", h);
    return create_cache(batch, kv_heads, max_len, head_dim, KV_DTYPE_FP8_E4M3, k_buf, v_buf, lens_dev, stream,
                        false, kNoWindow, k_scale, v_scale, nullptr, out);
}

kv_status kv_cache_create_ring(int32_t batch, int32_t kv_heads, int32_t capacity, int32_t head_dim,
                               kv_dtype dtype, int32_t window, void *k_buf, void *v_buf, int32_t *lens_dev,
                               void *stream, kv_cache **out) {
    if (out == nullptr) return fail(KV_ERR_INVALID_ARG, "out is null");
    *out = nullptr;
    if (capacity <= 0 || capacity % kRingAlign != 0)
        return fail(KV_ERR_INVALID_ARG, "ring capacity %d is not a positive multiple of %d", capacity, kRingAlign);
    if (window < 1 || window > capacity)
        return fail(KV_ERR_INVALID_ARG, "window %d outside 1..capacity %d", window, capacity);
    if (dtype == KV_DTYPE_FP8_E4M3) return fail(KV_ERR_UNSUPPORTED, "ring caches hold float32 or bfloat16");
    return create_cache(batch, kv_heads, capacity, head_dim, dtype, k_buf, v_buf, lens_dev, stream, true, window,
                        nullptr, nullptr, nullptr, out);
}

kv_status kv_cache_create_paged(int32_t batch, int32_t kv_heads, int32_t num_pages, int32_t page_size,
                                int32_t max_blocks, int32_t head_dim, kv_dtype dtype, void *k_pool, void *v_pool,
                                int32_t *block_table, int32_t *lens_dev, void *stream, kv_cache **out) {
    if (out == nullptr) return fail(KV_ERR_INVALID_ARG, "out is null");
    *out = nullptr;
    if (page_size < kMinPage || page_size > kMaxPage || (page_size & (page_size - 1)) != 0)
        return fail(KV_ERR_INVALID_ARG, "page_size %d is not a power of two in %d..%d", page_size, kMinPage,
                    kMaxPage);
    if (num_pages <= 0 || max_blocks <= 0)
        return fail(KV_ERR_INVALID_ARG, "bad pool num_pages=%d max_blocks=%d", num_pages, max_blocks);
    if ((int64_t)max_blocks * page_size > INT32_MAX - kRingAlign)
        return fail(KV_ERR_INVALID_ARG, "max_blocks * page_size out of range");
    if ((int64_t)batch * max_blocks > INT32_MAX) return fail(KV_ERR_INVALID_ARG, "block table too large");
    if ((int64_t)num_pages * kv_heads * page_size * head_dim >= (int64_t(1) << 40))
        return fail(KV_ERR_INVALID_ARG, "page pool too large");
    if (dtype == KV_DTYPE_FP8_E4M3) return fail(KV_ERR_UNSUPPORTED, "paged caches hold float32 or bfloat16");
    if (batch > 0 && block_table == nullptr) return fail(KV_ERR_INVALID_ARG, "block_table is null");
    if (!aligned16(block_table)) return fail(KV_ERR_INVALID_ARG, "buffers must be 16-byte aligned");
    const PagedSpec pg{num_pages, page_size, max_blocks, block_table};
    return create_cache(batch, kv_heads, max_blocks * page_size, head_dim, dtype, k_pool, v_pool, lens_dev, stream,
                        false, kNoWindow, nullptr, nullptr, &pg, out);
}

}  // extern "C"

namespace {
kv_status create_cache(int32_t batch, int32_t kv_heads, int32_t max_len, int32_t head_dim, kv_dtype dtype,
                       void *k_buf, void *v_buf, int32_t *lens_dev, void *stream, bool ring, int32_t window,
                       const float *k_scale, const float *v_scale, const PagedSpec *pg, kv_cache **out) {
    if (out == nullptr) return fail(KV_ERR_INVALID_ARG, "out is null");
    *out = nullptr;
    if (dtype != KV_DTYPE_F32 && dtype != KV_DTYPE_BF16 && dtype != KV_DTYPE_FP8_E4M3)
        return fail(KV_ERR_UNSUPPORTED, "unknown dtype %d", (int)dtype);
    if (head_dim != 16 && head_dim != 32 && head_dim != 64 && head_dim != 128)
        return fail(KV_ERR_UNSUPPORTED, "head_dim %d not in {16, 32, 64, 128}", head_dim);
    if (batch < 0 || kv_heads <= 0 || max_len <= 0)
        return fail(KV_ERR_INVALID_ARG, "bad shape batch=%d kv_heads=%d max_len=%d", batch, kv_heads, max_len);
    if (batch > 0 && (k_buf == nullptr || v_buf == nullptr))
        return fail(KV_ERR_INVALID_ARG, "k_buf/v_buf is null");
    if (!aligned16(k_buf) || !aligned16(v_buf) || !aligned16(lens_dev))
        return fail(KV_ERR_INVALID_ARG, "buffers must be 16-byte aligned");
    if (pg == nullptr && (int64_t)batch * kv_heads * max_len * head_dim >= (int64_t(1) << 40))
        return fail(KV_ERR_INVALID_ARG, "cache too large");
    kv_cache *c = new (std::nothrow) kv_cache;
    if (c == nullptr) return fail(KV_ERR_DEVICE, "out of host memory");
    c->batch = batch;
    c->kv_heads = kv_heads;
    c->max_len = max_len;
    c->head_dim = head_dim;
    c->dtype = dtype;
    c->elem_bytes = dtype == KV_DTYPE_F32 ? 4 : (dtype == KV_DTYPE_BF16 ? 2 : 1);
    c->io_bytes = dtype == KV_DTYPE_F32 ? 4 : 2;
    if (dtype == KV_DTYPE_FP8_E4M3) {
        c->k_scale.assign(k_scale, k_scale + kv_heads);
        c->v_scale.assign(v_scale, v_scale + kv_heads);
        for (int h = 0; h < kv_heads; ++h) {
            c->k_inv.push_back(1.0f / k_scale[h]);
            c->v_inv.push_back(1.0f / v_scale[h]);
        }
    }
    c->k = k_buf;
    c->v = v_buf;
    c->lens_dev = lens_dev;
    c->lens.assign(batch, 0);
    c->ring = ring;
    c->window = window;
    if (pg != nullptr) {
        c->paged = true;
        c->num_pages = pg->num_pages;
        c->page_size = pg->page_size;
        while ((1 << c->page_shift) < pg->page_size) ++c->page_shift;
        c->max_blocks = pg->max_blocks;
        c->table_dev = pg->table_dev;
        c->table.assign((size_t)batch * pg->max_blocks, -1);
        for (int32_t i = 0; i < pg->num_pages; ++i) c->free_pages.push(i);
        hipError_t e = launch_table_fill(c->table_dev, (int64_t)batch * pg->max_blocks, -1, (hipStream_t)stream);
        if (e != hipSuccess) {
            delete c;
            return device_fail(e, "kv_cache_create_paged");
        }
    }
    // the reservation starts as zeros ([GQA] "A strong answer" and [CH16]
    // "Layout and validity" both build the cache from zeros), so every byte
    // past a row's length is defined from the start
    if (batch > 0) {
        const int64_t bytes = pg != nullptr
            ? (int64_t)pg->num_pages * kv_heads * pg->page_size * head_dim * c->elem_bytes
            : (int64_t)batch * kv_heads * max_len * head_dim * c->elem_bytes;
        hipError_t e = launch_zero_bytes(k_buf, bytes, (hipStream_t)stream);
        if (e == hipSuccess) e = launch_zero_bytes(v_buf, bytes, (hipStream_t)stream);
        if (e != hipSuccess) {
            delete c;
            return device_fail(e, "kv_cache_create (zero fill)");
        }
    }
    if (lens_dev != nullptr) {
        for (int lo = 0; lo < batch; lo += kMaxRows) {
            LensTable t{};
            t.n_rows = std::min(kMaxRows, batch - lo);
            for (int i = 0; i < t.n_rows; ++i) {
                t.b[i] = lo + i;
                t.len[i] = 0;
            }
            hipError_t e = launch_set_lens(lens_dev, t, (hipStream_t)stream);
            if (e != hipSuccess) {
                delete c;
                return device_fail(e, "kv_cache_create");
            }
        }
    }
    *out = c;
    return ok();
}
}  // namespace

extern "C" {

kv_status kv_cache_destroy(kv_cache *c) {
    if (c == nullptr) return ok();
    side_stream_destroy(c->side);
    delete c;
    return ok();
}

kv_status kv_append(kv_cache *c, const void *k_new, const void *v_new, int32_t T, const int32_t *n_new,
                    void *stream) {
    int64_t pages = 0;
    kv_status s = append_check(c, k_new, v_new, T, n_new, &pages);
    if (s != KV_OK) return s;
    s = append_commit(c, k_new, v_new, T, n_new, pages, nullptr, stream);
    return s == KV_OK ? ok() : s;
}

kv_status gqa_attention_workspace_size(const kv_cache *c, int32_t q_heads, int32_t T, const int32_t *n_new,
                                       size_t *bytes) {
    if (bytes == nullptr) return fail(KV_ERR_INVALID_ARG, "bytes is null");
    *bytes = 0;
    kv_status s = check_attention_args(c, c == nullptr ? nullptr : c->lens.data(), q_heads, T, n_new);
    if (s != KV_OK) return s;
    if (c->batch == 0 || T == 0) return ok();
    *bytes = workspace_need(c, c->lens.data(), q_heads, T, n_new);
    return ok();
}

kv_status gqa_attention(kv_cache *c, const void *q, int32_t q_heads, int32_t T, const int32_t *n_new,
                        void *out, void *workspace, size_t workspace_bytes, void *stream) {
    return attention_call(c, q, q_heads, T, n_new, nullptr, out, workspace, workspace_bytes, stream);
}

kv_status gqa_attention_tree(kv_cache *c, const void *q, int32_t q_heads, int32_t T, const int32_t *n_new,
                             const int32_t *parents, void *out, void *workspace, size_t workspace_bytes,
                             void *stream) {
    kv_status s = check_attention_args(c, c == nullptr ? nullptr : c->lens.data(), q_heads, T, n_new);
    if (s != KV_OK) return s;
    s = check_tree(c, q_heads, T, n_new, parents);
    if (s != KV_OK) return s;
    return attention_call(c, q, q_heads, T, n_new, parents, out, workspace, workspace_bytes, stream);
}

kv_status kv_append_attention_workspace_size(const kv_cache *c, int32_t q_heads, int32_t T, const int32_t *n_new,
                                             size_t *bytes) {
    if (bytes == nullptr) return fail(KV_ERR_INVALID_ARG, "bytes is null");
    *bytes = 0;
    int64_t pages = 0;
    kv_status s = append_check(c, nullptr, nullptr, T, n_new, &pages, false);
    if (s != KV_OK) return s;
    std::vector<int32_t> after(c->lens);
    for (int b = 0; b < c->batch; ++b) after[b] += n_new[b];
    s = check_attention_args(c, after.data(), q_heads, T, n_new);
    if (s != KV_OK) return s;
    if (c->batch == 0 || T == 0) return ok();
    *bytes = workspace_need(c, after.data(), q_heads, T, n_new);
    return ok();
}

kv_status kv_append_attention(kv_cache *c, const void *k_new, const void *v_new, const void *q, int32_t q_heads,
                              int32_t T, const int32_t *n_new, void *out, void *workspace, size_t workspace_bytes,
                              void *stream) {
    return append_attention_call(c, k_new, v_new, q, q_heads, T, n_new, nullptr, out, workspace, workspace_bytes,
                                 stream);
}

kv_status kv_append_attention_noalloc(kv_cache *c, const void *k_new, const void *v_new, const void *q,
                                      int32_t q_heads, int32_t T, const int32_t *n_new, void *out, void *stream) {
    if (c == nullptr) return fail(KV_ERR_INVALID_ARG, "null cache handle");
    // the library's own scratch on the current device stands in for the
    // caller's workspace; every kernel runs on `stream`
    void *scratch = nullptr;
    const hipError_t e = scratch_region(&scratch);
    if (e != hipSuccess) return device_fail(e, "kv_append_attention_noalloc (scratch address)");
    const kv_status s = append_attention_call(c, k_new, v_new, q, q_heads, T, n_new, nullptr, out, scratch,
                                              kScratchBytes, stream, true);
    if (s == KV_ERR_WORKSPACE) {
        const std::string why = g_err;
        return fail(KV_ERR_WORKSPACE, "kv_append_attention_noalloc: %s; the entry point holds %zu bytes of scratch "
                    "per GPU (call kv_append_attention with a workspace instead)", why.c_str(), kScratchBytes);
    }
    return s;
}

kv_status kv_append_attention_tree(kv_cache *c, const void *k_new, const void *v_new, const void *q,
                                   int32_t q_heads, int32_t T, const int32_t *n_new, const int32_t *parents,
                                   void *out, void *workspace, size_t workspace_bytes, void *stream) {
    if (c == nullptr) return fail(KV_ERR_INVALID_ARG, "null cache handle");
    kv_status s = check_tree(c, q_heads, T, n_new, parents);
    if (s != KV_OK) return s;
    return append_attention_call(c, k_new, v_new, q, q_heads, T, n_new, parents, out, workspace, workspace_bytes,
                                 stream);
}

}  // extern "C"

namespace {
kv_status check_tree(const kv_cache *c, int32_t q_heads, int32_t T, const int32_t *n_new, const int32_t *parents) {
    if (q_heads <= 0 || q_heads % c->kv_heads != 0)
        return fail(KV_ERR_INVALID_ARG, "q_heads %d is not a positive multiple of kv_heads %d", q_heads,
                    c->kv_heads);
    if (T < 0 || (c->batch > 0 && n_new == nullptr)) return fail(KV_ERR_INVALID_ARG, "bad T or null n_new");
    if (T > kMaxTreeNodes || (int64_t)(q_heads / c->kv_heads) * T > 64)
        return fail(KV_ERR_UNSUPPORTED, "tree verify takes at most %d nodes and G * T <= 64", kMaxTreeNodes);
    if (c->ring) return fail(KV_ERR_UNSUPPORTED, "tree verify runs on linear caches");
    if (c->path_policy == 2) return fail(KV_ERR_UNSUPPORTED, "tree verify runs on the split-K decode kernel");
    if (c->batch > 0 && T > 0 && parents == nullptr) return fail(KV_ERR_INVALID_ARG, "parents is null");
    // [MASK] "What interviewers probe next": parent pointers; here every parent
    // is -1 (the committed prefix) or an earlier node of the same row
    for (int b = 0; b < c->batch; ++b) {
        if (n_new[b] < 0 || n_new[b] > T)
            return fail(KV_ERR_INVALID_ARG, "row %d: n_new %d outside 0..%d", b, n_new[b], T);
        for (int u = 0; u < n_new[b]; ++u) {
            const int p = parents[(int64_t)b * T + u];
            if (p < -1 || p >= u)
                return fail(KV_ERR_INVALID_ARG, "row %d node %d: parent %d is not -1 or an earlier node", b, u, p);
        }
    }
    return KV_OK;
}

kv_status append_attention_call(kv_cache *c, const void *k_new, const void *v_new, const void *q, int32_t q_heads,
                                int32_t T, const int32_t *n_new, const int32_t *parents, void *out,
                                void *workspace, size_t workspace_bytes, void *stream, bool one_stream) {
    // every check of both halves first, against the lengths after the append
    int64_t pages = 0;
    kv_status s = append_check(c, k_new, v_new, T, n_new, &pages);
    if (s != KV_OK) return s;
    std::vector<int32_t> after(c->lens);
    for (int b = 0; b < c->batch; ++b) after[b] += n_new[b];
    Plan p;
    s = attention_prepare(c, after.data(), q, q_heads, T, n_new, out, workspace, workspace_bytes, p,
                          parents != nullptr);
    if (s != KV_OK) return s;
    // rows of the decode kernel append themselves; prefill rows go through
    // the copy kernel (appending in the prefill kernel measured slower: it
    // costs that kernel registers on every tile)
    const bool fuse = !p.dec.empty();
    std::vector<char> skip(c->batch, 0);
    for (const RowPlan &r : p.dec) skip[r.b] = 1;
    s = append_commit(c, k_new, v_new, T, n_new, pages, &skip, stream);
    if (s != KV_OK) return s;
    Fused f;
    f.k_new = k_new;
    f.v_new = v_new;
    s = attention_launch(c, p, q, q_heads, T, n_new, parents, out, workspace, fuse ? &f : nullptr, stream,
                         one_stream);
    return s == KV_OK ? ok() : s;
}

kv_status append_check(const kv_cache *c, const void *k_new, const void *v_new, int32_t T, const int32_t *n_new,
                       int64_t *pages_out, bool check_pointers) {
    if (c == nullptr) return fail(KV_ERR_INVALID_ARG, "null cache handle");
    if (T < 0) return fail(KV_ERR_INVALID_ARG, "T %d < 0", T);
    if (c->batch > 0 && n_new == nullptr) return fail(KV_ERR_INVALID_ARG, "n_new is null");
    int64_t total = 0;
    // [GQA] "A strong answer": a row that would pass max_len raises; here every
    // row is checked before anything is enqueued, so a failure changes nothing
    for (int b = 0; b < c->batch; ++b) {
        if (n_new[b] < 0 || n_new[b] > T)
            return fail(KV_ERR_INVALID_ARG, "row %d: n_new %d outside 0..%d", b, n_new[b], T);
        const int64_t s = c->lens[b], n = n_new[b];
        if (!c->ring && s + n > c->max_len)
            return fail(KV_ERR_CAPACITY, "row %d: %lld tokens > max_len %d", b, (long long)(s + n), c->max_len);
        // a ring write may not evict a key the first new query still needs
        if (c->ring && n > 0 && oldest_kept(c, s + n) > lowest_needed(c, s))
            return fail(KV_ERR_CAPACITY, "row %d: %lld new tokens would evict keys the window still needs "
                        "(capacity %d, window %d)", b, (long long)n, c->max_len, c->window);
        if (s + n > INT32_MAX - kRingAlign)
            return fail(KV_ERR_CAPACITY, "row %d: position %lld out of range", b, (long long)(s + n));
        total += n;
    }
    // a paged cache takes the pages the new tokens need from the pool; the
    // call is refused whole if the pool cannot give them all
    int64_t pages_needed = 0;
    if (c->paged) {
        for (int b = 0; b < c->batch; ++b)
            pages_needed += blocks_of(c, (int64_t)c->lens[b] + n_new[b]) - blocks_of(c, c->lens[b]);
        if (pages_needed > (int64_t)c->free_pages.size())
            return fail(KV_ERR_CAPACITY, "%lld pages needed, %zu free in the pool", (long long)pages_needed,
                        c->free_pages.size());
    }
    if (total > 0 && check_pointers) {
        if (k_new == nullptr || v_new == nullptr) return fail(KV_ERR_INVALID_ARG, "k_new/v_new is null");
        if (!aligned16(k_new) || !aligned16(v_new))
            return fail(KV_ERR_INVALID_ARG, "k_new/v_new must be 16-byte aligned");
    }
    *pages_out = pages_needed;
    return KV_OK;
}

kv_status append_commit(kv_cache *c, const void *k_new, const void *v_new, int32_t T, const int32_t *n_new,
                        int64_t pages_needed, const std::vector<char> *skip, void *stream) {
    if (pages_needed > 0) {
        // row by row, each new block gets the lowest-numbered free page; the
        // device table learns the entries before the copy kernel reads them
        std::vector<std::pair<int32_t, int32_t>> upd;
        for (int b = 0; b < c->batch; ++b)
            for (int64_t i = blocks_of(c, c->lens[b]); i < blocks_of(c, (int64_t)c->lens[b] + n_new[b]); ++i) {
                const int32_t page = c->free_pages.top();
                c->free_pages.pop();
                const int32_t idx = (int32_t)((int64_t)b * c->max_blocks + i);
                c->table[idx] = page;
                upd.push_back({idx, page});
            }
        kv_status st = push_table_updates(c, upd, (hipStream_t)stream, "kv_append (block table)");
        if (st != KV_OK) return st;
    }
    std::vector<int> rows;
    for (int b = 0; b < c->batch; ++b)
        if (n_new[b] > 0 && (skip == nullptr || !(*skip)[b])) rows.push_back(b);
    const int64_t row_bytes = (int64_t)c->head_dim * c->io_bytes;      // of k_new / v_new
    for (size_t lo = 0; lo < rows.size(); lo += kMaxRows) {
        AppendArgs a{};
        a.k = c->k;
        a.v = c->v;
        a.k_new = k_new;
        a.v_new = v_new;
        a.lens_dev = c->lens_dev;
        a.row_bytes = row_bytes;
        a.quant = c->dtype == KV_DTYPE_FP8_E4M3;
        for (size_t h = 0; h < c->k_inv.size(); ++h) {
            a.k_inv[h] = c->k_inv[h];
            a.v_inv[h] = c->v_inv[h];
        }
        a.row_shift = 0;
        while ((int64_t(1) << a.row_shift) < row_bytes) ++a.row_shift;
        a.batch = c->batch;
        a.hkv = c->kv_heads;
        a.max_len = c->max_len;
        a.T = T;
        a.table = c->paged ? c->table_dev : nullptr;
        a.page_shift = c->page_shift;
        a.max_blocks = c->max_blocks;
        const size_t hi = std::min(rows.size(), lo + kMaxRows);
        a.t.n_rows = (int32_t)(hi - lo);
        int32_t blocks = 0;
        for (size_t i = lo; i < hi; ++i) {
            const int j = (int)(i - lo), b = rows[i];
            a.t.b[j] = b;
            a.t.start[j] = c->lens[b];
            a.t.slot0[j] = c->lens[b] % c->max_len;
            a.t.n[j] = n_new[b];
            a.t.nchunk[j] = (int32_t)ceil_div((int64_t)n_new[b] * row_bytes, kAppendChunk);
            a.t.block0[j] = blocks;
            blocks += c->kv_heads * a.t.nchunk[j];
        }
        a.t.block0[a.t.n_rows] = blocks;
        hipError_t e = launch_append(a, blocks, (hipStream_t)stream);
        if (e != hipSuccess) return device_fail(e, "kv_append");
    }
    // the length moves only after the write is enqueued ([GQA] "Common mistakes")
    for (int b = 0; b < c->batch; ++b) c->lens[b] += n_new[b];
    return KV_OK;
}

kv_status attention_prepare(const kv_cache *c, const int32_t *lens, const void *q, int32_t q_heads, int32_t T,
                            const int32_t *n_new, void *out, void *workspace, size_t workspace_bytes, Plan &p,
                            bool all_decode) {
    kv_status s = check_attention_args(c, lens, q_heads, T, n_new);
    if (s != KV_OK) return s;
    if (c->batch == 0 || T == 0) return KV_OK;           // an empty plan: nothing to launch
    if (q == nullptr || out == nullptr) return fail(KV_ERR_INVALID_ARG, "q/out is null");
    if (!aligned16(q) || !aligned16(out) || !aligned16(workspace))
        return fail(KV_ERR_INVALID_ARG, "q/out/workspace must be 16-byte aligned");
    plan_attention(c, lens, q_heads, T, n_new, p, all_decode);
    const size_t need = workspace_bytes_for(c, p);
    if (need > 0 && (workspace == nullptr || workspace_bytes < need))
        return fail(KV_ERR_WORKSPACE, "workspace of %zu bytes < %zu required", workspace_bytes, need);
    if (p.records > INT32_MAX / 2)
        return fail(KV_ERR_UNSUPPORTED, "too many split partials");
    // each launch's work items must fit one grid dimension
    for (const std::vector<RowPlan> *rows : {&p.dec, &p.pre})
        for (size_t lo = 0; lo < rows->size(); lo += kMaxRows) {
            int64_t items = 0;
            for (size_t i = lo; i < std::min(rows->size(), lo + kMaxRows); ++i)
                items += (int64_t)c->kv_heads * (*rows)[i].nq * (*rows)[i].nsplit;
            if (items > INT32_MAX) return fail(KV_ERR_UNSUPPORTED, "too many work items in one launch");
        }
    return KV_OK;
}

kv_status attention_call(kv_cache *c, const void *q, int32_t q_heads, int32_t T, const int32_t *n_new,
                         const int32_t *parents, void *out, void *workspace, size_t workspace_bytes,
                         void *stream) {
    Plan p;
    kv_status s = attention_prepare(c, c->lens.data(), q, q_heads, T, n_new, out, workspace, workspace_bytes, p,
                                    parents != nullptr);
    if (s != KV_OK) return s;
    s = attention_launch(c, p, q, q_heads, T, n_new, parents, out, workspace, nullptr, stream);
    return s == KV_OK ? ok() : s;
}

kv_status attention_launch(kv_cache *c, const Plan &p, const void *q, int32_t q_heads, int32_t T,
                           const int32_t *n_new, const int32_t *parents, void *out, void *workspace,
                           const Fused *fused, void *stream, bool one_stream) {
    if (p.dec.empty() && p.pre.empty() && p.pad_rows.empty()) return KV_OK;
    hipStream_t st = (hipStream_t)stream;
    const WsLayout w = ws_layout(c, p);
    char *ws = (char *)workspace;

    // A call with prefill rows runs the decode kernel and the zero fill on a
    // side stream forked from (and later joined back to) the caller's
    // stream, beside the prefill kernel: the MFMA-bound prefill then starts
    // at once and the HBM-bound work fills the chip around it. The three
    // write disjoint output slots.
    const bool mixed = !one_stream && !p.pre.empty() && (!p.dec.empty() || !p.pad_rows.empty());
    hipStream_t dec_stream = st;
    if (mixed) {
        hipError_t e = side_stream_init(c->side);
        if (e == hipSuccess) e = side_stream_fork(c->side, st);
        if (e != hipSuccess) return device_fail(e, "gqa_attention (side stream)");
        dec_stream = c->side.side;
    }

    AttnArgs a{};
    a.q = q;
    a.out = out;
    a.k = c->k;
    a.v = c->v;
    a.ws_acc = w.total ? (float *)(ws + w.acc) : nullptr;
    a.ws_ml = w.total ? (float *)(ws + w.ml) : nullptr;
    a.counters = w.total ? (unsigned long long *)(ws + w.cnt) : nullptr;
    a.merge_tag = merge_tag();
    a.batch = c->batch;
    a.T = T;
    a.hq = q_heads;
    a.hkv = c->kv_heads;
    a.group = p.group;
    a.max_len = c->max_len;
    a.head_dim = c->head_dim;
    a.window = c->window;
    a.table = c->paged ? c->table_dev : nullptr;
    a.page_shift = c->page_shift;
    a.max_blocks = c->max_blocks;
    for (size_t h = 0; h < c->k_scale.size(); ++h) {
        a.k_scale[h] = c->k_scale[h];
        a.v_scale[h] = c->v_scale[h];
        a.k_inv[h] = c->k_inv[h];
        a.v_inv[h] = c->v_inv[h];
    }
    a.records = p.records;
    a.scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)c->head_dim));

    a.tree = parents != nullptr;
    a.cols = p.dec_cols;
    if (fused != nullptr) {
        a.fuse = 1;
        a.k_new = fused->k_new;
        a.v_new = fused->v_new;
        a.lens_dev = c->lens_dev;
    }
    // padded slots: independent of the attention kernels. First on the
    // stream: in a mixed call the fill's small work groups share CUs with
    // the prefill kernel's (which leave registers to spare), where a decode
    // work group has to wait for a whole CU
    for (size_t lo = 0; lo < p.pad_rows.size(); lo += kMaxRows) {
        ZeroArgs z{};
        z.out = out;
        z.batch = c->batch;
        z.T = T;
        z.hq = q_heads;
        z.head_dim = c->head_dim;
        z.row_bytes = (int64_t)c->head_dim * c->io_bytes;
        z.slices = (int32_t)ceil_div((int64_t)T * z.row_bytes, kZeroSlice);
        const size_t hi = std::min(p.pad_rows.size(), lo + kMaxRows);
        z.rows.n_rows = (int32_t)(hi - lo);
        for (size_t i = lo; i < hi; ++i) {
            z.rows.b[i - lo] = p.pad_rows[i];
            z.rows.nnew[i - lo] = n_new[p.pad_rows[i]];
        }
        hipError_t e = launch_zero_fill(z, dec_stream);
        if (e != hipSuccess) return device_fail(e, "gqa_attention (zero fill)");
    }
    for (size_t lo = 0; lo < p.dec.size(); lo += kMaxRows) {
        fill_attn_rows(p.dec, lo, std::min(p.dec.size(), lo + kMaxRows), c->kv_heads, a.rows);
        if (a.tree) {
            std::memset(a.parent, -1, sizeof a.parent);
            for (int j = 0; j < a.rows.n_rows; ++j)
                for (int u = 0; u < a.rows.nnew[j]; ++u)
                    a.parent[j][u] = (int8_t)parents[(int64_t)a.rows.b[j] * T + u];
        }
        hipError_t e = launch_decode((int)c->dtype, c->head_dim, p.nsub, a, dec_stream);
        if (e != hipSuccess) return device_fail(e, "gqa_attention (decode kernel)");
    }

    a.cols = prefill_cols(c->dtype, c->head_dim);
    a.tree = 0;
    a.fuse = 0;                // prefill rows were appended by the copy kernel
    for (size_t lo = 0; lo < p.pre.size(); lo += kMaxRows) {
        fill_attn_rows(p.pre, lo, std::min(p.pre.size(), lo + kMaxRows), c->kv_heads, a.rows);
        hipError_t e = launch_prefill((int)c->dtype, c->head_dim, a, st);
        if (e != hipSuccess) return device_fail(e, "gqa_attention (prefill kernel)");
    }
    // rows split across work groups and not merged in the decode kernel:
    // merge their partials. The prefill rows' merge needs only the prefill
    // kernel, so it runs on the caller's stream before the join, beside the
    // decode kernel's tail; decode rows split more than kMergeMaxSplits ways
    // (only a small fixed keys-per-split policy asks for that) wait for it.
    auto combine = [&](const std::vector<std::pair<const RowPlan *, int>> &split_rows) -> kv_status {
        for (size_t lo = 0; lo < split_rows.size(); lo += kMaxRows) {
            CombineArgs m{};
            m.out = out;
            m.ws_acc = a.ws_acc;
            m.ws_ml = a.ws_ml;
            m.batch = c->batch;
            m.T = T;
            m.hq = q_heads;
            m.hkv = c->kv_heads;
            m.group = p.group;
            m.head_dim = c->head_dim;
            m.records = p.records;
            const size_t hi = std::min(split_rows.size(), lo + kMaxRows);
            m.rows.n_rows = (int32_t)(hi - lo);
            int32_t blocks = 0;
            for (size_t i = lo; i < hi; ++i) {
                const RowPlan &r = *split_rows[i].first;
                const int j = (int)(i - lo);
                m.rows.b[j] = r.b;
                m.rows.nnew[j] = r.nnew;
                m.rows.nsplit[j] = r.nsplit;
                m.rows.pbase[j] = (int32_t)r.pbase;
                m.rows.cols[j] = split_rows[i].second;
                m.rows.blk0[j] = blocks;
                const int per_group = (int)ceil_div((int64_t)split_rows[i].second * (c->head_dim / 4), 256);
                blocks += c->kv_heads * r.nq * per_group;
            }
            m.rows.blk0[m.rows.n_rows] = blocks;
            m.rows.total_blocks = blocks;
            hipError_t e = launch_combine((int)c->dtype, c->head_dim, m, st);
            if (e != hipSuccess) return device_fail(e, "gqa_attention (combine kernel)");
        }
        return KV_OK;
    };
    std::vector<std::pair<const RowPlan *, int>> pre_split, dec_split;
    for (auto &r : p.pre)
        if (r.nsplit > 1) pre_split.push_back({&r, prefill_cols(c->dtype, c->head_dim)});
    for (auto &r : p.dec)
        if (r.nsplit > kMergeMaxSplits) dec_split.push_back({&r, p.dec_cols});
    kv_status cs = combine(pre_split);
    if (cs != KV_OK) return cs;
    if (mixed) {
        hipError_t e = side_stream_join(c->side, st);
        if (e != hipSuccess) return device_fail(e, "gqa_attention (side stream)");
    }
    cs = combine(dec_split);
    if (cs != KV_OK) return cs;
    return KV_OK;
}
}  // namespace

extern "C" {

kv_status kv_truncate(kv_cache *c, const int32_t *new_lens, void *stream) {
    if (c == nullptr) return fail(KV_ERR_INVALID_ARG, "null cache handle");
    if (c->batch > 0 && new_lens == nullptr) return fail(KV_ERR_INVALID_ARG, "new_lens is null");
    // [CH16] "Layout and validity": 0 <= n <= current length; a ring must
    // still hold every key the next query (at position n) would see
    for (int b = 0; b < c->batch; ++b)
        if (new_lens[b] < 0 || new_lens[b] > c->lens[b] ||
            lowest_needed(c, new_lens[b]) < oldest_kept(c, c->lens[b]))
            return fail(KV_ERR_INVALID_ARG, "Invalid truncation length");
    if (c->lens_dev != nullptr) {
        std::vector<int> rows;
        for (int b = 0; b < c->batch; ++b)
            if (new_lens[b] != c->lens[b]) rows.push_back(b);
        for (size_t lo = 0; lo < rows.size(); lo += kMaxRows) {
            LensTable t{};
            const size_t hi = std::min(rows.size(), lo + kMaxRows);
            t.n_rows = (int32_t)(hi - lo);
            for (size_t i = lo; i < hi; ++i) {
                t.b[i - lo] = rows[i];
                t.len[i - lo] = new_lens[rows[i]];
            }
            hipError_t e = launch_set_lens(c->lens_dev, t, (hipStream_t)stream);
            if (e != hipSuccess) return device_fail(e, "kv_truncate");
        }
    }
    if (c->paged) {
        // blocks that no longer hold a token give their pages back to the pool
        std::vector<std::pair<int32_t, int32_t>> upd;
        for (int b = 0; b < c->batch; ++b)
            for (int64_t i = blocks_of(c, new_lens[b]); i < blocks_of(c, c->lens[b]); ++i)
                upd.push_back({(int32_t)((int64_t)b * c->max_blocks + i), -1});
        kv_status st = push_table_updates(c, upd, (hipStream_t)stream, "kv_truncate (block table)");
        if (st != KV_OK) return st;
        for (auto &u : upd) {
            c->free_pages.push(c->table[u.first]);
            c->table[u.first] = -1;
        }
    }
    for (int b = 0; b < c->batch; ++b) c->lens[b] = new_lens[b];
    return ok();
}

kv_status kv_get_block_table(const kv_cache *c, int32_t *table_host) {
    if (c == nullptr) return fail(KV_ERR_INVALID_ARG, "null cache handle");
    if (!c->paged) return fail(KV_ERR_INVALID_ARG, "not a paged cache");
    if (!c->table.empty() && table_host == nullptr) return fail(KV_ERR_INVALID_ARG, "table_host is null");
    std::copy(c->table.begin(), c->table.end(), table_host);
    return ok();
}

int32_t kv_free_pages(const kv_cache *c) { return (c != nullptr && c->paged) ? (int32_t)c->free_pages.size() : 0; }

kv_status kv_get_lens(const kv_cache *c, int32_t *lens_host) {
    if (c == nullptr) return fail(KV_ERR_INVALID_ARG, "null cache handle");
    if (c->batch > 0 && lens_host == nullptr) return fail(KV_ERR_INVALID_ARG, "lens_host is null");
    std::copy(c->lens.begin(), c->lens.end(), lens_host);
    return ok();
}

uint64_t kv_cache_bytes(const kv_cache *c) {
    if (c == nullptr) return 0;
    if (c->paged) return 2ull * (uint64_t)c->num_pages * c->kv_heads * c->page_size * c->head_dim * c->elem_bytes;
    return 2ull * (uint64_t)c->batch * c->kv_heads * c->max_len * c->head_dim * c->elem_bytes;
}

uint64_t kv_live_bytes(const kv_cache *c) {
    if (c == nullptr) return 0;
    uint64_t tokens = 0;      // a ring holds at most max_len tokens of a row
    for (int32_t l : c->lens) tokens += (uint64_t)(c->ring ? std::min(l, c->max_len) : l);
    return 2ull * tokens * c->kv_heads * c->head_dim * c->elem_bytes;
}

const char *kv_last_error(void) { return g_err.c_str(); }

kv_status kv_cache_set_policy(kv_cache *c, int32_t path, int32_t keys_per_split) {
    if (c == nullptr) return fail(KV_ERR_INVALID_ARG, "null cache handle");
    if (path < 0 || path > 2) return fail(KV_ERR_INVALID_ARG, "path %d not in 0..2", path);
    if (keys_per_split < 0) return fail(KV_ERR_INVALID_ARG, "keys_per_split %d < 0", keys_per_split);
    c->path_policy = path;
    c->keys_per_split = keys_per_split;
    return ok();
}

}  // extern "C"
