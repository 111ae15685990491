// Host-side stand-in for the kernel launchers of libgqakv (test infrastructure).
//
// Linked with the library's real host code (abi.cpp) instead of kernels.hip,
// it replays every launch the planner issues, block by block and column by
// column, using the same indexing functions the kernels use (indexing.h), and
// checks on the CPU that
//   * every K/V/q/out/workspace/lens access lies inside a registered buffer,
//   * append writes only the slots [lens, lens + n_new) of each row, once
//     (the copy kernel, or in kv_append_attention the attention kernels'
//     items, each token by exactly one item),
//   * each attention call writes every output row (b, h, t) exactly once,
//   * each split partial is written once before the combine kernel, or the
//     last work group of its group in the decode kernel, reads it; each
//     group's arrival counter lies in the workspace past the partials.
// Buffers are fake addresses registered by the test; nothing is dereferenced.

#include <hip/hip_runtime_api.h>

#include <cstdio>
#include <algorithm>
#include <cstring>
#include <map>
#include <string>
#include <vector>

#include "indexing.h"
#include "internal.h"

namespace {

struct Region {
    uintptr_t base;
    size_t size;
    std::string name;
};

std::vector<Region> g_regions;
std::vector<std::string> g_errors;
std::map<uintptr_t, int> g_out_rows;   // start address of an output row -> writes
std::map<int64_t, int> g_records;      // partial record -> writes
std::map<int64_t, int> g_arrivals;     // decode merge counter -> work groups arrived
std::map<uintptr_t, int> g_appended;   // 16-byte chunk of K -> writes
std::vector<int32_t> g_lens_dev;
std::vector<int32_t> g_table;          // the device block table of a paged cache, as the kernels see it
int64_t g_launches = 0;
int g_last_nsub = 0;                   // subtiles of the last decode launch

void err(const std::string &m) {
    if (g_errors.size() < 64) g_errors.push_back(m);
}

void access(const void *p, size_t bytes, const char *want, const char *what) {
    const uintptr_t a = reinterpret_cast<uintptr_t>(p);
    for (const Region &r : g_regions) {
        if (a >= r.base && a + bytes <= r.base + r.size) {
            if (r.name != want)
                err(std::string(what) + ": hits buffer " + r.name + ", expected " + want);
            return;
        }
    }
    char buf[160];
    snprintf(buf, sizeof buf, "%s: %zu bytes at %#lx outside every buffer (want %s)", what, bytes,
             (unsigned long)a, want);
    err(buf);
}

}  // namespace

extern "C" {

void hostcheck_reset() {
    g_regions.clear();
    g_errors.clear();
    g_out_rows.clear();
    g_records.clear();
    g_arrivals.clear();
    g_appended.clear();
    g_lens_dev.clear();
    g_table.clear();
    g_launches = 0;
}

void hostcheck_region(uintptr_t base, size_t size, const char *name) { g_regions.push_back({base, size, name}); }

// Start a new attention call: forget output-row and record counts.
void hostcheck_begin_call() {
    g_out_rows.clear();
    g_records.clear();
    g_arrivals.clear();
}

int hostcheck_error_count() { return (int)g_errors.size(); }

const char *hostcheck_error(int i) { return (i >= 0 && i < (int)g_errors.size()) ? g_errors[i].c_str() : ""; }

int64_t hostcheck_launches() { return g_launches; }

int hostcheck_last_decode_nsub() { return g_last_nsub; }

// Writes recorded for output row i of an [rows, row_bytes] array at base.
int hostcheck_out_row_writes(uintptr_t base, int64_t i, int64_t row_bytes) {
    auto it = g_out_rows.find(base + (uintptr_t)(i * row_bytes));
    return it == g_out_rows.end() ? 0 : it->second;
}

int64_t hostcheck_out_rows_total() {
    int64_t n = 0;
    for (auto &kv : g_out_rows) n += kv.second;
    return n;
}

// 16-byte chunks of K written by appends so far, and how many were written twice
int64_t hostcheck_appended_chunks() { return (int64_t)g_appended.size(); }
int64_t hostcheck_appended_dupes() {
    int64_t n = 0;
    for (auto &kv : g_appended) n += kv.second > 1;
    return n;
}

int32_t hostcheck_lens_dev(int b) { return (b >= 0 && b < (int)g_lens_dev.size()) ? g_lens_dev[b] : -1; }

// entry i of the simulated device block table (-2 when never written)
int32_t hostcheck_table(int64_t i) { return (i >= 0 && i < (int64_t)g_table.size()) ? g_table[i] : -2; }

}  // extern "C"

namespace gqakv {

hipError_t launch_append(const AppendArgs &a, int n_blocks, hipStream_t) {
    ++g_launches;
    if ((int)g_lens_dev.size() < a.batch) g_lens_dev.resize(a.batch, 0);
    for (int blk = 0; blk < n_blocks; ++blk) {
        const int r = find_row(a.t.block0, a.t.n_rows, blk);
        const int local = blk - a.t.block0[r];
        const int nch = a.t.nchunk[r];
        const int kvh = local / nch, chunk = local % nch;
        const int b = a.t.b[r];
        if (b < 0 || b >= a.batch || kvh < 0 || kvh >= a.hkv) err("append: block maps outside the cache");
        const int64_t span = (int64_t)a.t.n[r] * a.row_bytes;
        const int64_t head = (int64_t)b * a.hkv + kvh;
        for (int tid = 0; tid < 256; ++tid) {
            const int64_t off = (int64_t)chunk * kAppendChunk + tid * 16;
            if (off >= span) continue;
            if ((int64_t(1) << a.row_shift) != a.row_bytes) err("append: row_shift does not match row_bytes");
            if (a.t.slot0[r] != a.t.start[r] % a.max_len) err("append: slot0 is not start mod max_len");
            // the kernel's mapping: token i -> slot slot0 + i, wrapped once at
            // max_len; in a paged cache position p -> row p mod page of
            // (block_table[b][p / page], kv head) in the pool
            const int tok = (int)(off >> a.row_shift);
            int slot = a.t.slot0[r] + tok;
            if (slot >= a.max_len) slot -= a.max_len;
            int64_t crow = head * a.max_len + slot;
            if (a.table != nullptr) {
                const int p = a.t.start[r] + tok;
                const int64_t ti = (int64_t)b * a.max_blocks + (p >> a.page_shift);
                access(a.table + ti, 4, "table", "append block table");
                const int page = ti < (int64_t)g_table.size() ? g_table[ti] : -1;
                if (page < 0) err("append: block without a page");
                crow = (((int64_t)page * a.hkv + kvh) << a.page_shift) + (p & ((1 << a.page_shift) - 1));
                slot = p % a.max_len;                // the logical slot, for the check below
            }
            const int64_t src = head * a.T * a.row_bytes + off;
            // a quantizing append writes one code byte per two input bytes
            const int sh = a.quant ? a.row_shift - 1 : a.row_shift;
            const int64_t dst = (crow << sh) + ((off & (a.row_bytes - 1)) >> (a.quant ? 1 : 0));
            const int wbytes = a.quant ? 8 : 16;
            access((const char *)a.k_new + src, 16, "k_new", "append read k_new");
            access((const char *)a.v_new + src, 16, "v_new", "append read v_new");
            access((const char *)a.k + dst, wbytes, "k", "append write K");
            access((const char *)a.v + dst, wbytes, "v", "append write V");
            if (a.quant && (kvh >= kMaxScaleHeads || !(a.k_inv[kvh] > 0.f) || !(a.v_inv[kvh] > 0.f)))
                err("append: missing E4M3 scale");
            if (slot < 0 || slot >= a.max_len || slot != (a.t.start[r] + tok) % a.max_len || tok >= a.t.n[r])
                err("append: write outside the row's new slots");
            g_appended[(uintptr_t)a.k + dst]++;
        }
        if (a.lens_dev != nullptr && local == 0) {
            access(a.lens_dev + b, 4, "lens", "append lens_dev");
            g_lens_dev[b] = a.t.start[r] + a.t.n[r];
        }
    }
    return hipSuccess;
}

hipError_t launch_table_fill(int32_t *table, int64_t n, int32_t value, hipStream_t) {
    ++g_launches;
    access(table, (size_t)n * 4, "table", "table fill");
    g_table.assign((size_t)n, value);
    return hipSuccess;
}

// the no-allocation entry point's scratch: here the test's registered
// workspace region, so its accesses are checked like a caller's workspace
hipError_t scratch_region(void **ptr) {
    for (const Region &r : g_regions)
        if (r.name == "ws") {
            if (r.size < kScratchBytes) err("scratch: the ws region is smaller than the scratch array");
            *ptr = reinterpret_cast<void *>(r.base);
            return hipSuccess;
        }
    err("scratch: no ws region registered");
    return hipErrorInvalidValue;
}

hipError_t launch_zero_bytes(void *p, int64_t bytes, hipStream_t) {
    ++g_launches;
    if (bytes % 16 != 0 || (reinterpret_cast<uintptr_t>(p) & 15) != 0) err("zero bytes: not 16-byte granular");
    // the whole range must be one buffer: K or V
    const uintptr_t a = reinterpret_cast<uintptr_t>(p);
    bool inside = false;
    for (const Region &r : g_regions)
        if (a >= r.base && a + (uintptr_t)bytes <= r.base + r.size && (r.name == "k" || r.name == "v")) inside = true;
    if (bytes > 0 && !inside) err("zero bytes: range is not inside K or V");
    return hipSuccess;
}

hipError_t launch_table_set(const TableArgs &a, hipStream_t) {
    ++g_launches;
    if (a.n <= 0 || a.n > kMaxTableUpdates) err("table set: bad update count");
    for (int i = 0; i < a.n; ++i) {
        access(a.table + a.idx[i], 4, "table", "table set");
        if (a.idx[i] < 0 || a.idx[i] >= (int64_t)g_table.size()) err("table set: index outside the table");
        else g_table[a.idx[i]] = a.page[i];
    }
    return hipSuccess;
}

hipError_t launch_set_lens(int32_t *lens_dev, const LensTable &t, hipStream_t) {
    ++g_launches;
    for (int i = 0; i < t.n_rows; ++i) {
        access(lens_dev + t.b[i], 4, "lens", "set_lens");
        if ((int)g_lens_dev.size() <= t.b[i]) g_lens_dev.resize(t.b[i] + 1, 0);
        g_lens_dev[t.b[i]] = t.len[i];
    }
    return hipSuccess;
}

// merge: the decode kernel, whose work groups of a split row count their
// arrivals and the last one merges the row's partials
static void sim_attention(const AttnArgs &a, int cols, int key_tile, int elem, int cache_elem, bool merge) {
    ++g_launches;
    const AttnRows &R = a.rows;
    const int D = a.head_dim;
    const int64_t row_bytes = (int64_t)D * elem;             // q / out rows
    const int64_t cache_row = (int64_t)D * cache_elem;       // K / V rows
    if (R.item0[R.n_rows] != R.total_items) err("item0 does not end at total_items");
    const bool windowed = a.window != kNoWindow;
    if (windowed && (a.window < 1 || a.window > a.max_len || a.max_len % kRingAlign != 0))
        err("attention: bad ring window or capacity");
    for (int r = 0; r < R.n_rows; ++r) {
        if ((!windowed && R.len[r] > a.max_len) || R.nnew[r] > R.len[r] || R.nnew[r] <= 0 || R.nnew[r] > a.T)
            err("attention: bad row table entry");
        if (R.lsplit[r] % key_tile != 0 || R.nsplit[r] <= 0) err("attention: bad split");
    }
    const bool paged = a.table != nullptr;
    // kv_append_attention: the kernel writes its key range's new tokens and
    // reads keys at or past the row's first new position from k_new / v_new
    const bool fuse = a.fuse != 0;
    const int64_t in_row = (int64_t)D * elem;                 // k_new / v_new rows (input type)
    if (fuse && (a.k_new == nullptr || a.v_new == nullptr)) err("attention: fused append without k_new / v_new");
    if (fuse && cache_elem != elem) {
        // an E4M3 cache: codes of bfloat16 inputs, quantized with the append's 1 / scale
        if (cache_elem != 1 || elem != 2) err("attention: fused append with mismatched element sizes");
        for (int h = 0; h < a.hkv; ++h)
            if (h >= kMaxScaleHeads || !(a.k_inv[h] > 0.f) || !(a.v_inv[h] > 0.f) || !(a.k_scale[h] > 0.f))
                err("attention: fused E4M3 append without its scales");
    }
    auto new_row = [&](const Item &it, int r, int key) -> int64_t {   // k_new row of key `key`
        const int t = key - it.base;
        if (t < 0 || t >= R.nnew[r] || t >= a.T) err("attention: k_new row outside the row's new tokens");
        return ((int64_t)it.b * a.hkv + it.kvh) * a.T + t;
    };
    if (paged) {
        // no page is held by two blocks, and every block below a row's length has one
        std::map<int32_t, int> owners;
        for (int32_t e : g_table)
            if (e >= 0 && ++owners[e] > 1) err("attention: a page is held twice");
        if (windowed || (1 << a.page_shift) < kMinPage || a.max_len != a.max_blocks << a.page_shift)
            err("attention: bad paged geometry");
        for (int r = 0; r < R.n_rows; ++r)
            for (int i = 0; i < (R.len[r] + (1 << a.page_shift) - 1) >> a.page_shift; ++i) {
                const int64_t ti = (int64_t)R.b[r] * a.max_blocks + i;
                if (ti >= (int64_t)g_table.size() || g_table[ti] < 0) err("attention: block of a row without a page");
            }
    }
    for (int item = 0; item < R.total_items; ++item) {
        const Item it = decode_item(R, item, a.hkv, a.group, cols, a.window);
        const int r = find_row(R.item0, R.n_rows, item);
        if (it.b < 0 || it.b >= a.batch || it.kvh < 0 || it.kvh >= a.hkv || it.qtile < 0 || it.qtile >= it.nq ||
            it.split < 0 || it.split >= it.nsplit)
            err("attention: item decodes outside the launch");
        if (it.k_begin < 0 || it.k_end > R.len[r]) err("attention: key range outside the row");
        if (it.k_begin % key_tile != 0) err("attention: key range does not start on a tile");
        // the item's splits cover every key its queries may see: from the
        // first query's window start to the last query's position
        const int first_pos = it.base + it.t0;
        const int lo_visible = windowed ? std::max(0, first_pos - a.window + 1) : 0;
        if (it.split == 0 && range_start(first_pos, a.window) > lo_visible) err("attention: range starts too late");
        if (it.split == it.nsplit - 1 && it.k_end != it.base + it.t_end)
            err("attention: splits do not cover the item's keys");
        if (it.split < it.nsplit - 1 && it.k_end > it.k_begin + R.lsplit[r])
            err("attention: a split longer than lsplit before the last");
        // every visible key is still held by the ring (positions >= len - max_len)
        if (windowed && lo_visible < std::max(0, R.len[r] - a.max_len)) err("attention: window key evicted");
        const int64_t head = (int64_t)it.b * a.hkv + it.kvh;
        if (fuse) {
            // the item writes the new tokens of its own query tile that lie in its key split
            for (int p = std::max(it.k_begin, it.base + it.t0); p < std::min(it.k_end, it.base + it.t_end); ++p) {
                const int64_t src = new_row(it, r, p) * in_row;
                int64_t dst = head * a.max_len + p % a.max_len;
                if (paged) {
                    const int64_t ti = (int64_t)it.b * a.max_blocks + (p >> a.page_shift);
                    access(a.table + ti, 4, "table", "fused append block table");
                    const int page = ti < (int64_t)g_table.size() ? g_table[ti] : -1;
                    if (page < 0) err("fused append: block without a page");
                    dst = (((int64_t)page * a.hkv + it.kvh) << a.page_shift) + (p & ((1 << a.page_shift) - 1));
                }
                access((const char *)a.k_new + src, in_row, "k_new", "fused append read k_new");
                access((const char *)a.v_new + src, in_row, "v_new", "fused append read v_new");
                access((const char *)a.k + dst * cache_row, cache_row, "k", "fused append write K");
                access((const char *)a.v + dst * cache_row, cache_row, "v", "fused append write V");
                // one entry per 16 input bytes, at the bytes they land on (as the copy kernel's)
                for (int64_t o = 0; o < in_row; o += 16)
                    g_appended[(uintptr_t)a.k + dst * cache_row + o * cache_row / in_row]++;   // exactly once
            }
            if (a.lens_dev != nullptr && item == R.item0[r]) {
                access(a.lens_dev + it.b, 4, "lens", "fused append lens_dev");
                if ((int)g_lens_dev.size() <= it.b) g_lens_dev.resize(it.b + 1, 0);
                g_lens_dev[it.b] = R.len[r];
            }
        }
        // keys read: [k_begin, k_end) tile by tile; key j from slot j mod max_len,
        // and no tile may wrap inside the ring
        for (int t0 = it.k_begin; t0 < it.k_end; t0 += key_tile) {
            const int n = std::min(key_tile, it.k_end - t0);
            const int slot = t0 % a.max_len;
            if (slot + n > a.max_len) err("attention: key tile wraps");
            int64_t row0 = head * a.max_len + slot;   // cache row of the tile's first key (the kernels' KeyRows)
            if (paged) {
                const int psz = 1 << a.page_shift;
                const int64_t ti = (int64_t)it.b * a.max_blocks + (t0 >> a.page_shift);
                access(a.table + ti, 4, "table", "attention block table");
                const int page = ti < (int64_t)g_table.size() ? g_table[ti] : -1;
                if (page < 0) err("attention: tile in a block without a page");
                if ((t0 & (psz - 1)) + n > psz) err("attention: key tile crosses a page");
                row0 = (((int64_t)page * a.hkv + it.kvh) << a.page_shift) + (t0 & (psz - 1));
            }
            for (int64_t key : {row0, row0 + n - 1}) {
                access((const char *)a.k + key * cache_row, cache_row, "k", "attention K");
                access((const char *)a.v + key * cache_row, cache_row, "v", "attention V");
            }
            // a tile holding new keys reads them from k_new / v_new
            if (fuse && t0 + key_tile > it.base)
                for (int key : {std::max(t0, it.base), t0 + n - 1}) {
                    if (key < it.base) continue;
                    const int64_t src = new_row(it, r, key) * in_row;
                    access((const char *)a.k_new + src, in_row, "k_new", "fused attention k_new");
                    access((const char *)a.v_new + src, in_row, "v_new", "fused attention v_new");
                }
        }
        for (int col = 0; col < cols; ++col) {
            const int pos = column_position(it, col, a.group, cols);
            if (pos < 0) continue;
            const int t = column_t(it, col, a.group), h = column_head(it, col, a.group);
            if (t < 0 || t >= a.T || t >= R.nnew[r] || h < 0 || h >= a.hq) err("attention: column outside q");
            if (pos != R.len[r] - R.nnew[r] + t) err("attention: wrong absolute position");
            const int64_t qrow = ((int64_t)it.b * a.hq + h) * a.T + t;
            access((const char *)a.q + qrow * row_bytes, row_bytes, "q", "attention q");
            if (it.rec0 < 0) {
                const char *o = (const char *)a.out + qrow * row_bytes;
                access(o, row_bytes, "out", "attention out");
                g_out_rows[(uintptr_t)o]++;
            } else {
                const int64_t rec = (int64_t)it.rec0 + col;
                if (rec < 0 || rec >= a.records) err("attention: partial record out of range");
                access(a.ws_acc + rec * D, D * 4, "ws", "attention partial acc");
                access(a.ws_ml + rec * 2, 8, "ws", "attention partial m,l");
                g_records[rec]++;
            }
        }
        if (merge && it.rec0 >= 0 && it.nsplit <= kMergeMaxSplits) {
            const int64_t rec_first = (int64_t)it.rec0 - (int64_t)it.split * cols;
            if (rec_first < 0 || rec_first % cols != 0) err("decode merge: group's first record misplaced");
            const unsigned long long *cnt = a.counters + rec_first / cols;
            access(cnt, 8, "ws", "decode merge counter");
            if ((uintptr_t)cnt < (uintptr_t)(a.ws_ml + a.records * 2)) err("decode merge: counter overlaps partials");
            if (a.merge_tag == 0 || (a.merge_tag >> (64 - kMergeCountBits)) != 0) err("decode merge: bad tag");
            const int arrived = ++g_arrivals[rec_first / cols];
            if (arrived > it.nsplit) err("decode merge: more arrivals than splits");
            if (arrived == it.nsplit) {
                // the last work group reads every split's record of each column and writes the output
                for (int col = 0; col < cols; ++col) {
                    if (column_position(it, col, a.group, cols) < 0) continue;
                    for (int s = 0; s < it.nsplit; ++s) {
                        const int64_t rs = rec_first + col + (int64_t)s * cols;
                        auto w = g_records.find(rs);
                        if (w == g_records.end() || w->second != 1)
                            err("decode merge: partial not written exactly once");
                        access(a.ws_acc + rs * D, D * 4, "ws", "decode merge acc");
                        access(a.ws_ml + rs * 2, 8, "ws", "decode merge m,l");
                    }
                    const int t = column_t(it, col, a.group), h = column_head(it, col, a.group);
                    const char *o = (const char *)a.out + (((int64_t)it.b * a.hq + h) * a.T + t) * row_bytes;
                    access(o, row_bytes, "out", "decode merge out");
                    g_out_rows[(uintptr_t)o]++;
                }
            }
        }
    }
}

hipError_t launch_decode(int dtype, int head_dim, int nsub, const AttnArgs &a, hipStream_t) {
    if (head_dim != a.head_dim) err("decode: head_dim mismatch");
    // the kernel's register tiling holds 16 * nsub columns; the items use a.cols of them
    if (nsub != 1 && nsub != 2 && nsub != 4) err("decode: bad subtile count");
    g_last_nsub = nsub;
    if (a.cols < a.group || a.cols > 16 * nsub || (nsub > 1 && a.cols <= 8 * nsub))
        err("decode: item columns do not fit the kernel's tiling");
    sim_attention(a, a.cols, kDecodeKeyTile, dtype == 0 ? 4 : 2, dtype == 0 ? 4 : (dtype == 1 ? 2 : 1), true);
    return hipSuccess;
}

hipError_t launch_prefill(int dtype, int head_dim, const AttnArgs &a, hipStream_t) {
    if (head_dim != a.head_dim) err("prefill: head_dim mismatch");
    if (a.cols != prefill_cols(dtype, head_dim)) err("prefill: columns differ from the kernel's");
    if (a.fuse) err("prefill: fused append requested");
    sim_attention(a, a.cols, kPrefillKeyTile, dtype == 0 ? 4 : 2, dtype == 0 ? 4 : (dtype == 1 ? 2 : 1), false);
    return hipSuccess;
}

hipError_t launch_combine(int dtype, int head_dim, const CombineArgs &a, hipStream_t) {
    ++g_launches;
    const int64_t row_bytes = (int64_t)head_dim * (dtype == 0 ? 4 : 2);
    if (a.rows.blk0[a.rows.n_rows] != a.rows.total_blocks) err("combine: blk0 does not end at total_blocks");
    const int DC = head_dim / 4;
    for (int blk = 0; blk < a.rows.total_blocks; ++blk) {
        const int r = find_row(a.rows.blk0, a.rows.n_rows, blk);
        const int local = blk - a.rows.blk0[r];
        const int cols = a.rows.cols[r], nsplit = a.rows.nsplit[r], n = a.rows.nnew[r];
        const int tq = cols / a.group;
        const int nq = (n + tq - 1) / tq;
        const int per_group = (cols * DC + 255) / 256;
        const int grp = local / per_group, part = local % per_group;
        const int kvh = grp / nq, qtile = grp % nq;
        if (kvh >= a.hkv || nsplit < 2) err("combine: block maps outside the row");
        const int64_t rec_first = a.rows.pbase[r] + (int64_t)((kvh * nq + qtile) * nsplit) * cols;
        for (int tid = 0; tid < 256; ++tid) {
            const int task = part * 256 + tid;
            if (task >= cols * DC) continue;
            const int col = task / DC, d = (task % DC) * 4;
            const int t = qtile * tq + col / a.group;
            if (col >= tq * a.group || t >= n) continue;
            const int h = kvh * a.group + col % a.group;
            for (int s = 0; s < nsplit; ++s) {
                const int64_t rs = rec_first + col + (int64_t)s * cols;
                if (rs < 0 || rs >= a.records) err("combine: record out of range");
                auto w = g_records.find(rs);
                if (w == g_records.end() || w->second != 1) err("combine: partial not written exactly once");
                access(a.ws_acc + rs * head_dim + d, 16, "ws", "combine acc");
                access(a.ws_ml + rs * 2, 8, "ws", "combine m,l");
            }
            const char *o = (const char *)a.out + (((int64_t)a.rows.b[r] * a.hq + h) * a.T + t) * row_bytes + d * (dtype == 0 ? 4 : 2);
            access(o, 4 * (dtype == 0 ? 4 : 2), "out", "combine out");
            if (d == 0) g_out_rows[(uintptr_t)((const char *)a.out + (((int64_t)a.rows.b[r] * a.hq + h) * a.T + t) * row_bytes)]++;
        }
    }
    return hipSuccess;
}

// stream fork/join only orders work; the simulator runs launches in call order
hipError_t side_stream_init(SideStream &s) {
    s.side = reinterpret_cast<hipStream_t>(0x5);
    return hipSuccess;
}
void side_stream_destroy(SideStream &s) { s = SideStream{}; }
hipError_t side_stream_fork(SideStream &, hipStream_t) { return hipSuccess; }
hipError_t side_stream_join(SideStream &, hipStream_t) { return hipSuccess; }

hipError_t launch_zero_fill(const ZeroArgs &a, hipStream_t) {
    ++g_launches;
    // block-by-block, as the kernel maps block ids to slices
    if (a.slices != (a.T * a.row_bytes + kZeroSlice - 1) / kZeroSlice) err("zero fill: slice count");
    for (int64_t blk = 0; blk < (int64_t)a.rows.n_rows * a.hq * a.slices; ++blk) {
        const int slice = (int)(blk % a.slices);
        const int rh = (int)(blk / a.slices);
        const int r = rh / a.hq, h = rh % a.hq;
        const int64_t head_off = ((int64_t)a.rows.b[r] * a.hq + h) * a.T * a.row_bytes;
        const int64_t lo = (int64_t)slice * kZeroSlice;
        const int64_t begin = head_off + std::max(lo, (int64_t)a.rows.nnew[r] * a.row_bytes);
        const int64_t end = head_off + std::min(lo + kZeroSlice, (int64_t)a.T * a.row_bytes);
        for (int j = 0; j < kZeroSlice / 16; ++j) {
            const int64_t off = head_off + lo + (int64_t)j * 16;
            if (off < begin || off >= end) continue;
            const char *o = (const char *)a.out + off;
            access(o, 16, "out", "zero fill");
            if ((off - head_off) % a.row_bytes == 0) g_out_rows[(uintptr_t)o]++;
        }
    }
    return hipSuccess;
}

}  // namespace gqakv
