// Launch tables shared by the host planner (abi.cpp) and the kernels
// (kernels.hip). Per-row metadata travels in the kernel arguments: the host
// already holds every row's length, so no host-to-device copy is ever needed
// and every launch is self-contained (graph-capturable). Rows beyond
// kMaxRows are split over several launches.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace gqakv {

constexpr int kMaxRows = 64;

// Decode rows split into at most this many work groups are merged by the last
// of them to finish, in the decode kernel; rows split further (only under a
// small keys-per-split policy) are merged by the combine kernel.
constexpr int kMergeMaxSplits = 64;
constexpr int kMergeCountBits = 8;     // arrivals field of a counter word (> log2 kMergeMaxSplits)
static_assert(kMergeMaxSplits < (1 << kMergeCountBits), "arrival count field too narrow");

// ---------------------------------------------------------------- append
struct AppendTable {
    int32_t n_rows;
    int32_t b[kMaxRows];       // batch row
    int32_t start[kMaxRows];   // row length before the append (position of the first token)
    int32_t slot0[kMaxRows];   // slot of the first token: start mod max_len (a ring wraps there)
    int32_t n[kMaxRows];       // tokens written
    int32_t nchunk[kMaxRows];  // 4 KiB copy chunks per (row, kv head)
    int32_t block0[kMaxRows + 1];
};

// E4M3 caches carry one scale per KV head for K and one for V.
constexpr int kMaxScaleHeads = 64;
// Tree verify: at most this many draft nodes per row.
constexpr int kMaxTreeNodes = 16;

struct AppendArgs {
    void *k;                   // cache K [B, Hkv, max_len, d], or the page pool [pages, Hkv, page, d]
    void *v;
    const void *k_new;         // [B, Hkv, T, d]
    const void *v_new;
    int32_t *lens_dev;         // optional
    int64_t row_bytes;         // bytes of one k_new row: d * input element size (a power of two)
    int32_t row_shift;         // log2(row_bytes)
    int32_t batch, hkv, max_len, T;
    int32_t quant;             // 1: bfloat16 inputs stored as E4M3 codes of x * inv scale
    float k_inv[kMaxScaleHeads], v_inv[kMaxScaleHeads];   // float32 1 / scale per KV head
    const int32_t *table;      // paged cache: block table [B, max_blocks] (null: linear or ring)
    int32_t page_shift;        // log2(page size)
    int32_t max_blocks;
    AppendTable t;
};

// Paged caches: entries of the device block table set in stream order, carried
// in the kernel arguments (no host-to-device copy).
constexpr int kMaxTableUpdates = 480;
struct TableArgs {
    int32_t *table;
    int32_t n;
    int32_t idx[kMaxTableUpdates];    // b * max_blocks + block
    int32_t page[kMaxTableUpdates];   // page, or -1
};

struct LensTable {
    int32_t n_rows;
    int32_t b[kMaxRows];
    int32_t len[kMaxRows];
};

// ------------------------------------------------------------- attention
// Work item = (row, kv head, query tile, key split). Items of one row are
// numbered with the kv head fastest, then the split, then the query tile from
// the last (longest key range) to the first.
struct AttnRows {
    int32_t n_rows;
    int32_t total_items;
    int32_t b[kMaxRows];
    int32_t len[kMaxRows];     // keys valid after the append
    int32_t nnew[kMaxRows];    // real queries of the row
    int32_t nsplit[kMaxRows];  // key splits per (kv head, query tile)
    int32_t lsplit[kMaxRows];  // keys per split (multiple of the key tile)
    int32_t pbase[kMaxRows];   // first partial record of the row; -1: write out directly
    int32_t item0[kMaxRows + 1];
};

struct AttnArgs {
    const void *q;             // [B, Hq, T, d]
    void *out;                 // [B, Hq, T, d]
    const void *k;             // cache [B, Hkv, max_len, d], or the page pool [pages, Hkv, page, d]
    const void *v;
    float *ws_acc;             // partial records: unnormalised acc [rec][d]
    float *ws_ml;              // partial records: (running max in log2 units, sum) [rec][2]
    int32_t batch, T, hq, hkv, group, max_len, head_dim;
    int32_t cols;              // columns (query, head pairs) per work item of this launch
    int32_t window;            // keys a query sees: pos - window < key <= pos (kNoWindow: no lower bound)
    int64_t records;           // partial records available in the workspace
    float scale_log2;          // log2(e) / sqrt(d)
    float k_scale[kMaxScaleHeads], v_scale[kMaxScaleHeads];   // E4M3 caches: code x scale per KV head
    float k_inv[kMaxScaleHeads], v_inv[kMaxScaleHeads];       // and the float32 1 / scale the append uses
    const int32_t *table;      // paged cache: block table [B, max_blocks] (null: linear or ring)
    int32_t page_shift;        // log2(page size)
    int32_t max_blocks;
    // kv_append_attention on decode-kernel rows: the kernel writes each row's
    // new tokens from k_new / v_new ([B, Hkv, T, d]) into the cache (E4M3:
    // their codes) and reads those keys from k_new / v_new; one work group per
    // row sets lens_dev
    int32_t fuse;
    const void *k_new;
    const void *v_new;
    int32_t *lens_dev;         // optional
    // rows split across decode work groups into at most kMergeMaxSplits
    // splits are merged in the decode kernel: one arrival counter per (row,
    // kv head, query tile) group, at the group's first partial record / cols;
    // each word holds (merge_tag << kMergeCountBits) | arrivals
    unsigned long long *counters;
    unsigned long long merge_tag;   // nonzero, below 2^(64 - kMergeCountBits), fixed per process
    int32_t tree;              // 1: the new tokens of each row form a tree (parent below)
    int8_t parent[kMaxRows][kMaxTreeNodes];   // per launch row: parent node of node u, -1 = the committed prefix
    AttnRows rows;
};

// Combine of rows split across work groups: one block per (row, kv head, query tile).
struct CombineRows {
    int32_t n_rows;
    int32_t total_blocks;
    int32_t b[kMaxRows];
    int32_t nnew[kMaxRows];
    int32_t nsplit[kMaxRows];
    int32_t pbase[kMaxRows];
    int32_t cols[kMaxRows];    // columns per query tile of the kernel that wrote the partials
    int32_t blk0[kMaxRows + 1];
};

struct CombineArgs {
    void *out;
    const float *ws_acc;
    const float *ws_ml;
    int32_t batch, T, hq, hkv, group, head_dim;
    int64_t records;
    CombineRows rows;
};

// Zero fill of padded query slots: rows r get out[b, :, nnew[r]:T, :] = +0.0.
struct ZeroRows {
    int32_t n_rows;
    int32_t b[kMaxRows];
    int32_t nnew[kMaxRows];
};

struct ZeroArgs {
    void *out;
    int32_t batch, T, hq, head_dim;
    int32_t slices;            // kZeroSlice-byte slices per (row, query head): ceil(T * row_bytes / kZeroSlice)
    int64_t row_bytes;         // d * element size
    ZeroRows rows;
};

// Scratch of the no-allocation entry point (kv_append_attention_noalloc): a
// file-scope device array of this many bytes in kernels.hip, one copy per GPU,
// held until the process ends. It holds a call's split partial records.
constexpr size_t kScratchBytes = size_t(16) << 20;
// The device address of that array on the current device, looked up with
// hipGetSymbolAddress on the first call on each device and kept per device.
hipError_t scratch_region(void **ptr);

// element type codes match kv_dtype
hipError_t launch_append(const AppendArgs &a, int n_blocks, hipStream_t s);
hipError_t launch_set_lens(int32_t *lens_dev, const LensTable &t, hipStream_t s);
hipError_t launch_table_set(const TableArgs &a, hipStream_t s);
hipError_t launch_table_fill(int32_t *table, int64_t n, int32_t value, hipStream_t s);
// +0 into `bytes` bytes from p (16-byte aligned, a multiple of 16 bytes): the
// cache buffers at creation
hipError_t launch_zero_bytes(void *p, int64_t bytes, hipStream_t s);
// nsub: 16-column subtiles per decode work item (1, 2 or 4); a.table selects
// the paged kernels (float32 and bfloat16 caches)
hipError_t launch_decode(int dtype, int head_dim, int nsub, const AttnArgs &a, hipStream_t s);
hipError_t launch_prefill(int dtype, int head_dim, const AttnArgs &a, hipStream_t s);
hipError_t launch_combine(int dtype, int head_dim, const CombineArgs &a, hipStream_t s);

// Side stream for running the decode kernel beside the prefill kernel of a
// mixed batch. `fork` makes `side` wait for all work enqueued on `main` so far;
// `join` makes `main` wait for all work enqueued on `side`. The stream and
// events are created once (default priority) and owned by the caller.
struct SideStream {
    hipStream_t side = nullptr;
    hipEvent_t fork_ev = nullptr, join_ev = nullptr;
};
hipError_t side_stream_init(SideStream &s);
void side_stream_destroy(SideStream &s);
hipError_t side_stream_fork(SideStream &s, hipStream_t main);
hipError_t side_stream_join(SideStream &s, hipStream_t main);
hipError_t launch_zero_fill(const ZeroArgs &a, hipStream_t s);

constexpr int kDecodeKeyTile = 32;
constexpr int kDecodeWaves = 8;       // waves per decode work group (they split the keys)
constexpr int kPrefillKeyTile = 64;
// Waves per prefill work group (32 columns each): 8, one work group per CU;
// float32 at d = 128 keeps 4 (its accumulators need the full register file
// of one wave per SIMD). The planner and the kernels take the count from here.
inline constexpr int prefill_waves(int dtype, int head_dim) { return (dtype == 0 && head_dim == 128) ? 4 : 8; }
// 16-column subtiles per prefill wave (2: 32 columns)
inline constexpr int prefill_subtiles(int dtype, int head_dim) { return (void)dtype, (void)head_dim, 2; }
inline constexpr int prefill_cols(int dtype, int head_dim) {
    return 16 * prefill_subtiles(dtype, head_dim) * prefill_waves(dtype, head_dim);
}
// Window of a linear cache: pos - kNoWindow < 0 <= every key, so no lower bound.
constexpr int32_t kNoWindow = 0x7fffffff;
// Ring caches hold a multiple of this many slots, and key ranges start at a
// multiple of it, so no key tile of either kernel wraps inside the ring.
constexpr int32_t kRingAlign = 64;
constexpr int kZeroSlice = 16384;   // bytes of output one zero-fill block clears
constexpr int kAppendChunk = 4096;
// Pages of a paged cache hold a power of two of tokens in this range: a key
// tile of either kernel (32 or 64 keys from a multiple of its size) never
// crosses a page.
constexpr int32_t kMinPage = 64;
constexpr int32_t kMaxPage = 65536;

}  // namespace gqakv
