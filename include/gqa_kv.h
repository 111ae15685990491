/*
 * gqa_kv.h -- grouped-query attention over a contiguous, preallocated KV cache
 * on one AMD Instinct MI355X (gfx950).
 *
 * The operations follow three pages:
 *   [GQA]  "Implement grouped-query attention over a preallocated KV cache, with
 *          no torch.cat, for both prefill chunks and decode" (inferenceinterviews.com)
 *   [MASK] "Write the causal mask for a decode step with a KV cache, where the
 *          query is shorter than the keys" (inferenceinterviews.com)
 *   [CH16] "16. Prefill, decode and the KV cache" (inference.shantanugoel.com)
 *
 * Ownership. The caller owns every device buffer (K, V, the optional device
 * copy of the lengths, q, out, k_new, v_new, the workspace) and every stream.
 * The library owns only the opaque handle and its host copies of the per-row
 * lengths (and of a paged cache's block table); it never allocates device
 * memory.
 *
 * Layout. All device arrays are dense and row-major:
 *   K, V            [B, Hkv, max_len, d]   ([GQA] "A strong answer")
 *   k_new, v_new    [B, Hkv, T, d]         (slots t >= n_new[b] are padding)
 *   q, out          [B, Hq,  T, d]
 * q, out, k_new, v_new and the cache share one element type. Every device
 * pointer must be 16-byte aligned. Supported d: 16, 32, 64, 128. Hq must be a
 * positive multiple of Hkv, with group size G = Hq / Hkv <= 128.
 *
 * Ordering. Calls are enqueued on the given HIP stream (NULL = the null
 * stream) and return without waiting for the device. The host copy of the
 * lengths is updated when a call is enqueued, so host-side validation of the
 * next call sees it at once. All calls on one handle must be issued from one
 * host thread at a time and kept in stream order by the caller.
 *
 * Graph capture. kv_append, gqa_attention, gqa_attention_tree,
 * kv_append_attention and kv_truncate enqueue only kernel launches (and, for
 * a call with prefill rows beside other rows, an event fork and join with the
 * handle's side stream, created by the first such call): no copies, memsets
 * or device allocations, so they may be captured into a HIP graph. The host
 * state (lengths, pages) moves once, when the call is captured; each replay
 * repeats the captured lengths and block-table entries. A step that appends
 * at a fixed length and rolls back replays correctly; a growing decode loop
 * needs a new capture (or eager calls) as the lengths move.
 *
 * Errors. Every call validates all of its arguments on the host before it
 * enqueues anything. KV_ERR_INVALID_ARG, KV_ERR_CAPACITY, KV_ERR_UNSUPPORTED
 * and KV_ERR_WORKSPACE mean nothing was enqueued and no state changed: not
 * the host lengths, not the device lengths, not a byte of K or V, not a page
 * of a paged cache. KV_ERR_DEVICE means a HIP launch failed part way through
 * a call that enqueues several kernels; the handle's state is then
 * unspecified and it should be destroyed. kv_last_error() returns the message
 * of the last failing call on the calling thread.
 */
#ifndef GQA_KV_H
#define GQA_KV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct kv_cache kv_cache;

typedef enum kv_status {
    KV_OK = 0,
    KV_ERR_INVALID_ARG = 1,   /* bad pointer, shape, n_new or truncation length */
    KV_ERR_CAPACITY = 2,      /* an append would pass max_len (or, in a ring,
                                 evict keys the window still needs)              */
    KV_ERR_UNSUPPORTED = 3,   /* head_dim, dtype or group size not built         */
    KV_ERR_WORKSPACE = 4,     /* workspace missing or smaller than required      */
    KV_ERR_DEVICE = 5         /* a HIP call failed                               */
} kv_status;

typedef enum kv_dtype {
    KV_DTYPE_F32 = 0,         /* IEEE float32 storage and float32 arithmetic     */
    KV_DTYPE_BF16 = 1,        /* bfloat16 storage, float32 accumulation          */
    KV_DTYPE_FP8_E4M3 = 2     /* E4M3 codes with one scale per KV head; q, out,
                                 k_new and v_new are bfloat16 (kv_cache_create_fp8) */
} kv_dtype;

/*
 * Wrap caller-allocated cache buffers in a handle.
 * [GQA] "A strong answer" (the cache is allocated once as [B, Hkv, max_len, d]
 * plus a length per row); [CH16] "Layout and validity" (capacity vs length).
 *   k_buf, v_buf  device, B*Hkv*max_len*d elements each, set to zero here
 *                 on `stream` by a fill kernel ([GQA] "A strong answer" and
 *                 [CH16] "Layout and validity" build the cache from zeros), so
 *                 every byte past a row's length is defined. Bytes outside a
 *                 row's valid prefix are never read by attention.
 *   lens_dev      optional device int32[B] that the library keeps equal to the
 *                 per-row lengths in stream order (append, truncate). May be NULL.
 *                 When given, it is set to zero on `stream` here.
 *   out           receives the handle.
 * All rows start empty. Returns KV_ERR_UNSUPPORTED for a head_dim outside
 * {16,32,64,128} or an unknown dtype, KV_ERR_INVALID_ARG for non-positive
 * kv_heads/max_len, negative batch or NULL/misaligned buffers.
 */
kv_status kv_cache_create(int32_t batch, int32_t kv_heads, int32_t max_len, int32_t head_dim,
                          kv_dtype dtype, void *k_buf, void *v_buf, int32_t *lens_dev,
                          void *stream, kv_cache **out);

/*
 * Sliding-window cache: wrap caller-allocated buffers as a ring of `capacity`
 * slots per row, keeping only the latest tokens, with attention limited to a
 * window. [MASK] "A strong answer", the reversal paragraph (a window adds a
 * lower limit on the visible keys, and once tokens sit in ring slots the
 * visibility test has to compare positions, since a slot number no longer
 * says where a token came in) and
 * [CH16] exercise 3 (a cache that keeps only the last positions in a ring).
 *   capacity      slots per row, a positive multiple of 64; k_buf and v_buf
 *                 hold B*Hkv*capacity*d elements each, laid out as
 *                 [B, Hkv, capacity, d].
 *   window        1 <= window <= capacity: a query at absolute position p
 *                 sees keys p - window < j <= p.
 * Token p of a row lives in slot p mod capacity. Lengths count every token
 * ever appended (the next absolute position; below 2^31 - 64), and
 * kv_get_lens, kv_truncate, lens_dev and the query positions of
 * gqa_attention use those absolute positions. kv_append refuses (with
 * KV_ERR_CAPACITY, "row {b}: {n} new tokens would evict keys the window still
 * needs (capacity {C}, window {W})") a write that would overwrite a key its
 * own first new query still needs, so at most capacity - window + 1 tokens
 * per call once a row has wrapped. kv_truncate also refuses a rollback to a
 * length whose next query would need a key already overwritten.
 * Other arguments and errors as kv_cache_create; KV_ERR_INVALID_ARG for a
 * capacity that is not a positive multiple of 64 or a window outside
 * 1..capacity.
 */
kv_status kv_cache_create_ring(int32_t batch, int32_t kv_heads, int32_t capacity, int32_t head_dim,
                               kv_dtype dtype, int32_t window, void *k_buf, void *v_buf,
                               int32_t *lens_dev, void *stream, kv_cache **out);

/*
 * FP8 cache: K and V stored as E4M3 codes with one scale per KV head, read back
 * dequantized. [CH16] exercise 4 (store the cache in FP8, E4M3 with one scale
 * per head, and dequantize on read) and "How big is the cache?" (half the
 * bytes of a bfloat16 cache, which a bandwidth-bound decode reads every step).
 *   k_buf, v_buf  device, B*Hkv*max_len*d BYTES each, [B, Hkv, max_len, d].
 *   k_scale, v_scale  HOST float[kv_heads], finite and > 0, copied here: a
 *                 code c of KV head h stands for c * scale[h] (E4M3 is the
 *                 OCP format: bias 7, largest finite 448, no infinities).
 * kv_append then takes bfloat16 k_new/v_new and stores, for each element x of
 * head h, the E4M3 code of x * (1 / scale[h]) computed in float32, saturated
 * to +-448 and rounded to the nearest code, ties to even. gqa_attention takes
 * bfloat16 q and writes bfloat16 out; scores use the dequantized keys and the
 * output the dequantized values (every E4M3 value is exact in bfloat16). At
 * most 64 KV heads. Other arguments, errors and the linear-cache rules as
 * kv_cache_create (kv_cache_create refuses this dtype).
 */
kv_status kv_cache_create_fp8(int32_t batch, int32_t kv_heads, int32_t max_len, int32_t head_dim,
                              const float *k_scale, const float *v_scale, void *k_buf, void *v_buf,
                              int32_t *lens_dev, void *stream, kv_cache **out);

/*
 * Paged cache: one pool of fixed-size pages shared by every row, and a block
 * table per row that maps the row's logical blocks to pages, so memory is held
 * in proportion to the tokens stored instead of max_len per row. [GQA] "A
 * strong answer" (preallocating max_len per row is the waste a paged cache
 * removes) and its reversal paragraph (rows whose lengths differ by orders of
 * magnitude leave most of a dense reservation empty; a per-row page table
 * and a kernel that follows it fix that); [CH16] "16. Prefill, decode and the KV cache",
 * design choices (a paged cache keeps the in-place O(1) write without
 * reserving the maximum up front).
 *   num_pages     pages in the pool; k_pool and v_pool are device arrays of
 *                 num_pages * Hkv * page_size * d elements each, laid out
 *                 [num_pages, Hkv, page_size, d].
 *   page_size     tokens per page: a power of two, 64 <= page_size <= 65536.
 *   max_blocks    table entries per row: a row holds at most
 *                 max_blocks * page_size tokens (its max_len).
 *   block_table   device int32[B * max_blocks], caller-allocated, written only
 *                 by the library, in stream order: entry b * max_blocks + i is
 *                 the page holding tokens i * page_size .. (i + 1) *
 *                 page_size - 1 of row b, or -1. Set to -1 here on `stream`.
 * kv_append gives each row the pages its new tokens need, row by row, each
 * time the lowest-numbered free page; if the pool cannot give them all it
 * returns KV_ERR_CAPACITY ("{n} pages needed, {m} free in the pool") and
 * changes nothing. kv_truncate returns to the pool the pages of blocks that
 * no longer hold a token. gqa_attention and gqa_attention_tree compute what
 * they compute on a linear cache with max_len = max_blocks * page_size, the
 * keys gathered through the table. float32 and bfloat16 only
 * (KV_ERR_UNSUPPORTED for E4M3); KV_ERR_INVALID_ARG for a page_size, num_pages
 * or max_blocks outside the ranges above; other arguments and errors as
 * kv_cache_create.
 */
kv_status kv_cache_create_paged(int32_t batch, int32_t kv_heads, int32_t num_pages, int32_t page_size,
                                int32_t max_blocks, int32_t head_dim, kv_dtype dtype, void *k_pool,
                                void *v_pool, int32_t *block_table, int32_t *lens_dev, void *stream,
                                kv_cache **out);

/*
 * Copy a paged cache's host block table (B * max_blocks entries, as of the
 * last enqueued call; -1 = no page) into table_host. KV_ERR_INVALID_ARG for a
 * cache that is not paged.
 */
kv_status kv_get_block_table(const kv_cache *c, int32_t *table_host);

/* Pages of a paged cache's pool that hold no token (0 for other caches). */
int32_t kv_free_pages(const kv_cache *c);

/*
 * Release the handle (never the caller's buffers); KV_OK, also for NULL. Work
 * already enqueued on the caller's streams is not waited for: the buffers must
 * outlive it.
 */
kv_status kv_cache_destroy(kv_cache *c);

/*
 * Append in place: for each row b, write k_new[b,:,0:n_new[b]] and
 * v_new[b,:,0:n_new[b]] into K and V at positions lens[b] .. lens[b]+n_new[b]-1,
 * then advance lens[b] by n_new[b]. History is never moved and nothing is
 * concatenated. [GQA] "A strong answer" (in-place write at the row's length),
 * [CH16] "Layout and validity" (capacity checked before the copy).
 *   k_new, v_new  device [B, Hkv, T, d]; padded slots are never read.
 *   T             slots per row in k_new (>= 0).
 *   n_new         HOST int32[B], 0 <= n_new[b] <= T.
 * Every row is checked before anything is written: if lens[b] + n_new[b] >
 * max_len for any b the call returns KV_ERR_CAPACITY with the message
 * "row {b}: {lens[b]+n_new[b]} tokens > max_len {max_len}" and changes nothing.
 * The bytes are copied bit for bit. In a ring cache (kv_cache_create_ring)
 * token p goes to slot p mod capacity and the capacity rule is the ring's.
 */
kv_status kv_append(kv_cache *c, const void *k_new, const void *v_new, int32_t T,
                    const int32_t *n_new, void *stream);

/*
 * Workspace that gqa_attention needs for this call (split-K partial results),
 * in bytes, written to *bytes. Depends on the current lengths and n_new.
 * Zero means no workspace is needed. The figure also covers the tree-verify
 * variants of the call (gqa_attention_tree, which keeps every row on the
 * split-K decode kernel), so one size serves both.
 */
kv_status gqa_attention_workspace_size(const kv_cache *c, int32_t q_heads, int32_t T,
                                       const int32_t *n_new, size_t *bytes);

/*
 * Grouped-query attention for the n_new[b] tokens each row just appended
 * (call it after kv_append of the same step).
 * [GQA] "A strong answer" and TL;DR: query head h reads KV head h / G with no
 * repeated KV; query t of row b sits at absolute position
 * lens[b] - n_new[b] + t and sees key j iff j <= lens[b] - n_new[b] + t and
 * j < lens[b] ([MASK] TL;DR: the bottom-right-aligned rule j <= i + (S - T),
 * evaluated as index arithmetic, never as a mask tensor); in a ring cache also
 * j > lens[b] - n_new[b] + t - window, with key j read from slot j mod
 * capacity ([MASK] "A strong answer", the reversal). Scores are scaled by
 * 1/sqrt(d). Slots t >= n_new[b], rows with n_new[b] == 0, B == 0 and T == 0
 * give +0.0 (never NaN).
 *   q             device [B, q_heads, T, d]; out device [B, q_heads, T, d].
 *   n_new         HOST int32[B] with 0 <= n_new[b] <= min(T, lens[b]).
 *   workspace     device scratch of at least gqa_attention_workspace_size()
 *                 bytes (may be NULL when that size is 0). It holds the
 *                 unnormalised partial outputs and (max, sum) pairs of key
 *                 ranges split across work groups, and one arrival counter per
 *                 split (row, KV head, query tile) of the decode kernel, whose
 *                 last work group merges the partials. Every partial is
 *                 written before it is read in the same call, and a counter
 *                 word that no call of this process has left behind is
 *                 recognised as such (it matches a random per-process 56-bit
 *                 tag only with probability 2^-56), so the contents need no
 *                 initialisation. Two calls in flight at once must not share a
 *                 workspace.
 * A call with prefill-kernel rows runs its decode kernel and its zero fill of
 * padded slots on a stream the handle owns, forked from `stream` by an event
 * before any of the call's work and joined back to it before the call's last
 * kernel, so the call as a whole stays in `stream` order.
 * Returns KV_ERR_INVALID_ARG for a bad shape, a q_heads that is not a positive
 * multiple of kv_heads, or a bad n_new; KV_ERR_UNSUPPORTED when G > 128;
 * KV_ERR_WORKSPACE when the workspace is too small.
 */
kv_status gqa_attention(kv_cache *c, const void *q, int32_t q_heads, int32_t T,
                        const int32_t *n_new, void *out, void *workspace,
                        size_t workspace_bytes, void *stream);

/*
 * Tree-based speculative verify: as gqa_attention, but the n_new[b] tokens just
 * appended to row b are the nodes of a draft tree rather than a chain. [MASK]
 * "What interviewers probe next": with a tree-shaped draft, the block of the
 * mask among the new tokens follows the tree (a node sees the committed keys,
 * itself and the nodes on its path to the root, given by parent pointers)
 * instead of a triangle.
 *   parents       HOST int32[B * T]; parents[b * T + u] for u < n_new[b] is -1
 *                 (node u follows the committed prefix) or the index of an
 *                 earlier node (0 <= parent < u). Entries for u >= n_new[b]
 *                 are ignored.
 * Node u of row b is the key at absolute position lens[b] - n_new[b] + u, and
 * query t sees key j iff j < lens[b] - n_new[b] (committed) or j is node t or
 * one of its ancestors. Needs T <= 16, G * T <= 64 and a linear cache (not a
 * ring); runs on the split-K decode kernel (KV_ERR_UNSUPPORTED when the
 * policy forces the prefill kernel). The workspace is that of gqa_attention
 * for the same arguments. A chain (parent u - 1 for every u) gives the bits
 * gqa_attention gives. KV_ERR_INVALID_ARG for a parent outside -1 .. u - 1.
 */
kv_status gqa_attention_tree(kv_cache *c, const void *q, int32_t q_heads, int32_t T,
                             const int32_t *n_new, const int32_t *parents, void *out,
                             void *workspace, size_t workspace_bytes, void *stream);

/*
 * Append and attention in one call: exactly kv_append(c, k_new, v_new, T,
 * n_new) followed by gqa_attention(c, q, q_heads, T, n_new, out, ...), the
 * cache bytes, lengths and outputs bit for bit the same. [GQA] "A strong
 * answer" (each step writes the new tokens at the row's length, then attends
 * over the cache) and [CH16] "Layout and validity" (append, then attend).
 * Every check of both halves runs before anything is enqueued, with the
 * lengths the append will leave; any error other than KV_ERR_DEVICE changes
 * nothing. Rows that run on the split-K decode kernel are appended by that
 * kernel, which reads those keys from k_new / v_new (an E4M3 cache: it stores
 * their codes and attends to the same codes), so one launch does the append
 * and the attention of a decode step; other rows are appended by the copy
 * kernel first.
 *   k_new, v_new  device [B, Hkv, T, d]; q, out device [B, q_heads, T, d]
 *   n_new         HOST int32[B]
 *   workspace     as gqa_attention, of at least
 *                 kv_append_attention_workspace_size() bytes.
 */
kv_status kv_append_attention(kv_cache *c, const void *k_new, const void *v_new, const void *q,
                              int32_t q_heads, int32_t T, const int32_t *n_new, void *out,
                              void *workspace, size_t workspace_bytes, void *stream);

/*
 * kv_append_attention for a draft tree: exactly kv_append followed by
 * gqa_attention_tree with the same parents ([MASK] "What interviewers probe
 * next"), bit for bit, in one launch of the decode kernel. Arguments and
 * limits as both; parents HOST int32 [B, T]. Any error other than
 * KV_ERR_DEVICE changes nothing.
 */
kv_status kv_append_attention_tree(kv_cache *c, const void *k_new, const void *v_new, const void *q,
                                   int32_t q_heads, int32_t T, const int32_t *n_new, const int32_t *parents,
                                   void *out, void *workspace, size_t workspace_bytes, void *stream);

/*
 * kv_append_attention for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same call, with the same cache bytes, lengths and output
 * bits, but no workspace argument. The split partial records live in a
 * scratch array of 16 MiB that the library holds in device memory, one copy
 * per GPU, from the first call on that GPU until the process ends; the call
 * itself allocates nothing (no device memory, stream or event), and every
 * kernel runs on `stream`, with a mixed batch's decode and prefill kernels
 * one after the other. Call it with the cache's device current: the scratch
 * of the current device is used. Every call on a GPU shares that GPU's
 * scratch, which keeps whatever the last call left (nothing in it needs to
 * start at any value, as for a workspace): two calls
 * that may overlap on one GPU, on different streams or from different
 * threads, race and must be ordered by the caller.
 * Returns KV_ERR_WORKSPACE, with nothing changed, for a call whose partials
 * need more than the 16 MiB (the size kv_append_attention_workspace_size
 * reports for it, before the tree-verify margin); KV_ERR_DEVICE if the
 * scratch address cannot be looked up; otherwise as kv_append_attention.
 */
kv_status kv_append_attention_noalloc(kv_cache *c, const void *k_new, const void *v_new, const void *q,
                                      int32_t q_heads, int32_t T, const int32_t *n_new, void *out, void *stream);

/*
 * Workspace kv_append_attention needs for these arguments (the
 * gqa_attention workspace for the lengths after the append), in bytes; it
 * also covers kv_append_attention_tree.
 */
kv_status kv_append_attention_workspace_size(const kv_cache *c, int32_t q_heads, int32_t T,
                                             const int32_t *n_new, size_t *bytes);

/*
 * Roll back: set lens[b] = new_lens[b] for every row, copying and clearing
 * nothing. [CH16] "Layout and validity" (truncate for speculative rollback;
 * stale slots stay and are never read). new_lens is a HOST int32[B] with
 * 0 <= new_lens[b] <= lens[b] (and, in a ring cache, new_lens[b] no lower
 * than the ring still supports); otherwise KV_ERR_INVALID_ARG with the message
 * "Invalid truncation length". Truncating every row to 0 is a reset.
 */
kv_status kv_truncate(kv_cache *c, const int32_t *new_lens, void *stream);

/* Copy the host lengths (as of the last enqueued call) into lens_host[B]. */
kv_status kv_get_lens(const kv_cache *c, int32_t *lens_host);

/*
 * Bytes of the reservation, 2 * B * Hkv * max_len * d * element size
 * ([CH16] "Layout and validity", the bytes property); for a paged cache the
 * pool, 2 * num_pages * Hkv * page_size * d * element size.
 */
uint64_t kv_cache_bytes(const kv_cache *c);

/*
 * Bytes of valid K and V, 2 * sum(lens) * Hkv * d * element size
 * ([CH16] "How big is the cache?" with tokens = the current lengths; a ring
 * row counts at most `capacity` tokens).
 */
uint64_t kv_live_bytes(const kv_cache *c);

/* Message of the last non-OK status returned on this thread ("" if none). */
const char *kv_last_error(void);

/*
 * Kernel selection, for tests and tuning. path: 0 = automatic (rows with
 * G * n_new[b] <= 32 use the split-K decode kernel, the others the tiled
 * chunked-prefill kernel), 1 = every row through the split-K decode kernel,
 * 2 = every row through the chunked-prefill kernel. keys_per_split: 0 =
 * automatic, otherwise the key range of one split (rounded up to the key
 * tile). The result is the same attention up to float32 rounding order.
 */
kv_status kv_cache_set_policy(kv_cache *c, int32_t path, int32_t keys_per_split);

#ifdef __cplusplus
}
#endif

#endif /* GQA_KV_H */
