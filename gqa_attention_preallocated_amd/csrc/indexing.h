// Work-item indexing shared by the attention kernels (device) and the host-side
// launch simulator used by the tests (host): one definition of how a block id
// becomes (row, kv head, query tile, key split), which key range it reads and
// which partial records it writes.
#pragma once

#include <stdint.h>

#include "internal.h"

#if defined(__HIP__)
#define GQAKV_HD __host__ __device__
#else
#define GQAKV_HD
#endif

namespace gqakv {

GQAKV_HD inline int imin(int a, int b) { return a < b ? a : b; }
GQAKV_HD inline int imax(int a, int b) { return a > b ? a : b; }

// Largest r in [0, n_rows) with item0[r] <= item (item0 is nondecreasing
// from item0[0] = 0): the number of rows r >= 1 whose first item is <= item.
// The kernels take the same count with one ballot over a wave whose lane l
// holds item0[l] (all lanes load at once, so a block finds its row after one
// round of loads); here it is a loop.
GQAKV_HD inline int find_row(const int32_t *item0, int n_rows, int item) {
    int r = 0;
    for (int i = 1; i < n_rows; ++i) r += item0[i] <= item;
    return r;
}

// One work item of an attention launch (see AttnRows for the numbering).
struct Item {
    int r;                // row of the launch table
    int b, kvh, qtile, split, nq, nsplit;
    int base;             // absolute position of the row's query 0 = len - n_new
    int t0, t_end;        // queries [t0, t_end) of this tile
    int k_begin, k_end;   // key positions of this split that some query of the tile may see
    int rec0;             // first partial record of the item, or -1: direct write
};

// First key position an item's range starts from: the lowest key its first
// query sees under the window, rounded down to kRingAlign (0 without a window).
GQAKV_HD inline int range_start(int first_pos, int window) {
    const int lo = first_pos - window + 1;
    return lo <= 0 ? 0 : lo - lo % kRingAlign;
}

// The row table entries of one row.
struct RowFields {
    int item0, nnew, nsplit, b, len, lsplit, pbase;
};

GQAKV_HD inline RowFields row_fields(const AttnRows &R, int r) {
    return RowFields{R.item0[r], R.nnew[r], R.nsplit[r], R.b[r], R.len[r], R.lsplit[r], R.pbase[r]};
}

// Item `item` of row r, whose table entries are f.
GQAKV_HD inline Item decode_item_at(const RowFields &f, int r, int item, int hkv, int group, int cols, int window) {
    Item it;
    it.r = r;
    const int n = f.nnew;
    const int tq = cols / group;                  // queries per tile
    it.nq = (n + tq - 1) / tq;
    it.nsplit = f.nsplit;
    const int local = item - f.item0;
    it.kvh = local % hkv;
    const int rest = local / hkv;
    it.split = rest % it.nsplit;
    it.qtile = it.nq - 1 - rest / it.nsplit;      // longest key range first
    it.b = f.b;
    it.base = f.len - n;
    it.t0 = it.qtile * tq;
    it.t_end = imin(it.t0 + tq, n);
    // bottom-right rule: the tile's last query sits at base + t_end - 1 and sees
    // keys up to that position, never past the row's length; with a window the
    // tile's first query sees nothing below base + t0 - window + 1. Splits
    // of lsplit keys each, the last one up to the tile's last key (the
    // planner may hand it more than lsplit)
    const int keys_hi = it.base + it.t_end;
    it.k_begin = range_start(it.base + it.t0, window) + it.split * f.lsplit;
    it.k_end = it.split == it.nsplit - 1 ? keys_hi : imin(it.k_begin + f.lsplit, keys_hi);
    it.rec0 = f.pbase < 0 ? -1 : f.pbase + ((it.kvh * it.nq + it.qtile) * it.nsplit + it.split) * cols;
    return it;
}

GQAKV_HD inline Item decode_item(const AttnRows &R, int item, int hkv, int group, int cols, int window) {
    const int r = find_row(R.item0, R.n_rows, item);
    return decode_item_at(row_fields(R, r), r, item, hkv, group, cols, window);
}

// Absolute position of the query in column `col` of the item, or -1 for a
// padding column (no key visible). Column col holds query t0 + col / G of
// query head kvh * G + col % G.
GQAKV_HD inline int column_position(const Item &it, int col, int group, int cols) {
    const int tq = cols / group;
    const int t = it.t0 + col / group;
    return (col < tq * group && t < it.t_end) ? it.base + t : -1;
}

GQAKV_HD inline int column_t(const Item &it, int col, int group) { return it.t0 + col / group; }
GQAKV_HD inline int column_head(const Item &it, int col, int group) { return it.kvh * group + col % group; }

}  // namespace gqakv
