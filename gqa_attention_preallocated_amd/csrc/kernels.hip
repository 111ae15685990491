// HIP kernels for grouped-query attention over a preallocated KV cache, gfx950.
//
// Pages cited (titles; sections named where used):
//   [GQA]  "Implement grouped-query attention over a preallocated KV cache, with
//          no torch.cat, for both prefill chunks and decode"
//   [MASK] "Write the causal mask for a decode step with a KV cache, where the
//          query is shorter than the keys"
//   [CH16] "16. Prefill, decode and the KV cache"
//
// Matrix-core formulation. Both attention kernels compute, for one KV head,
//   S^T[key][col] = K[key][:] . Q[col][:]          (MFMA, m = key, n = col)
//   O^T[d][col]  += V^T[d][key] . P^T[key][col]    (MFMA, m = d,   n = col)
// where a "column" is one (query, group member) pair: the G query heads that
// share KV head kvh sit side by side, so every K/V element loaded feeds all G
// heads and no repeated KV exists ([GQA] "A strong answer", decision 1).
// With v_mfma_f32_16x16x32_bf16 a lane l holds, for A, row (l%16) and k-slots
// 8*(l/16)..+7; for B, column (l%16) and the same k-slots; for C, rows
// 4*(l/16)+i and column (l%16). Putting the key on S^T's m axis leaves each
// lane with 4 scores of one column; two 16-key blocks give 8 scores, exactly
// the 8 k-slots the lane needs as B operand of the O^T product, so the
// probabilities never move between lanes. Only V needs a transpose (k-slots
// must run along keys), done through LDS.
//
// Float32 caches use v_mfma_f32_16x16x4_f32 with the same operand layout
// (8 values per lane, issued as 8 instructions), so they never round to bf16.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <mutex>
#include <type_traits>
#include <vector>

#include "indexing.h"
#include "internal.h"

namespace gqakv {

// ---------------------------------------------------------------------------
// Scratch of the no-allocation entry point: the split partial records of one
// call (what the caller's workspace holds in the other entry points). Each GPU
// the library runs on gets its own copy at its own address. In host code the
// name below is only a host-side handle for the symbol, never a device
// address: host code uses the pointer scratch_region() returns.
// ---------------------------------------------------------------------------
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

hipError_t scratch_region(void **ptr) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    static std::mutex mu;
    static std::vector<void *> addr;      // device address of `scratch`, per device
    std::lock_guard<std::mutex> lock(mu);
    if ((size_t)dev >= addr.size()) addr.resize((size_t)dev + 1, nullptr);
    if (addr[dev] == nullptr) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));   // with device `dev` current
        if (e != hipSuccess) return e;
        if (p == nullptr) return hipErrorInvalidSymbol;
        addr[dev] = p;
    }
    *ptr = addr[dev];
    return hipSuccess;
}

// every launch passes its tables by value: keep them inside the kernel-argument space
static_assert(sizeof(AttnArgs) <= 4096 && sizeof(AppendArgs) <= 4096 && sizeof(CombineArgs) <= 4096 &&
              sizeof(ZeroArgs) <= 4096 && sizeof(TableArgs) <= 4096, "kernel arguments too large");

typedef __bf16 bf16_t;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(8))) float f32x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;

// K and V are read once per call: non-temporal loads keep them from displacing
// other lines and measured faster for streaming reads on MI355X
__device__ inline uint4 load_stream(const void *p) {
    const u32x4 t = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
    return make_uint4(t.x, t.y, t.z, t.w);
}

// Buffer view of `bytes` bytes from `base`: a load at a byte offset at or past
// the end returns zeros without touching memory, so a tile that runs past the
// valid keys needs no per-lane predicate. The last descriptor word is the
// raw (untyped, unswizzled) buffer setting of CDNA parts.
// `base` and `bytes` must be the same in every lane of the wave (they are
// moved to scalar registers).
__device__ inline __amdgpu_buffer_rsrc_t buffer_view(const void *base, int bytes) {
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
    void *p = reinterpret_cast<void *>(((uint64_t)hi << 32) | lo);
    return __builtin_amdgcn_make_buffer_rsrc(p, (short)0, __builtin_amdgcn_readfirstlane(bytes), 0x00020000);
}

// 16 bytes at byte offset `off` of a buffer view, non-temporal (cache policy nt)
__device__ inline uint4 buffer_load_stream(__amdgpu_buffer_rsrc_t r, int off) {
    const u32x4 t = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 2);
    return make_uint4(t.x, t.y, t.z, t.w);
}
// The same load without the non-temporal hint: for data other work groups of
// the same XCD read soon after (the query tiles of one (row, KV head) in the
// prefill kernel), so their reads hit in L2.
__device__ inline uint4 buffer_load_shared(__amdgpu_buffer_rsrc_t r, int off) {
    const u32x4 t = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
    return make_uint4(t.x, t.y, t.z, t.w);
}

// ---------------------------------------------------------------------------
// element traits: 8-element MFMA operands and the 16x16 product
// ---------------------------------------------------------------------------
template <typename E> struct Op;

template <> struct Op<bf16_t> {
    using vec = bf16x8;
    static constexpr int kBytes = 2;
    __device__ static inline vec zero() { return __builtin_bit_cast(vec, make_uint4(0, 0, 0, 0)); }
    __device__ static inline vec ones() {      // bf16 1.0 = 0x3f80 in every slot
        return __builtin_bit_cast(vec, make_uint4(0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u));
    }
    __device__ static inline vec gload(const bf16_t *p) {
        return __builtin_bit_cast(vec, *reinterpret_cast<const uint4 *>(p));
    }
    __device__ static inline vec gload_stream(const bf16_t *p) { return __builtin_bit_cast(vec, load_stream(p)); }
    __device__ static inline vec lds_load(const unsigned char *p) {
        return __builtin_bit_cast(vec, *reinterpret_cast<const uint4 *>(p));
    }
    __device__ static inline f32x4 mma(const vec &a, const vec &b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
    __device__ static inline vec from_f32(const f32x8 &x) { return __builtin_convertvector(x, vec); }
    // c * v, rounded to bfloat16 (to nearest, even)
    __device__ static inline vec scaled(const vec &v, float c) {
        return __builtin_convertvector(__builtin_convertvector(v, f32x8) * c, vec);
    }
    // elements j, j+1 (j even) of an operand from two floats (one packed convert)
    __device__ static inline void set_pair(vec &v, int j, float x, float y) {
        typedef __attribute__((ext_vector_type(2))) float f32x2;
        typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
        const bf16x2 w = __builtin_convertvector((f32x2){x, y}, bf16x2);
        uint4 u = __builtin_bit_cast(uint4, v);
        const uint32_t bits = __builtin_bit_cast(uint32_t, w);
        if (j == 0) u.x = bits; else if (j == 2) u.y = bits; else if (j == 4) u.z = bits; else u.w = bits;
        v = __builtin_bit_cast(vec, u);
    }
    // LDS row stride for a K/V tile: 32 bytes of padding put the rows that one
    // transposed read touches on disjoint banks
    static constexpr int kPad = 32;
    // A operand of O^T += V^T P^T for output rows d0..d0+15 and the 32 keys
    // key0.. of a row-major LDS tile: lane (i, g) needs V[key][d0 + i] for the
    // keys k-slot j of group g stands for (4g + j, then 16 + 4g + j). The
    // gfx950 transpose read gives lane i of a 16-lane group element i%4 of the
    // 8-byte segments read by lanes i/4 + 4j, so lane a + 4j reads
    // V[key_j][d0 + 4a .. +3].
    __device__ static inline vec vt_operand(const unsigned char *tile, int rs, int key0, int d0, int lane) {
        typedef short v4s __attribute__((ext_vector_type(4)));
        const int src = lane & 15, g = lane >> 4;
        const unsigned char *p = tile + (key0 + g * 4 + (src >> 2)) * rs + (d0 + 4 * (src & 3)) * 2;
        const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) v4s *)(p));
        const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) v4s *)(p + 16 * rs));
        const uint2 a = __builtin_bit_cast(uint2, lo), b = __builtin_bit_cast(uint2, hi);
        return __builtin_bit_cast(vec, make_uint4(a.x, a.y, b.x, b.y));
    }
    __device__ static inline void store4(bf16_t *p, f32x4 v) {
        typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
        bf16x4 b = __builtin_convertvector(v, bf16x4);
        *reinterpret_cast<uint2 *>(p) = __builtin_bit_cast(uint2, b);
    }
};

template <> struct Op<float> {
    using vec = f32x8;
    static constexpr int kBytes = 4;
    __device__ static inline vec zero() { return vec{0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f}; }
    __device__ static inline vec ones() { return vec{1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f}; }
    __device__ static inline vec gload(const float *p) {
        float4 a = reinterpret_cast<const float4 *>(p)[0];
        float4 b = reinterpret_cast<const float4 *>(p)[1];
        return vec{a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    }
    __device__ static inline vec gload_stream(const float *p) {
        const float4 a = __builtin_bit_cast(float4, load_stream(p));
        const float4 b = __builtin_bit_cast(float4, load_stream(p + 4));
        return vec{a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    }
    __device__ static inline vec lds_load(const unsigned char *p) {
        float4 a = reinterpret_cast<const float4 *>(p)[0];
        float4 b = reinterpret_cast<const float4 *>(p)[1];
        return vec{a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    }
    __device__ static inline f32x4 mma(const vec &a, const vec &b, f32x4 c) {
#pragma unroll
        for (int j = 0; j < 8; ++j) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[j], b[j], c, 0, 0, 0);
        return c;
    }
    __device__ static inline vec from_f32(const f32x8 &x) { return x; }
    __device__ static inline vec scaled(const vec &v, float c) { return v * c; }
    __device__ static inline void set_pair(vec &v, int j, float x, float y) {
        v[j] = x;
        v[j + 1] = y;
    }
    // the contraction over the first 16 elements only (4 of the 8 steps)
    __device__ static inline f32x4 mma16(const vec &a, const vec &b, f32x4 c) {
#pragma unroll
        for (int j = 0; j < 4; ++j) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[j], b[j], c, 0, 0, 0);
        return c;
    }
    // vt_operand over a 16-key tile: keys 4g..4g+3 only (elements 4..7 unused)
    __device__ static inline vec vt_operand16(const unsigned char *tile, int rs, int d0, int lane) {
        const int lr = lane & 15, lg = lane >> 4;
        vec r = zero();
#pragma unroll
        for (int j = 0; j < 4; ++j) r[j] = *reinterpret_cast<const float *>(tile + (lg * 4 + j) * rs + (d0 + lr) * 4);
        return r;
    }
    static constexpr int kPad = 16;
    // A operand of O^T += V^T P^T (see the bf16 version): 8 single-element reads
    __device__ static inline vec vt_operand(const unsigned char *tile, int rs, int key0, int d0, int lane) {
        const int lr = lane & 15, lg = lane >> 4;
        vec r;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int key = key0 + ((j < 4) ? lg * 4 + j : 16 + lg * 4 + (j - 4));
            r[j] = *reinterpret_cast<const float *>(tile + key * rs + (d0 + lr) * 4);
        }
        return r;
    }
    __device__ static inline void store4(float *p, f32x4 v) {
        *reinterpret_cast<float4 *>(p) = make_float4(v[0], v[1], v[2], v[3]);
    }
};

// ---------------------------------------------------------------------------
// cache storage: the kernel's own element type, or (F8) E4M3 codes that are
// widened exactly to bfloat16 on read ([CH16] exercise 4: dequantize on read;
// the head's scale is applied to the scores and to the output instead of to
// every element). The gfx950 conversion is exact for every E4M3 value.
// ---------------------------------------------------------------------------
template <typename E, bool F8> struct Stor {
    using vec = typename Op<E>::vec;
    using kraw = vec;                                 // K operand as loaded
    static constexpr int kBytes = Op<E>::kBytes;      // bytes per cached element
    static constexpr int kLdsPerChunk = 16;           // LDS bytes a 16-byte cache chunk becomes
    __device__ static inline kraw load_k(const unsigned char *p) {
        return Op<E>::gload_stream(reinterpret_cast<const E *>(p));
    }
    __device__ static inline kraw zero_k() { return Op<E>::zero(); }
    __device__ static inline vec widen_k(const kraw &r) { return r; }
    __device__ static inline void stage(unsigned char *dst, const uint4 &raw) {
        *reinterpret_cast<uint4 *>(dst) = raw;
    }
};

template <> struct Stor<bf16_t, true> {
    using vec = bf16x8;
    typedef __attribute__((ext_vector_type(2))) unsigned int u32x2;
    using kraw = uint2;                               // 8 codes
    static constexpr int kBytes = 1;
    static constexpr int kLdsPerChunk = 32;           // 16 codes -> 16 bfloat16
    __device__ static inline kraw load_k(const unsigned char *p) {
        const u32x2 t = __builtin_nontemporal_load(reinterpret_cast<const u32x2 *>(p));
        return make_uint2(t.x, t.y);
    }
    __device__ static inline kraw zero_k() { return make_uint2(0, 0); }
    // codes in bytes 0,1 (HI false) or 2,3 (HI true) of w -> two bfloat16 (exact; scale 1)
    template <bool HI> __device__ static inline uint32_t widen2(uint32_t w) {
        return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
    }
    __device__ static inline uint4 widen4x2(uint32_t a, uint32_t b) {
        return make_uint4(widen2<false>(a), widen2<true>(a), widen2<false>(b), widen2<true>(b));
    }
    __device__ static inline vec widen_k(const kraw &r) { return __builtin_bit_cast(vec, widen4x2(r.x, r.y)); }
    __device__ static inline void stage(unsigned char *dst, const uint4 &raw) {
        reinterpret_cast<uint4 *>(dst)[0] = widen4x2(raw.x, raw.y);
        reinterpret_cast<uint4 *>(dst)[1] = widen4x2(raw.z, raw.w);
    }
};

// 2^x with the hardware instruction alone. exp2f adds a range fix for
// results below 2^-126; a probability that small is zero for every purpose here.
__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Max of scores, which are finite or -inf (masked keys), never NaN. The
// NaN-propagating maximum needs no quieting of its inputs, where fmaxf makes
// the compiler canonicalize every operand that is not the result of another
// max first (one extra VALU instruction per score), and it pairs into the
// three-input v_maximum3_f32.
__device__ inline float smax(float a, float b) { return __builtin_elementwise_maximum(a, b); }
__device__ inline float smax8(float a, float b, float c, float d, float e, float f, float g, float h) {
    return smax(smax(smax(smax(a, b), c), smax(smax(d, e), f)), smax(g, h));
}

__device__ inline float wave_max_across_groups(float v) {
    // lanes l, l^16, l^32, l^48 hold the same column. A gfx950 lane-half swap
    // returns (own, partner) in some order, so the max of the pair is the max
    // over the two lanes, with no LDS traffic.
    const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = smax(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return smax(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

__device__ inline float wave_sum_across_groups(float v) {
    v += __shfl_xor(v, 16);
    v += __shfl_xor(v, 32);
    return v;
}

// ---------------------------------------------------------------------------
// append: bit copy of the new tokens into their slots ([GQA] "A strong answer":
// written in place at the row's current length; nothing else moves). In a ring
// cache token p lands in slot p mod max_len ([CH16] exercise 3).
// ---------------------------------------------------------------------------
// E4M3 codes of 8 bfloat16 values (a 16-byte chunk) times inv, in memory order
__device__ inline uint32_t quant4(uint32_t lo, uint32_t hi, float inv) {
    auto f = [&](uint32_t bits) {                 // bfloat16 -> float32 is exact
        const float y = __uint_as_float(bits << 16) * inv;
        return fminf(fmaxf(y, -448.f), 448.f);    // saturate: the conversion rounds to nearest even
    };
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(f(lo & 0xffffu), f(lo >> 16), 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(f(hi & 0xffffu), f(hi >> 16), w, true);
    return (uint32_t)w;
}

__device__ inline uint2 quant8(const uint4 &x, float inv) {
    return make_uint2(quant4(x.x, x.y, inv), quant4(x.z, x.w, inv));
}

// ---------------------------------------------------------------------------
// Row lookup from the launch tables in the kernel arguments. Lane l of a wave
// loads entry l of each table (at most kMaxRows rows: one wave holds them
// all), so every entry arrives after one round of loads; the block's row is
// the ballot count of find_row, and its entries are read from that row's lane.
// (A search over the table would chain one dependent load per step before a
// block could issue its first memory access.)
// ---------------------------------------------------------------------------
// Entry `lane` of a launch table of kMaxRows (or kMaxRows + 1) entries, pad
// past the n in use. The load does not wait for n: every lane's entry lies
// inside the table.
__device__ inline int lane_entry(const int32_t *table, int n, int pad) {
    const int l = threadIdx.x & 63;
    const int v = table[l];
    return l < n ? v : pad;
}

// find_row over `first` (nondecreasing, first[0] = 0) with one ballot
__device__ inline int wave_find_row(int first_mine, int idx) {
    const int l = threadIdx.x & 63;
    return (int)__builtin_popcountll(__ballot(l >= 1 && first_mine <= idx));
}

__device__ inline int row_entry(int mine, int r) { return __builtin_amdgcn_readlane(mine, r); }

__device__ inline Item decode_item_wave(const AttnRows &R, int item, int hkv, int group, int cols, int window) {
    const int n = R.n_rows;
    const int i0 = lane_entry(R.item0, n, 0x7fffffff);
    const int nn = lane_entry(R.nnew, n, 0), ns = lane_entry(R.nsplit, n, 1), bb = lane_entry(R.b, n, 0);
    const int ln = lane_entry(R.len, n, 0), ls = lane_entry(R.lsplit, n, 0), pb = lane_entry(R.pbase, n, -1);
    const int r = wave_find_row(i0, item);
    const RowFields f{row_entry(i0, r), row_entry(nn, r), row_entry(ns, r), row_entry(bb, r),
                      row_entry(ln, r), row_entry(ls, r), row_entry(pb, r)};
    return decode_item_at(f, r, item, hkv, group, cols, window);
}

// A wave-uniform 64-bit value moved to scalar registers (each half through
// its own readfirstlane, as unsigned 32-bit values: the builtin returns int)
__device__ inline uint64_t uniform_u64(uint64_t v) {
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return ((uint64_t)hi << 32) | lo;
}

// Partial records written and read by different work groups of one launch
// (the decode kernel's merge): agent-scope accesses, which reach the
// device-coherent level rather than stopping in (or hitting a stale line of)
// one XCD's L2. Two floats per access: 64 bits is the widest atomic access.
__device__ inline float2 coherent_load2(const float *p) {
    const unsigned long long u =
        __hip_atomic_load(reinterpret_cast<const unsigned long long *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return __builtin_bit_cast(float2, u);
}
__device__ inline void coherent_store2(float *p, float x, float y) {
    __hip_atomic_store(reinterpret_cast<unsigned long long *>(p), __builtin_bit_cast(unsigned long long, make_float2(x, y)),
                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Split partials: the nsplit partial records rec, rec + stride, ... of one
// column hold unnormalised sums acc and (running max m in log2 units, sum l).
// Their outputs d..d+3 are merged by log-sum-exp in split order, BATCH splits
// per batch of loads, and normalised (0 when no split saw a key).
// COHERENT: the records were written in this launch by other work groups
// (the decode kernel's in-kernel merge), else by an earlier launch. Eight
// splits per batch (one round trip for up to eight), four in the decode
// kernel's merge at d < 64, whose smaller instances would otherwise lose
// occupancy to these registers.
template <int D, bool COHERENT = false>
__device__ inline f32x4 merge_partials(const float *ws_acc, const float *ws_ml, int64_t rec, int64_t stride,
                                       int nsplit, int d) {
    constexpr int BATCH = COHERENT && D < 64 ? 4 : 8;
    float M = -INFINITY, L = 0.f;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int s0 = 0; s0 < nsplit; s0 += BATCH) {
        float2 ml[BATCH];
        float4 x[BATCH];
#pragma unroll
        for (int j = 0; j < BATCH; ++j) {
            const int64_t rs = rec + (int64_t)(s0 + j) * stride;
            if (s0 + j < nsplit) {
                if constexpr (COHERENT) {
                    const float *px = ws_acc + rs * D + d;
                    ml[j] = coherent_load2(ws_ml + rs * 2);
                    const float2 lo = coherent_load2(px), hi = coherent_load2(px + 2);
                    x[j] = make_float4(lo.x, lo.y, hi.x, hi.y);
                } else {
                    ml[j] = *reinterpret_cast<const float2 *>(ws_ml + rs * 2);
                    x[j] = *reinterpret_cast<const float4 *>(ws_acc + rs * D + d);
                }
            } else {
                ml[j] = make_float2(-INFINITY, 0.f);
                x[j] = make_float4(0.f, 0.f, 0.f, 0.f);
            }
        }
        float bm = M;
#pragma unroll
        for (int j = 0; j < BATCH; ++j) bm = fmaxf(bm, ml[j].x);
        if (bm == -INFINITY) continue;            // no split so far saw a key of this column
        const float c = fast_exp2(M - bm);        // M = -inf: c = 0 (acc and L are still 0)
        acc *= c;
        L *= c;
#pragma unroll
        for (int j = 0; j < BATCH; ++j) {
            const float w = fast_exp2(ml[j].x - bm);   // a split that saw no key: w = 0
            acc[0] += w * x[j].x; acc[1] += w * x[j].y; acc[2] += w * x[j].z; acc[3] += w * x[j].w;
            L += w * ml[j].y;
        }
        M = bm;
    }
    return acc * (L > 0.f ? 1.f / L : 0.f);
}

__global__ __launch_bounds__(256) void append_kernel(AppendArgs a) {
    const int nrow = a.t.n_rows;
    const int first = lane_entry(a.t.block0, nrow, 0x7fffffff);
    const int r = wave_find_row(first, blockIdx.x);
    const int local = blockIdx.x - row_entry(first, r);
    const int nch = row_entry(lane_entry(a.t.nchunk, nrow, 1), r);
    const int kvh = local / nch;
    const int chunk = local % nch;
    const int b = row_entry(lane_entry(a.t.b, nrow, 0), r);
    const int start = row_entry(lane_entry(a.t.start, nrow, 0), r);
    const int slot0 = row_entry(lane_entry(a.t.slot0, nrow, 0), r);
    const int ntok = row_entry(lane_entry(a.t.n, nrow, 0), r);
    const int64_t span = (int64_t)ntok * a.row_bytes;
    const int64_t off = (int64_t)chunk * kAppendChunk + threadIdx.x * 16;
    const int64_t head = (int64_t)b * a.hkv + kvh;
    if (off < span) {
        // token i of the row goes to slot slot0 + i, wrapping at max_len (a
        // ring; a linear cache never reaches the wrap)
        const int tok = (int)(off >> a.row_shift);
        int64_t crow;                             // cache row of the token
        if (a.table == nullptr) {
            int slot = slot0 + tok;
            if (slot >= a.max_len) slot -= a.max_len;
            crow = head * a.max_len + slot;
        } else {
            // paged: position p sits in row p mod page of (page, kv head) in the
            // pool, page = block_table[b][p / page] ([GQA] reversal); the table
            // entries were set earlier on the stream
            const int p = start + tok;
            const int page = a.table[(int64_t)b * a.max_blocks + (p >> a.page_shift)];
            crow = (((int64_t)page * a.hkv + kvh) << a.page_shift) + (p & ((1 << a.page_shift) - 1));
        }
        const int64_t src = head * a.T * a.row_bytes + off;
        const uint4 kx = *reinterpret_cast<const uint4 *>((const char *)a.k_new + src);
        const uint4 vx = *reinterpret_cast<const uint4 *>((const char *)a.v_new + src);
        if (!a.quant) {
            const int64_t dst = (crow << a.row_shift) + (off & (a.row_bytes - 1));
            *reinterpret_cast<uint4 *>((char *)a.k + dst) = kx;
            *reinterpret_cast<uint4 *>((char *)a.v + dst) = vx;
        } else {
            // E4M3 cache ([CH16] exercise 4): 8 bfloat16 in, 8 codes out, each
            // the code of x * (1 / scale) in float32, saturated to +-448,
            // rounded to the nearest code (ties to even)
            const int64_t dst = (crow << (a.row_shift - 1)) + ((off & (a.row_bytes - 1)) >> 1);
            *reinterpret_cast<uint2 *>((char *)a.k + dst) = quant8(kx, a.k_inv[kvh]);
            *reinterpret_cast<uint2 *>((char *)a.v + dst) = quant8(vx, a.v_inv[kvh]);
        }
    }
    // the row's new length becomes visible to later kernels in stream order
    if (a.lens_dev != nullptr && local == 0 && threadIdx.x == 0) a.lens_dev[b] = start + ntok;
}

__global__ __launch_bounds__(64) void set_lens_kernel(int32_t *lens_dev, LensTable t) {
    const int i = threadIdx.x;
    if (i < t.n_rows) lens_dev[t.b[i]] = t.len[i];
}

// paged caches: block-table entries set by the host's page assignment
__global__ __launch_bounds__(256) void table_set_kernel(TableArgs a) {
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i < a.n) a.table[a.idx[i]] = a.page[i];
}

__global__ __launch_bounds__(256) void table_fill_kernel(int32_t *table, int64_t n, int32_t value) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n) table[i] = value;
}

// zero K and V at creation: 16-byte stores over a grid-stride loop (a kernel,
// not a memset, so a captured graph holds no memset node)
__global__ __launch_bounds__(256) void zero_bytes_kernel(uint4 *p, int64_t n16) {
    const int64_t stride = (int64_t)gridDim.x * 256;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += stride) p[i] = make_uint4(0, 0, 0, 0);
}

// ---------------------------------------------------------------------------
// shared pieces of the two attention kernels
// ---------------------------------------------------------------------------

// q row of a column (only read when the column is real)
template <typename E>
__device__ inline const E *column_q(const AttnArgs &a, const Item &it, int col, int D) {
    const int t = column_t(it, col, a.group), h = column_head(it, col, a.group);
    return reinterpret_cast<const E *>(a.q) + (((int64_t)it.b * a.hq + h) * a.T + t) * D;
}

template <typename E>
__device__ inline E *column_out(const AttnArgs &a, const Item &it, int col, int D) {
    const int t = column_t(it, col, a.group), h = column_head(it, col, a.group);
    return reinterpret_cast<E *>(a.out) + (((int64_t)it.b * a.hq + h) * a.T + t) * D;
}

// Where the keys of a work item live. Key position j of (row b, kv head h): a
// linear or ring cache holds it in slot j mod max_len of the head's
// [max_len, d] block; a paged cache in row j mod page of block (page, h) of
// the pool, page = block_table[b][j / page] ([GQA] reversal: a block table
// and a paged kernel). row(tile) is the cache row of a tile's first key; no
// tile crosses a page or the end of a ring. A paged lookup keeps 64
// consecutive table entries of the row, one per lane, and reads the one it
// needs across lanes; tiles are asked for in increasing order, so the entries
// are reloaded once per 64 blocks.
template <bool PG> struct KeyRows;

template <> struct KeyRows<false> {
    int64_t head_row;
    int max_len;
    __device__ KeyRows(const AttnArgs &a, const Item &it, int)
        : head_row(((int64_t)it.b * a.hkv + it.kvh) * a.max_len), max_len(a.max_len) {}
    __device__ int64_t row(int tile) const { return head_row + tile % max_len; }
};

template <> struct KeyRows<true> {
    const int32_t *tbl;
    int nblk, shift, kvh, hkv;
    int blk0, ent;
    __device__ KeyRows(const AttnArgs &a, const Item &it, int first_key)
        : tbl(a.table + (int64_t)it.b * a.max_blocks), nblk(a.max_blocks), shift(a.page_shift), kvh(it.kvh),
          hkv(a.hkv) {
        refill(__builtin_amdgcn_readfirstlane(first_key >> shift));
    }
    __device__ void refill(int blk) {
        blk0 = blk;
        const int i = blk + (int)(threadIdx.x & 63);
        ent = i < nblk ? tbl[i] : 0;
    }
    __device__ int64_t row(int tile) {
        const int blk = __builtin_amdgcn_readfirstlane(tile >> shift);
        if (blk - blk0 >= 64) refill(blk);
        const int page = __builtin_amdgcn_readlane(ent, blk - blk0);
        return (((int64_t)page * hkv + kvh) << shift) + (tile & ((1 << shift) - 1));
    }
};

// Cache row (in units of one K or V row) of key position p of (row b, kv head
// h), for the few keys a fused append writes: linear and ring caches use slot
// p mod max_len, paged caches the block table.
template <bool PG>
__device__ inline int64_t cache_row(const AttnArgs &a, int b, int h, int p) {
    if constexpr (PG) {
        const int page = a.table[(int64_t)b * a.max_blocks + (p >> a.page_shift)];
        return (((int64_t)page * a.hkv + h) << a.page_shift) + (p & ((1 << a.page_shift) - 1));
    } else {
        return ((int64_t)b * a.hkv + h) * a.max_len + p % a.max_len;
    }
}

// kv_append_attention on decode-kernel rows. Each new token is written by
// exactly one work item: the one whose query tile holds the token's own
// query and whose key split holds the token (every new position p = base + t
// lies in the key range of the tile of query t, and the splits of a tile
// partition that range). The kernel reads the new keys from k_new / v_new
// ([B, Hkv, T, d] rows of NROWB input bytes), so no read waits for these
// writes.
template <int D, bool F8, bool PG, int NROWB>
__device__ inline void write_new_tokens(const AttnArgs &a, const Item &it, int tid, int nthreads) {
    constexpr int CROWB = F8 ? D : NROWB;             // cache bytes of a row
    constexpr int PPR = NROWB / 16;                   // 16-byte input pieces per row
    const int lo = imax(it.k_begin, it.base + it.t0), hi = imin(it.k_end, it.base + it.t_end);
    const int n_tok = hi - lo;
    if (n_tok <= 0) return;
    const int64_t new0 = ((int64_t)it.b * a.hkv + it.kvh) * a.T + (lo - it.base);
    for (int task = tid; task < 2 * n_tok * PPR; task += nthreads) {
        const int tv = task / (n_tok * PPR), rem = task % (n_tok * PPR);
        const int tok = rem / PPR, part = rem % PPR;
        const unsigned char *sb = reinterpret_cast<const unsigned char *>(tv ? a.v_new : a.k_new);
        unsigned char *db = reinterpret_cast<unsigned char *>(const_cast<void *>(tv ? a.v : a.k));
        const uint4 x = *reinterpret_cast<const uint4 *>(sb + (new0 + tok) * NROWB + part * 16);
        const int64_t crow = cache_row<PG>(a, it.b, it.kvh, lo + tok);
        // an E4M3 cache stores the codes of x * (1 / scale), as the append kernel does
        if constexpr (F8)
            *reinterpret_cast<uint2 *>(db + crow * CROWB + part * 8) =
                quant8(x, tv ? a.v_inv[it.kvh] : a.k_inv[it.kvh]);
        else
            *reinterpret_cast<uint4 *>(db + crow * CROWB + part * 16) = x;
    }
}

// 16 storage bytes at storage byte `off` of new token t of a (row, kv head)
// whose k_new / v_new rows start at nb: an E4M3 cache gets the 16 codes of
// 16 bfloat16 inputs, exactly as they are stored
template <bool F8, int NROWB>
__device__ inline uint4 new_chunk(const unsigned char *nb, int t, int off, float inv) {
    if constexpr (F8) {
        const unsigned char *p = nb + (int64_t)t * NROWB + off * 2;
        const uint2 c0 = quant8(load_stream(p), inv), c1 = quant8(load_stream(p + 16), inv);
        return make_uint4(c0.x, c0.y, c1.x, c1.y);
    } else {
        return load_stream(nb + (int64_t)t * NROWB + off);
    }
}

// One online-softmax step for the 8 scores a lane holds for its column
// (two 16-key blocks: s0 = keys 4g..4g+3, s1 = keys 16+4g..16+4g+3 of a
// 32-key chunk, g = lane/16). Scores arrive unscaled; `pos` is the column's
// absolute position; `kfirst` the key index of s0[0]'s block row 0. Keys past
// pos (or past k_end) get probability 0. Returns the rescale factor for the
// accumulator and writes the probabilities back into s0/s1.
struct ColState {
    float m;   // reference max, log2 units (-inf until a key is visible)
    float l;   // this lane's share of the running denominator
};

// The accumulator is rescaled only when a column's max grows past the
// reference by more than this (log2 units): between rescales exp2 arguments
// stay <= 8, so probabilities stay <= 256, far inside float32 and bfloat16
// range, and acc / l is unchanged algebraically.
constexpr float kRescaleLog2 = 8.f;

// One online-softmax step for the N raw scores q.k a lane holds for its
// column (16-key blocks: v[0..3] = keys 4g..4g+3, v[4..7] = keys
// 16+4g..16+4g+3 of a 32-key tile, g = lane/16; N = 4: one 16-key block);
// invisible keys are -inf. c = log2(e)/sqrt(d) > 0, so the max of raw scores
// scaled by c is the max of the scaled scores. Writes p = exp2(v*c - m)
// (p[N..7] untouched) and updates the state.
template <int NB, int N>
__device__ inline void softmax_step(const float (&v)[N], float c, ColState &st, f32x4 (&acc)[NB], f32x8 &p) {
    static_assert(N == 4 || N == 8, "one or two 16-key blocks");
    float tmax = N == 8 ? smax8(v[0], v[1], v[2], v[3], v[4], v[5], v[6], v[7])
                        : smax(smax(v[0], v[1]), smax(v[2], v[3 % N]));
    tmax = wave_max_across_groups(tmax) * c;
    if (tmax > st.m + kRescaleLog2) {             // st.m = -inf: the first visible key sets it
        const float alpha = fast_exp2(st.m - tmax);   // 0 when st.m = -inf (acc and l are still 0)
        st.l *= alpha;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) acc[nb] *= alpha;
        st.m = tmax;
    }
    const float m_use = (st.m == -INFINITY) ? 0.f : st.m;   // no key seen yet: every p is 0
    float lsum = 0.f;
#pragma unroll
    for (int j = 0; j < N; ++j) {
        const float e = fast_exp2(fmaf(v[j], c, -m_use));
        p[j] = e;
        lsum += e;
    }
    st.l += lsum;
}

// ---------------------------------------------------------------------------
// split-K decode / verify kernel. One work group of W waves per work item
// (row, kv head, query tile, key split) with 16*NSUB columns. The item's
// 32-key tiles are dealt to the waves in turn (wave w takes tiles w, w + W,
// ...: a fixed assignment, so results are bitwise reproducible, and the work
// group reads one contiguous run of K and of V at a time); each wave streams
// its tiles from HBM with the next tile in flight while one is computed, then
// the waves merge their partial results through LDS (reusing the V staging
// space), so a split-free row needs no second pass. In kv_append_attention
// the kernel also writes its share of the new tokens into the cache and reads
// the new keys from k_new / v_new.
// ---------------------------------------------------------------------------
template <typename E, int D, int NSUB, int W, bool F8, bool PG>
__global__ __launch_bounds__(64 * W) void decode_kernel(AttnArgs a) {
    using O = Op<E>;
    using S = Stor<E, F8>;
    using vec = typename O::vec;
    using kraw = typename S::kraw;
    // 32 keys per tile; float32 at d = 128 takes 16-key tiles (half the K and V
    // registers: with 32 its instances spilled), two per planner tile
    constexpr int KT = (std::is_same<E, float>::value && D == 128) ? 16 : kDecodeKeyTile;
    constexpr int NKS = KT / 16;                  // 16-key blocks per tile
    static_assert(kDecodeKeyTile % KT == 0 && (NKS == 2 || std::is_same<E, float>::value), "key tile");
    constexpr int KC = D >= 32 ? D / 32 : 1;      // 32-wide chunks of d
    constexpr int NB = D / 16;                    // 16-row blocks of O^T
    // columns per work item: a.cols (the planner's choice, at most 16 * NSUB;
    // columns past it are padding and see no key)
    constexpr int ROWB = D * O::kBytes;           // LDS bytes of one V row (compute type)
    constexpr int RS = ROWB + O::kPad;            // padded LDS row: conflict-free transposed reads
    constexpr int CROWB = D * S::kBytes;          // cache bytes of one K or V row
    constexpr int CPK = CROWB / 16;               // 16-byte cache chunks per key row
    constexpr int VCH = (KT * CPK + 63) / 64;     // V chunks per lane per tile
    constexpr int STAGE = KT * RS;                // per-wave V staging bytes
    constexpr int PSTR = D + 4;                   // floats per column in the merge area
    constexpr int MERGE = W * 16 * PSTR * 4 + W * 16 * 2 * 4;
    constexpr int LDS_BYTES = (W * STAGE > MERGE) ? W * STAGE : MERGE;
    __shared__ __attribute__((aligned(16))) unsigned char lds_all[LDS_BYTES];

    const int tid = threadIdx.x;
    // the wave index is the same in every lane: a scalar, so that tile
    // positions and per-wave conditions stay in scalar registers
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int lr = lane & 15, lg = lane >> 4;
    unsigned char *lds = lds_all + wave * STAGE;
    Item it = decode_item_wave(a.rows, blockIdx.x, a.hkv, a.group, a.cols, a.window);
    // the key range in scalar registers: tile positions and cache rows are
    // then scalar work
    it.k_begin = __builtin_amdgcn_readfirstlane(it.k_begin);
    it.k_end = __builtin_amdgcn_readfirstlane(it.k_end);

    // this wave's share of the item's keys: every W-th 32-key tile from its
    // own, so at any time the work group streams one contiguous run of K and
    // one of V (fewer concurrent DRAM streams than a contiguous range per wave)
    const int w_begin = it.k_begin + wave * KT;
    const int w_end = it.k_end;
    constexpr int step = W * KT;

    // k-slots of lane group lg in 32-wide chunk kc: d = dmap(kc) .. +7. The
    // contraction over d is a sum, so Q and K only need the same map: for an
    // E4M3 cache with an even chunk count, chunks 2j and 2j+1 take the two
    // halves of 16 contiguous codes (one 16-byte load per lane for both)
    constexpr bool KPAIR = F8 && KC % 2 == 0;
    auto dmap = [&](int kc) { return KPAIR ? 64 * (kc >> 1) + 16 * lg + 8 * (kc & 1) : kc * 32 + lg * 8; };

    // ---- columns: absolute positions and Q operands (B of S^T)
    int pos[NSUB];
    vec qop[NSUB][KC];
#pragma unroll
    for (int s = 0; s < NSUB; ++s) {
        const int col = s * 16 + lr;
        pos[s] = column_position(it, col, a.group, a.cols);
        const E *qp = pos[s] >= 0 ? column_q<E>(a, it, col, D) : nullptr;
#pragma unroll
        for (int kc = 0; kc < KC; ++kc) {
            const int d0 = dmap(kc);
            qop[s][kc] = (qp != nullptr && d0 < D) ? O::gload(qp + d0) : O::zero();
        }
    }

    const unsigned char *kbase = reinterpret_cast<const unsigned char *>(a.k);
    const unsigned char *vbase = reinterpret_cast<const unsigned char *>(a.v);
    KeyRows<PG> km(a, it, w_begin);
    // rows of k_new / v_new hold d input elements (bfloat16 for an E4M3 cache)
    constexpr int NROWB = D * (int)sizeof(E);
    if (a.fuse) {
        // kv_append_attention: this item's share of the new tokens goes into
        // the cache here; the attention below reads them from k_new / v_new
        write_new_tokens<D, F8, PG, NROWB>(a, it, tid, 64 * W);
        // the first item of a row (kv head 0, split 0, its last query tile)
        // sets the row's device length
        if (a.lens_dev != nullptr && tid == 0 && it.kvh == 0 && it.split == 0 && it.qtile == it.nq - 1)
            a.lens_dev[it.b] = a.rows.len[it.r];
    }
    // an E4M3 cache stands for code x scale of the head: the K scale joins the
    // score scale, the V scale multiplies the output
    const float score_c = F8 ? a.scale_log2 * a.k_scale[it.kvh] : a.scale_log2;
    const float out_c = F8 ? a.v_scale[it.kvh] : 1.f;

    f32x4 acc[NSUB][NB];
    ColState st[NSUB];
#pragma unroll
    for (int s = 0; s < NSUB; ++s) {
        st[s].m = -INFINITY;
        st[s].l = 0.f;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) acc[s][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    // ---- prefetch: the next tile is in flight while one is computed (a
    //      bfloat16 tile is 64 VGPRs a lane; a second set would cost occupancy).
    //      An E4M3 tile is half the bytes, so two are kept in flight to keep
    //      the same bytes outstanding per CU (up to 32 columns; wider items
    //      have no registers to spare).
    constexpr int PF = (F8 && NSUB <= 2) ? 2 : 1;
    kraw kA[NKS][KC], kB[NKS][KC];
    uint4 vA[VCH], vB[VCH];
    // a tile's keys are consecutive cache rows from km.row(tile): no tile
    // wraps (ring capacities are multiples of kRingAlign, pages of kMinPage,
    // and tiles start at multiples of KT)
    // kv_append_attention: keys at or past the row's first new position come
    // from k_new / v_new [B, Hkv, T, d] (FRESH tiles)
    const unsigned char *knew = nullptr, *vnew = nullptr;
    if (a.fuse) {
        const int64_t r0 = ((int64_t)it.b * a.hkv + it.kvh) * a.T;
        knew = reinterpret_cast<const unsigned char *>(a.k_new) + r0 * NROWB;
        vnew = reinterpret_cast<const unsigned char *>(a.v_new) + r0 * NROWB;
    }
    const float kinv = F8 ? a.k_inv[it.kvh] : 1.f, vinv = F8 ? a.v_inv[it.kvh] : 1.f;
    auto load_tile_as = [&](kraw (&kop)[NKS][KC], uint4 (&vreg)[VCH], int tile, auto fresh) {
        constexpr bool FRESH = decltype(fresh)::value;
        const int64_t row0 = km.row(tile);
        const unsigned char *kt = kbase + row0 * CROWB;
        const unsigned char *vt = vbase + row0 * CROWB;
        // A key at or past the range end (only in a range's last tile) is read
        // from the range's last key when the tile holds no new keys: its score
        // is masked and its p is 0, so any finite row will do, and the loads
        // then need no condition (loads under a condition made the compiler
        // wait for the tiles in flight before the next tile's work)
        const int last = w_end - 1 - tile;                    // >= 0: the tile starts below w_end
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
            const int key = ks * 16 + lr;
            const bool ok = tile + key < w_end;
            const bool nw = FRESH && tile + key >= it.base;       // a new key: from k_new
            const int t = tile + key - it.base;
            const int keyc = ok ? key : last;
            if constexpr (KPAIR) {
#pragma unroll
                for (int j = 0; j < KC / 2; ++j) {
                    const int off = dmap(2 * j);                  // codes: byte = d
                    uint4 w;
                    if constexpr (FRESH)
                        w = !ok ? make_uint4(0, 0, 0, 0)
                            : nw ? new_chunk<F8, NROWB>(knew, t, off, kinv) : load_stream(kt + key * CROWB + off);
                    else
                        w = load_stream(kt + keyc * CROWB + off);
                    kop[ks][2 * j] = make_uint2(w.x, w.y);
                    kop[ks][2 * j + 1] = make_uint2(w.z, w.w);
                }
            } else {
#pragma unroll
                for (int kc = 0; kc < KC; ++kc) {
                    const int d0 = dmap(kc);
                    if constexpr (!FRESH && D >= 32) {
                        kop[ks][kc] = S::load_k(kt + keyc * CROWB + d0 * S::kBytes);   // d0 < D for every lane
                    } else if (!(ok && d0 < D)) {
                        kop[ks][kc] = S::zero_k();
                    } else if (nw) {
                        if constexpr (F8)
                            kop[ks][kc] = quant8(*reinterpret_cast<const uint4 *>(knew + (int64_t)t * NROWB + d0 * 2), kinv);
                        else
                            kop[ks][kc] = S::load_k(knew + (int64_t)t * NROWB + d0 * S::kBytes);
                    } else {
                        kop[ks][kc] = S::load_k(kt + key * CROWB + d0 * S::kBytes);
                    }
                }
            }
        }
#pragma unroll
        for (int i = 0; i < VCH; ++i) {
            const int c = lane + 64 * i;
            const int key = c / CPK, part = c % CPK;
            if constexpr (!FRESH && (KT * CPK) % 64 == 0) {
                vreg[i] = load_stream(vt + (tile + key < w_end ? key : last) * CROWB + part * 16);
            } else {
                const bool ok = (c < KT * CPK) && (tile + key < w_end);
                const bool nw = FRESH && tile + key >= it.base;
                vreg[i] = !ok ? make_uint4(0, 0, 0, 0)
                        : nw ? new_chunk<F8, NROWB>(vnew, tile + key - it.base, part * 16, vinv)
                             : load_stream(vt + key * CROWB + part * 16);
            }
        }
    };
    auto load_tile = [&](kraw (&kop)[NKS][KC], uint4 (&vreg)[VCH], int tile) {
        if (a.fuse && tile + KT > it.base) {               // uniform over the wave
            load_tile_as(kop, vreg, tile, std::true_type{});
            return;
        }
        load_tile_as(kop, vreg, tile, std::false_type{});
    };

    // tree verify ([MASK] "What interviewers probe next"): the new tokens of
    // the row are tree nodes; a column's query (node t) sees the committed keys
    // and the nodes on its path to the root. anc = that path as a bit set.
    uint32_t anc[NSUB];
#pragma unroll
    for (int s = 0; s < NSUB; ++s) {
        anc[s] = 0;
        if (a.tree && pos[s] >= 0) {
            const int8_t *par = a.parent[it.r];
            int u = column_t(it, s * 16 + lr, a.group);
            for (int k = 0; k < kMaxTreeNodes && u >= 0; ++k) {   // parents point to earlier nodes
                anc[s] |= 1u << u;
                u = par[u];
            }
        }
    }

    // smallest position among this item's real columns: tiles ending at or
    // before it need no mask ([MASK] "A strong answer", tile cases); with a
    // window, tiles starting at or below the largest position minus the
    // window hold keys below some column's window
    const int pos_min = it.base + it.t0;
    const int pos_max = it.base + it.t_end - 1;
    int lo_key[NSUB];                              // lowest key each column sees (clamped at 0)
#pragma unroll
    for (int s = 0; s < NSUB; ++s) lo_key[s] = pos[s] - a.window + 1 > 0 ? pos[s] - a.window + 1 : 0;

    // compute the tile held in (kop, vreg), refilling the set with the next tile
    // The order the waves take the tiles in. Each round gives wave w its
    // tile w; rows of a linear or ring cache sit max_len keys apart, and with
    // a row stride that is not a multiple of 2 MiB the work groups, which all
    // start together, would stream from unrelated offsets modulo 2 MiB: the
    // decode step measured up to 23% slower (max_len 8,256 against 8,192). So
    // a work group starts at the full round that brings its byte address back
    // to the offset a 2 MiB-aligned row would have, takes the full rounds from
    // there, wrapping around, and the last, partial round last. phys maps a
    // tile of the plain order to the tile read in its place. A 2 MiB-aligned
    // row, and a paged cache (whose pages are not rows), keep the plain order;
    // so does an E4M3 cache (two tiles in flight), whose registers are full.
    const int full_end = it.k_begin + (it.k_end - it.k_begin) / step * step;   // end of the full rounds
    int rot = 0;                                                     // keys the full rounds are rotated by
    if constexpr (!PG && PF == 1) {
        constexpr int64_t kPhase = int64_t(1) << 21;
        const int64_t base = (((int64_t)it.b * a.hkv + it.kvh) * a.max_len + it.k_begin % a.max_len) * CROWB;
        const int64_t rb = (int64_t)step * CROWB;                   // bytes of one round
        const int rf = (full_end - it.k_begin) / step;
        if (rf > 1) rot = (int)((((kPhase - (base & (kPhase - 1))) & (kPhase - 1)) / rb) % rf) * step;
    }
    auto phys = [&](int vt) {
        if (vt >= full_end) return vt;
        const int t = vt + rot;
        return t >= full_end ? t - (full_end - it.k_begin) : t;
    };

    // compute the tile held in (kop, vreg), refilling the set with the next
    // one; vt is the tile in the plain order, tile the one read in its place
    // STEADY: the caller knows the tile PF rounds ahead exists and holds no
    // new keys, so the prefetch needs no test and takes the plain load path
    auto process = [&](kraw (&kop)[NKS][KC], uint4 (&vreg)[VCH], int vt, auto steady) {
        const int tile = phys(vt);
        // V tile into this wave's LDS stage (row-major, padded, compute type)
#pragma unroll
        for (int i = 0; i < VCH; ++i) {
            const int c = lane + 64 * i;
            if (c < KT * CPK) {
                const int key = c / CPK, part = c % CPK;
                S::stage(lds + key * RS + part * S::kLdsPerChunk, vreg[i]);
            }
        }
        // ---- S^T = K Q^T for the 32 keys
        f32x4 sc[NSUB][NKS];
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
            vec kv[KC];
#pragma unroll
            for (int kc = 0; kc < KC; ++kc) kv[kc] = S::widen_k(kop[ks][kc]);
#pragma unroll
            for (int s = 0; s < NSUB; ++s) {
                f32x4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kc = 0; kc < KC; ++kc) c = O::mma(kv[kc], qop[s][kc], c);
                sc[s][ks] = c;
            }
        }
        if constexpr (decltype(steady)::value) {
            load_tile_as(kop, vreg, phys(vt + PF * step), std::false_type{});
            // the loads stay here: left to itself the scheduler sank them past
            // the pair's second tile, a tile's work later
            __builtin_amdgcn_sched_barrier(0);
        } else if (vt + PF * step < w_end) {
            load_tile(kop, vreg, phys(vt + PF * step));
        }

        // ---- mask (only tiles that straddle the diagonal or the range end),
        //      online softmax in log2 units
        const bool need_mask = (tile + KT > w_end) || (tile + KT - 1 > pos_min) || (tile <= pos_max - a.window) ||
                               (a.tree && tile + KT > it.base);
        f32x8 p[NSUB];
#pragma unroll
        for (int s = 0; s < NSUB; ++s) {
            float v[4 * NKS];
#pragma unroll
            for (int j = 0; j < 4 * NKS; ++j) v[j] = sc[s][j >> 2][j & 3];
            if (need_mask) {                      // uniform over the wave
                // key j is visible iff lo_key <= j <= pos and j < the range end,
                // and (tree) j is committed or on the column's path to the root
                const int lim = imin(pos[s] + 1, w_end) - (tile + lg * 4);
                const int lim_lo = lo_key[s] - (tile + lg * 4);
                const int node0 = tile + lg * 4 - it.base;        // node index of offset 0
#pragma unroll
                for (int j = 0; j < 4 * NKS; ++j) {
                    const int off = (j >> 2) * 16 + (j & 3);
                    const int u = node0 + off;
                    const bool on_path = u < 0 || (u < 32 && ((anc[s] >> (u & 31)) & 1u));
                    v[j] = (off < lim && off >= lim_lo && (!a.tree || on_path)) ? v[j] : -INFINITY;
                }
            }
            softmax_step<NB, 4 * NKS>(v, score_c, st[s], acc[s], p[s]);
        }

        __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): this wave's V stores have landed
        __builtin_amdgcn_wave_barrier();

        // ---- O^T += V^T P^T
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            if constexpr (NKS == 2) {
                const vec vt = O::vt_operand(lds, RS, 0, nb * 16, lane);
#pragma unroll
                for (int s = 0; s < NSUB; ++s) acc[s][nb] = O::mma(vt, O::from_f32(p[s]), acc[s][nb]);
            } else {                              // float32, 16-key tiles
                const vec vt = O::vt_operand16(lds, RS, nb * 16, lane);
#pragma unroll
                for (int s = 0; s < NSUB; ++s) acc[s][nb] = O::mma16(vt, p[s], acc[s][nb]);
            }
        }
        __builtin_amdgcn_s_waitcnt(0xc07f);   // V^T reads done before the stage is overwritten
        __builtin_amdgcn_wave_barrier();
    };

    if constexpr (PF == 2) {
        // While both tiles of a pair and both of their prefetches exist and
        // hold no new keys, every pass issues the same loads: the compiler can
        // then count them and waits for the current tile only, leaving the
        // next one in flight (with a test on each prefetch it waited for both).
        // The first two tiles then take the same plain loads, on a path of
        // their own, so the loop is entered with the loads in flight that it
        // loops with.
        const int lim = a.fuse ? imin(w_end, it.base) : w_end;
        int tile = w_begin;
        if (w_begin + 3 * step + KT <= lim) {
            load_tile_as(kA, vA, phys(w_begin), std::false_type{});
            __builtin_amdgcn_sched_barrier(0);     // all of A's loads before B's, as in the loop
            load_tile_as(kB, vB, phys(w_begin + step), std::false_type{});
            __builtin_amdgcn_sched_barrier(0);
            for (; tile + 3 * step + KT <= lim; tile += 2 * step) {
                process(kA, vA, tile, std::true_type{});
                process(kB, vB, tile + step, std::true_type{});
            }
        } else {
            if (w_begin < w_end) load_tile(kA, vA, phys(w_begin));
            if (w_begin + step < w_end) load_tile(kB, vB, phys(w_begin + step));
        }
        for (; tile < w_end; tile += 2 * step) {
            process(kA, vA, tile, std::false_type{});
            if (tile + step < w_end) process(kB, vB, tile + step, std::false_type{});
        }
    } else {
        if (w_begin < w_end) load_tile(kA, vA, phys(w_begin));
        for (int tile = w_begin; tile < w_end; tile += step) process(kA, vA, tile, std::false_type{});
    }

    // ---- merge the W waves' partials in LDS, one 16-column subtile at a time
    float *part = reinterpret_cast<float *>(lds_all);                 // [W][16][PSTR]
    float *pml = part + W * 16 * PSTR;                                // [W][16][2]
    constexpr int DC = D / 4;
#pragma unroll
    for (int s = 0; s < NSUB; ++s) {
        const float l = wave_sum_across_groups(st[s].l);
        __syncthreads();                       // stages (or the previous subtile) no longer read
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
            *reinterpret_cast<float4 *>(part + (wave * 16 + lr) * PSTR + nb * 16 + lg * 4) =
                make_float4(acc[s][nb][0], acc[s][nb][1], acc[s][nb][2], acc[s][nb][3]);
        if (lg == 0) *reinterpret_cast<float2 *>(pml + (wave * 16 + lr) * 2) = make_float2(st[s].m, l);
        __syncthreads();
        for (int task = tid; task < 16 * DC; task += 64 * W) {
            const int c16 = task / DC, d = (task % DC) * 4;
            const int col = s * 16 + c16;
            if (column_position(it, col, a.group, a.cols) < 0) continue;
            float M = -INFINITY;
#pragma unroll
            for (int w = 0; w < W; ++w) M = fmaxf(M, pml[(w * 16 + c16) * 2]);
            const float m_use = (M == -INFINITY) ? 0.f : M;
            f32x4 o = {0.f, 0.f, 0.f, 0.f};
            float L = 0.f;
#pragma unroll
            for (int w = 0; w < W; ++w) {
                const float2 ml = *reinterpret_cast<const float2 *>(pml + (w * 16 + c16) * 2);
                const float wt = fast_exp2(ml.x - m_use);      // a wave that saw no key: weight 0
                const float4 x = *reinterpret_cast<const float4 *>(part + (w * 16 + c16) * PSTR + d);
                o[0] += wt * x.x; o[1] += wt * x.y; o[2] += wt * x.z; o[3] += wt * x.w;
                L += wt * ml.y;
            }
            o *= out_c;                            // the V scale of an E4M3 cache (1 otherwise)
            if (it.rec0 < 0) {
                E *op = column_out<E>(a, it, col, D) + d;
                O::store4(op, o * (L > 0.f ? 1.f / L : 0.f));
            } else {
                // a partial of a row split across work groups, written through
                // to the device-coherent level for the merge below
                float *ap = a.ws_acc + (it.rec0 + col) * (int64_t)D + d;
                coherent_store2(ap, o[0], o[1]);
                coherent_store2(ap + 2, o[2], o[3]);
                if (d == 0) coherent_store2(a.ws_ml + (it.rec0 + col) * 2, M, L);
            }
        }
    }

    // ---- rows split across work groups: the last work group of a (row, kv
    //      head, query tile) group to finish merges the group's nsplit
    //      partials, in split order (so the result does not depend on which
    //      group is last). Each work group waits until its partial stores have
    //      completed, which for stores at agent scope means they are at the
    //      device-coherent level, then counts its arrival with one atomic add;
    //      the last arrival reads every partial at agent scope. No cache
    //      write-back is needed (a release fence per work group measured
    //      slower than a separate merge launch). A counter word holds (tag,
    //      arrivals) and the last arrival leaves it at (tag, 0), ready for the
    //      next call on this workspace (or the next replay of a captured
    //      graph). The tag is fixed for the process: a word that does not hold
    //      it, or holds a count the group cannot reach, is memory no call has
    //      used yet. Such an arrival's add is void: it counts itself with an
    //      exchange that takes the word as zero arrivals, and the first
    //      exchange rewrites the whole word (adds that landed on the old word
    //      are discarded with it; their arrivals count themselves the same way).
    if (it.rec0 >= 0 && it.nsplit <= kMergeMaxSplits) {
        __shared__ int last_arrival;
        const int64_t rec_first = it.rec0 - (int64_t)it.split * a.cols;
        unsigned long long *cnt = a.counters + rec_first / a.cols;
        __builtin_amdgcn_s_waitcnt(0x0f70);            // vmcnt(0): this thread's partial stores completed
        __syncthreads();
        if (tid == 0) {
            constexpr unsigned long long kCountMask = (1ull << kMergeCountBits) - 1;
            const unsigned long long base = a.merge_tag << kMergeCountBits;
            auto arrivals = [&](unsigned long long w) -> int {   // -1: a word no call has used yet
                return (w & ~kCountMask) == base && (int)(w & kCountMask) < it.nsplit ? (int)(w & kCountMask) : -1;
            };
            unsigned long long old = __hip_atomic_fetch_add(cnt, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            int arrived = arrivals(old);
            if (arrived < 0) {
                old += 1;                                   // the word as this add left it (a first guess)
                unsigned long long want;
                do {
                    arrived = arrivals(old);
                    if (arrived < 0) arrived = 0;
                    want = base | (unsigned long long)(arrived + 1);
                } while (!__hip_atomic_compare_exchange_strong(cnt, &old, want, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                                               __HIP_MEMORY_SCOPE_AGENT));
            }
            const bool last = arrived + 1 == it.nsplit;
            if (last) __hip_atomic_store(cnt, base, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            last_arrival = last;
        }
        __syncthreads();
        if (last_arrival) {
            for (int task = tid; task < a.cols * DC; task += 64 * W) {
                const int col = task / DC, d = (task % DC) * 4;
                if (column_position(it, col, a.group, a.cols) < 0) continue;
                O::store4(column_out<E>(a, it, col, D) + d,
                          merge_partials<D, true>(a.ws_acc, a.ws_ml, rec_first + col, a.cols, it.nsplit, d));
            }
        }
    }
}


// ---------------------------------------------------------------------------
// chunked-prefill kernel: PW waves x 32 columns per work item, 64-key tiles
// of K and V shared by the waves through LDS. With PW = 8 one work group
// fills a CU at two waves per SIMD; eight waves rather than four halve the
// staging (global loads, LDS stores, their registers) per FLOP. The two waves
// of a SIMD run each tile's matrix work and softmax in opposite orders, so
// one's exponentials and vector work run beside the other's MFMAs (on gfx950
// a wave's exponentials overlap another wave's MFMAs, but stall its own).
// float32 at d = 128 runs PW = 4 at one wave per SIMD (prefill_waves).
// Key tiles past the last query's position are never loaded; tiles wholly at
// or below the first query's position are not masked; only tiles straddling
// the diagonal compare indices ([MASK] "A strong answer", tiled-kernel rule).
// ---------------------------------------------------------------------------
template <typename E, int D, bool F8, bool PG, int PW, int NS>
__global__ __launch_bounds__(64 * PW) __attribute__((amdgpu_waves_per_eu(PW == 8 ? 2 : 1))) void prefill_kernel(AttnArgs a) {
    using O = Op<E>;
    using S = Stor<E, F8>;
    using vec = typename O::vec;
    constexpr int KT = kPrefillKeyTile;           // 64 keys per tile
    constexpr int KC = D >= 32 ? D / 32 : 1;
    constexpr int NB = D / 16;
    constexpr int WC = 16 * NS;                   // columns per wave (NS 16-column subtiles)
    constexpr int C = WC * PW;                    // columns per item
    constexpr int NT = 64 * PW;                   // threads per work group
    constexpr int ROWB = D * O::kBytes;           // LDS bytes of a K or V row (compute type)
    // padded LDS rows keep the operand reads conflict-free
    constexpr int RS = ROWB + O::kPad;
    constexpr int CROWB = D * S::kBytes;          // cache bytes of a row
    constexpr int CPK = CROWB / 16;               // 16-byte cache chunks per row
    constexpr int TILE_BYTES = KT * RS;
    constexpr int PCH = (KT * CPK + NT - 1) / NT; // 16-byte chunks per thread per tensor
    // With 8 waves, waves w and w + 4 share a SIMD and run a tile's work in
    // opposite orders (PING, below); a K or V tile is then read in two
    // iterations, and each tensor gets three slots. With 4 waves (one per
    // SIMD) every wave takes the same order, and two slots suffice.
    constexpr bool PING = PW == 8;
    constexpr int SL = PING ? 3 : 2;
    __shared__ __attribute__((aligned(16))) unsigned char lds_k[SL][TILE_BYTES];
    __shared__ __attribute__((aligned(16))) unsigned char lds_v[SL][TILE_BYTES];
    static_assert(2 * SL * TILE_BYTES <= 160 * 1024, "prefill LDS tiles exceed the CU's 160 KiB");

    const int tid = threadIdx.x;
    // the wave index is the same in every lane: a scalar, so that per-wave
    // conditions and tile positions stay in scalar registers and branches
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int lr = lane & 15, lg = lane >> 4;
    Item it = decode_item_wave(a.rows, blockIdx.x, a.hkv, a.group, C, a.window);
    // the key range in scalar registers: the loop's tile positions, cache rows
    // and buffer views are then scalar work (more item fields in scalar
    // registers made this instance spill)
    it.k_begin = __builtin_amdgcn_readfirstlane(it.k_begin);
    it.k_end = __builtin_amdgcn_readfirstlane(it.k_end);

    int pos[NS];
    vec qop[NS][KC];
    int wave_pos_max = -1, wave_pos_min = 0x7fffffff;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        const int col = wave * WC + s * 16 + lr;
        pos[s] = column_position(it, col, a.group, C);
        // every lane loads from a valid address (a padding column from the
        // item's column 0, which is always real); the zeros of padding
        // columns and of d0 >= D are selected when Q is scaled, after the
        // first K and V loads have gone out (loads under a condition made the
        // compiler wait for each before issuing the next)
        const E *qp = column_q<E>(a, it, pos[s] >= 0 ? col : 0, D);
#pragma unroll
        for (int kc = 0; kc < KC; ++kc) {
            const int d0 = kc * 32 + lg * 8;
            qop[s][kc] = O::gload(qp + (d0 < D ? d0 : 0));
        }
    }
    {
        // range of real positions among the wave's columns (uniform over the wave)
        const int tq = C / a.group;
        const int c_lo = wave * WC, c_hi = min(wave * WC + WC - 1, tq * a.group - 1);
        if (c_lo <= c_hi) {
            const int t_lo = it.t0 + c_lo / a.group;
            const int t_hi = min(it.t0 + c_hi / a.group, it.t_end - 1);
            if (t_lo <= t_hi) {
                wave_pos_min = it.base + t_lo;
                wave_pos_max = it.base + t_hi;
            }
        }
    }

    const unsigned char *kbase = reinterpret_cast<const unsigned char *>(a.k);
    const unsigned char *vbase = reinterpret_cast<const unsigned char *>(a.v);
    KeyRows<PG> km(a, it, it.k_begin);
    if constexpr (!PG) {
        // linear and ring caches: K and V of the (row, KV head) block from
        // scalar registers (the item's fields are vector values), so a tile's
        // address is scalar arithmetic, not 64-bit vector work per load
        const int64_t off = (int64_t)uniform_u64((uint64_t)km.head_row) * CROWB;
        kbase += off;
        vbase += off;
    }
    // cache row of a tile's first key: within the block above (linear and
    // ring), or of the whole pool (paged)
    auto tile_row = [&](int tile) -> int64_t {
        if constexpr (PG) return km.row(tile);
        else return tile % a.max_len;
    };
    // an E4M3 cache: the K scale joins the score scale, the V scale the output
    const float score_c = F8 ? a.scale_log2 * a.k_scale[it.kvh] : a.scale_log2;
    const float out_c = F8 ? a.v_scale[it.kvh] : 1.f;
    // Q carries the score scale (log2 e / sqrt(d), times the K scale of an
    // E4M3 cache), so the score MFMAs give scaled scores; their accumulators
    // start at -m, the column's reference max, so they give the exponent of
    // p = exp2(s - m) directly ([GQA] "A strong answer": the 1/sqrt(d) scale).
    // Rounding q * scale to bfloat16 adds an error of at most 2^-9 of each
    // product q_i k_i, with random signs over the d terms of a score. The
    // scaling waits for the Q loads, so it runs after the first K and V loads
    // are issued (one memory round trip for both).
    auto scale_q = [&]() {
#pragma unroll
        for (int s = 0; s < NS; ++s)
#pragma unroll
            for (int kc = 0; kc < KC; ++kc)
                qop[s][kc] = (pos[s] >= 0 && kc * 32 + lg * 8 < D) ? O::scaled(qop[s][kc], score_c) : O::zero();
    };

    // acc[s][0..NB-1]: O^T rows; acc[s][NB]: a 16-row block whose A operand is
    // all ones, so each of its rows is the column's running sum of p (the
    // same rounded p the output rows use)
    f32x4 acc[NS][NB + 1];
    ColState st[NS];
    f32x4 bias[NS];          // -m, the reference the scores are taken against (0 before any key)
    float thr[NS];           // the reference moves when the tile's max exceeds it: -inf before any key
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        bias[s] = f32x4{0.f, 0.f, 0.f, 0.f};
        thr[s] = -INFINITY;
        st[s].m = -INFINITY;
        st[s].l = 0.f;
#pragma unroll
        for (int nb = 0; nb <= NB; ++nb) acc[s][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    const vec ones = O::ones();
    uint4 kreg[PCH], vreg[PCH];
    // thread chunk c = tid + 256 i is key c / CPK, bytes (c % CPK) * 16.. of the
    // tile: byte offset c * 16 from the tile's first key. Keys at or past
    // k_end (and chunks past the tile) fall outside the view and read as zero.
    // a tile's keys are consecutive cache rows from tile_row(tile), which the
    // K load of a tile looks up and the V load of the same tile reuses (no
    // tile wraps or crosses a page: see decode)
    auto load = [&](uint4 (&reg)[PCH], const unsigned char *base, int64_t row0, int tile) {
        const __amdgpu_buffer_rsrc_t r = buffer_view(base + row0 * CROWB, imin(it.k_end - tile, KT) * CROWB);
#pragma unroll
        for (int i = 0; i < PCH; ++i) reg[i] = buffer_load_shared(r, (tid + NT * i) * 16);
    };
    // into LDS in the compute type (an E4M3 chunk of 16 codes becomes 32 bytes)
    auto store = [&](const uint4 (&reg)[PCH], unsigned char *dst) {
#pragma unroll
        for (int i = 0; i < PCH; ++i) {
            const int c = tid + NT * i;
            if ((KT * CPK) % NT == 0 || c < KT * CPK) S::stage(dst + (c / CPK) * RS + (c % CPK) * S::kLdsPerChunk, reg[i]);
        }
    };
    // straddling tiles only: key (ch, ks, j) = tile + ch*32 + ks*16 + 4*lg + j
    // is visible iff it is <= the column's position, > that position minus
    // the window, and < the split end
    auto mask = [&](int tile, f32x4 (&sc)[2][NS][2]) {
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            const int lim = imin(pos[s] + 1, it.k_end) - (tile + lg * 4);
            const int lo_key = pos[s] - a.window + 1 > 0 ? pos[s] - a.window + 1 : 0;
            const int lim_lo = lo_key - (tile + lg * 4);
#pragma unroll
            for (int ch = 0; ch < 2; ++ch)
#pragma unroll
                for (int ks = 0; ks < 2; ++ks)
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const int off = ch * 32 + ks * 16 + j;
                        sc[ch][s][ks][j] = (off < lim && off >= lim_lo) ? sc[ch][s][ks][j] : -INFINITY;
                    }
        }
    };
    // Software pipeline over the item's key tiles, one iteration per tile i
    // between barriers. A wave's work for a tile is a matrix block (MFMAs
    // with their LDS operand reads: PV of one tile, the scores of another)
    // and a softmax block (vector work: column max, rescale decision,
    // probabilities). Group A (waves 0-3) runs the matrix block first, PV of
    // tile i-1 and the scores of tile i, then the softmax of tile i; group B
    // (waves 4-7, the other wave of each SIMD) runs the softmax of tile i
    // first (its scores came with the previous iteration), then PV of tile i
    // and the scores of tile i+1. So on every SIMD one wave's softmax runs
    // beside the other wave's MFMAs. With 4 waves there are no pairs: every
    // wave takes group B's order.
    // Staging: iteration i stores K(i+1) and V(i) into slot (i+1) % SL and
    // i % SL of their tensors, issues the global loads of K(i+2) and V(i+1)
    // into the registers just stored, then the barrier. In iteration i the
    // waves read K(i), K(i+1), V(i-1) and V(i) (group A the first and third,
    // group B the others); a wave that is still in iteration i-1 when another
    // stores reads K(i-1), K(i), V(i-2), V(i-1); with three slots (two without
    // group A) the slots written are never among them. A wave computes tiles
    // 0..wave_last only (tiles past its last query are skipped); it still
    // takes part in staging and barriers, and group A finishes the PV of its
    // last tile in the first skipped iteration or after the loop.
    // waves w and w + 4 share a SIMD (the waves of a work group go to the
    // SIMDs in turn)
    const bool grp_a = PING && wave < 4;
    // an empty asm that takes v in registers: v is computed by this point
    auto pin = [](vec &v) {
        if constexpr (sizeof(vec) == 16) {
            uint4 u = __builtin_bit_cast(uint4, v);
            asm volatile("" : "+v"(u.x), "+v"(u.y), "+v"(u.z), "+v"(u.w));
            v = __builtin_bit_cast(vec, u);
        } else {
            struct U8 { uint4 a, b; };
            U8 u = __builtin_bit_cast(U8, v);
            asm volatile("" : "+v"(u.a.x), "+v"(u.a.y), "+v"(u.a.z), "+v"(u.a.w));
            asm volatile("" : "+v"(u.b.x), "+v"(u.b.y), "+v"(u.b.z), "+v"(u.b.w));
            v = __builtin_bit_cast(vec, u);
        }
    };
    const int ntiles = it.k_end > it.k_begin ? (it.k_end - it.k_begin + KT - 1) / KT : 0;
    const int wave_last = wave_pos_max < it.k_begin ? -1 : imin(ntiles - 1, (wave_pos_max - it.k_begin) / KT);
    f32x4 sc[2][NS][2];      // scores of tile i (chunk, subtile, 16-key block)
    vec pb[2][NS];           // PV B operands: the probabilities of one tile, both chunks
#pragma unroll
    for (int ch = 0; ch < 2; ++ch)
#pragma unroll
        for (int s = 0; s < NS; ++s) pb[ch][s] = O::zero();

    // probability pair u (0..4 NS - 1) of chunk ch of tile i: subtile u / 4,
    // elements 2 (u % 4) and 2 (u % 4) + 1, packed into the PV operand
    auto prob_pair = [&](int ch, int u) {
        const int ps = u >> 2, j = (u & 3) * 2;
        O::set_pair(pb[ch][ps], j, fast_exp2(sc[ch][ps][j >> 2][j & 3]), fast_exp2(sc[ch][ps][(j + 1) >> 2][(j + 1) & 3]));
    };
    // S^T of one 64-key tile for the wave's columns (prologue: tile 0)
    auto scores = [&](const unsigned char *kl, f32x4 (&out)[2][NS][2]) {
#pragma unroll
        for (int ch = 0; ch < 2; ++ch)
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const int krow = ch * 32 + ks * 16 + lr;
#pragma unroll
                for (int s = 0; s < NS; ++s) out[ch][s][ks] = bias[s];
#pragma unroll
                for (int kc = 0; kc < KC; ++kc) {
                    const int d0 = kc * 32 + lg * 8;
                    const vec kv = (d0 < D) ? O::lds_load(kl + krow * RS + d0 * O::kBytes) : O::zero();
#pragma unroll
                    for (int s = 0; s < NS; ++s) out[ch][s][ks] = O::mma(kv, qop[s][kc], out[ch][s][ks]);
                }
            }
    };
    // PV of one 32-key chunk (outside the phases: a wave's last tile)
    auto pv_chunk = [&](const unsigned char *vl, int ch, const vec (&b)[NS]) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            const vec vt = O::vt_operand(vl, RS, ch * 32, nb * 16, lane);
#pragma unroll
            for (int s = 0; s < NS; ++s) acc[s][nb] = O::mma(vt, b[s], acc[s][nb]);
        }
#pragma unroll
        for (int s = 0; s < NS; ++s) acc[s][NB] = O::mma(ones, b[s], acc[s][NB]);
    };

    // Half of a matrix block: NSTEP = NB + 2 KC steps of NS MFMAs. PV steps
    // (NB of them: output block nb of chunk c of the V tile vl, B operand
    // pb[c]) and score steps (2 KC: (kc, ks) of chunk c of the K tile kl into
    // scn) are spread evenly, so the LDS reads of both kinds interleave; a
    // score accumulator is updated every other score step. Operands are read
    // from LDS two steps ahead; steps are fenced with sched_barrier so the
    // order holds. The all-ones row-sum MFMAs of the PV chunk close it.
    constexpr int NSTEP = NB + 2 * KC;
    auto half_block = [&](const unsigned char *vl, const unsigned char *kl, int c, f32x4 (&scn)[2][NS][2]) {
        // step g is a PV step iff the Bresenham count of PV steps grows at g
        auto is_pv = [](int g) { return ((g + 1) * NB) / NSTEP != (g * NB) / NSTEP; };
        auto pv_idx = [](int g) { return (g * NB) / NSTEP; };
        auto operand = [&](int g) -> vec {
            if (is_pv(g)) return O::vt_operand(vl, RS, c * 32, pv_idx(g) * 16, lane);
            const int q = g - pv_idx(g), kc = q >> 1, ks = q & 1;
            const int d0 = kc * 32 + lg * 8;
            return (d0 < D) ? O::lds_load(kl + (c * 32 + ks * 16 + lr) * RS + d0 * O::kBytes) : O::zero();
        };
        vec op[3];
        op[0] = operand(0);
        if (NSTEP > 1) op[1] = operand(1);
#pragma unroll
        for (int g = 0; g < NSTEP; ++g) {
            if (g + 2 < NSTEP) op[(g + 2) % 3] = operand(g + 2);
            if (is_pv(g)) {
                const int nb = pv_idx(g);
#pragma unroll
                for (int s = 0; s < NS; ++s) acc[s][nb] = O::mma(op[g % 3], pb[c][s], acc[s][nb]);
            } else {
                const int q = g - pv_idx(g), kc = q >> 1, ks = q & 1;
#pragma unroll
                for (int s = 0; s < NS; ++s) {
                    const f32x4 c0 = kc == 0 ? bias[s] : scn[c][s][ks];
                    scn[c][s][ks] = O::mma(op[g % 3], qop[s][kc], c0);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int s = 0; s < NS; ++s) acc[s][NB] = O::mma(ones, pb[c][s], acc[s][NB]);
    };
    // The softmax of tile i as one block of vector work: the column max of
    // the tile, the rescale decision (the reference max moves only when a
    // column's max outgrows it by more than kRescaleLog2; acc then holds every
    // PV product of the tiles before i), and the probabilities of both chunks
    // against the reference, packed into the PV operands pb. Each result is
    // pinned at the end of the block, so the block stays where it is placed
    // and its exponentials run while the other wave of the SIMD issues MFMAs.
    auto softmax_block = [&](int tile) {
        if ((tile + KT > it.k_end) || (tile + KT - 1 > wave_pos_min) || (tile <= wave_pos_max - a.window))
            mask(tile, sc);                              // uniform over the wave
        // the max of the lane's scores per subtile, relative to the reference
        // the scores carry
        float rel[NS];
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            float q4[4];
#pragma unroll
            for (int qq = 0; qq < 4; ++qq) {
                const f32x4 x = sc[qq >> 1][s][qq & 1];
                q4[qq] = smax(smax(smax(x[0], x[1]), x[2]), x[3]);
            }
            rel[s] = smax(smax(smax(q4[0], q4[1]), q4[2]), q4[3]);
        }
        // the reference moves (rarely) when a column's first keys arrive or its
        // max outgrows the reference by more than kRescaleLog2 (thr): acc,
        // holding every PV product of the tiles before, takes the factor, and
        // this tile's scores are taken against the new reference. A column's
        // max exceeds thr iff one of its lanes' maxima does, so the column
        // maxima are only formed when some lane's does.
        bool moves = false;
#pragma unroll
        for (int s = 0; s < NS; ++s) moves |= rel[s] > thr[s];
        if (__builtin_amdgcn_ballot_w64(moves)) {        // uniform over the wave
#pragma unroll
            for (int s = 0; s < NS; ++s) {
                float shift = 0.f;
                rel[s] = wave_max_across_groups(rel[s]);
                if (rel[s] > thr[s]) {
                    const float m_new = (st[s].m == -INFINITY ? 0.f : st[s].m) + rel[s];
                    const float alpha = fast_exp2(st[s].m - m_new);  // st.m = -inf: 0 (acc is still 0)
#pragma unroll
                    for (int nb = 0; nb <= NB; ++nb) acc[s][nb] *= alpha;
                    st[s].m = m_new;
                    thr[s] = kRescaleLog2;
                    shift = rel[s];
                    bias[s] = f32x4{-m_new, -m_new, -m_new, -m_new};
                }
#pragma unroll
                for (int q = 0; q < 4; ++q) sc[q >> 1][s][q & 1] -= shift;
            }
        }
#pragma unroll
        for (int ch = 0; ch < 2; ++ch)
#pragma unroll
            for (int u = 0; u < 4 * NS; ++u) prob_pair(ch, u);
#pragma unroll
        for (int ch = 0; ch < 2; ++ch)
#pragma unroll
            for (int s = 0; s < NS; ++s) pin(pb[ch][s]);
        __builtin_amdgcn_sched_barrier(0);
    };
    // The matrix block: PV of both chunks of the V tile vl with pb, and the
    // scores of both chunks of the K tile kl into scn.
    auto matrix_block = [&](const unsigned char *vl, const unsigned char *kl, f32x4 (&scn)[2][NS][2]) {
        half_block(vl, kl, 0, scn);
        half_block(vl, kl, 1, scn);
        __builtin_amdgcn_sched_barrier(0);
    };

    int64_t row_next = 0;                              // cache row of tile i + 1
    if (ntiles > 0) {
        // K(0), V(0) and K(1) go out together: one round trip to memory
        // before the first tile, not two (a short item is mostly this)
        const int64_t row0 = tile_row(it.k_begin);
        uint4 k0[PCH];
        load(k0, kbase, row0, it.k_begin);
        load(vreg, vbase, row0, it.k_begin);
        if (ntiles > 1) {
            row_next = tile_row(it.k_begin + KT);
            load(kreg, kbase, row_next, it.k_begin + KT);
        }
        scale_q();
        store(k0, lds_k[0]);
        __syncthreads();
        if (!grp_a && wave_last >= 0) scores(lds_k[0], sc);   // group A computes them in its first step
    }
    int sl = 0;                                        // slot of K(i) and V(i): i % SL
    for (int i = 0; i < ntiles; ++i) {
        const int tile = it.k_begin + i * KT;
        const bool has_next = i + 1 < ntiles;          // uniform over the work group
        const int sn = sl == SL - 1 ? 0 : sl + 1, sp = sl == 0 ? SL - 1 : sl - 1;
        if (has_next) store(kreg, lds_k[sn]);          // K(i+1)
        store(vreg, lds_v[sl]);                        // V(i)
        // the registers are free again: the next loads go out before the
        // barrier, so they have the barrier wait as well as one iteration
        int64_t row_k2 = 0;
        if (i + 2 < ntiles) {
            row_k2 = tile_row(tile + 2 * KT);
            load(kreg, kbase, row_k2, tile + 2 * KT);
        }
        if (has_next) load(vreg, vbase, row_next, tile + KT);
        row_next = row_k2;
        __syncthreads();
        const int cur = sl;
        sl = sn;
        if (i > wave_last) {
            // group A still owes the PV of its last computed tile
            if (grp_a && i == wave_last + 1 && wave_last >= 0) {
                pv_chunk(lds_v[sp], 0, pb[0]);
                pv_chunk(lds_v[sp], 1, pb[1]);
            }
            continue;
        }
        // group B: the softmax of tile i (its scores came with the previous
        // iteration), then PV of tile i and the scores of tile i+1. Group A:
        // PV of tile i-1 and the scores of tile i, then the softmax of tile i.
        // The matrix block is one piece of code for both groups. Tile 0 has no
        // predecessor: group A's pb is still zero then, and V(0) (finite,
        // already staged) stands in for V(-1), so those products add nothing.
        if (!grp_a) softmax_block(tile);
        __builtin_amdgcn_s_setprio(1);
        // the V slot of group A's PV: V(i-1), or V(0) for tile 0; the choice is
        // hidden from the optimizer, which would otherwise peel iteration 0
        // into a second copy of the loop body
        int va = __builtin_amdgcn_readfirstlane(i > 0 ? sp : cur);
        asm volatile("" : "+s"(va));
        matrix_block(grp_a ? lds_v[va] : lds_v[cur], grp_a ? lds_k[cur] : lds_k[sn], sc);
        __builtin_amdgcn_s_setprio(0);
        if (grp_a) softmax_block(tile);
    }
    // group A: the PV of the last tile (V(last) was staged in the last
    // iteration, before its barrier)
    if (grp_a && ntiles > 0 && wave_last == ntiles - 1) {
        const int last = (ntiles - 1) % SL;
        pv_chunk(lds_v[last], 0, pb[0]);
        pv_chunk(lds_v[last], 1, pb[1]);
    }

#pragma unroll
    for (int s = 0; s < NS; ++s) {
        const float l = acc[s][NB][0];
        const int col = wave * WC + s * 16 + lr;
        if (pos[s] < 0) continue;
        if (it.rec0 < 0) {
            E *op = column_out<E>(a, it, col, D);
            const float inv = l > 0.f ? out_c / l : 0.f;
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) O::store4(op + nb * 16 + lg * 4, acc[s][nb] * inv);
        } else {
            const int64_t rec = it.rec0 + col;
            float *ap = a.ws_acc + rec * D;
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
                *reinterpret_cast<float4 *>(ap + nb * 16 + lg * 4) =
                    make_float4(acc[s][nb][0] * out_c, acc[s][nb][1] * out_c, acc[s][nb][2] * out_c,
                                acc[s][nb][3] * out_c);
            if (lg == 0) *reinterpret_cast<float2 *>(a.ws_ml + rec * 2) = make_float2(st[s].m, l);
        }
    }
}

// ---------------------------------------------------------------------------
// ---------------------------------------------------------------------------
// zero fill: +0.0 into every padded slot t >= n_new[b] (and every slot of a
// row with no new tokens). [GQA] "A strong answer": such rows give zeros,
// never NaN. Each block clears one 16 KiB slice of a (row, query head) region
// [0, T) x d, clipped to the padded part; 16-byte stores, 4 per thread.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void zero_fill_kernel(ZeroArgs a) {
    const int slice = blockIdx.x % a.slices;
    const int rh = blockIdx.x / a.slices;
    const int r = rh / a.hq;
    const int h = rh % a.hq;
    const int b = a.rows.b[r];
    const int n = a.rows.nnew[r];
    const int64_t head_off = ((int64_t)b * a.hq + h) * a.T * a.row_bytes;
    const int64_t lo = (int64_t)slice * kZeroSlice;
    const int64_t begin = head_off + (lo > (int64_t)n * a.row_bytes ? lo : (int64_t)n * a.row_bytes);
    const int64_t hi = lo + kZeroSlice;
    const int64_t end = head_off + (hi < (int64_t)a.T * a.row_bytes ? hi : (int64_t)a.T * a.row_bytes);
    char *out = reinterpret_cast<char *>(a.out);
#pragma unroll
    for (int j = 0; j < kZeroSlice / (256 * 16); ++j) {
        const int64_t off = head_off + lo + (j * 256 + threadIdx.x) * 16;
        if (off >= begin && off < end) *reinterpret_cast<uint4 *>(out + off) = make_uint4(0, 0, 0, 0);
    }
}

// ---------------------------------------------------------------------------
// combine: for rows split across work groups, merge the nsplit partials of
// every column by log-sum-exp in split order, normalise and cast. One thread
// per (column, 4 outputs) of a (row, kv head, query tile); loads of 8 splits
// are issued together.
// ---------------------------------------------------------------------------
template <typename E, int D>
__global__ __launch_bounds__(256) void combine_kernel(CombineArgs a) {
    using O = Op<E>;
    constexpr int DC = D / 4;
    const int nrow = a.rows.n_rows;
    const int first = lane_entry(a.rows.blk0, nrow, 0x7fffffff);
    const int r = wave_find_row(first, blockIdx.x);
    const int local = blockIdx.x - row_entry(first, r);
    const int cols = row_entry(lane_entry(a.rows.cols, nrow, 16), r);
    const int nsplit = row_entry(lane_entry(a.rows.nsplit, nrow, 1), r);
    const int n = row_entry(lane_entry(a.rows.nnew, nrow, 0), r);
    const int tq = cols / a.group;
    const int nq = (n + tq - 1) / tq;
    const int per_group = (cols * DC + 255) / 256;   // blocks per (kv head, query tile)
    const int grp = local / per_group, part = local % per_group;
    const int kvh = grp / nq, qtile = grp % nq;
    const int b = row_entry(lane_entry(a.rows.b, nrow, 0), r);
    const int64_t rec_first = row_entry(lane_entry(a.rows.pbase, nrow, 0), r) +
                              (int64_t)((kvh * nq + qtile) * nsplit) * cols;
    const int task = part * 256 + threadIdx.x;       // one (column, 4 outputs) per thread
    if (task >= cols * DC) return;
    const int col = task / DC, d = (task % DC) * 4;
    const int t = qtile * tq + col / a.group;
    if (col >= tq * a.group || t >= n) return;
    const int h = kvh * a.group + col % a.group;
    const int64_t rec = rec_first + col;
    E *op = reinterpret_cast<E *>(a.out) + (((int64_t)b * a.hq + h) * a.T + t) * D + d;
    O::store4(op, merge_partials<D>(a.ws_acc, a.ws_ml, rec, cols, nsplit, d));
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
hipError_t launch_append(const AppendArgs &a, int n_blocks, hipStream_t s) {
    if (n_blocks <= 0) return hipSuccess;
    hipLaunchKernelGGL(append_kernel, dim3(n_blocks), dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_set_lens(int32_t *lens_dev, const LensTable &t, hipStream_t s) {
    if (t.n_rows <= 0) return hipSuccess;
    hipLaunchKernelGGL(set_lens_kernel, dim3(1), dim3(64), 0, s, lens_dev, t);
    return hipGetLastError();
}

hipError_t launch_table_set(const TableArgs &a, hipStream_t s) {
    if (a.n <= 0) return hipSuccess;
    hipLaunchKernelGGL(table_set_kernel, dim3((a.n + 255) / 256), dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_table_fill(int32_t *table, int64_t n, int32_t value, hipStream_t s) {
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(table_fill_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, table, n, value);
    return hipGetLastError();
}

hipError_t launch_zero_bytes(void *p, int64_t bytes, hipStream_t s) {
    const int64_t n16 = bytes / 16;
    if (n16 <= 0) return hipSuccess;
    // at most 8,192 blocks of 256 threads; each thread stores 16 bytes per pass
    const int64_t blocks = std::min<int64_t>(8192, (n16 + 255) / 256);
    hipLaunchKernelGGL(zero_bytes_kernel, dim3((unsigned)blocks), dim3(256), 0, s, reinterpret_cast<uint4 *>(p), n16);
    return hipGetLastError();
}

// dtype codes (kv_dtype): 0 float32, 1 bfloat16, 2 E4M3 cache with bfloat16 q/out
template <typename E, int D, bool F8, bool PG>
static hipError_t decode_d(int nsub, const AttnArgs &a, hipStream_t s) {
    constexpr int W = kDecodeWaves;
    const dim3 grid(a.rows.total_items), block(64 * W);
    switch (nsub) {
        case 1: hipLaunchKernelGGL((decode_kernel<E, D, 1, W, F8, PG>), grid, block, 0, s, a); break;
        case 2:
            // float32 at d = 128: two subtiles need more registers than two
            // waves per SIMD leave a wave; one wave per SIMD
            if constexpr (std::is_same<E, float>::value && D == 128)
                hipLaunchKernelGGL((decode_kernel<E, D, 2, 4, F8, PG>), grid, dim3(256), 0, s, a);
            else
                hipLaunchKernelGGL((decode_kernel<E, D, 2, W, F8, PG>), grid, block, 0, s, a);
            break;
        case 4:
            // four subtiles over rows of 256 bytes or more (in the compute type)
            // need more registers than two waves per SIMD leave a wave, and
            // spilled heavily: their work groups are 4 waves at one per SIMD
            if constexpr (D * sizeof(E) >= 256)
                hipLaunchKernelGGL((decode_kernel<E, D, 4, 4, F8, PG>), grid, dim3(256), 0, s, a);
            else
                hipLaunchKernelGGL((decode_kernel<E, D, 4, W, F8, PG>), grid, block, 0, s, a);
            break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <typename E, bool F8, bool PG>
static hipError_t decode_e(int head_dim, int nsub, const AttnArgs &a, hipStream_t s) {
    switch (head_dim) {
        case 16: return decode_d<E, 16, F8, PG>(nsub, a, s);
        case 32: return decode_d<E, 32, F8, PG>(nsub, a, s);
        case 64: return decode_d<E, 64, F8, PG>(nsub, a, s);
        case 128: return decode_d<E, 128, F8, PG>(nsub, a, s);
        default: return hipErrorInvalidValue;
    }
}

// paged caches hold float32 or bfloat16 (dtype 0 or 1)
hipError_t launch_decode(int dtype, int head_dim, int nsub, const AttnArgs &a, hipStream_t s) {
    if (a.rows.total_items <= 0) return hipSuccess;
    const bool pg = a.table != nullptr;
    switch (dtype) {
        case 0: return pg ? decode_e<float, false, true>(head_dim, nsub, a, s)
                          : decode_e<float, false, false>(head_dim, nsub, a, s);
        case 1: return pg ? decode_e<bf16_t, false, true>(head_dim, nsub, a, s)
                          : decode_e<bf16_t, false, false>(head_dim, nsub, a, s);
        case 2: return pg ? hipErrorInvalidValue : decode_e<bf16_t, true, false>(head_dim, nsub, a, s);
        default: return hipErrorInvalidValue;
    }
}

template <typename E, int D, bool F8, bool PG>
static void prefill_d(const AttnArgs &a, hipStream_t s) {
    constexpr int dt = std::is_same<E, float>::value ? 0 : 1;
    constexpr int PW = prefill_waves(dt, D), NS = prefill_subtiles(dt, D);
    hipLaunchKernelGGL((prefill_kernel<E, D, F8, PG, PW, NS>), dim3(a.rows.total_items), dim3(64 * PW), 0, s, a);
}

template <typename E, bool F8, bool PG>
static hipError_t prefill_e(int head_dim, const AttnArgs &a, hipStream_t s) {
    switch (head_dim) {
        case 16: prefill_d<E, 16, F8, PG>(a, s); break;
        case 32: prefill_d<E, 32, F8, PG>(a, s); break;
        case 64: prefill_d<E, 64, F8, PG>(a, s); break;
        case 128: prefill_d<E, 128, F8, PG>(a, s); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_prefill(int dtype, int head_dim, const AttnArgs &a, hipStream_t s) {
    if (a.rows.total_items <= 0) return hipSuccess;
    const bool pg = a.table != nullptr;
    switch (dtype) {
        case 0: return pg ? prefill_e<float, false, true>(head_dim, a, s) : prefill_e<float, false, false>(head_dim, a, s);
        case 1: return pg ? prefill_e<bf16_t, false, true>(head_dim, a, s)
                          : prefill_e<bf16_t, false, false>(head_dim, a, s);
        case 2: return pg ? hipErrorInvalidValue : prefill_e<bf16_t, true, false>(head_dim, a, s);
        default: return hipErrorInvalidValue;
    }
}

template <typename E>
static hipError_t combine_e(int head_dim, const CombineArgs &a, hipStream_t s) {
    const dim3 grid(a.rows.total_blocks), block(256);
    switch (head_dim) {
        case 16: hipLaunchKernelGGL((combine_kernel<E, 16>), grid, block, 0, s, a); break;
        case 32: hipLaunchKernelGGL((combine_kernel<E, 32>), grid, block, 0, s, a); break;
        case 64: hipLaunchKernelGGL((combine_kernel<E, 64>), grid, block, 0, s, a); break;
        case 128: hipLaunchKernelGGL((combine_kernel<E, 128>), grid, block, 0, s, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_combine(int dtype, int head_dim, const CombineArgs &a, hipStream_t s) {
    if (a.rows.total_blocks <= 0) return hipSuccess;
    return dtype == 0 ? combine_e<float>(head_dim, a, s) : combine_e<bf16_t>(head_dim, a, s);
}

hipError_t side_stream_init(SideStream &s) {
    if (s.side != nullptr) return hipSuccess;
    hipError_t e = hipStreamCreateWithFlags(&s.side, hipStreamNonBlocking);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&s.fork_ev, hipEventDisableTiming);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&s.join_ev, hipEventDisableTiming);
    if (e != hipSuccess) side_stream_destroy(s);
    return e;
}

void side_stream_destroy(SideStream &s) {
    if (s.fork_ev) (void)hipEventDestroy(s.fork_ev);
    if (s.join_ev) (void)hipEventDestroy(s.join_ev);
    if (s.side) (void)hipStreamDestroy(s.side);
    s = SideStream{};
}

hipError_t side_stream_fork(SideStream &s, hipStream_t main) {
    hipError_t e = hipEventRecord(s.fork_ev, main);
    return e == hipSuccess ? hipStreamWaitEvent(s.side, s.fork_ev, 0) : e;
}

hipError_t side_stream_join(SideStream &s, hipStream_t main) {
    hipError_t e = hipEventRecord(s.join_ev, s.side);
    return e == hipSuccess ? hipStreamWaitEvent(main, s.join_ev, 0) : e;
}

hipError_t launch_zero_fill(const ZeroArgs &a, hipStream_t s) {
    if (a.rows.n_rows <= 0 || a.hq <= 0) return hipSuccess;
    hipLaunchKernelGGL(zero_fill_kernel, dim3(a.rows.n_rows * a.hq * a.slices), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace gqakv
