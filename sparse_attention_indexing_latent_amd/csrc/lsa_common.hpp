// Shared device-side definitions of the LSA HIP kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/lsa.h"

namespace lsa {

constexpr int kLatent = LSA_LATENT_DIM;           // 64
constexpr int kPool = LSA_POOL;                   // 4
constexpr int kBlockEntries = LSA_BLOCK_ENTRIES;  // 512
constexpr int kBlockTokens = LSA_BLOCK_TOKENS;    // 2048
constexpr int kLeavesPerBlock = LSA_LEAVES_PER_BLOCK;
constexpr int kMaxBucket = LSA_MAX_BUCKET;
constexpr int kMaxGroup = LSA_MAX_GROUP;
constexpr int kMaxLevels = 40;
constexpr int kCandCap = 512;      // candidates per (query, KV head) the fused flat search sorts
constexpr int kCandStride = 1024;  // candidate list slots per (query, KV head) in the fused flat search
constexpr int kSubCap = kCandStride / 4;   // the list is 4 sub-lists of this many slots
constexpr int kFullTake = 0xFFFF;  // "every eligible token of this bucket"

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------- cache view
// Device pointers of one bucket cache; strides are element counts between
// consecutive (b, g) slices.
struct CacheView {
    void* cent;            // [B, H_kv, leaves_max, 64]  dtype
    float* sums;           // [B, H_kv, leaves_max, 64]  fp32
    uint32_t* meta;        // [B, H_kv, leaves_max]      size | first-member offset << 8
    uint16_t* members;     // [B, H_kv, n_blocks_max, 512]
    uint8_t* eleaf;        // [B, H_kv, n_blocks_max, 512]
    void* tcent;           // [B, H_kv, nodes_max, 64]   dtype (tree levels >= 1)
    float* tsums;          // [B, H_kv, nodes_max, 64]
    uint8_t* epos;         // [B, H_kv, n_blocks_max, 512] position of each entry in its bucket's member list
    void* edge;            // [B, H_kv, n_blocks_max + 1, n_lev_cap, 64] dtype: node straddling 64 nb leaves
    int8_t* cq;            // bf16 only: [B, H_kv, leaves_max / 16 tiles, 1 KB] int8 codes of the centroids
    float* csc;            // bf16 only: [B, H_kv, leaves_max] their scales
    int64_t s_cent, s_sums, s_meta, s_members, s_eleaf, s_tcent, s_tsums, s_epos, s_edge, s_cq, s_csc;
    int32_t n_blocks;      // full blocks bucketed
    int32_t n_leaves;
    int32_t n_levels;      // tree levels including the leaves
    int32_t bf16;          // centroid storage dtype
    int32_t n_leaves_cap;  // leaves_max: the tree levels are laid out for it
    int32_t n_lev_cap;     // levels of a tree over leaves_max leaves (edge table rows)
};

// bf16 leaf centroids are stored in tiles of 16 buckets (2 KB, 1024
// elements) in the operand order of the scoring MFMA: element dim of bucket
// `leaf` sits at tile * 1024 + m * 512 + (r + 16 h) * 8 + e, with r = leaf %
// 16, h = dim / 16, m = (dim / 8) % 2, e = dim % 8.  Lane l = r + 16 h of a
// wave then reads its two 8-element k-steps of a tile as the 16-byte words
// l and 64 + l, so each load instruction covers 1 KB contiguously.
// (fp32 centroids and the tree levels above the leaves stay row-major.)
__device__ __forceinline__ int64_t cent_tile_word(int64_t leaf, int h, int m) {
    return (leaf >> 4) * 128 + m * 64 + (leaf & 15) + 16 * h;   // 16-byte word index
}

// Tree level l >= 1 holds ceil(n_leaves / 2^l) nodes (pairing (2j, 2j+1) level
// by level); levels are stored one after the other from level 1, each with
// room for the nodes over leaves_max leaves, so a node keeps its place as the
// cache grows (tree_level_off takes leaves_max).
__device__ __forceinline__ int64_t tree_level_size(int64_t n_leaves, int lev) {
    return (n_leaves + ((int64_t)1 << lev) - 1) >> lev;
}
__device__ __forceinline__ int64_t tree_level_off(int64_t n_leaves, int lev) {
    int64_t off = 0;
    for (int i = 1; i < lev; ++i) off += tree_level_size(n_leaves, i);
    return off;
}

// ---------------------------------------------------------------- numerics
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float(((uint32_t)h) << 16); }

// Round to nearest even (inputs here are finite).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// Maximum without the canonicalisation fmaxf needs (v_maximum3_f32 on gfx950; a NaN operand gives NaN,
// which the scores and outputs here never hold), and 2^x as the bare hardware instruction (results
// below 2^-126 flush to 0: softmax weights that small never matter).
__device__ __forceinline__ float fmax_nc(float a, float b) { return __builtin_elementwise_maximum(a, b); }
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

template <typename T> __device__ __forceinline__ float load_f32(const T* p);
template <> __device__ __forceinline__ float load_f32<float>(const float* p) { return *p; }
template <> __device__ __forceinline__ float load_f32<uint16_t>(const uint16_t* p) { return bf16_to_f32(*p); }

// Monotone map float -> uint32 (larger float -> larger key); -0 folded into +0.
__device__ __forceinline__ uint32_t ord_key(float f) {
    uint32_t u = __float_as_uint(f + 0.0f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float ord_key_inv(uint32_t k) {
    uint32_t u = (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
    return __uint_as_float(u);
}
// Ranking key of a bucket: score descending, then id ascending.
__device__ __forceinline__ uint64_t rank_key(float score, uint32_t id) {
    return ((uint64_t)ord_key(score) << 32) | (uint64_t)(0xFFFFFFFFu - id);
}
__device__ __forceinline__ uint32_t rank_key_id(uint64_t k) { return 0xFFFFFFFFu - (uint32_t)(k & 0xFFFFFFFFu); }

// ---------------------------------------------------------------- wave helpers (wave64)
__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
    return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    return v;
}
__device__ __forceinline__ int wave_max_i(int v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = max(v, __shfl_xor(v, o));
    return v;
}
__device__ __forceinline__ int wave_min_i(int v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = min(v, __shfl_xor(v, o));
    return v;
}
__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int o) {
    uint32_t lo = (uint32_t)v, hi = (uint32_t)(v >> 32);
    lo = __shfl_xor(lo, o);
    hi = __shfl_xor(hi, o);
    return ((uint64_t)hi << 32) | lo;
}
__device__ __forceinline__ uint64_t shfl_u64(uint64_t v, int src) {
    uint32_t lo = (uint32_t)v, hi = (uint32_t)(v >> 32);
    lo = __shfl(lo, src);
    hi = __shfl(hi, src);
    return ((uint64_t)hi << 32) | lo;
}
__device__ __forceinline__ uint64_t wave_min_u64(uint64_t v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
        uint64_t w = shfl_xor_u64(v, o);
        v = w < v ? w : v;
    }
    return v;
}
// Inclusive prefix sum over the wave.
__device__ __forceinline__ int wave_incl_scan(int v) {
    const int l = lane_id();
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        int w = __shfl_up(v, o);
        if (l >= o) v += w;
    }
    return v;
}

// ---------------------------------------------------------------- device-coherent accesses
// Data one workgroup hands to another within a kernel goes through relaxed
// agent-scope atomic stores and loads: on gfx950 they carry the system-
// coherence bit, so they are visible across the XCDs' separate L2 caches
// without the full L2 write-back and invalidate that an agent-scope fence
// costs.  The writer waits for its stores to complete (s_waitcnt) before the
// atomic that signals the reader; the reader's loads issue after it has seen
// that atomic.
__device__ __forceinline__ void store_coherent_u64(void* p, uint64_t v) {
    __hip_atomic_store(reinterpret_cast<uint64_t*>(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_coherent_u32(void* p, uint32_t v) {
    __hip_atomic_store(reinterpret_cast<uint32_t*>(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t load_coherent_u64(const void* p) {
    return __hip_atomic_load(reinterpret_cast<uint64_t*>(const_cast<void*>(p)), __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t load_coherent_u32(const void* p) {
    return __hip_atomic_load(reinterpret_cast<uint32_t*>(const_cast<void*>(p)), __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_coherent_f32(const float* p) { return __uint_as_float(load_coherent_u32(p)); }
__device__ __forceinline__ uint64_t pack_f32x2(float a, float b) {
    return (uint64_t)__float_as_uint(a) | ((uint64_t)__float_as_uint(b) << 32);
}
// Wait until every memory access this wave issued has completed.
__device__ __forceinline__ void wait_all_memory() {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// ---------------------------------------------------------------- query geometry
// nvis selectable blocks, sinks [0, sink_end), local window [l0, t];
// eligible long-range tokens are [sink_end, l0).
struct Geom {
    int64_t t;
    int32_t nvis;
    int64_t sink_end;
    int64_t l0;
};
__device__ __forceinline__ Geom query_geom(int64_t t, int32_t n_blocks, int32_t n_sinks, int32_t window) {
    Geom G;
    G.t = t;
    int64_t bq = t / kBlockTokens;
    G.nvis = (int32_t)(bq < n_blocks ? bq : n_blocks);
    G.sink_end = (int64_t)n_sinks < t + 1 ? (int64_t)n_sinks : t + 1;
    int64_t lw = t - (int64_t)window + 1;
    int64_t lb = (int64_t)kBlockTokens * G.nvis;
    int64_t l0 = lw < lb ? lw : lb;
    G.l0 = l0 > 0 ? l0 : 0;
    return G;
}

// The member entries of one bucket (<= 16, ascending, starting at entry
// `off` of the block's member array) as 16-bit values in registers: the
// aligned 48-byte window holding them is read with three 16-byte loads (none
// past the block's 512 entries) and shifted into place.
__device__ __forceinline__ void load_members(const uint16_t* blk_members, int off, uint16_t (&e)[16]) {
    const int a = off & ~7;
    const uint4* p = reinterpret_cast<const uint4*>(blk_members + a);
    const uint4 z = {0, 0, 0, 0};
    const uint4 w0 = p[0], w1 = (a + 8 < kBlockEntries) ? p[1] : z, w2 = (a + 16 < kBlockEntries) ? p[2] : z;
    const uint32_t w[12] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w, w2.x, w2.y, w2.z, w2.w};
    const int sh = off - a;        // 0..7 entries
    const int s2 = sh >> 1;        // whole 32-bit words to skip
    uint32_t ww[9];
#pragma unroll
    for (int m = 0; m < 9; ++m)
        ww[m] = s2 == 0 ? w[m] : (s2 == 1 ? w[m + 1] : (s2 == 2 ? w[m + 2] : w[m + 3]));
#pragma unroll
    for (int m = 0; m < 8; ++m) {
        const uint32_t v = (sh & 1) ? __builtin_amdgcn_alignbit(ww[m + 1], ww[m], 16) : ww[m];
        e[2 * m] = (uint16_t)(v & 0xFFFFu);
        e[2 * m + 1] = (uint16_t)(v >> 16);
    }
}

// Eligible tokens of one bucket: its tokens in [sink_end, l0).  m is the
// bucket's meta word (size | first-member offset << 8).
__device__ __forceinline__ int leaf_weight_m(const CacheView& cv, int64_t bg, uint32_t leaf, uint32_t m,
                                             const Geom& q) {
    const int blk = leaf / kLeavesPerBlock;
    const int64_t lo = (int64_t)blk * kBlockTokens, hi = lo + kBlockTokens;
    const int sz = m & 0xFF;
    if (lo >= q.sink_end && hi <= q.l0) return kPool * sz;
    if (hi <= q.sink_end || lo >= q.l0) return 0;
    uint16_t e[16];
    load_members(cv.members + bg * cv.s_members + (int64_t)blk * kBlockEntries, (m >> 8) & 0x3FF, e);
    int w = 0;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        const int64_t t0 = lo + (int64_t)e[j] * kPool;
#pragma unroll
        for (int jj = 0; jj < kPool; ++jj) w += (j < sz && t0 + jj >= q.sink_end && t0 + jj < q.l0) ? 1 : 0;
    }
    return w;
}
__device__ __forceinline__ int leaf_weight(const CacheView& cv, int64_t bg, uint32_t leaf, const Geom& q) {
    return leaf_weight_m(cv, bg, leaf, cv.meta[bg * cv.s_meta + leaf], q);
}

}  // namespace lsa
