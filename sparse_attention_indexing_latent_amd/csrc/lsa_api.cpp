// C ABI of the LSA hot path: argument validation, cache and workspace
// layouts, and kernel launches on the caller's stream.  See include/lsa.h.

#include <hip/hip_runtime.h>

#include <atomic>
#include <chrono>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>

#include "../../include/lsa.h"
#include "lsa_launch.hpp"

namespace {

thread_local std::string g_err;

lsa_status fail(lsa_status s, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_err = buf;
    return s;
}

lsa_status ok() {
    g_err.clear();
    return LSA_OK;
}

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

bool misaligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) != 0; }

lsa_status check_layout(const lsa_layout* L) {
    if (!L) return fail(LSA_ERR_INVALID_ARG, "layout is NULL");
    if (L->latent_dim != LSA_LATENT_DIM) return fail(LSA_ERR_SHAPE, "latent_dim must be %d", LSA_LATENT_DIM);
    if (L->pool != LSA_POOL) return fail(LSA_ERR_SHAPE, "pool must be %d", LSA_POOL);
    if (L->block_entries != LSA_BLOCK_ENTRIES) return fail(LSA_ERR_SHAPE, "block_entries must be %d", LSA_BLOCK_ENTRIES);
    if (L->mean_bucket != LSA_MEAN_BUCKET) return fail(LSA_ERR_SHAPE, "mean_bucket must be %d", LSA_MEAN_BUCKET);
    if (L->max_bucket != LSA_MAX_BUCKET) return fail(LSA_ERR_SHAPE, "max_bucket must be %d", LSA_MAX_BUCKET);
    if (L->head_dim != 64 && L->head_dim != 128) return fail(LSA_ERR_SHAPE, "head_dim must be 64 or 128, got %d", L->head_dim);
    if (L->n_kv_heads < 1 || L->n_q_heads < 1) return fail(LSA_ERR_SHAPE, "head counts must be >= 1");
    if (L->n_q_heads % L->n_kv_heads != 0) return fail(LSA_ERR_SHAPE, "n_q_heads must be a multiple of n_kv_heads");
    if (L->n_q_heads / L->n_kv_heads > LSA_MAX_GROUP)
        return fail(LSA_ERR_SHAPE, "group size %d exceeds %d", L->n_q_heads / L->n_kv_heads, LSA_MAX_GROUP);
    if (L->dtype != LSA_F32 && L->dtype != LSA_BF16) return fail(LSA_ERR_DTYPE, "dtype must be LSA_F32 or LSA_BF16");
    if (L->build_tree != 0 && L->build_tree != 1) return fail(LSA_ERR_INVALID_ARG, "build_tree must be 0 or 1");
    return LSA_OK;
}

struct CacheGeom {
    int64_t nbm, nlm, nnm;
    int64_t n_blocks, n_leaves;
    int32_t n_levels;
    int32_t elt;
    int64_t level_off[lsa::kMaxLevels];
    int64_t level_size[lsa::kMaxLevels];
    int32_t n_lev_cap;   // levels of a tree over leaves_max leaves
    size_t s_cent, s_sums, s_meta, s_members, s_eleaf, s_tcent, s_tsums, s_epos, s_edge, s_cq, s_csc;   // per (b, g)
    size_t off_cent, off_sums, off_meta, off_members, off_eleaf, off_tcent, off_tsums, off_epos, off_edge, off_cq,
        off_csc, total;
};

int64_t tree_nodes_above(int64_t nl) {
    int64_t tot = 0;
    while (nl > 1) {
        nl = (nl + 1) / 2;
        tot += nl;
    }
    return tot;
}

void cache_geom(const lsa_layout* L, int64_t B, int64_t t_max, int64_t T, CacheGeom& c) {
    memset(&c, 0, sizeof(c));
    c.elt = L->dtype == LSA_BF16 ? 2 : 4;
    c.nbm = t_max / LSA_BLOCK_TOKENS;
    c.nlm = c.nbm * LSA_LEAVES_PER_BLOCK;
    c.nnm = L->build_tree ? tree_nodes_above(c.nlm) : 0;
    c.n_lev_cap = 1;
    for (int64_t nl = c.nlm; nl > 1; nl = (nl + 1) / 2) ++c.n_lev_cap;
    c.n_blocks = T / LSA_BLOCK_TOKENS;
    c.n_leaves = c.n_blocks * LSA_LEAVES_PER_BLOCK;
    if (c.n_leaves > 0) {
        // sizes from the current leaves, offsets from the capacity (stable as the cache grows)
        int64_t nl = c.n_leaves, ncap = c.nlm, off = 0;
        int lev = 0;
        c.level_size[0] = nl;
        c.level_off[0] = 0;
        while (nl > 1 && lev + 1 < lsa::kMaxLevels) {
            nl = (nl + 1) / 2;
            ncap = (ncap + 1) / 2;
            ++lev;
            c.level_off[lev] = off;
            c.level_size[lev] = nl;
            off += ncap;
        }
        c.n_levels = lev + 1;
    }
    const int64_t HB = B * L->n_kv_heads;
    c.s_cent = align256((size_t)c.nlm * LSA_LATENT_DIM * c.elt);
    c.s_sums = align256((size_t)c.nlm * LSA_LATENT_DIM * 4);
    c.s_meta = align256((size_t)c.nlm * 4);
    c.s_members = align256((size_t)c.nbm * LSA_BLOCK_ENTRIES * 2);
    c.s_eleaf = align256((size_t)c.nbm * LSA_BLOCK_ENTRIES);
    c.s_tcent = align256((size_t)c.nnm * LSA_LATENT_DIM * c.elt);
    c.s_tsums = align256((size_t)c.nnm * LSA_LATENT_DIM * 4);
    c.s_epos = align256((size_t)c.nbm * LSA_BLOCK_ENTRIES);
    c.s_edge = L->build_tree ? align256((size_t)(c.nbm + 1) * c.n_lev_cap * LSA_LATENT_DIM * c.elt) : 0;
    c.s_cq = L->dtype == LSA_BF16 ? align256((size_t)c.nlm * LSA_LATENT_DIM) : 0;   // int8 codes
    c.s_csc = L->dtype == LSA_BF16 ? align256((size_t)c.nlm * 4) : 0;              // fp32 scales
    size_t o = 0;
    c.off_cent = o;    o += c.s_cent * HB;
    c.off_sums = o;    o += c.s_sums * HB;
    c.off_meta = o;    o += c.s_meta * HB;
    c.off_members = o; o += c.s_members * HB;
    c.off_eleaf = o;   o += c.s_eleaf * HB;
    c.off_tcent = o;   o += c.s_tcent * HB;
    c.off_tsums = o;   o += c.s_tsums * HB;
    c.off_epos = o;    o += c.s_epos * HB;
    c.off_edge = o;    o += c.s_edge * HB;
    c.off_cq = o;      o += c.s_cq * HB;
    c.off_csc = o;     o += c.s_csc * HB;
    c.total = o > 0 ? o : 256;
}

lsa::CacheView make_view(const CacheGeom& c, void* cache, bool bf16) {
    lsa::CacheView v;
    memset(&v, 0, sizeof(v));
    char* base = static_cast<char*>(cache);
    v.cent = base + c.off_cent;
    v.sums = reinterpret_cast<float*>(base + c.off_sums);
    v.meta = reinterpret_cast<uint32_t*>(base + c.off_meta);
    v.members = reinterpret_cast<uint16_t*>(base + c.off_members);
    v.eleaf = reinterpret_cast<uint8_t*>(base + c.off_eleaf);
    v.tcent = base + c.off_tcent;
    v.tsums = reinterpret_cast<float*>(base + c.off_tsums);
    v.epos = reinterpret_cast<uint8_t*>(base + c.off_epos);
    v.edge = base + c.off_edge;
    v.cq = reinterpret_cast<int8_t*>(base + c.off_cq);
    v.csc = reinterpret_cast<float*>(base + c.off_csc);
    v.s_cq = (int64_t)c.s_cq;
    v.s_csc = (int64_t)(c.s_csc / 4);
    v.s_cent = (int64_t)(c.s_cent / c.elt);
    v.s_sums = (int64_t)(c.s_sums / 4);
    v.s_meta = (int64_t)(c.s_meta / 4);
    v.s_members = (int64_t)(c.s_members / 2);
    v.s_eleaf = (int64_t)c.s_eleaf;
    v.s_tcent = (int64_t)(c.s_tcent / c.elt);
    v.s_tsums = (int64_t)(c.s_tsums / 4);
    v.s_epos = (int64_t)c.s_epos;
    v.s_edge = (int64_t)(c.s_edge / c.elt);
    v.n_lev_cap = c.n_lev_cap;
    v.n_blocks = (int32_t)c.n_blocks;
    v.n_leaves = (int32_t)c.n_leaves;
    v.n_levels = c.n_levels;
    v.n_leaves_cap = (int32_t)c.nlm;
    v.bf16 = bf16 ? 1 : 0;
    return v;
}

lsa_status check_cfg(const lsa_select_cfg* C, int64_t T) {
    if (!C) return fail(LSA_ERR_INVALID_ARG, "select cfg is NULL");
    if (C->k < 0 || C->n_sinks < 0) return fail(LSA_ERR_INVALID_ARG, "k and n_sinks must be >= 0");
    if (C->window < 1) return fail(LSA_ERR_INVALID_ARG, "window must be >= 1");
    if (C->search != LSA_SEARCH_FLAT && C->search != LSA_SEARCH_TREE) return fail(LSA_ERR_INVALID_ARG, "unknown search");
    if (C->strategy < LSA_STRATEGY_AUTO || C->strategy > LSA_STRATEGY_MATERIALIZED)
        return fail(LSA_ERR_INVALID_ARG, "unknown strategy");
    if (C->k > LSA_MAX_K && (int64_t)C->k < T)
        return fail(LSA_ERR_CAPACITY, "k=%d exceeds %d and is below the %lld bucketed tokens", C->k, LSA_MAX_K,
                    (long long)T);
    if (C->search == LSA_SEARCH_TREE && (C->beam < 1 || C->beam > LSA_MAX_BEAM))
        return fail(LSA_ERR_CAPACITY, "beam must be in 1..%d", LSA_MAX_BEAM);
    if (C->causal_tree != 0 && C->causal_tree != 1) return fail(LSA_ERR_INVALID_ARG, "causal_tree must be 0 or 1");
    if (C->skip_recorded_lists != 0 && C->skip_recorded_lists != 1)
        return fail(LSA_ERR_INVALID_ARG, "skip_recorded_lists must be 0 or 1");
    return LSA_OK;
}

struct SelectWs {
    size_t off_qhat, off_tau, off_cnt, off_counters, off_cand, off_fb, off_scores, off_tmax, zero_off, zero_bytes, total;
    int64_t score_stride, tmax_stride;
    int fb_slots;
    int strategy;
};

constexpr int kFallbackSlots = 256;

// Split-key attention workspace: fp32 partials (max, denominator, d values
// per split and head), then one 64-bit arrival word per unit.
size_t attend_part_bytes(int64_t units, int splits, int G, int d) {
    return align256((size_t)units * splits * G * (d + 2) * 4);
}
size_t attend_ws_bytes(int64_t units, int splits, int G, int d) {
    return splits > 1 ? attend_part_bytes(units, splits, G, d) + align256((size_t)units * 8) : 0;
}

// Tag that tells one attention call's arrival words from another's: a
// process-wide counter, started from the clock so that words left by another
// process in reused memory are unlikely to carry a live tag; 0 is skipped.
uint32_t next_call_tag() {
    static std::atomic<uint32_t> tag{(uint32_t)std::chrono::steady_clock::now().time_since_epoch().count() | 1u};
    uint32_t t = tag.fetch_add(1, std::memory_order_relaxed);
    if (t == 0) t = tag.fetch_add(1, std::memory_order_relaxed);
    return t;
}

// Workspace of one bucket-major pass over nqp queries per sequence: the
// per-bin counts and offsets, the per-unit pair counts, slot offsets and
// staging rows (kBmUnitCap pair records each), the pair records grouped by
// bin, the work records, and the partials (fp32 max, denominator and scale,
// D fp16 values) of every pool slot.  The pool holds
// kBmPoolPerUnit slots per unit on average (a unit takes one per bucket it
// reads from, about k / 32 with buckets of 8 entries, 64 at k = 2048) and at
// least one full unit; pool slots are handed out in unit order, so a pass
// whose units need more runs its last units through the gather path.
constexpr int64_t kBmPoolPerUnit = 80;
// most units per pass: keeps every pair and slot index inside 32 bits
constexpr int64_t kBmMaxUnits = (int64_t)1 << 23;

struct BmWs {
    int64_t units, leaves_max, nbins, nbins_pad, nuch;
    uint32_t pool_cap;
    size_t off_lcnt, off_loff, off_ctot, off_csum, off_gpre, off_uoff, off_unp, off_utot, off_ucsum, off_stage,
        off_srec, off_work, off_po, off_pml, total;
};

void bm_ws(const lsa_layout* L, int64_t B, int64_t nqp, int64_t t_max, BmWs& w) {
    memset(&w, 0, sizeof(w));
    const int64_t H_kv = L->n_kv_heads, G = L->n_q_heads / L->n_kv_heads, D = L->head_dim;
    w.units = B * nqp * H_kv;
    w.leaves_max = (t_max / LSA_BLOCK_TOKENS) * LSA_LEAVES_PER_BLOCK;
    w.nbins = B * H_kv * w.leaves_max;
    const int64_t nch = (w.nbins + lsa::kBmScanChunk - 1) / lsa::kBmScanChunk;
    w.nbins_pad = (nch > 0 ? nch : 1) * lsa::kBmScanChunk;
    w.nuch = (w.units + lsa::kBmScanChunk - 1) / lsa::kBmScanChunk;
    if (w.nuch < 1) w.nuch = 1;
    int64_t pool = w.units * kBmPoolPerUnit;
    if (pool < lsa::kBmUnitCap) pool = lsa::kBmUnitCap;
    if (pool > ((int64_t)1 << 31)) pool = (int64_t)1 << 31;
    w.pool_cap = (uint32_t)pool;
    size_t o = 0;
    w.off_lcnt = o;   o = align256(o + (size_t)(w.nbins_pad + 4) * 4);
    w.off_loff = o;   o = align256(o + (size_t)w.nbins_pad * 4);
    w.off_ctot = o;   o = align256(o + (size_t)(w.nbins_pad / lsa::kBmScanChunk) * 8);
    w.off_csum = o;   o = align256(o + (size_t)(w.nbins_pad / lsa::kBmScanChunk) * 8);
    w.off_gpre = o;   o = align256(o + (size_t)(w.nbins_pad / 64) * 4);
    w.off_uoff = o;   o = align256(o + (size_t)w.units * 4);
    w.off_unp = o;    o = align256(o + (size_t)w.units * 4);
    w.off_utot = o;   o = align256(o + (size_t)w.nuch * 4);
    w.off_ucsum = o;  o = align256(o + (size_t)w.nuch * 4);
    w.off_stage = o;  o = align256(o + (size_t)w.units * lsa::kBmUnitCap * 16);
    w.off_srec = o;   o = align256(o + (size_t)pool * 16);
    w.off_work = o;   o = align256(o + (size_t)w.nbins * 17 * 16);
    w.off_po = o;     o = align256(o + (size_t)pool * G * (2 * D));   // fp16 rows
    w.off_pml = o;    o = align256(o + (size_t)pool * G * 16);
    w.total = o;
}

int resolve_strategy(const lsa_select_cfg* C, int64_t units) {
    if (C->search == LSA_SEARCH_TREE) return -1;
    if (C->strategy != LSA_STRATEGY_AUTO) return C->strategy;
    return units <= 4096 ? LSA_STRATEGY_MATERIALIZED : LSA_STRATEGY_FUSED;
}

void select_ws(const lsa_layout* L, const lsa_select_cfg* C, int64_t B, int64_t n_q, int64_t t_max, SelectWs& w) {
    memset(&w, 0, sizeof(w));
    const int64_t units = B * n_q * L->n_kv_heads;
    const int elt = L->dtype == LSA_BF16 ? 2 : 4;
    const int64_t nlm = (t_max / LSA_BLOCK_TOKENS) * LSA_LEAVES_PER_BLOCK;
    w.strategy = resolve_strategy(C, units);
    w.score_stride = (nlm + 63) & ~(int64_t)63;
    size_t o = 0;
    w.off_qhat = o;     o = align256(o + (size_t)(B * n_q * L->n_q_heads) * LSA_LATENT_DIM * elt);
    w.off_counters = o; o = align256(o + 64);
    w.off_tau = o;      o = align256(o + (size_t)units * 4);
    w.off_cnt = o;      o = align256(o + (size_t)units * 16);   // fused: 4 sub-list counts per unit
    if (w.strategy == LSA_STRATEGY_FUSED) {
        w.off_cand = o; o = align256(o + (size_t)units * lsa::kCandStride * 8);
        w.off_fb = o;   o = align256(o + (size_t)units * 4);
        w.fb_slots = (int)(units < kFallbackSlots ? (units > 0 ? units : 1) : kFallbackSlots);
        w.off_scores = o; o = align256(o + (size_t)w.fb_slots * w.score_stride * 4);
    } else if (w.strategy == LSA_STRATEGY_MATERIALIZED) {   // the finish runs its exact fallback in place
        w.off_scores = o; o = align256(o + (size_t)units * w.score_stride * 4);
        w.tmax_stride = w.score_stride / 16;
        w.off_tmax = o; o = align256(o + (size_t)units * w.tmax_stride * 4);
    }
    w.total = o;
}

}  // namespace

namespace lsa {
// Records a failure for lsa_last_error() from another translation unit of the library.
lsa_status set_error(lsa_status s, const char* msg) { return fail(s, "%s", msg); }
}  // namespace lsa

extern "C" {

int32_t lsa_abi_version(void) { return LSA_ABI_VERSION; }

const char* lsa_status_string(lsa_status s) {
    switch (s) {
        case LSA_OK: return "LSA_OK";
        case LSA_ERR_INVALID_ARG: return "LSA_ERR_INVALID_ARG";
        case LSA_ERR_SHAPE: return "LSA_ERR_SHAPE";
        case LSA_ERR_DTYPE: return "LSA_ERR_DTYPE";
        case LSA_ERR_ALIGN: return "LSA_ERR_ALIGN";
        case LSA_ERR_WORKSPACE: return "LSA_ERR_WORKSPACE";
        case LSA_ERR_CAPACITY: return "LSA_ERR_CAPACITY";
        case LSA_ERR_HIP: return "LSA_ERR_HIP";
        case LSA_ERR_UNSUPPORTED: return "LSA_ERR_UNSUPPORTED";
    }
    return "LSA_ERR_UNKNOWN";
}

const char* lsa_last_error(void) { return g_err.c_str(); }

lsa_status lsa_cache_bytes(const lsa_layout* layout, int64_t batch, int64_t t_max, size_t* bytes) {
    lsa_status s = check_layout(layout);
    if (s) return s;
    if (!bytes) return fail(LSA_ERR_INVALID_ARG, "bytes is NULL");
    if (batch < 0 || t_max < 0) return fail(LSA_ERR_INVALID_ARG, "batch and t_max must be >= 0");
    CacheGeom c;
    cache_geom(layout, batch, t_max, t_max, c);
    *bytes = c.total;
    return ok();
}

lsa_status lsa_cache_describe(const lsa_layout* layout, int64_t batch, int64_t t_max, int64_t T,
                              lsa_cache_info* info) {
    lsa_status s = check_layout(layout);
    if (s) return s;
    if (!info) return fail(LSA_ERR_INVALID_ARG, "info is NULL");
    if (batch < 0 || t_max < 0 || T < 0) return fail(LSA_ERR_INVALID_ARG, "sizes must be >= 0");
    if (T > t_max) return fail(LSA_ERR_CAPACITY, "T=%lld exceeds t_max=%lld", (long long)T, (long long)t_max);
    CacheGeom c;
    cache_geom(layout, batch, t_max, T, c);
    memset(info, 0, sizeof(*info));
    info->n_blocks_max = c.nbm;
    info->leaves_max = c.nlm;
    info->nodes_max = c.nnm;
    info->n_blocks = c.n_blocks;
    info->n_leaves = c.n_leaves;
    info->n_levels = c.n_levels;
    info->elt_bytes = c.elt;
    for (int i = 0; i < 40 && i < lsa::kMaxLevels; ++i) {
        info->level_off[i] = c.level_off[i];
        info->level_size[i] = c.level_size[i];
    }
    info->off_cent = c.off_cent;
    info->off_sums = c.off_sums;
    info->off_meta = c.off_meta;
    info->off_members = c.off_members;
    info->off_entry_leaf = c.off_eleaf;
    info->off_tree_cent = c.off_tcent;
    info->off_tree_sums = c.off_tsums;
    info->stride_cent = c.s_cent;
    info->stride_sums = c.s_sums;
    info->stride_meta = c.s_meta;
    info->stride_members = c.s_members;
    info->stride_entry_leaf = c.s_eleaf;
    info->stride_tree_cent = c.s_tcent;
    info->stride_tree_sums = c.s_tsums;
    info->total_bytes = c.total;
    info->off_entry_pos = c.off_epos;
    info->stride_entry_pos = c.s_epos;
    info->off_edge_cent = c.off_edge;
    info->stride_edge_cent = c.s_edge;
    info->edge_levels = c.n_lev_cap;
    info->off_cent_i8 = c.off_cq;
    info->stride_cent_i8 = c.s_cq;
    info->off_cent_scale = c.off_csc;
    info->stride_cent_scale = c.s_csc;
    return ok();
}

lsa_status lsa_build_buckets(const lsa_layout* layout, const void* K, int64_t batch, int64_t t_cap, int64_t T,
                             const void* W_k, void* cache, size_t cache_bytes, int64_t t_max, void* stream) {
    lsa_status s = check_layout(layout);
    if (s) return s;
    if (batch < 0 || t_cap < 0 || T < 0 || t_max < 0) return fail(LSA_ERR_INVALID_ARG, "sizes must be >= 0");
    if (T > t_cap) return fail(LSA_ERR_CAPACITY, "T=%lld exceeds t_cap=%lld", (long long)T, (long long)t_cap);
    if (T > t_max) return fail(LSA_ERR_CAPACITY, "T=%lld exceeds t_max=%lld", (long long)T, (long long)t_max);
    if (!K || !W_k || !cache) return fail(LSA_ERR_INVALID_ARG, "K, W_k and cache must be non-NULL");
    if (misaligned(K) || misaligned(W_k) || misaligned(cache)) return fail(LSA_ERR_ALIGN, "pointers must be 16-byte aligned");
    CacheGeom c;
    cache_geom(layout, batch, t_max, T, c);
    if (cache_bytes < c.total)
        return fail(LSA_ERR_WORKSPACE, "cache has %zu bytes, needs %zu", cache_bytes, c.total);
    if (batch == 0 || c.n_blocks == 0) return ok();
    const bool bf16 = layout->dtype == LSA_BF16;
    lsa::CacheView v = make_view(c, cache, bf16);
    hipStream_t st = static_cast<hipStream_t>(stream);
    hipError_t e = lsa::launch_build(v, K, bf16, t_cap, layout->head_dim, (int)batch, layout->n_kv_heads, W_k, st);
    if (e == hipSuccess && layout->build_tree)
        e = lsa::launch_tree(v, c.level_off, c.level_size, (int)batch, layout->n_kv_heads, st);
    if (e == hipSuccess && layout->build_tree) e = lsa::launch_edges(v, (int)batch, layout->n_kv_heads, 1, st);
    if (e != hipSuccess) return fail(LSA_ERR_HIP, "launch failed: %s", hipGetErrorString(e));
    return ok();
}

lsa_status lsa_extend_buckets(const lsa_layout* layout, const void* K, int64_t batch, int64_t t_cap, int64_t T_old,
                              int64_t T_new, const void* W_k, void* cache, size_t cache_bytes, int64_t t_max,
                              void* stream) {
    lsa_status s = check_layout(layout);
    if (s) return s;
    if (batch < 0 || t_cap < 0 || T_old < 0 || t_max < 0) return fail(LSA_ERR_INVALID_ARG, "sizes must be >= 0");
    if (T_new < T_old) return fail(LSA_ERR_INVALID_ARG, "T_new=%lld is below T_old=%lld", (long long)T_new, (long long)T_old);
    if (T_new > t_cap) return fail(LSA_ERR_CAPACITY, "T_new=%lld exceeds t_cap=%lld", (long long)T_new, (long long)t_cap);
    if (T_new > t_max) return fail(LSA_ERR_CAPACITY, "T_new=%lld exceeds t_max=%lld", (long long)T_new, (long long)t_max);
    if (!K || !W_k || !cache) return fail(LSA_ERR_INVALID_ARG, "K, W_k and cache must be non-NULL");
    if (misaligned(K) || misaligned(W_k) || misaligned(cache)) return fail(LSA_ERR_ALIGN, "pointers must be 16-byte aligned");
    CacheGeom c;
    cache_geom(layout, batch, t_max, T_new, c);
    if (cache_bytes < c.total)
        return fail(LSA_ERR_WORKSPACE, "cache has %zu bytes, needs %zu", cache_bytes, c.total);
    const int64_t b0 = T_old / LSA_BLOCK_TOKENS;
    if (batch == 0 || c.n_blocks == b0) return ok();
    const bool bf16 = layout->dtype == LSA_BF16;
    lsa::CacheView v = make_view(c, cache, bf16);
    hipStream_t st = static_cast<hipStream_t>(stream);
    hipError_t e = lsa::launch_build(v, K, bf16, t_cap, layout->head_dim, (int)batch, layout->n_kv_heads, W_k, st,
                                     (int)b0);
    if (e == hipSuccess && layout->build_tree)
        e = lsa::launch_tree(v, c.level_off, c.level_size, (int)batch, layout->n_kv_heads, st,
                             b0 * LSA_LEAVES_PER_BLOCK);
    if (e == hipSuccess && layout->build_tree)
        e = lsa::launch_edges(v, (int)batch, layout->n_kv_heads, (int)b0 + 1, st);
    if (e != hipSuccess) return fail(LSA_ERR_HIP, "launch failed: %s", hipGetErrorString(e));
    return ok();
}

lsa_status lsa_select_workspace_bytes(const lsa_layout* layout, const lsa_select_cfg* cfg, int64_t batch,
                                      int64_t n_q, int64_t t_max, size_t* bytes) {
    lsa_status s = check_layout(layout);
    if (s) return s;
    if (!cfg || !bytes) return fail(LSA_ERR_INVALID_ARG, "cfg and bytes must be non-NULL");
    if (batch < 0 || n_q < 0 || t_max < 0) return fail(LSA_ERR_INVALID_ARG, "sizes must be >= 0");
    s = check_cfg(cfg, t_max);
    if (s) return s;
    SelectWs w;
    select_ws(layout, cfg, batch, n_q, t_max, w);
    *bytes = w.total;
    return ok();
}

lsa_status lsa_select(const lsa_layout* layout, const lsa_select_cfg* cfg, const void* cache, size_t cache_bytes,
                      int64_t t_max, int64_t T, const void* Q, const int64_t* q_pos, int64_t batch, int64_t n_q,
                      const void* W_q, int32_t* lr_idx, int32_t* lr_cnt, void* bucket_recs, int32_t* bucket_cnt,
                      void* workspace, size_t workspace_bytes, void* stream) {
    lsa_status s = check_layout(layout);
    if (s) return s;
    if (batch < 0 || n_q < 0 || T < 0 || t_max < 0) return fail(LSA_ERR_INVALID_ARG, "sizes must be >= 0");
    if (T > t_max) return fail(LSA_ERR_CAPACITY, "T=%lld exceeds t_max=%lld", (long long)T, (long long)t_max);
    s = check_cfg(cfg, T);
    if (s) return s;
    if (cfg->search == LSA_SEARCH_TREE && !layout->build_tree)
        return fail(LSA_ERR_UNSUPPORTED, "tree search needs a cache built with build_tree = 1");
    const int64_t units = batch * n_q * layout->n_kv_heads;
    if (units == 0) return ok();
    if (!cache || !Q || !q_pos || !W_q || !lr_cnt || (!lr_idx && cfg->k > 0) || !workspace)
        return fail(LSA_ERR_INVALID_ARG, "a required pointer is NULL");
    if ((bucket_recs == nullptr) != (bucket_cnt == nullptr))
        return fail(LSA_ERR_INVALID_ARG, "bucket_recs and bucket_cnt must both be NULL or both be set");
    if (misaligned(cache) || misaligned(Q) || misaligned(q_pos) || misaligned(W_q) || misaligned(lr_cnt) ||
        (lr_idx && misaligned(lr_idx)) || misaligned(workspace) || (bucket_recs && misaligned(bucket_recs)) ||
        (bucket_cnt && misaligned(bucket_cnt)))
        return fail(LSA_ERR_ALIGN, "pointers must be 16-byte aligned");
    CacheGeom c;
    cache_geom(layout, batch, t_max, T, c);
    if (cache_bytes < c.total) return fail(LSA_ERR_WORKSPACE, "cache has %zu bytes, needs %zu", cache_bytes, c.total);
    SelectWs w;
    select_ws(layout, cfg, batch, n_q, t_max, w);
    if (workspace_bytes < w.total)
        return fail(LSA_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes, w.total);
    const bool bf16 = layout->dtype == LSA_BF16;
    lsa::CacheView v = make_view(c, const_cast<void*>(cache), bf16);
    char* wb = static_cast<char*>(workspace);
    lsa::SelectBuffers sb;
    sb.qhat = wb + w.off_qhat;
    sb.tau = reinterpret_cast<float*>(wb + w.off_tau);
    sb.cnt = reinterpret_cast<int*>(wb + w.off_cnt);
    sb.counters = reinterpret_cast<int*>(wb + w.off_counters);
    sb.cand = reinterpret_cast<uint64_t*>(wb + w.off_cand);
    sb.fb_list = reinterpret_cast<int*>(wb + w.off_fb);
    sb.scores = reinterpret_cast<float*>(wb + w.off_scores);
    sb.score_stride = w.score_stride;
    sb.tmax = reinterpret_cast<float*>(wb + w.off_tmax);
    sb.tmax_stride = w.tmax_stride;
    sb.fb_slots = w.fb_slots;
    lsa::SelArgs sa;
    sa.k = cfg->k;
    sa.n_sinks = cfg->n_sinks;
    sa.window = cfg->window;
    sa.beam = cfg->beam;
    sa.causal_tree = cfg->search == LSA_SEARCH_TREE ? cfg->causal_tree : 0;
    sa.H_q = layout->n_q_heads;
    sa.H_kv = layout->n_kv_heads;
    sa.G = layout->n_q_heads / layout->n_kv_heads;
    sa.n_q = n_q;
    sa.n_units = units;
    sa.brec = static_cast<lsa::u32x4*>(bucket_recs);
    sa.bcnt = bucket_cnt;
    sa.skip_lists = bucket_recs != nullptr ? cfg->skip_recorded_lists : 0;
    hipStream_t st = static_cast<hipStream_t>(stream);
    int32_t* lr = lr_idx ? lr_idx : lr_cnt;  // k == 0: rows are empty, never written
    hipError_t e = bucket_cnt ? lsa::launch_fill_i32(bucket_cnt, units, -1, st) : hipSuccess;
    // the bf16 materialized scan computes its own query latents
    const bool own_qhat = cfg->search == LSA_SEARCH_FLAT && w.strategy == LSA_STRATEGY_MATERIALIZED && bf16;
    if (e == hipSuccess && !own_qhat)
        e = lsa::launch_qlatent(Q, W_q, bf16, layout->head_dim, batch * n_q * layout->n_q_heads, sb.qhat,
                                       sb.counters, wb + w.zero_off, w.zero_bytes, st);
    if (e == hipSuccess) {
        if (cfg->search == LSA_SEARCH_TREE)
            e = lsa::launch_select_tree(v, bf16, q_pos, sa, sb, lr, lr_cnt, st);
        else if (w.strategy == LSA_STRATEGY_FUSED)
            e = lsa::launch_select_fused(v, bf16, q_pos, sa, (int)batch, sb, lr, lr_cnt, st);
        else
            e = lsa::launch_select_materialized(v, bf16, q_pos, sa, sb, lr, lr_cnt, Q, W_q, layout->head_dim,
                                                batch * n_q * layout->n_q_heads, st);
    }
    if (e != hipSuccess) return fail(LSA_ERR_HIP, "launch failed: %s", hipGetErrorString(e));
    return ok();
}

lsa_status lsa_attend_workspace_bytes(const lsa_layout* layout, const lsa_select_cfg* cfg, int64_t batch,
                                      int64_t n_q, size_t* bytes) {
    lsa_status s = check_layout(layout);
    if (s) return s;
    if (!cfg || !bytes) return fail(LSA_ERR_INVALID_ARG, "cfg and bytes must be non-NULL");
    if (batch < 0 || n_q < 0) return fail(LSA_ERR_INVALID_ARG, "sizes must be >= 0");
    const int64_t units = batch * n_q * layout->n_kv_heads;
    *bytes = attend_ws_bytes(units, lsa::attend_splits(units, cfg->window, cfg->k),
                             layout->n_q_heads / layout->n_kv_heads, layout->head_dim);
    return ok();
}

lsa_status lsa_sparse_attend(const lsa_layout* layout, const lsa_select_cfg* cfg, const void* Q, const void* K,
                             const void* V, int64_t t_cap, int64_t T, const int64_t* q_pos, int64_t batch,
                             int64_t n_q, const int32_t* lr_idx, const int32_t* lr_cnt, float scale, void* O,
                             void* workspace, size_t workspace_bytes, void* stream) {
    lsa_status s = check_layout(layout);
    if (s) return s;
    if (!cfg) return fail(LSA_ERR_INVALID_ARG, "cfg is NULL");
    if (batch < 0 || n_q < 0 || t_cap < 0 || T < 0) return fail(LSA_ERR_INVALID_ARG, "sizes must be >= 0");
    if (cfg->k < 0 || cfg->n_sinks < 0 || cfg->window < 1) return fail(LSA_ERR_INVALID_ARG, "bad k / n_sinks / window");
    if (T > t_cap) return fail(LSA_ERR_CAPACITY, "T=%lld exceeds t_cap=%lld", (long long)T, (long long)t_cap);
    if (!std::isfinite(scale)) return fail(LSA_ERR_INVALID_ARG, "scale must be finite");
    const int64_t units = batch * n_q * layout->n_kv_heads;
    if (units == 0) return ok();
    if (!Q || !K || !V || !q_pos || !lr_cnt || (!lr_idx && cfg->k > 0) || !O)
        return fail(LSA_ERR_INVALID_ARG, "a required pointer is NULL");
    if (misaligned(Q) || misaligned(K) || misaligned(V) || misaligned(q_pos) || misaligned(lr_cnt) ||
        (lr_idx && misaligned(lr_idx)) || misaligned(O))
        return fail(LSA_ERR_ALIGN, "pointers must be 16-byte aligned");
    const int splits = lsa::attend_splits(units, cfg->window, cfg->k);
    const int G = layout->n_q_heads / layout->n_kv_heads;
    const size_t need = attend_ws_bytes(units, splits, G, layout->head_dim);
    if (workspace_bytes < need || (need > 0 && !workspace))
        return fail(LSA_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes, need);
    if (need > 0 && misaligned(workspace)) return fail(LSA_ERR_ALIGN, "workspace must be 16-byte aligned");
    lsa::AttArgs aa;
    memset(&aa, 0, sizeof(aa));
    aa.n_q = n_q;
    aa.q0 = 0;
    aa.nqp = n_q;
    aa.n_units = units;
    aa.t_cap = t_cap;
    aa.B = (int32_t)batch;
    aa.H_kv = layout->n_kv_heads;
    aa.H_q = layout->n_q_heads;
    aa.G = G;
    aa.n_sinks = cfg->n_sinks;
    aa.window = cfg->window;
    aa.n_blocks = (int32_t)(T / LSA_BLOCK_TOKENS);
    aa.k = cfg->k;
    aa.splits = splits;
    aa.scale = scale;
    aa.arrive = need > 0 ? reinterpret_cast<unsigned long long*>(static_cast<char*>(workspace) +
                                                                 attend_part_bytes(units, splits, G, layout->head_dim))
                         : nullptr;
    aa.tag = next_call_tag();
    hipError_t e = lsa::launch_attend(Q, K, V, q_pos, lr_idx ? lr_idx : lr_cnt, lr_cnt, aa, layout->head_dim,
                                      layout->dtype == LSA_BF16, O, static_cast<float*>(workspace),
                                      static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(LSA_ERR_HIP, "launch failed: %s", hipGetErrorString(e));
    return ok();
}

lsa_status lsa_attend_bucket_major_workspace_bytes(const lsa_layout* layout, const lsa_select_cfg* cfg,
                                                   int64_t batch, int64_t n_q_pass, int64_t t_max, size_t* bytes) {
    lsa_status s = check_layout(layout);
    if (s) return s;
    if (!cfg || !bytes) return fail(LSA_ERR_INVALID_ARG, "cfg and bytes must be non-NULL");
    if (batch < 0 || n_q_pass < 0 || t_max < 0) return fail(LSA_ERR_INVALID_ARG, "sizes must be >= 0");
    BmWs w;
    bm_ws(layout, batch, n_q_pass, t_max, w);
    *bytes = w.total;
    return ok();
}

lsa_status lsa_sparse_attend_bucket_major(const lsa_layout* layout, const lsa_select_cfg* cfg, const void* cache,
                                          size_t cache_bytes, int64_t t_max, const void* Q, const void* K,
                                          const void* V, int64_t t_cap, int64_t T, const int64_t* q_pos,
                                          int64_t batch, int64_t n_q, const int32_t* lr_idx, const int32_t* lr_cnt,
                                          const void* bucket_recs, const int32_t* bucket_cnt, float scale, void* O,
                                          void* workspace, size_t workspace_bytes, uint32_t* fallback_counts,
                                          void* stream) {
    lsa_status s = check_layout(layout);
    if (s) return s;
    if (!cfg) return fail(LSA_ERR_INVALID_ARG, "cfg is NULL");
    if (layout->dtype != LSA_BF16) return fail(LSA_ERR_UNSUPPORTED, "bucket-major attention is bf16 only");
    if (batch < 0 || n_q < 0 || t_cap < 0 || T < 0 || t_max < 0)
        return fail(LSA_ERR_INVALID_ARG, "sizes must be >= 0");
    if (cfg->k < 0 || cfg->n_sinks < 0 || cfg->window < 1) return fail(LSA_ERR_INVALID_ARG, "bad k / n_sinks / window");
    if (T > t_cap) return fail(LSA_ERR_CAPACITY, "T=%lld exceeds t_cap=%lld", (long long)T, (long long)t_cap);
    if (T > t_max) return fail(LSA_ERR_CAPACITY, "T=%lld exceeds t_max=%lld", (long long)T, (long long)t_max);
    if (!std::isfinite(scale)) return fail(LSA_ERR_INVALID_ARG, "scale must be finite");
    const int64_t units = batch * n_q * layout->n_kv_heads;
    if (units == 0) return ok();
    if (!cache || !Q || !K || !V || !q_pos || !lr_cnt || (!lr_idx && cfg->k > 0) || !O || !workspace)
        return fail(LSA_ERR_INVALID_ARG, "a required pointer is NULL");
    if ((bucket_recs == nullptr) != (bucket_cnt == nullptr))
        return fail(LSA_ERR_INVALID_ARG, "bucket_recs and bucket_cnt must both be NULL or both be set");
    if (misaligned(cache) || misaligned(Q) || misaligned(K) || misaligned(V) || misaligned(q_pos) ||
        misaligned(lr_cnt) || (lr_idx && misaligned(lr_idx)) || misaligned(O) || misaligned(workspace) ||
        (bucket_recs && misaligned(bucket_recs)) || (bucket_cnt && misaligned(bucket_cnt)) ||
        (fallback_counts && misaligned(fallback_counts)))
        return fail(LSA_ERR_ALIGN, "pointers must be 16-byte aligned");
    CacheGeom c;
    cache_geom(layout, batch, t_max, T, c);
    if (cache_bytes < c.total) return fail(LSA_ERR_WORKSPACE, "cache has %zu bytes, needs %zu", cache_bytes, c.total);
    if (batch * layout->n_kv_heads > kBmMaxUnits)
        return fail(LSA_ERR_CAPACITY, "more than %lld (sequence, KV head) slices", (long long)kBmMaxUnits);
    // queries per pass: the most the workspace holds (the size is increasing in the pass length), and at
    // most kBmMaxUnits units
    BmWs w;
    bm_ws(layout, batch, 1, t_max, w);
    if (workspace_bytes < w.total)
        return fail(LSA_ERR_WORKSPACE, "workspace has %zu bytes, needs at least %zu", workspace_bytes, w.total);
    int64_t lo = 1, hi = n_q;
    if (hi > kBmMaxUnits / (batch * layout->n_kv_heads)) hi = kBmMaxUnits / (batch * layout->n_kv_heads);
    while (lo < hi) {
        const int64_t mid = lo + (hi - lo + 1) / 2;
        bm_ws(layout, batch, mid, t_max, w);
        if (w.total <= workspace_bytes) lo = mid; else hi = mid - 1;
    }
    const int64_t nqp_max = lo;
    if (w.nbins > (int64_t)0xFFFFFFFF) return fail(LSA_ERR_CAPACITY, "too many buckets for one pass");
    const int G = layout->n_q_heads / layout->n_kv_heads;
    lsa::CacheView v = make_view(c, const_cast<void*>(cache), true);
    hipStream_t st = static_cast<hipStream_t>(stream);
    char* wb = static_cast<char*>(workspace);
    for (int64_t q0 = 0; q0 < n_q; q0 += nqp_max) {
        const int64_t nqp = n_q - q0 < nqp_max ? n_q - q0 : nqp_max;
        bm_ws(layout, batch, nqp, t_max, w);
        lsa::BmBuffers bm;
        bm.leaves_max = w.leaves_max;
        bm.nbins = w.nbins;
        bm.nbins_pad = w.nbins_pad;
        bm.nuch = w.nuch;
        bm.pool_cap = w.pool_cap;
        bm.lcnt = reinterpret_cast<uint32_t*>(wb + w.off_lcnt);
        bm.loff = reinterpret_cast<uint32_t*>(wb + w.off_loff);
        bm.ctot = reinterpret_cast<uint32_t*>(wb + w.off_ctot);
        bm.csum = reinterpret_cast<uint32_t*>(wb + w.off_csum);
        bm.gpre = reinterpret_cast<uint32_t*>(wb + w.off_gpre);
        bm.unit_off = reinterpret_cast<uint32_t*>(wb + w.off_uoff);
        bm.unit_np = reinterpret_cast<int32_t*>(wb + w.off_unp);
        bm.utot = reinterpret_cast<uint32_t*>(wb + w.off_utot);
        bm.ucsum = reinterpret_cast<uint32_t*>(wb + w.off_ucsum);
        bm.stage = reinterpret_cast<lsa::u32x4*>(wb + w.off_stage);
        bm.srec = reinterpret_cast<lsa::u32x4*>(wb + w.off_srec);
        bm.fallback = fallback_counts;
        bm.work = reinterpret_cast<lsa::u32x4*>(wb + w.off_work);
        bm.po = reinterpret_cast<uint32_t*>(wb + w.off_po);
        bm.pml = reinterpret_cast<float*>(wb + w.off_pml);
        lsa::AttArgs aa;
        memset(&aa, 0, sizeof(aa));
        aa.n_q = n_q;
        aa.q0 = q0;
        aa.nqp = nqp;
        aa.n_units = w.units;
        aa.t_cap = t_cap;
        aa.B = (int32_t)batch;
        aa.H_kv = layout->n_kv_heads;
        aa.H_q = layout->n_q_heads;
        aa.G = G;
        aa.n_sinks = cfg->n_sinks;
        aa.window = cfg->window;
        aa.n_blocks = (int32_t)(T / LSA_BLOCK_TOKENS);
        aa.k = cfg->k;
        aa.splits = 1;
        aa.scale = scale;
        aa.bm_off = bm.unit_off;
        aa.bm_np = bm.unit_np;
        aa.bm_po = bm.po;
        aa.bm_ml = bm.pml;
        aa.bm_brec = static_cast<const lsa::u32x4*>(bucket_recs);
        aa.bm_bcnt = bucket_cnt;
        const int32_t* lr = lr_idx ? lr_idx : lr_cnt;
        hipError_t e = lsa::launch_bucket_partials(v, Q, K, V, q_pos, lr, lr_cnt, aa, bm, layout->head_dim, st);
        if (e == hipSuccess)
            e = lsa::launch_attend_local(v, Q, K, V, q_pos, lr, lr_cnt, aa, layout->head_dim, O, st);
        if (e != hipSuccess) return fail(LSA_ERR_HIP, "launch failed: %s", hipGetErrorString(e));
    }
    return ok();
}

lsa_status lsa_pca_workspace_bytes(const lsa_layout* layout, size_t* bytes) {
    lsa_status s = check_layout(layout);
    if (s) return s;
    if (!bytes) return fail(LSA_ERR_INVALID_ARG, "bytes is NULL");
    *bytes = lsa::pca_workspace_bytes(layout->head_dim);
    return ok();
}

lsa_status lsa_pca_projection(const lsa_layout* layout, const void* K, int64_t batch, int64_t t_cap, int64_t T,
                              void* W, float* eigvals, void* workspace, size_t workspace_bytes, void* stream) {
    lsa_status s = check_layout(layout);
    if (s) return s;
    if (batch < 1 || T < 1 || t_cap < T) return fail(LSA_ERR_INVALID_ARG, "need batch >= 1 and 1 <= T <= t_cap");
    if (!K || !W || !workspace) return fail(LSA_ERR_INVALID_ARG, "K, W and workspace must be non-NULL");
    if (misaligned(K) || misaligned(W) || misaligned(workspace) || (eigvals && misaligned(eigvals)))
        return fail(LSA_ERR_ALIGN, "pointers must be 16-byte aligned");
    const size_t need = lsa::pca_workspace_bytes(layout->head_dim);
    if (workspace_bytes < need) return fail(LSA_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes, need);
    hipError_t e = lsa::launch_pca(K, layout->dtype == LSA_BF16, layout->head_dim, t_cap, T,
                                   (int)(batch * layout->n_kv_heads), W, eigvals, workspace,
                                   static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(LSA_ERR_HIP, "launch failed: %s", hipGetErrorString(e));
    return ok();
}

}  // extern "C"
