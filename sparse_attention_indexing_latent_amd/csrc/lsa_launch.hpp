// Host-side launch interface between the C ABI (lsa_api.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lsa_common.hpp"

namespace lsa {

struct SelArgs {
    int32_t k;
    int32_t n_sinks;
    int32_t window;
    int32_t beam;
    int32_t causal_tree;   // tree: straddling nodes scored from the cache's edge table
    int32_t H_q;
    int32_t G;
    int32_t H_kv;
    int64_t n_q;
    int64_t n_units;   // B * n_q * H_kv
    u32x4* brec;       // optional: [n_units, LSA_BUCKET_RECS] bucket records of the selection
    int32_t* bcnt;     // optional: [n_units] their count (-1: none; the caller fills -1 first)
    int32_t skip_lists;   // rows that get records: no token list written
};

struct SelectBuffers {
    void* qhat;
    float* tau;
    int* cnt;
    uint64_t* cand;
    int* fb_list;
    int* counters;
    float* scores;
    int64_t score_stride;
    float* tmax;           // materialized: the largest score of each 16-bucket tile
    int64_t tmax_stride;
    int fb_slots;
};

struct AttArgs {
    int64_t n_q;
    int64_t q0, nqp;   // this launch covers queries [q0, q0 + nqp) of every sequence
    int64_t n_units;   // B * nqp * H_kv
    int64_t t_cap;
    int32_t B, H_kv, H_q, G;
    int32_t n_sinks, window, n_blocks, k;
    int32_t splits;
    float scale;
    unsigned long long* arrive;   // splits > 1: per-unit arrival words (tag << 32 | count)
    uint32_t tag;                 // distinct per call
    // bucket-major merge (null bm_np: plain gather of the long-range list)
    const uint32_t* bm_off;       // [n_units] first partial slot of the unit
    const int32_t* bm_np;         // [n_units] partials of the unit; -1: gather its list; -2: gather its records' keys
    const uint32_t* bm_po;        // [slots, G, D/2] words: unnormalised partial output / its scale, fp16
                                  //   (layout: see BmBuffers)
    const float* bm_ml;           // [slots, G, 4] partial max, denominator, scale (a power of two), 0
    const u32x4* bm_brec;         // optional: [units of the call, LSA_BUCKET_RECS] the selection's bucket records
    const int32_t* bm_bcnt;       // optional: their counts (-1: derive the pairs from the list)
};

// Workspace of one bucket-major pass.  A "bin" is one bucket of one (b, g):
// bin = (b * H_kv + g) * leaves_max + bucket id.  A pair is one (query, KV
// head) unit together with one bucket it selected keys from.  The pairs of a
// unit are staged in its own row of kBmUnitCap records; an exclusive scan of
// the units' pair counts (in unit order) then gives every unit its range of
// partial slots in the pool, so which slots a unit gets, and which units do
// not fit the pool, never depend on the order in which waves run.
struct BmBuffers {
    int64_t leaves_max;
    int64_t nbins;             // B * H_kv * leaves_max
    int64_t nbins_pad;         // nbins rounded up to the scan chunk
    int64_t nuch;              // unit scan chunks: ceil(units / kBmScanChunk)
    uint32_t pool_cap;
    uint32_t* lcnt;            // [nbins_pad + 4] pairs per bin, then: unused, the work count, two unused
    uint32_t* loff;            // [nbins_pad] offset of the bin's pairs inside its scan chunk
    uint32_t* ctot;            // [2 * nbins_pad / chunk] pairs, then bins with pairs, per scan chunk
    uint32_t* csum;            // [2 * nbins_pad / chunk] exclusive scans of both halves of ctot
    uint32_t* gpre;            // [nbins_pad / 64] bins with pairs before each 64-bin group, inside its chunk
    uint32_t* unit_off;        // [n_units] first pool slot of the unit (after the rank step; before it: the
                               //   offset inside its scan chunk)
    int32_t* unit_np;          // [n_units] pairs of the unit; -1: gather its token list instead; -2: gather the
                               //   keys its bucket records name (records row whose pairs do not fit the pool)
    uint32_t* utot;            // [nuch] pairs per unit scan chunk
    uint32_t* ucsum;           // [nuch] their exclusive scan
    u32x4* stage;              // [n_units, kBmUnitCap] the unit's pairs: (bin, rank in the bin, key mask lo, hi);
                               //   mask bit j: key j of the bucket (member order) is listed
    u32x4* srec;               // [pool_cap] grouped by bin: (Q row of the unit's first head, pair slot, key mask
                               //   lo, hi)
    u32x4* work;               // [nbins, 17] one record per bin with pairs: (pair start, pairs, keys, b * H_kv + g),
                               //   then the bucket's 64 key tokens (member order; past the bucket: its first)
    uint32_t* po;              // [pool_cap, G, D/2] fp16 partial outputs (layout below)
    float* pml;                // [pool_cap, G, 4] (max, denominator, scale, 0)
    uint32_t* fallback;        // optional, [2]: rows gathered whole are added to [0], those sent there because
                               //   the pool was full also to [1]
};
// A partial output row of D values o is stored as fp16 values o * 2^-e and
// 2^e as the fp32 scale: e = 0 when every value fits fp16 with its relative
// precision (largest magnitude below 2^15 and, unless zero, at least 2^-8),
// else the power of two with the largest magnitude times 2^-e in [2^14, 2^15)
// (no overflow, fp16's relative precision for every value down to 2^-10 of
// the largest).  Layout [pair][m < D/32][head][reading lane r < 4], 16 bytes
// each: the 8 dims 32m + 8r + [0,8) of (pair, head); a pair's heads of one m
// are contiguous, so the writes of a group m and the merge's reads are whole
// G x 64-byte runs.
constexpr int kBmScanChunk = 4096;   // bins (or units) per workgroup of an offset scan
constexpr int kBmUnitCap = 256;      // most buckets one unit may take through the bucket-major path

// Sets lsa_last_error()'s message (and returns s) for a failure found outside lsa_api.cpp.
lsa_status set_error(lsa_status s, const char* msg);

hipError_t launch_build(const CacheView& cv, const void* K, bool bf16, int64_t t_cap, int d, int B, int H_kv,
                        const void* W, hipStream_t st, int blk0 = 0);
hipError_t launch_tree(const CacheView& cv, const int64_t* level_off, const int64_t* level_size, int B, int H_kv,
                       hipStream_t st, int64_t first_leaf = 0);
// Edge table of the tree: for every block boundary nb in [nb_first, n_blocks] and
// level, the centroid of the node straddling leaf 64 nb, over its leaves below it.
hipError_t launch_edges(const CacheView& cv, int B, int H_kv, int nb_first, hipStream_t st);
hipError_t launch_qlatent(const void* Q, const void* W, bool bf16, int d, int64_t rows, void* qhat, int* counters,
                          void* zero, size_t zero_bytes, hipStream_t st);
hipError_t launch_select_fused(const CacheView& cv, bool bf16, const int64_t* q_pos, const SelArgs& sa, int B,
                               const SelectBuffers& sb, int32_t* lr_idx, int32_t* lr_cnt, hipStream_t st);
// bf16: the scan computes the q_hat rows from Q and W itself (no latent launch before it)
hipError_t launch_select_materialized(const CacheView& cv, bool bf16, const int64_t* q_pos, const SelArgs& sa,
                                      const SelectBuffers& sb, int32_t* lr_idx, int32_t* lr_cnt, const void* Q,
                                      const void* W, int d, int64_t q_rows, hipStream_t st);
hipError_t launch_select_tree(const CacheView& cv, bool bf16, const int64_t* q_pos, const SelArgs& sa,
                              const SelectBuffers& sb, int32_t* lr_idx, int32_t* lr_cnt, hipStream_t st);
int attend_splits(int64_t n_units, int window, int k);
hipError_t launch_attend(const void* Q, const void* K, const void* V, const int64_t* q_pos, const int32_t* lr_idx,
                         const int32_t* lr_cnt, const AttArgs& aa, int D, bool bf16, void* O, float* part,
                         hipStream_t st);
size_t pca_workspace_bytes(int D);
hipError_t launch_fill_i32(int32_t* p, int64_t n, int32_t v, hipStream_t st);
hipError_t launch_pca(const void* K, bool bf16, int D, int64_t t_cap, int64_t T, int BH, void* W, float* eig,
                      void* workspace, hipStream_t st);
hipError_t launch_attend_local(const CacheView& cv, const void* Q, const void* K, const void* V,
                               const int64_t* q_pos, const int32_t* lr_idx, const int32_t* lr_cnt, const AttArgs& aa,
                               int D, void* O, hipStream_t st);
hipError_t launch_bucket_partials(const CacheView& cv, const void* Q, const void* K, const void* V,
                                  const int64_t* q_pos, const int32_t* lr_idx, const int32_t* lr_cnt,
                                  const AttArgs& aa, const BmBuffers& bm, int D, hipStream_t st);

}  // namespace lsa
