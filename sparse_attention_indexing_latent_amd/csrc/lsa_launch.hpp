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
    const int32_t* bm_np;         // [n_units] partials of the unit; -1: gather its list instead
    const uint32_t* bm_po;        // [slots, G, 3D/8] words: unnormalised partial output / its scale, packed
                                  //   12-bit integers (kPartialWords layout)
    const float* bm_ml;           // [slots, G, 4] partial max, denominator, scale (largest |output| / 2047), 0
    const u32x4* bm_brec;         // optional: [units of the call, LSA_BUCKET_RECS] the selection's bucket records
    const int32_t* bm_bcnt;       // optional: their counts (-1: derive the pairs from the list)
};

// Workspace of one bucket-major pass.  A "bin" is one bucket of one (b, g):
// (a pair's partial output row is kept as fp16 values in [-1, 1] times an
// fp32 scale, the row's largest magnitude: half the bytes of fp32 with an
// absolute rounding error of at most 2^-12 of that scale)
// bin = (b * H_kv + g) * leaves_max + bucket id.  A pair is one (query, KV
// head) unit together with one bucket it selected tokens from; pair slots
// are handed out per unit from a pool of pool_cap.
struct BmBuffers {
    int64_t leaves_max;
    int64_t nbins;             // B * H_kv * leaves_max
    int64_t nbins_pad;         // nbins rounded up to the scan chunk
    uint32_t pool_cap;
    uint32_t* lcnt;            // [nbins_pad + 2 + kBmCursors] pairs per bin, unused, the work count, then
                               //   the pool cursors (cursor c hands out slots of pool slice c)
    uint32_t* loff;            // [nbins_pad] offset of the bin's pairs inside its scan chunk
    uint32_t* ctot;            // [2 * nbins_pad / chunk] pairs, then bins with pairs, per scan chunk
    uint32_t* csum;            // [2 * nbins_pad / chunk] exclusive scans of both halves of ctot
    uint32_t* gpre;            // [nbins_pad / 64] bins with pairs before each 64-bin group, inside its chunk
    uint32_t* unit_off;        // [n_units]
    int32_t* unit_np;          // [n_units]
    u32x4* rec;                // [pool_cap] (bin, arrival rank in the bin, key mask lo, hi); mask bit j:
                               //   key j of the bucket (member order) is listed
    u32x4* srec;               // [pool_cap] grouped by bin: (local unit, pair slot, key mask lo, hi)
    u32x4* work;               // [nbins, 17] one record per bin with pairs: (pair start, pairs, keys, b * H_kv + g),
                               //   then the bucket's 64 key tokens (member order; past the bucket: its first)
    uint32_t* po;              // [pool_cap, G, 3D/8] packed 12-bit partial outputs (layout below)
    float* pml;                // [pool_cap, G, 4] (max, denominator, scale, 0)
};
// A partial output row of D values is stored as integers q = round(o / scale) with
// scale = max |o| / 2047, so |q| <= 2047 fits 12 bits (worst-case error scale / 2, the
// same as fp16's for the row's largest values).  The row is 4 runs of 3D/32 words,
// run r holding the D/4 dims 32m + 8r + i (m < D/32, i < 8, value index 8m + i) of
// one reading lane: first D/16 words of high bytes (bits 4..11 of q, two's
// complement; value v in byte v % 4 of word v / 4), then D/32 words of low nibbles
// (bits 0..3; value v in nibble v % 8 of word D/16 + v / 8).
template <int D>
constexpr int kPartialWords = 3 * D / 32;   // words of one run (one reading lane)
constexpr int kBmScanChunk = 4096;   // bins per workgroup of the offset scan
constexpr int kBmUnitCap = 256;      // most buckets one unit may take through the bucket-major path
constexpr int kBmCursors = 256;      // pool slices, so that the units' slot requests spread over many words

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
hipError_t launch_select_materialized(const CacheView& cv, bool bf16, const int64_t* q_pos, const SelArgs& sa,
                                      const SelectBuffers& sb, int32_t* lr_idx, int32_t* lr_cnt, hipStream_t st);
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
hipError_t launch_attend_local(const void* Q, const void* K, const void* V, const int64_t* q_pos,
                               const int32_t* lr_idx, const int32_t* lr_cnt, const AttArgs& aa, int D, void* O,
                               hipStream_t st);
hipError_t launch_bucket_partials(const CacheView& cv, const void* Q, const void* K, const void* V,
                                  const int64_t* q_pos, const int32_t* lr_idx, const int32_t* lr_cnt,
                                  const AttArgs& aa, const BmBuffers& bm, int D, hipStream_t st);

}  // namespace lsa
