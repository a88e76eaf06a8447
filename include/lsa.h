/*
 * lsa.h — C ABI of the Latent Sparse Attention (LSA) layer hot path on one
 * AMD Instinct MI355X (gfx950).
 *
 * The method (zhichai.net explainer "卡片柜", ch.2–ch.4; diosapp.com.cn LSA
 * tutorial, section 二):
 *   key side   — every key is projected to a 64-d latent and L2-normalised,
 *                4 consecutive latents are pooled into one entry, each block
 *                of 512 entries is clustered once with Ward's method into
 *                buckets of mean 8 / max 16 entries, and the normalised bucket
 *                means ("cards") form the bucket cache; optionally a complete
 *                binary tree of merged buckets is kept above the leaves.
 *   query side — the query is projected the same way, every visible card is
 *                scored (max over the query heads of a GQA group), the best
 *                buckets are expanded into k long-range token indices, and
 *                exact softmax attention runs over sinks + local window +
 *                those tokens.
 *
 * Three calls follow that problem statement:
 *   lsa_build_buckets(K)              -> cache
 *   lsa_select(Q, cache)              -> long-range indices
 *   lsa_sparse_attend(Q, K, V, idx)   -> O
 *
 * Conventions shared by every call
 *   - All tensor pointers are DEVICE pointers owned by the caller; the
 *     library never allocates or frees device memory and keeps no device
 *     state between calls.  Pointers must be 16-byte aligned.
 *   - Work is enqueued on the given HIP stream (a hipStream_t passed as
 *     void*; NULL = the default stream) and is asynchronous: a call returns
 *     once its kernels are queued, never synchronises the host with the
 *     device, and so may be captured into a HIP graph.
 *   - Arguments are validated on the host before anything is queued; on any
 *     error nothing is written and a status other than LSA_OK is returned
 *     (lsa_last_error() then holds a per-thread message).  Faults inside a
 *     kernel surface at the caller's next synchronisation.
 *   - Layouts are row-major and contiguous:
 *       K, V   [B, H_kv, t_cap, d]   (a pooled entry's 4 keys are 4*d
 *                                      consecutive elements)
 *       Q, O   [B, n_q, H_q, d]
 *       W_k, W_q [d, 64]
 *       q_pos  [B, n_q] int64, absolute position of each query
 *       lr_idx [B, n_q, H_kv, k] int32, lr_cnt [B, n_q, H_kv] int32
 *     Query head h reads KV head h / G, G = H_q / H_kv.
 *   - Token geometry of a query at position t, with T tokens bucketed
 *     (n_blocks = T / 2048 full blocks; a trailing partial block is not
 *     bucketed):  nvis = min(t / 2048, n_blocks) blocks are selectable;
 *     sinks = [0, min(n_sinks, t+1)); local window = [l0, t] with
 *     l0 = max(0, min(t - window + 1, 2048 * nvis)), i.e. the last `window`
 *     tokens widened back to the first token that is not selectable.
 *     The long-range list holds only tokens outside sinks and window.
 */
#ifndef LSA_H
#define LSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LSA_BUCKET_RECS 256   /* bucket records per (query, KV head) in lsa_select's optional output */
#define LSA_ABI_VERSION 7

#define LSA_LATENT_DIM 64         /* latent width (ch.2: 64-d index space) */
#define LSA_POOL 4                /* keys pooled per entry (ch.2)            */
#define LSA_BLOCK_ENTRIES 512     /* entries per Ward block (ch.2)           */
#define LSA_BLOCK_TOKENS 2048     /* = LSA_POOL * LSA_BLOCK_ENTRIES          */
#define LSA_MEAN_BUCKET 8         /* mean entries per bucket (ch.2)          */
#define LSA_MAX_BUCKET 16         /* max entries per bucket (ch.2)           */
#define LSA_LEAVES_PER_BLOCK 64   /* = 512 / 8 buckets per full block        */
#define LSA_MAX_GROUP 8           /* largest supported G = H_q / H_kv        */
#define LSA_MAX_K 4096            /* largest k short of "every eligible token" */
#define LSA_MAX_BEAM 64           /* largest tree beam width                 */

typedef enum lsa_status {
    LSA_OK = 0,
    LSA_ERR_INVALID_ARG = 1,  /* NULL pointer, negative size, unknown enum value     */
    LSA_ERR_SHAPE = 2,        /* unsupported d / latent / pool / block / bucket / G  */
    LSA_ERR_DTYPE = 3,        /* dtype not LSA_F32 or LSA_BF16                       */
    LSA_ERR_ALIGN = 4,        /* a pointer not 16-byte aligned                       */
    LSA_ERR_WORKSPACE = 5,    /* cache or workspace smaller than the size query says */
    LSA_ERR_CAPACITY = 6,     /* T > t_max or T > t_cap, k or beam out of range      */
    LSA_ERR_HIP = 7,          /* a HIP launch returned an error                      */
    LSA_ERR_UNSUPPORTED = 8   /* e.g. tree search on a cache built without a tree    */
} lsa_status;

typedef enum lsa_dtype { LSA_F32 = 0, LSA_BF16 = 1 } lsa_dtype;

typedef enum lsa_search { LSA_SEARCH_FLAT = 0, LSA_SEARCH_TREE = 1 } lsa_search;

/* How lsa_select finds the top buckets of a flat search.  Every strategy
 * returns identical results; they differ only in speed. */
typedef enum lsa_strategy {
    LSA_STRATEGY_AUTO = 0,         /* fused for many queries, materialised for few       */
    LSA_STRATEGY_FUSED = 1,        /* one MFMA scoring pass per query tile that keeps the
                                      buckets above a rising per-query bound, then an exact
                                      finish over those (fp32: a bound pass, then a
                                      candidate pass)                                     */
    LSA_STRATEGY_MATERIALIZED = 2  /* every score and every 16-bucket tile maximum written
                                      to the workspace; the tile maxima bound a small
                                      candidate set that is ranked exactly (an exact radix
                                      select when it is not small); decode: few queries,
                                      many buckets                                        */
} lsa_strategy;

/* Shape of the layer.  latent_dim, pool, block_entries, mean_bucket and
 * max_bucket must equal the LSA_* constants above (the method's values);
 * they are spelled out so a caller states them and a mismatch is caught. */
typedef struct lsa_layout {
    int32_t head_dim;       /* d: 64 or 128                                        */
    int32_t latent_dim;     /* 64                                                  */
    int32_t n_kv_heads;     /* H_kv >= 1                                           */
    int32_t n_q_heads;      /* H_q, a multiple of H_kv, G = H_q / H_kv in 1..8     */
    int32_t pool;           /* 4                                                   */
    int32_t block_entries;  /* 512                                                 */
    int32_t mean_bucket;    /* 8                                                   */
    int32_t max_bucket;     /* 16                                                  */
    int32_t dtype;          /* lsa_dtype of K, V, Q, O, W and the stored centroids */
    int32_t build_tree;     /* 1: also keep the binary tree of merged buckets      */
} lsa_layout;

/* Query-side parameters (ch.3: k long-range keys, sinks, local window; ch.4:
 * tree beam). */
typedef struct lsa_select_cfg {
    int32_t k;         /* long-range budget: 0..LSA_MAX_K, or >= T (take every eligible token) */
    int32_t n_sinks;   /* >= 0                                                          */
    int32_t window;    /* >= 1                                                          */
    int32_t search;    /* lsa_search                                                    */
    int32_t beam;      /* tree only: 1..LSA_MAX_BEAM                                    */
    int32_t strategy;  /* lsa_strategy (flat search only)                               */
    int32_t causal_tree; /* tree only, 0 or 1: score a node that straddles the query's
                          * visible leaves by the centroid of its visible part (the
                          * node as a tree built over the visible blocks has it), so a
                          * prefill query selects what a decode step at its position
                          * does on a cache grown to that point; 0: stored centroids */
    int32_t skip_recorded_lists; /* 0 or 1; with bucket records requested, 1 leaves the
                          * lr_idx row of every (query, KV head) that gets records
                          * unwritten (its lr_cnt is written): for callers that
                          * pass the records to lsa_sparse_attend_bucket_major,
                          * which then reads only the other rows' lists */
} lsa_select_cfg;

/* Byte offsets of the cache regions, for inspection (tests, tools).  Per
 * (b, g): cent [leaves_max, 64] (dtype; in bf16 stored in tiles of 16
 * buckets: element d of bucket x at (x/16)*1024 + ((d/8)%2)*512 +
 * (x%16 + 16*(d/16))*8 + d%8, the scoring operand order), sums [leaves_max, 64] fp32,
 * meta [leaves_max] uint32 (bits 0-7 = entries in the bucket, bits 8-17 =
 * offset of its first member in the block's member list), members
 * [n_blocks_max, 512] uint16 (each block's entry indices grouped by bucket,
 * ascending inside a bucket), entry_leaf [n_blocks_max, 512] uint8 (bucket
 * rank of every entry), tree_cent / tree_sums [nodes_max, 64] for the tree
 * levels above the leaves (level l >= 1 starts at node level_off[l]; each
 * level has room for ceil(leaves_max / 2^l) nodes, so offsets depend on
 * t_max only and a node keeps its place as the cache grows),
 * entry_pos [n_blocks_max, 512] uint8 (position of every entry inside its
 * bucket's member list, so token 4e + j of a bucket is its key number
 * 4 * entry_pos[e] + j in member order), and with a tree edge_cent
 * [n_blocks_max + 1, edge_levels, 64] (dtype): row (nb, l) is the centroid
 * of the level-l node that straddles leaf 64 nb, taken over its leaves
 * below 64 nb only, i.e. that node as a tree over the first nb blocks has it
 * (normalised sum of its visible children's sums; rows of levels with no
 * straddling node are unused). */
typedef struct lsa_cache_info {
    int64_t n_blocks_max;
    int64_t leaves_max;
    int64_t nodes_max;
    int64_t n_blocks;          /* for the T passed to lsa_cache_describe */
    int64_t n_leaves;
    int32_t n_levels;          /* tree levels including the leaves (1 + ceil(log2 n_leaves)) */
    int32_t elt_bytes;         /* 2 (bf16) or 4 (fp32) */
    int64_t level_off[40];     /* node offset of tree level l (l >= 1); level_size = nodes in use */
    int64_t level_size[40];
    size_t off_cent, off_sums, off_meta, off_members, off_entry_leaf, off_tree_cent, off_tree_sums;
    size_t stride_cent, stride_sums, stride_meta, stride_members, stride_entry_leaf,
           stride_tree_cent, stride_tree_sums;   /* bytes between consecutive (b, g) */
    size_t total_bytes;
    size_t off_entry_pos, stride_entry_pos;
    size_t off_edge_cent, stride_edge_cent;   /* tree only: see below */
    int32_t edge_levels;
    /* bf16 only (else 0): each leaf centroid also as int8 codes with one fp32
     * scale per leaf, code = round(centroid / scale), scale = max |component|
     * / 127 (0 for a zero centroid), the codes in tiles of 16 leaves (1 KB:
     * leaf r's 16 codes of dims [16 h, 16 h + 16) at byte 16 (r + 16 h));
     * the flat decode scan bounds the bf16 scores with them */
    size_t off_cent_i8, stride_cent_i8, off_cent_scale, stride_cent_scale;
} lsa_cache_info;

/* Bytes of a bucket cache for `batch` sequences of up to t_max tokens.
 * Host only; no device work. */
lsa_status lsa_cache_bytes(const lsa_layout* layout, int64_t batch, int64_t t_max, size_t* bytes);

/* Region offsets of such a cache when T tokens are bucketed. Host only. */
lsa_status lsa_cache_describe(const lsa_layout* layout, int64_t batch, int64_t t_max, int64_t T,
                              lsa_cache_info* info);

/* Key side (ch.2; ch.4 for the tree).  For every sequence b < batch and KV
 * head g, and every full 2048-token block of the first T tokens: project
 * each key with W_k (64-d), L2-normalise, pool 4 -> 1, run capped Ward down
 * to 64 buckets (<= 16 entries each, ties to the lowest cluster-id pair) and
 * store each bucket's fp32 member sum, its centroid (sum / ||sum||, rounded
 * to nearest even in the dtype), size and members.  With
 * layout->build_tree, also the tree levels (node sum = sum of its children,
 * centroid likewise).  K: [batch, H_kv, t_cap, d] in layout->dtype, T <= t_cap,
 * T <= t_max; cache: cache_bytes >= lsa_cache_bytes(layout, batch, t_max).
 * The cache is then read-only for the other calls. */
lsa_status lsa_build_buckets(const lsa_layout* layout, const void* K, int64_t batch, int64_t t_cap,
                             int64_t T, const void* W_k, void* cache, size_t cache_bytes,
                             int64_t t_max, void* stream);

/* Cache growth (ch.2: each block of 512 pooled keys is clustered once, as
 * the keys stream in, and never again).  The cache holds a build (or
 * extensions) of the first T_old tokens with this layout, batch and t_max;
 * the full blocks of tokens [T_old, T_new) are clustered and their buckets
 * appended exactly as lsa_build_buckets would store them, and with
 * layout->build_tree the tree nodes over the new leaves (the right edge of
 * every level, and any new levels) are recomputed: the cache then equals,
 * bit for bit, a build of the first T_new tokens.  Buckets and nodes over
 * older leaves are not touched, so readers of them may run concurrently on
 * other streams.  K: [batch, H_kv, t_cap, d], T_old <= T_new <= t_cap,
 * T_new <= t_max; errors as lsa_build_buckets (nothing is launched). */
lsa_status lsa_extend_buckets(const lsa_layout* layout, const void* K, int64_t batch, int64_t t_cap,
                              int64_t T_old, int64_t T_new, const void* W_k, void* cache,
                              size_t cache_bytes, int64_t t_max, void* stream);

/* Workspace bytes lsa_select needs for this many queries. Host only. */
lsa_status lsa_select_workspace_bytes(const lsa_layout* layout, const lsa_select_cfg* cfg,
                                      int64_t batch, int64_t n_q, int64_t t_max, size_t* bytes);

/* Query side selection (ch.3 flat search, ch.4 tree search).  For each
 * (b, i, g): q_hat_h = round(normalise(Q[b,i,h] W_q)) for the G heads of
 * group g; score(x) = max_h <q_hat_h, c_x> over the visible buckets x
 * (blocks < nvis; tree: visible nodes on the beam); buckets ranked by
 * (score desc, bucket id asc) are taken whole until k eligible tokens
 * (tokens outside sinks and window), the last one giving its lowest-index
 * eligible tokens.  Writes lr_idx[b,i,g,:] ascending, padded with -1, and
 * lr_cnt[b,i,g] = min(k, eligible tokens of the visible buckets).  A query
 * position outside [0, t_cap) of the K/V it will attend is not checked here;
 * positions < 0 give lr_cnt = -1.  T is the number of bucketed tokens the
 * cache was built with.
 * Optional (both NULL, or both set and 16-byte aligned): bucket_recs
 * [batch, n_q, H_kv, LSA_BUCKET_RECS] records of four uint32 and bucket_cnt
 * [batch, n_q, H_kv] int32, the same selection one record per selected
 * bucket: {leaf id, key mask bits 0..31, bits 32..63, 0}, ascending in leaf
 * id, where key j of a bucket is token 4 members[j / 4] + j % 4 of its block
 * and is in lr_idx's row exactly when bit j is set.  bucket_cnt holds the
 * number of records; it is -1 where the row came from the exact fallback or
 * a trivial case (no ranking needed, or position
 * < 0).  lsa_sparse_attend_bucket_major takes them in place of the token
 * rows' bucket lookups. */
lsa_status lsa_select(const lsa_layout* layout, const lsa_select_cfg* cfg, const void* cache,
                      size_t cache_bytes, int64_t t_max, int64_t T, const void* Q,
                      const int64_t* q_pos, int64_t batch, int64_t n_q, const void* W_q,
                      int32_t* lr_idx, int32_t* lr_cnt, void* bucket_recs, int32_t* bucket_cnt,
                      void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes lsa_sparse_attend needs (split-key partial results). */
lsa_status lsa_attend_workspace_bytes(const lsa_layout* layout, const lsa_select_cfg* cfg,
                                      int64_t batch, int64_t n_q, size_t* bytes);

/* Exact attention over the selected keys (diosapp section 二:
 * softmax(q K[keys]^T / sqrt(d)) V[keys]).  For each (b, i, h):
 * O[b,i,h] = sum_{j in S} softmax_j(scale * <Q[b,i,h], K[b,g,j]>) V[b,g,j]
 * over S = sinks U [l0, t] U lr_idx[b,i,g,:lr_cnt], fp32 softmax with the
 * running max subtracted, O written in the dtype.  K, V: [batch, H_kv,
 * t_cap, d] with every position <= t valid; T = tokens bucketed (fixes the
 * geometry exactly as in lsa_select).  Rows with lr_cnt < 0 are written as
 * zeros. */
lsa_status lsa_sparse_attend(const lsa_layout* layout, const lsa_select_cfg* cfg, const void* Q,
                             const void* K, const void* V, int64_t t_cap, int64_t T,
                             const int64_t* q_pos, int64_t batch, int64_t n_q,
                             const int32_t* lr_idx, const int32_t* lr_cnt, float scale, void* O,
                             void* workspace, size_t workspace_bytes, void* stream);

/* lsa_sparse_attend for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same call with the same arguments and result, except that
 * the split-key partials (needed when few (query, KV head) units are split
 * over their key lists, as in decode) live in a fixed 4 MiB device array of
 * the library instead of a caller workspace.  The call allocates nothing;
 * its first call on a device looks up that device's copy of the array
 * (hipGetSymbolAddress, with the device current; no stream work), so a
 * caller that captures graphs makes one call before capturing.  A call that
 * would need more than 4 MiB (lsa_attend_workspace_bytes; only for G = 8
 * with d = 128 and fewer than 1024 units) fails with LSA_ERR_WORKSPACE
 * before anything is queued.  All calls on one device share its array:
 * calls that overlap in time on one device race and must be ordered (one
 * stream, or events).  Nothing in the array needs clearing between calls. */
lsa_status lsa_sparse_attend_noalloc(const lsa_layout* layout, const lsa_select_cfg* cfg, const void* Q,
                                     const void* K, const void* V, int64_t t_cap, int64_t T,
                                     const int64_t* q_pos, int64_t batch, int64_t n_q,
                                     const int32_t* lr_idx, const int32_t* lr_cnt, float scale, void* O,
                                     void* stream);

/* Workspace bytes lsa_sparse_attend_bucket_major needs to process n_q_pass
 * queries per sequence in one pass (a cache for t_max tokens).  Host only.
 * Dominated by the pool of partials, 80 slots per (query, KV head) on
 * average, one per (query, KV head, bucket) pair (fp32 max, denominator and
 * scale, d fp16 values per head), and a staging row of 256 pair records per
 * (query, KV head): about 80 * (16 + G * (2 d + 16)) + 4104 bytes per
 * (query, KV head). */
lsa_status lsa_attend_bucket_major_workspace_bytes(const lsa_layout* layout, const lsa_select_cfg* cfg,
                                                   int64_t batch, int64_t n_q_pass, int64_t t_max, size_t* bytes);

/* The same attention as lsa_sparse_attend, computed bucket-major (diosapp
 * section 二 for the attention; zhichai.net "卡片柜" ch.3 for the long-range
 * keys being whole buckets): the (query, bucket) pairs of a pass of queries
 * are grouped by bucket through the cache's entry_leaf / entry_pos maps, each
 * bucket's keys and values are read once for every query that listed any of
 * them, and the per-pair softmax partials are merged with the sinks + window
 * part by a log-sum-exp combine.  Arguments as for lsa_sparse_attend plus the
 * cache (built with T tokens for t_max; layout must be the one it was built
 * with, build_tree included, since the cache's regions are found from it)
 * and a workspace of at least
 * lsa_attend_bucket_major_workspace_bytes(.., 1, ..); the call then runs
 * ceil(n_q / P) passes, P the most queries the workspace holds.
 * Precision: each partial's unnormalised output is stored as fp16 values
 * times an exact power-of-two scale per (pair, head), so a value differs
 * from lsa_sparse_attend's by the order of the fp32 sums plus the fp16
 * rounding of each partial value (relative 2^-11 of that value, weighted by
 * the partial's share of the softmax).
 * Rows gathered whole instead (same result, slower): a (query, KV head)
 * whose list is not strictly ascending, holds a token outside
 * [sink end, window start), or touches more than 256 buckets (its list is
 * gathered); and one whose pairs do not fit in the pass's pool of partial
 * slots, which are handed out in query order (its list is gathered, or, for
 * a row with bucket records, the keys its records name, so a row whose list
 * the selection skipped is still attended exactly).  bf16 only
 * (LSA_ERR_UNSUPPORTED otherwise); lr_idx rows must not be modified while
 * the call's kernels run.
 * Optional bucket_recs / bucket_cnt (both NULL, or both set): the records
 * lsa_select wrote with these rows.  A (query, KV head) with bucket_cnt >= 0
 * takes its (query, bucket) pairs from its records instead of looking up
 * every listed token: the same pairs in the same order, so the same output
 * bit for bit.  If a record's bucket lies outside the blocks the query's
 * long-range keys come from, or the masks' bits do not add up to the row's
 * count, the row's list is used instead.
 * Optional fallback_counts (device, two uint32, NULL for none): the call
 * adds the number of rows it gathered whole to [0], and of those the rows
 * whose pairs did not fit in the pool to [1] (the caller zeroes them). */
lsa_status lsa_sparse_attend_bucket_major(const lsa_layout* layout, const lsa_select_cfg* cfg, const void* cache,
                                          size_t cache_bytes, int64_t t_max, const void* Q, const void* K,
                                          const void* V, int64_t t_cap, int64_t T, const int64_t* q_pos,
                                          int64_t batch, int64_t n_q, const int32_t* lr_idx, const int32_t* lr_cnt,
                                          const void* bucket_recs, const int32_t* bucket_cnt, float scale, void* O,
                                          void* workspace, size_t workspace_bytes, uint32_t* fallback_counts,
                                          void* stream);

/* Workspace bytes lsa_pca_projection needs for this layout's head_dim.  Host only. */
lsa_status lsa_pca_workspace_bytes(const lsa_layout* layout, size_t* bytes);

/* Training-free projection (zhichai.net "卡片柜" ch.5: the D-LSA variant
 * that needs no training takes the leading principal directions of the
 * keys).  Over every key K[b, g, t, :] with b < batch, g < H_kv, t < T
 * (N = batch * H_kv * T rows): C = (1/N) sum (k - mean)(k - mean)^T,
 * eigen-decomposed; W [d, 64] (row-major, layout->dtype, rounded to nearest
 * even in bf16) receives the eigenvectors of the 64 largest eigenvalues as
 * columns, in descending order, each with its largest-magnitude component
 * positive.  eigvals (optional, fp32 [d]) receives all eigenvalues,
 * descending.  W serves as both W_k and W_q; the rest of the path depends on
 * it only through the spanned subspace (every latent is normalised).
 * Accumulation in fp32 per workgroup and fp64 across workgroups; the
 * eigen-solver is a cyclic Jacobi in fp32. */
lsa_status lsa_pca_projection(const lsa_layout* layout, const void* K, int64_t batch, int64_t t_cap, int64_t T,
                              void* W, float* eigvals, void* workspace, size_t workspace_bytes, void* stream);

/* Human-readable status name; detail of the last failed call on this thread. */
const char* lsa_status_string(lsa_status status);
const char* lsa_last_error(void);
int32_t lsa_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LSA_H */
