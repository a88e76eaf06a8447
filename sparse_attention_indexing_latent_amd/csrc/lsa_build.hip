// Key side of LSA on gfx950: latent projection, L2 normalisation, 4-key
// pooling and capped Ward clustering per 512-entry block, then the centroids
// and the binary tree of merged buckets.
//
// Method: zhichai.net explainer "卡片柜", ch.2 (project to 64-d, normalise,
// pool 4 keys, Ward inside each 512-entry block to buckets of mean 8 / max
// 16, normalised bucket mean as the card) and ch.4 (complete binary tree,
// node centroid = mean of all keys below).
//
// One workgroup of 512 threads clusters one block; thread i owns entry i and,
// while it is alive, the cluster whose smallest member is i (its id).  Each
// thread keeps its cluster mean (64 fp32) in registers together with its
// nearest allowed partner among larger ids (nn, delta).  A merge step is a
// workgroup argmin over (delta, id, nn) — the lowest (id_A, id_B) wins ties —
// followed by recomputing, from broadcast means, the partner of the merged
// cluster and of every cluster whose partner was A or B; every other
// cluster only compares its partner with the merged cluster.  This is the
// same greedy decision sequence as rescanning all pairs every step.

#include "lsa_launch.hpp"

namespace lsa {

namespace {

constexpr int kWardThreads = 512;
constexpr int kRows = 16;             // broadcast rows per recompute round
constexpr float kInf = __builtin_huge_valf();

// Wave minimum of a 64-bit key with DPP moves (no LDS round trips): pairs
// within quads, then halves and rows of 16 (mirrors), then rows 0+1 and
// 2+3 (row broadcast of lane 15), then all four (broadcast of lane 31); the
// minimum ends in lane 63 and is read from there by every lane.
template <int CTRL, int ROWS>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t v) {
    const int lo = (int)(uint32_t)v, hi = (int)(uint32_t)(v >> 32);
    const int dlo = __builtin_amdgcn_update_dpp(lo, lo, CTRL, ROWS, 0xF, false);
    const int dhi = __builtin_amdgcn_update_dpp(hi, hi, CTRL, ROWS, 0xF, false);
    return ((uint64_t)(uint32_t)dhi << 32) | (uint32_t)dlo;
}
__device__ __forceinline__ uint64_t min_u64(uint64_t a, uint64_t b) { return b < a ? b : a; }
__device__ __forceinline__ uint64_t wave_min_u64_dpp(uint64_t v) {
    v = min_u64(v, dpp_u64<0xB1, 0xF>(v));    // quad_perm [1,0,3,2]
    v = min_u64(v, dpp_u64<0x4E, 0xF>(v));    // quad_perm [2,3,0,1]
    v = min_u64(v, dpp_u64<0x141, 0xF>(v));   // row_half_mirror
    v = min_u64(v, dpp_u64<0x140, 0xF>(v));   // row_mirror
    v = min_u64(v, dpp_u64<0x142, 0xA>(v));   // row_bcast:15 into rows 1 and 3
    v = min_u64(v, dpp_u64<0x143, 0xC>(v));   // row_bcast:31 into rows 2 and 3
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, 63);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), 63);
    return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ uint64_t pair_key(float d, int id, int nn) {
    return ((uint64_t)__float_as_uint(d) << 32) | ((uint64_t)id << 16) | (uint64_t)nn;
}

// Register budget: 128 VGPRs (4 waves per SIMD), so two 512-thread workgroups
// share a CU.  A block's 448 merges are a chain of barriers and workgroup
// reductions, so a second block on the CU fills the first one's waits; the
// values that do not fit (88 VGPRs, mostly the cluster mean's components
// between recomputes) spill to scratch.  Measured on the 1M layer (4096 x 8
// blocks): 53.7 ms with one workgroup per CU (156 VGPRs, no spills), 32.2 ms
// with two, 44.1 and 133 ms with three and four (more spills).
template <typename TIN>
__global__ __launch_bounds__(kWardThreads) __attribute__((amdgpu_waves_per_eu(4, 4))) void ward_kernel(const TIN* __restrict__ K, int64_t t_cap, int d,
                                                            int H_kv, const TIN* __restrict__ W, CacheView cv,
                                                            int blk0) {
    const int blk = blk0 + blockIdx.x, g = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int64_t bg = (int64_t)b * H_kv + g;

    __shared__ __align__(16) float Wsh[128 * kLatent];     // projection (phase 1) / entry chunks (phase 2 init)
    __shared__ __align__(16) float rowv[kRows][kLatent];   // broadcast means
    __shared__ int row_id[kRows], row_n[kRows];
    __shared__ uint64_t red[8];
    __shared__ uint64_t red2[8][kRows];
    __shared__ __align__(16) float sBmu[kLatent];
    __shared__ int sBn, nrows;
    __shared__ short lab[kWardThreads];
    __shared__ short rank_of[kWardThreads];
    __shared__ int size_by_rank[kLeavesPerBlock];
    __shared__ int wcnt[8];

    // ---------------- phase 1: pooled entry e_i = mean of the 4 unit latents
    for (int i = tid; i < d * kLatent; i += kWardThreads) Wsh[i] = load_f32(W + i);
    __syncthreads();
    float mu[kLatent];
#pragma unroll
    for (int c = 0; c < kLatent; ++c) mu[c] = 0.f;
    const int64_t tok0 = (int64_t)blk * kBlockTokens + (int64_t)kPool * tid;
    const TIN* kr = K + (bg * t_cap + tok0) * d;
    for (int j = 0; j < kPool; ++j) {
        float z[kLatent];
#pragma unroll
        for (int c = 0; c < kLatent; ++c) z[c] = 0.f;
        const TIN* row = kr + (int64_t)j * d;
        for (int dd = 0; dd < d; ++dd) {
            const float kv = load_f32(row + dd);
            const float4* wr = reinterpret_cast<const float4*>(Wsh + dd * kLatent);
#pragma unroll
            for (int c4 = 0; c4 < kLatent / 4; ++c4) {
                const float4 w = wr[c4];
                z[4 * c4 + 0] = fmaf(kv, w.x, z[4 * c4 + 0]);
                z[4 * c4 + 1] = fmaf(kv, w.y, z[4 * c4 + 1]);
                z[4 * c4 + 2] = fmaf(kv, w.z, z[4 * c4 + 2]);
                z[4 * c4 + 3] = fmaf(kv, w.w, z[4 * c4 + 3]);
            }
        }
        float ss = 0.f;
#pragma unroll
        for (int c = 0; c < kLatent; ++c) ss = fmaf(z[c], z[c], ss);
        const float inv = ss > 0.f ? 1.0f / sqrtf(ss) : 0.f;
#pragma unroll
        for (int c = 0; c < kLatent; ++c) mu[c] = fmaf(z[c], inv, mu[c]);
    }
#pragma unroll
    for (int c = 0; c < kLatent; ++c) mu[c] *= 0.25f;

    // ---------------- phase 2: capped Ward
    int n = 1;
    bool act = true;
    lab[tid] = (short)tid;
    float nd = kInf;
    int nn = -1;
    // initial partners: singletons, delta = |e_i - e_j|^2 / 2 over j > i
    for (int c0 = 0; c0 < kWardThreads; c0 += 32) {
        __syncthreads();
        if (tid >= c0 && tid < c0 + 32) {
#pragma unroll
            for (int c = 0; c < kLatent; ++c) Wsh[(tid - c0) * kLatent + c] = mu[c];
        }
        __syncthreads();
        if (c0 + 31 > tid) {
            for (int jj = 0; jj < 32; ++jj) {
                const int j = c0 + jj;
                if (j <= tid) continue;
                const float4* er = reinterpret_cast<const float4*>(Wsh + jj * kLatent);
                float dist = 0.f;
#pragma unroll
                for (int c4 = 0; c4 < kLatent / 4; ++c4) {
                    const float4 e = er[c4];
                    float t0 = mu[4 * c4 + 0] - e.x, t1 = mu[4 * c4 + 1] - e.y;
                    float t2 = mu[4 * c4 + 2] - e.z, t3 = mu[4 * c4 + 3] - e.w;
                    dist = fmaf(t0, t0, dist);
                    dist = fmaf(t1, t1, dist);
                    dist = fmaf(t2, t2, dist);
                    dist = fmaf(t3, t3, dist);
                }
                const float dl = 0.5f * dist;
                if (dl < nd) {
                    nd = dl;
                    nn = j;
                }
            }
        }
    }

    const int n_merge = kBlockEntries - kLeavesPerBlock;
    for (int step = 0; step < n_merge; ++step) {
        uint64_t key = (act && nn >= 0) ? pair_key(nd, tid, nn) : ~0ull;
        key = wave_min_u64_dpp(key);
        if (lane == 0) red[wid] = key;
        if (tid == 0) nrows = 1;
        __syncthreads();
        key = red[0];
#pragma unroll
        for (int w = 1; w < 8; ++w) key = red[w] < key ? red[w] : key;
        if (key == ~0ull) break;  // no allowed pair: impossible before 64 clusters remain
        const int A = (int)((key >> 16) & 0xFFFF), B = (int)(key & 0xFFFF);
        bool redo = act && tid != A && tid != B && (nn == A || nn == B);
        if (tid == B) {
#pragma unroll
            for (int c = 0; c < kLatent; ++c) sBmu[c] = mu[c];
            sBn = n;
            act = false;
            nn = -1;
            nd = kInf;
        }
        __syncthreads();
        if (tid == A) {
            const float fa = (float)n, fb = (float)sBn, inv = 1.0f / (float)(n + sBn);
#pragma unroll
            for (int c = 0; c < kLatent; ++c) {
                mu[c] = (fa * mu[c] + fb * sBmu[c]) * inv;
                rowv[0][c] = mu[c];
            }
            n += sBn;
            row_id[0] = A;
            row_n[0] = n;
            // its partner is recomputed from scratch below
            nn = -1;
            nd = kInf;
        }
        if (lab[tid] == B) lab[tid] = (short)A;

        bool first = true;
        while (true) {
            if (!first) {
                if (tid == 0) nrows = 0;
                __syncthreads();
            }
            if (redo) {
                const int s = atomicAdd(&nrows, 1);
                if (s < kRows) {
#pragma unroll
                    for (int c = 0; c < kLatent; ++c) rowv[s][c] = mu[c];
                    row_id[s] = tid;
                    row_n[s] = n;
                    redo = false;
                }
            }
            __syncthreads();
            const int nr = nrows < kRows ? nrows : kRows;
            for (int r = 0; r < nr; ++r) {
                const int Kr = row_id[r], nK = row_n[r];
                const bool ok = act && tid != Kr && (nK + n <= kMaxBucket);
                float dl = kInf;
                if (ok) {
                    const float4* rv = reinterpret_cast<const float4*>(rowv[r]);
                    float dist = 0.f;
#pragma unroll
                    for (int c4 = 0; c4 < kLatent / 4; ++c4) {
                        const float4 e = rv[c4];
                        float t0 = mu[4 * c4 + 0] - e.x, t1 = mu[4 * c4 + 1] - e.y;
                        float t2 = mu[4 * c4 + 2] - e.z, t3 = mu[4 * c4 + 3] - e.w;
                        dist = fmaf(t0, t0, dist);
                        dist = fmaf(t1, t1, dist);
                        dist = fmaf(t2, t2, dist);
                        dist = fmaf(t3, t3, dist);
                    }
                    dl = ((float)(nK * n) / (float)(nK + n)) * dist;
                }
                // clusters with smaller ids only compare their partner with the merged one
                if (first && r == 0 && ok && tid < Kr && !(nn == A || nn == B)) {
                    if (dl < nd || (dl == nd && Kr < nn)) {
                        nd = dl;
                        nn = Kr;
                    }
                }
                uint64_t k2 = (ok && tid > Kr) ? (((uint64_t)__float_as_uint(dl) << 32) | (uint64_t)tid) : ~0ull;
                k2 = wave_min_u64_dpp(k2);
                if (lane == 0) red2[wid][r] = k2;
            }
            __syncthreads();
            for (int r = 0; r < nr; ++r) {
                if (tid == row_id[r]) {
                    uint64_t k = red2[0][r];
#pragma unroll
                    for (int w = 1; w < 8; ++w) k = red2[w][r] < k ? red2[w][r] : k;
                    if (k == ~0ull) {
                        nn = -1;
                        nd = kInf;
                    } else {
                        nn = (int)(k & 0xFFFF);
                        nd = __uint_as_float((uint32_t)(k >> 32));
                    }
                }
            }
            first = false;
            if (!__syncthreads_or(redo ? 1 : 0)) break;
        }
    }
    __syncthreads();

    // ---------------- phase 3: leaves of this block, ordered by id
    const uint64_t bal = __ballot(act);
    if (lane == 0) wcnt[wid] = __popcll(bal);
    __syncthreads();
    int base = 0;
    for (int w = 0; w < wid; ++w) base += wcnt[w];
    const int rank = base + __popcll(bal & ((1ull << lane) - 1ull));
    rank_of[tid] = act ? (short)rank : (short)-1;
    if (act) size_by_rank[rank] = n;
    __syncthreads();
    cv.eleaf[bg * cv.s_eleaf + (int64_t)blk * kBlockEntries + tid] = (uint8_t)rank_of[lab[tid]];
    if (act) {
        int off = 0;
        for (int r = 0; r < rank; ++r) off += size_by_rank[r];
        const int64_t leaf = (int64_t)blk * kLeavesPerBlock + rank;
        float* srow = cv.sums + bg * cv.s_sums + leaf * kLatent;
        float ss = 0.f;
#pragma unroll
        for (int c = 0; c < kLatent; ++c) {
            srow[c] = mu[c] * (float)n;
            ss = fmaf(mu[c], mu[c], ss);
        }
        const float inv = ss > 0.f ? 1.0f / sqrtf(ss) : 0.f;
        if (cv.bf16) {   // tile-swizzled: eight 16-byte words (h, m) of 8 consecutive dims
            uint4* cw = reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(cv.cent) + bg * cv.s_cent);
#pragma unroll
            for (int h = 0; h < 4; ++h)
#pragma unroll
                for (int m = 0; m < 2; ++m) {
                    const int c = 16 * h + 8 * m;
                    uint32_t w[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        w[e] = (uint32_t)f32_to_bf16(mu[c + 2 * e] * inv) |
                               ((uint32_t)f32_to_bf16(mu[c + 2 * e + 1] * inv) << 16);
                    cw[cent_tile_word(leaf, h, m)] = uint4{w[0], w[1], w[2], w[3]};
                }
            // int8 codes of the rounded centroid: scale = max |c| / 127, code = round(c / scale)
            float amax = 0.f;
#pragma unroll
            for (int c = 0; c < kLatent; ++c) amax = fmaxf(amax, fabsf(bf16_to_f32(f32_to_bf16(mu[c] * inv))));
            const float sc = amax / 127.0f;
            uint4* qw = reinterpret_cast<uint4*>(cv.cq + bg * cv.s_cq);
#pragma unroll
            for (int h = 0; h < 4; ++h) {
                uint32_t w[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    uint32_t word = 0;
#pragma unroll
                    for (int b = 0; b < 4; ++b) {
                        const float c = bf16_to_f32(f32_to_bf16(mu[16 * h + 4 * e + b] * inv));
                        const int code = sc > 0.f ? (int)fminf(fmaxf(rintf(c / sc), -127.f), 127.f) : 0;
                        word |= (uint32_t)(uint8_t)(int8_t)code << (8 * b);
                    }
                    w[e] = word;
                }
                qw[(leaf >> 4) * 64 + (leaf & 15) + 16 * h] = uint4{w[0], w[1], w[2], w[3]};
            }
            cv.csc[bg * cv.s_csc + leaf] = sc;
        } else {
            float* crow = reinterpret_cast<float*>(cv.cent) + bg * cv.s_cent + leaf * kLatent;
#pragma unroll
            for (int c = 0; c < kLatent; ++c) crow[c] = mu[c] * inv;
        }
        cv.meta[bg * cv.s_meta + leaf] = (uint32_t)n | ((uint32_t)off << 8);
        uint16_t* mem = cv.members + bg * cv.s_members + (int64_t)blk * kBlockEntries + off;
        int cnt = 0;
        uint8_t* pos = cv.epos + bg * cv.s_epos + (int64_t)blk * kBlockEntries;
        for (int j = tid; j < kWardThreads && cnt < n; ++j)
            if (lab[j] == tid) {
                pos[j] = (uint8_t)cnt;
                mem[cnt++] = (uint16_t)j;
            }
    }
}

// One wave per tree node: sum of the two children (an odd last node has
// one), its norm, and the rounded centroid (ch.4: node centroid = mean of
// every key below it; the normalisation makes mean and sum equivalent).
__global__ __launch_bounds__(256) void tree_level_kernel(CacheView cv, int lev, int64_t n_child, int64_t n_par,
                                                         int64_t child_off, int64_t par_off, int64_t first) {
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    const int64_t node = first + (int64_t)blockIdx.x * 4 + wid;
    if (node >= n_par) return;
    const int64_t bg = blockIdx.y;
    const float* cs = lev == 1 ? cv.sums + bg * cv.s_sums : cv.tsums + bg * cv.s_tsums + child_off * kLatent;
    const int64_t c0 = 2 * node, c1 = c0 + 1;
    float s = cs[c0 * kLatent + lane];
    if (c1 < n_child) s += cs[c1 * kLatent + lane];
    const int64_t o = (par_off + node) * kLatent + lane;
    cv.tsums[bg * cv.s_tsums + o] = s;
    const float ss = wave_sum(s * s);
    const float v = ss > 0.f ? s * (1.0f / sqrtf(ss)) : 0.f;
    if (cv.bf16)
        reinterpret_cast<uint16_t*>(cv.tcent)[bg * cv.s_tcent + o] = f32_to_bf16(v);
    else
        reinterpret_cast<float*>(cv.tcent)[bg * cv.s_tcent + o] = v;
}

// Edge table: one wave per (b, g) and block boundary nb (m = 64 nb leaves).
// At level l the node straddling leaf m is j = (m - 1) >> l (none when m is
// a multiple of 2^l); as a node of the tree over the first m leaves its sum
// is its left child's sum (complete when m >= the children's midpoint) plus
// its right child's partial sum (the straddling node one level down) when
// m passes the midpoint, else its left child's partial sum: the additions
// tree_level_kernel makes for a tree built over m leaves, so the centroid
// is bit for bit that tree's.  Rows are written for every level of a tree
// over leaves_max leaves.
__global__ __launch_bounds__(256) void tree_edge_kernel(CacheView cv, int nb_first) {
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    const int64_t nb = nb_first + (int64_t)blockIdx.x * 4 + wid;
    if (nb > cv.n_blocks) return;
    const int64_t bg = blockIdx.y;
    const int64_t m = nb * kLeavesPerBlock;
    float part = 0.f;   // partial sum of the straddling node one level down
    // every level of the capacity tree: above the current top, node 0 straddles and only reads
    // nodes that exist (m <= the midpoint), so the rows do not depend on when they were written
    for (int lev = 1; lev < cv.n_lev_cap; ++lev) {
        if ((m & (((int64_t)1 << lev) - 1)) == 0) continue;   // no straddling node at this level
        const int64_t j = (m - 1) >> lev;
        const int64_t mid = (2 * j + 1) << (lev - 1);
        float s;
        if (m >= mid) {
            const int64_t c0 = 2 * j;
            s = lev == 1 ? cv.sums[bg * cv.s_sums + c0 * kLatent + lane]
                         : cv.tsums[bg * cv.s_tsums + (tree_level_off(cv.n_leaves_cap, lev - 1) + c0) * kLatent + lane];
            if (m > mid) s += part;
        } else {
            s = part;
        }
        part = s;
        const float ss = wave_sum(s * s);
        const float v = ss > 0.f ? s * (1.0f / sqrtf(ss)) : 0.f;
        const int64_t o = bg * cv.s_edge + (nb * cv.n_lev_cap + lev) * kLatent + lane;
        if (cv.bf16)
            reinterpret_cast<uint16_t*>(cv.edge)[o] = f32_to_bf16(v);
        else
            reinterpret_cast<float*>(cv.edge)[o] = v;
    }
}

}  // namespace

hipError_t launch_edges(const CacheView& cv, int B, int H_kv, int nb_first, hipStream_t st) {
    if (nb_first > cv.n_blocks) return hipSuccess;
    const int64_t n = cv.n_blocks - nb_first + 1;
    dim3 grid((unsigned)((n + 3) / 4), (unsigned)(B * H_kv));
    hipLaunchKernelGGL(tree_edge_kernel, grid, dim3(256), 0, st, cv, nb_first);
    return hipGetLastError();
}

hipError_t launch_build(const CacheView& cv, const void* K, bool bf16, int64_t t_cap, int d, int B, int H_kv,
                        const void* W, hipStream_t st, int blk0) {
    if (cv.n_blocks > blk0) {
        dim3 grid(cv.n_blocks - blk0, H_kv, B);
        if (bf16)
            hipLaunchKernelGGL(ward_kernel<uint16_t>, grid, dim3(kWardThreads), 0, st,
                               static_cast<const uint16_t*>(K), t_cap, d, H_kv, static_cast<const uint16_t*>(W), cv,
                               blk0);
        else
            hipLaunchKernelGGL(ward_kernel<float>, grid, dim3(kWardThreads), 0, st, static_cast<const float*>(K),
                               t_cap, d, H_kv, static_cast<const float*>(W), cv, blk0);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t launch_tree(const CacheView& cv, const int64_t* level_off, const int64_t* level_size, int B, int H_kv,
                       hipStream_t st, int64_t first_leaf) {
    // nodes from the one over first_leaf on (all of them for a build; the new right edge when the
    // cache grows: the nodes over older leaves only are unchanged)
    for (int lev = 1; lev < cv.n_levels; ++lev) {
        const int64_t n_child = level_size[lev - 1], n_par = level_size[lev];
        const int64_t first = first_leaf >> lev;
        if (first >= n_par) continue;
        dim3 grid((unsigned)((n_par - first + 3) / 4), (unsigned)(B * H_kv));
        hipLaunchKernelGGL(tree_level_kernel, grid, dim3(256), 0, st, cv, lev, n_child, n_par, level_off[lev - 1],
                           level_off[lev], first);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace lsa
