// Query side of LSA on gfx950: latent query, centroid scoring with a max
// over the GQA group's heads, top-bucket selection (flat or tree beam) and
// expansion into sorted long-range token indices.
//
// Method: zhichai.net explainer "卡片柜", ch.3 (score every card, take the
// best p buckets and expand them until k long-range keys, plus sinks and a
// recent window), ch.4 (beam descent of the bucket tree) and ch.5 (the
// bucket score is the max over heads); diosapp.com.cn tutorial, section 二
// (the query is projected by the same latent map).
//
// Exact selection rule: buckets ranked by (score desc, id asc) are taken
// whole until k eligible tokens, the last giving its lowest-index eligible
// tokens.  Three ways to reach it:
//   fused (many queries): a 64-query x bucket-tile bf16 MFMA scan per KV
//     head.  Pass 1 keeps, per query and cluster block, the best bucket and
//     its size and builds a 256-bin histogram of those block maxima weighted
//     by bucket tokens; the bin where the weight reaches k gives a bound tau
//     that the true boundary score cannot undercut.  Pass 2 rescans and keeps
//     every bucket scoring >= tau as a candidate (<= 512).  A per-query wave
//     then sorts the candidates, walks them and expands.  A query with more
//     candidates falls back to the exact path below.
//   materialised (few queries, e.g. decode): all scores are written out,
//     then one workgroup per query finds the boundary key with a weighted
//     4 x 8-bit radix select and collects the selected buckets in id order.
//   tree: one wave per query descends the bucket tree keeping the best
//     `beam` visible children per level, then walks the final beam.

#include "lsa_launch.hpp"

namespace lsa {

namespace {

constexpr float kNegInf = -__builtin_huge_valf();

__device__ __forceinline__ void wave_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

struct Unit {
    int64_t b, i, g, u;
};
__device__ __forceinline__ Unit unit_of(int64_t u, const SelArgs& sa) {
    Unit r;
    r.u = u;
    r.g = u % sa.H_kv;
    const int64_t bi = u / sa.H_kv;
    r.i = bi % sa.n_q;
    r.b = bi / sa.n_q;
    return r;
}

// ------------------------------------------------------------------ q latent
// q_hat = round(normalise(q W)) per (b, i, h) row; one wave handles 4 rows,
// lane c produces latent coordinate c.
template <typename TIN>
__global__ __launch_bounds__(256) void qlatent_kernel(const TIN* __restrict__ Q, const TIN* __restrict__ W, int d,
                                                      int64_t rows, void* qhat, int out_bf16, int* counters) {
    __shared__ float Wsh[128 * kLatent];
    if (blockIdx.x == 0 && threadIdx.x < 4) counters[threadIdx.x] = 0;
    for (int i = threadIdx.x; i < d * kLatent; i += 256) Wsh[i] = load_f32(W + i);
    __syncthreads();
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    for (int64_t r0 = ((int64_t)blockIdx.x * 4 + wid) * 4; r0 < rows; r0 += (int64_t)gridDim.x * 16) {
        float z[4] = {0.f, 0.f, 0.f, 0.f};
        const TIN* q0 = Q + r0 * d;
        for (int dd = 0; dd < d; ++dd) {
            const float w = Wsh[dd * kLatent + lane];
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                const float qv = (r0 + rr < rows) ? load_f32(q0 + (int64_t)rr * d + dd) : 0.f;
                z[rr] = fmaf(qv, w, z[rr]);
            }
        }
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            const float ss = wave_sum(z[rr] * z[rr]);
            const float v = ss > 0.f ? z[rr] * (1.0f / sqrtf(ss)) : 0.f;
            if (r0 + rr < rows) {
                if (out_bf16)
                    reinterpret_cast<uint16_t*>(qhat)[(r0 + rr) * kLatent + lane] = f32_to_bf16(v);
                else
                    reinterpret_cast<float*>(qhat)[(r0 + rr) * kLatent + lane] = v;
            }
        }
    }
}

// ------------------------------------------------------------------ scoring tiles
// Scores of the 16 buckets x0..x0+15 against 16 query slots, max over the
// group's heads.  Output (MFMA C layout): lane l holds buckets
// x0 + 4*(l/16) + v, v = 0..3, for query slot l % 16.
//
// bf16: A = 16 centroids (lane (r = l%16, h = l/16) loads latent dims
// [16h, 16h+16) of bucket x0 + r as two 8-element k-steps), B = the query
// latents of one head with the same dim order, fp32 accumulate.
struct QFragBF16 {
    bf16x8 f[kMaxGroup][2];
};

__device__ __forceinline__ void load_qfrag_bf16(QFragBF16& qf, const uint16_t* qrow_h0, bool valid, int G) {
    const int h = lane_id() >> 4;
#pragma unroll
    for (int hh = 0; hh < kMaxGroup; ++hh) {
        uint4 a = {0, 0, 0, 0}, c = {0, 0, 0, 0};
        if (valid && hh < G) {
            const uint4* p = reinterpret_cast<const uint4*>(qrow_h0 + hh * kLatent + 16 * h);
            a = p[0];
            c = p[1];
        }
        qf.f[hh][0] = as_bf16x8(a);
        qf.f[hh][1] = as_bf16x8(c);
    }
}

__device__ __forceinline__ f32x4 score_tile_bf16(const uint16_t* cent_bg, int64_t x0, const QFragBF16& qf, int G) {
    const int l = lane_id(), r = l & 15, h = l >> 4;
    const uint4* p = reinterpret_cast<const uint4*>(cent_bg + (x0 + r) * kLatent + 16 * h);
    const bf16x8 a0 = as_bf16x8(p[0]), a1 = as_bf16x8(p[1]);
    f32x4 best = {kNegInf, kNegInf, kNegInf, kNegInf};
#pragma unroll
    for (int hh = 0; hh < kMaxGroup; ++hh) {
        if (hh < G) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, qf.f[hh][0], acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, qf.f[hh][1], acc, 0, 0, 0);
            best[0] = fmaxf(best[0], acc[0]);
            best[1] = fmaxf(best[1], acc[1]);
            best[2] = fmaxf(best[2], acc[2]);
            best[3] = fmaxf(best[3], acc[3]);
        }
    }
    return best;
}

// fp32: plain fp32 dot products in the same output layout.
__device__ __forceinline__ f32x4 score_tile_f32(const float* cent_bg, int64_t x0, const float* qrow_h0, bool valid,
                                                int G) {
    const int l = lane_id(), h = l >> 4;
    f32x4 best = {kNegInf, kNegInf, kNegInf, kNegInf};
    if (!valid) return best;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        const float* c = cent_bg + (x0 + 4 * h + v) * kLatent;
        float m = kNegInf;
        for (int hh = 0; hh < G; ++hh) {
            const float* q = qrow_h0 + hh * kLatent;
            float s = 0.f;
            for (int j = 0; j < kLatent; ++j) s = fmaf(q[j], c[j], s);
            m = fmaxf(m, s);
        }
        best[v] = m;
    }
    return best;
}

// ------------------------------------------------------------------ fused flat scan
// PASS 0: per-query bound tau; PASS 1: candidates with score >= tau.
// grid (ceil(n_q / 64), H_kv, B), 4 waves, wave w owns queries 16w..16w+15
// of the tile; every wave scans all buckets visible to any of its queries.
template <bool BF16, int PASS>
__global__ __launch_bounds__(256) void fused_scan_kernel(CacheView cv, const void* __restrict__ qhat,
                                                         const int64_t* __restrict__ q_pos, SelArgs sa,
                                                         float* __restrict__ tau, int* __restrict__ cnt,
                                                         uint64_t* __restrict__ cand) {
    __shared__ uint32_t hist[PASS == 0 ? 4 : 1][16][256];
    __shared__ int lcnt[4][16];
    const int l = lane_id(), wid = threadIdx.x >> 6, n = l & 15, h = l >> 4;
    const int64_t b = blockIdx.z, g = blockIdx.y;
    const int64_t i = (int64_t)blockIdx.x * 64 + wid * 16 + n;
    const bool qv = i < sa.n_q;
    const int64_t t = qv ? q_pos[b * sa.n_q + i] : -1;
    const Geom q = query_geom(t < 0 ? 0 : t, cv.n_blocks, sa.n_sinks, sa.window);
    const int NLv = (t < 0) ? 0 : kLeavesPerBlock * q.nvis;
    const int64_t u = (b * sa.n_q + i) * sa.H_kv + g;
    const int64_t bg = b * sa.H_kv + g;
    const int maxNLv = wave_max_i(NLv), minNLv = wave_min_i(NLv);
    const int64_t qrow = ((b * sa.n_q + i) * sa.H_q + g * sa.G) * kLatent;

    QFragBF16 qf;
    if constexpr (BF16) load_qfrag_bf16(qf, reinterpret_cast<const uint16_t*>(qhat) + (qv ? qrow : 0), qv, sa.G);
    const float* qf32 = reinterpret_cast<const float*>(qhat) + (qv ? qrow : 0);

    float tau_n = 0.f;
    if constexpr (PASS == 0) {
        for (int j = l; j < 16 * 256; j += 64) (&hist[wid][0][0])[j] = 0u;
    } else {
        if (l < 16) lcnt[wid][l] = 0;
        tau_n = qv ? tau[u] : 0.f;
    }
    wave_sync();

    const uint16_t* cb16 = reinterpret_cast<const uint16_t*>(cv.cent) + bg * cv.s_cent;
    const float* cb32 = reinterpret_cast<const float*>(cv.cent) + bg * cv.s_cent;
    const uint32_t* meta = cv.meta + bg * cv.s_meta;

    for (int blk = 0; blk * kLeavesPerBlock < maxNLv; ++blk) {
        uint32_t bmax = 0;
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
            const int64_t x0 = (int64_t)blk * kLeavesPerBlock + 16 * tt;
            f32x4 vals;
            if constexpr (BF16)
                vals = score_tile_bf16(cb16, x0, qf, sa.G);
            else
                vals = score_tile_f32(cb32, x0, qf32, qv, sa.G);
            const int64_t xb = x0 + 4 * h;
            const bool edge = x0 + 16 > minNLv;
            if constexpr (PASS == 0) {
                const uint4 m4 = *reinterpret_cast<const uint4*>(meta + xb);
                const uint32_t mm[4] = {m4.x, m4.y, m4.z, m4.w};
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const uint32_t key = (__float_as_uint(vals[v] + 2.0f) & ~0xFu) | ((mm[v] & 0xFFu) - 1u);
                    const bool ok = !edge || (xb + v < NLv);
                    bmax = (ok && key > bmax) ? key : bmax;
                }
            } else {
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const bool pred = (!edge || (xb + v < NLv)) && qv && vals[v] >= tau_n;
                    if (pred) {
                        const int pos = atomicAdd(&lcnt[wid][n], 1);
                        if (pos < kCandCap) cand[u * kCandCap + pos] = rank_key(vals[v], (uint32_t)(xb + v));
                    }
                }
            }
        }
        if constexpr (PASS == 0) {
            uint32_t o = __shfl_xor(bmax, 16);
            bmax = o > bmax ? o : bmax;
            o = __shfl_xor(bmax, 32);
            bmax = o > bmax ? o : bmax;
            const int64_t lo = (int64_t)blk * kBlockTokens;
            if (h == 0 && qv && bmax != 0u && lo >= q.sink_end && lo + kBlockTokens <= q.l0) {
                const float s = __uint_as_float(bmax & ~0xFu) - 2.0f;
                int bin = (int)floorf((s + 1.0f) * 128.0f);
                bin = bin < 0 ? 0 : (bin > 255 ? 255 : bin);
                hist[wid][n][bin] += (uint32_t)kPool * ((bmax & 0xFu) + 1u);
            }
        }
    }
    wave_sync();
    if constexpr (PASS == 0) {
        if (h == 0 && qv) {
            uint32_t cum = 0;
            float tv = kNegInf;
            for (int bin = 255; bin >= 1; --bin) {
                cum += hist[wid][n][bin];
                if (cum >= (uint32_t)sa.k) {
                    tv = (float)bin * (1.0f / 128.0f) - 1.0f;
                    break;
                }
            }
            tau[u] = tv;
        }
    } else {
        if (h == 0 && qv) cnt[u] = lcnt[wid][n];
    }
}

// ------------------------------------------------------------------ wave-level finish
// Bitonic sort of P (power of two) 64-bit keys in LDS, descending.
__device__ void wave_sort_desc(uint64_t* a, int P) {
    const int l = lane_id();
    for (int size = 2; size <= P; size <<= 1) {
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            for (int j = l; j < (P >> 1); j += 64) {
                const int lo = 2 * stride * (j / stride) + (j % stride), hi = lo + stride;
                const bool desc = (lo & size) == 0;
                const uint64_t x = a[lo], y = a[hi];
                if (desc ? (x < y) : (x > y)) {
                    a[lo] = y;
                    a[hi] = x;
                }
            }
            wave_sync();
        }
    }
}

__device__ __forceinline__ int pow2_at_least(int n) {
    int p = 2;
    while (p < n) p <<= 1;
    return p;
}

// Writes the tokens of the selected buckets in ascending order.  sel[] holds
// (leaf << 16 | take) sorted by leaf; take = kFullTake or, for the single
// boundary bucket, the count of its lowest eligible tokens.  tk[] is a
// 64-entry scratch.  Returns the number of tokens written.
__device__ int wave_expand(const uint64_t* sel, int nsel, const CacheView& cv, int64_t bg, const Geom& q,
                           int32_t* out, int* tk) {
    const int l = lane_id();
    int count = 0;
    int i = 0;
    while (i < nsel) {
        const uint32_t blk = (uint32_t)(sel[i] >> 16) / kLeavesPerBlock;
        int j = i;
        while (true) {
            const int idx = j + l;
            const bool same = idx < nsel && (uint32_t)(sel[idx] >> 16) / kLeavesPerBlock == blk;
            const uint64_t bal = __ballot(same);
            const int run = __popcll(bal);
            j += run;
            if (run < 64) break;
        }
        tk[l] = 0;
        wave_sync();
        for (int idx = i + l; idx < j; idx += 64) {
            const uint64_t s = sel[idx];
            tk[(uint32_t)(s >> 16) % kLeavesPerBlock] = (int)(s & 0xFFFF);
        }
        wave_sync();
        const int my = tk[l];
        const bool is_part = my != 0 && my != kFullTake;
        const uint64_t pb = __ballot(is_part);
        const int prank = pb ? __builtin_ctzll(pb) : -1;
        const int quota = pb ? __shfl(my, prank) : 0;

        const uint64_t rk8 = *reinterpret_cast<const uint64_t*>(cv.eleaf + bg * cv.s_eleaf +
                                                               (int64_t)blk * kBlockEntries + 8 * l);
        const int64_t T0 = (int64_t)blk * kBlockTokens + 32 * l;
        uint32_t emit = 0;   // bit (4e + jj) set when token T0 + 4e + jj is emitted
        uint32_t part = 0;   // eligible tokens of the boundary bucket
        int npart = 0;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int rk = (int)((rk8 >> (8 * e)) & 0x3F);
            const int take = tk[rk];
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const int64_t tok = T0 + 4 * e + jj;
                const bool el = tok >= q.sink_end && tok < q.l0;
                if (!el || take == 0) continue;
                if (take == kFullTake) {
                    emit |= 1u << (4 * e + jj);
                } else {
                    part |= 1u << (4 * e + jj);
                    ++npart;
                }
            }
        }
        if (prank >= 0) {
            const int pre = wave_incl_scan(npart) - npart;
            int seen = pre;
            for (int bit = 0; bit < 32; ++bit) {
                if (part & (1u << bit)) {
                    if (seen < quota) emit |= 1u << bit;
                    ++seen;
                }
            }
        }
        const int ne = __popc(emit);
        const int base = wave_incl_scan(ne) - ne;
        int w = count + base;
        for (int bit = 0; bit < 32; ++bit)
            if (emit & (1u << bit)) out[w++] = (int32_t)(T0 + bit);
        count += __shfl(base + ne, 63);
        wave_sync();
        i = j;
    }
    return count;
}

// Walk keys[0..n) (sorted by rank), pick the buckets until k eligible
// tokens, sort the picks by id into sel[] and expand.  Returns the count.
__device__ int wave_walk_expand(uint64_t* keys, int n, uint64_t* sel, int* tk, const CacheView& cv, int64_t bg,
                                const Geom& q, int k, int32_t* out) {
    const int l = lane_id();
    int have = 0, nsel = 0;
    bool done = false;
    for (int c0 = 0; c0 < n && !done; c0 += 64) {
        const int r = c0 + l;
        const bool in = r < n && keys[r] != 0ull;
        const uint32_t leaf = in ? rank_key_id(keys[r]) : 0u;
        const int w = in ? leaf_weight(cv, bg, leaf, q) : 0;
        const int cum = wave_incl_scan(w) + have;
        const int before = cum - w;
        const bool take = w > 0 && before < k;
        const int tk_n = take ? ((cum <= k) ? kFullTake : (k - before)) : 0;
        const uint64_t bal = __ballot(take);
        const int pos = __popcll(bal & ((1ull << l) - 1ull));
        if (take) sel[nsel + pos] = ((uint64_t)leaf << 16) | (uint64_t)tk_n;
        nsel += __popcll(bal);
        have = __shfl(cum, 63);
        if (have >= k) done = true;
    }
    wave_sync();
    const int P = pow2_at_least(nsel);
    for (int j = nsel + l; j < P; j += 64) sel[j] = ~0ull;   // pads sort after every real entry
    wave_sync();
    // ascending by leaf: sort descending on the complement
    for (int j = l; j < P; j += 64) sel[j] = ~sel[j];
    wave_sync();
    wave_sort_desc(sel, P);
    for (int j = l; j < P; j += 64) sel[j] = ~sel[j];
    wave_sync();
    return wave_expand(sel, nsel, cv, bg, q, out, tk);
}

__device__ void write_pad(int32_t* out, int from, int k) {
    for (int j = from + lane_id(); j < k; j += 64) out[j] = -1;
}

// Handles the cases that need no ranking: invalid position (count -1), and
// a budget covering every eligible token (the whole range [sink_end, l0)).
__device__ bool trivial_unit(int64_t t, const Geom& q, int k, int32_t* out, int32_t* cnt_out) {
    const int l = lane_id();
    if (t < 0) {
        write_pad(out, 0, k);
        if (l == 0) *cnt_out = -1;
        return true;
    }
    if (k == 0) {
        if (l == 0) *cnt_out = 0;
        return true;
    }
    const int64_t total = q.l0 > q.sink_end ? q.l0 - q.sink_end : 0;
    if ((int64_t)k >= total) {
        for (int64_t j = l; j < total; j += 64) out[j] = (int32_t)(q.sink_end + j);
        write_pad(out, (int)total, k);
        if (l == 0) *cnt_out = (int32_t)total;
        return true;
    }
    return false;
}

// ------------------------------------------------------------------ fused finalize
__global__ __launch_bounds__(256) void fused_finalize_kernel(CacheView cv, const int64_t* __restrict__ q_pos, SelArgs sa,
                                                             const int* __restrict__ cnt,
                                                             const uint64_t* __restrict__ cand, int* fb_list,
                                                             int* counters, int32_t* lr_idx, int32_t* lr_cnt) {
    __shared__ uint64_t keys[4][kCandCap];
    __shared__ uint64_t sel[4][kCandCap];
    __shared__ int tk[4][64];
    const int l = lane_id(), wid = threadIdx.x >> 6;
    const int64_t u = (int64_t)blockIdx.x * 4 + wid;
    if (u >= sa.n_units) return;
    const Unit un = unit_of(u, sa);
    const int64_t t = q_pos[un.b * sa.n_q + un.i];
    const Geom q = query_geom(t < 0 ? 0 : t, cv.n_blocks, sa.n_sinks, sa.window);
    int32_t* out = lr_idx + u * sa.k;
    if (trivial_unit(t, q, sa.k, out, lr_cnt + u)) return;
    const int c = cnt[u];
    if (c > kCandCap) {
        if (l == 0) {
            const int pos = atomicAdd(&counters[0], 1);
            fb_list[pos] = (int)u;
        }
        return;
    }
    const int P = pow2_at_least(c);
    for (int j = l; j < P; j += 64) keys[wid][j] = j < c ? cand[u * kCandCap + j] : 0ull;
    wave_sync();
    wave_sort_desc(keys[wid], P);
    const int64_t bg = un.b * sa.H_kv + un.g;
    const int got = wave_walk_expand(keys[wid], c, sel[wid], tk[wid], cv, bg, q, sa.k, out);
    write_pad(out, got, sa.k);
    if (l == 0) lr_cnt[u] = got;
}

// ------------------------------------------------------------------ materialised scores
// grid (n_units, splits): all visible bucket scores of one (query, KV head).
template <bool BF16>
__global__ __launch_bounds__(256) void score_all_kernel(CacheView cv, const void* __restrict__ qhat,
                                                        const int64_t* __restrict__ q_pos, SelArgs sa,
                                                        float* __restrict__ scores, int64_t score_stride) {
    const int l = lane_id(), wid = threadIdx.x >> 6, n = l & 15, h = l >> 4;
    const int64_t u = blockIdx.x;
    const Unit un = unit_of(u, sa);
    const int64_t t = q_pos[un.b * sa.n_q + un.i];
    if (t < 0) return;
    const Geom q = query_geom(t, cv.n_blocks, sa.n_sinks, sa.window);
    const int NLv = kLeavesPerBlock * q.nvis;
    const int ntiles = NLv / 16;
    const int per = (ntiles + gridDim.y - 1) / gridDim.y;
    const int t0 = blockIdx.y * per, t1 = min(ntiles, t0 + per);
    const int64_t bg = un.b * sa.H_kv + un.g;
    const int64_t qrow = ((un.b * sa.n_q + un.i) * sa.H_q + un.g * sa.G) * kLatent;
    QFragBF16 qf;
    if constexpr (BF16) load_qfrag_bf16(qf, reinterpret_cast<const uint16_t*>(qhat) + qrow, n == 0, sa.G);
    const float* qf32 = reinterpret_cast<const float*>(qhat) + qrow;
    float* sc = scores + u * score_stride;
    for (int tt = t0 + wid; tt < t1; tt += 4) {
        const int64_t x0 = (int64_t)tt * 16;
        f32x4 vals;
        if constexpr (BF16)
            vals = score_tile_bf16(reinterpret_cast<const uint16_t*>(cv.cent) + bg * cv.s_cent, x0, qf, sa.G);
        else
            vals = score_tile_f32(reinterpret_cast<const float*>(cv.cent) + bg * cv.s_cent, x0, qf32, n == 0, sa.G);
        if (n == 0) *reinterpret_cast<f32x4*>(sc + x0 + 4 * h) = vals;
    }
}

// Workgroup-wide exclusive scan over 256 threads (4 waves).
__device__ __forceinline__ int wg_excl_scan(int v, int* sh4, int& total) {
    const int l = lane_id(), wid = threadIdx.x >> 6;
    const int inc = wave_incl_scan(v);
    if (l == 63) sh4[wid] = inc;
    __syncthreads();
    int base = 0;
    total = 0;
    for (int w = 0; w < 4; ++w) {
        const int s = sh4[w];
        if (w < wid) base += s;
        total += s;
    }
    __syncthreads();
    return base + inc - v;
}

constexpr int kExactSel = LSA_MAX_K + 2 * kLeavesPerBlock;   // selected buckets held per query

// One workgroup per (query, KV head): weighted radix select of the boundary
// key over materialised scores, then the selected buckets in id order.
// With unit_list, loops over the fallback list and scores its units itself.
template <bool BF16>
__global__ __launch_bounds__(256) void exact_select_kernel(CacheView cv, const void* __restrict__ qhat,
                                                           const int64_t* __restrict__ q_pos, SelArgs sa,
                                                           const int* unit_list, const int* counters,
                                                           float* scores, int64_t score_stride,
                                                           int32_t* lr_idx, int32_t* lr_cnt) {
    __shared__ uint32_t hist[256];
    __shared__ uint64_t sel[kExactSel];
    __shared__ int tk[64];
    __shared__ int sh4[4];
    __shared__ uint32_t bc[4];
    const int tid = threadIdx.x, l = lane_id(), wid = tid >> 6, n = l & 15, h = l >> 4;
    const int n_items = unit_list ? counters[0] : (int)sa.n_units;
    for (int slot = blockIdx.x; slot < n_items; slot += gridDim.x) {
        const int64_t u = unit_list ? unit_list[slot] : slot;
        const Unit un = unit_of(u, sa);
        const int64_t t = q_pos[un.b * sa.n_q + un.i];
        const Geom q = query_geom(t < 0 ? 0 : t, cv.n_blocks, sa.n_sinks, sa.window);
        int32_t* out = lr_idx + u * sa.k;
        if (wid == 0) trivial_unit(t, q, sa.k, out, lr_cnt + u);
        const int64_t total = q.l0 > q.sink_end ? q.l0 - q.sink_end : 0;
        if (t < 0 || sa.k == 0 || (int64_t)sa.k >= total) {
            __syncthreads();
            continue;
        }
        const int NLv = kLeavesPerBlock * q.nvis;
        const int64_t bg = un.b * sa.H_kv + un.g;
        float* sc = scores + (unit_list ? (int64_t)blockIdx.x : u) * score_stride;
        if (unit_list) {
            const int64_t qrow = ((un.b * sa.n_q + un.i) * sa.H_q + un.g * sa.G) * kLatent;
            QFragBF16 qf;
            if constexpr (BF16) load_qfrag_bf16(qf, reinterpret_cast<const uint16_t*>(qhat) + qrow, n == 0, sa.G);
            const float* qf32 = reinterpret_cast<const float*>(qhat) + qrow;
            for (int tt = wid; tt < NLv / 16; tt += 4) {
                const int64_t x0 = (int64_t)tt * 16;
                f32x4 vals;
                if constexpr (BF16)
                    vals = score_tile_bf16(reinterpret_cast<const uint16_t*>(cv.cent) + bg * cv.s_cent, x0, qf, sa.G);
                else
                    vals = score_tile_f32(reinterpret_cast<const float*>(cv.cent) + bg * cv.s_cent, x0, qf32, n == 0,
                                          sa.G);
                if (n == 0) *reinterpret_cast<f32x4*>(sc + x0 + 4 * h) = vals;
            }
            __threadfence_block();
            __syncthreads();
        }
        // weighted radix select: the key K* where the weight of keys >= K* first reaches k
        uint32_t prefix = 0;
        uint32_t target = (uint32_t)sa.k;
        for (int pass = 0; pass < 4; ++pass) {
            hist[tid] = 0u;
            __syncthreads();
            const int shift = 24 - 8 * pass;
            for (int x = tid; x < NLv; x += 256) {
                const uint32_t key = ord_key(sc[x]);
                if (pass > 0 && (key >> (shift + 8)) != prefix) continue;
                const int w = leaf_weight(cv, bg, (uint32_t)x, q);
                if (w > 0) atomicAdd(&hist[(key >> shift) & 0xFFu], (uint32_t)w);
            }
            __syncthreads();
            if (tid == 0) {
                uint32_t cum = 0;
                int dsel = 0;
                for (int dg = 255; dg >= 0; --dg) {
                    const uint32_t hv = hist[dg];
                    if (cum + hv >= target) {
                        dsel = dg;
                        break;
                    }
                    cum += hv;
                }
                bc[0] = (prefix << 8) | (uint32_t)dsel;
                bc[1] = target - cum;
            }
            __syncthreads();
            prefix = bc[0];
            target = bc[1];
            __syncthreads();
        }
        const uint32_t kstar = prefix;   // boundary key; `target` tokens still needed among keys == K*
        // selected buckets in id order
        int nsel = 0, eq_have = 0;
        for (int x0 = 0; x0 < NLv; x0 += 256) {
            const int x = x0 + tid;
            uint32_t key = 0;
            int w = 0;
            if (x < NLv) {
                key = ord_key(sc[x]);
                if (key >= kstar) w = leaf_weight(cv, bg, (uint32_t)x, q);
            }
            const bool gt = w > 0 && key > kstar, eq = w > 0 && key == kstar;
            int eq_tot;
            const int eb = wg_excl_scan(eq ? w : 0, sh4, eq_tot) + eq_have;
            int tkn = 0;
            if (gt) tkn = kFullTake;
            if (eq && eb < (int)target) tkn = (eb + w <= (int)target) ? kFullTake : ((int)target - eb);
            int s_tot;
            const int pos = wg_excl_scan(tkn != 0 ? 1 : 0, sh4, s_tot);
            if (tkn != 0 && nsel + pos < kExactSel) sel[nsel + pos] = ((uint64_t)x << 16) | (uint64_t)tkn;
            nsel += s_tot;
            eq_have += eq_tot;
        }
        __syncthreads();
        if (wid == 0) {
            const int ns = nsel < kExactSel ? nsel : kExactSel;
            const int got = wave_expand(sel, ns, cv, bg, q, out, tk);
            write_pad(out, got, sa.k);
            if (l == 0) lr_cnt[u] = got;
        }
        __syncthreads();
    }
}

// ------------------------------------------------------------------ tree beam descent
// One wave per (query, KV head).  A = the group's query latents (heads as
// rows), B = 16 candidate node centroids per MFMA, so lane l ends with the
// scores of heads 4*(l/16)..+3 for candidate l % 16.
template <bool BF16>
__global__ __launch_bounds__(256) void tree_kernel(CacheView cv, const void* __restrict__ qhat,
                                                   const int64_t* __restrict__ q_pos, SelArgs sa, int32_t* lr_idx,
                                                   int32_t* lr_cnt) {
    __shared__ uint64_t keys[4][2 * LSA_MAX_BEAM];
    __shared__ uint32_t front[4][LSA_MAX_BEAM];
    __shared__ uint64_t sel[4][2 * LSA_MAX_BEAM];
    __shared__ int tk[4][64];
    const int l = lane_id(), wid = threadIdx.x >> 6, n = l & 15, h = l >> 4;
    const int64_t u = (int64_t)blockIdx.x * 4 + wid;
    if (u >= sa.n_units) return;
    const Unit un = unit_of(u, sa);
    const int64_t t = q_pos[un.b * sa.n_q + un.i];
    const Geom q = query_geom(t < 0 ? 0 : t, cv.n_blocks, sa.n_sinks, sa.window);
    int32_t* out = lr_idx + u * sa.k;
    if (trivial_unit(t, q, sa.k, out, lr_cnt + u)) return;
    const int64_t NLv = (int64_t)kLeavesPerBlock * q.nvis;
    const int64_t bg = un.b * sa.H_kv + un.g;
    const int64_t qrow = ((un.b * sa.n_q + un.i) * sa.H_q + un.g * sa.G) * kLatent;
    const int G = sa.G;

    // A fragments (query heads as rows)
    bf16x8 qa0, qa1;
    const float* qrow32 = reinterpret_cast<const float*>(qhat) + qrow;
    if constexpr (BF16) {
        uint4 a = {0, 0, 0, 0}, c = {0, 0, 0, 0};
        if (n < G) {
            const uint4* p =
                reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(qhat) + qrow + n * kLatent + 16 * h);
            a = p[0];
            c = p[1];
        }
        qa0 = as_bf16x8(a);
        qa1 = as_bf16x8(c);
    }

    const int top = cv.n_levels - 1;
    int nf = 1;
    if (l == 0) {
        front[wid][0] = 0;
        keys[wid][0] = rank_key(0.f, 0);
    }
    wave_sync();
    for (int lev = top - 1; lev >= 0; --lev) {
        const int64_t n_lev = cv.level_size[lev];
        const int64_t span = (int64_t)1 << lev;
        const int ncand = 2 * nf;
        const int ntiles = (ncand + 15) / 16;
        for (int tt = 0; tt < ntiles; ++tt) {
            const int c = 16 * tt + n;
            int64_t node = -1;
            if (c < ncand) {
                node = 2 * (int64_t)front[wid][c >> 1] + (c & 1);
                if (node >= n_lev || node * span >= NLv) node = -1;
            }
            float sc = kNegInf;
            if constexpr (BF16) {
                uint4 b0 = {0, 0, 0, 0}, b1 = {0, 0, 0, 0};
                if (node >= 0) {
                    const uint16_t* base =
                        lev == 0 ? reinterpret_cast<const uint16_t*>(cv.cent) + bg * cv.s_cent + node * kLatent
                                 : reinterpret_cast<const uint16_t*>(cv.tcent) + bg * cv.s_tcent +
                                       (cv.level_off[lev] + node) * kLatent;
                    const uint4* p = reinterpret_cast<const uint4*>(base + 16 * h);
                    b0 = p[0];
                    b1 = p[1];
                }
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa0, as_bf16x8(b0), acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa1, as_bf16x8(b1), acc, 0, 0, 0);
#pragma unroll
                for (int v = 0; v < 4; ++v)
                    if (4 * h + v < G) sc = fmaxf(sc, acc[v]);
            } else {
                if (node >= 0) {
                    const float* base = lev == 0 ? reinterpret_cast<const float*>(cv.cent) + bg * cv.s_cent +
                                                       node * kLatent
                                                 : reinterpret_cast<const float*>(cv.tcent) + bg * cv.s_tcent +
                                                       (cv.level_off[lev] + node) * kLatent;
#pragma unroll
                    for (int v = 0; v < 4; ++v) {
                        const int hh = 4 * h + v;
                        if (hh < G) {
                            float s = 0.f;
                            for (int j = 0; j < kLatent; ++j) s = fmaf(qrow32[hh * kLatent + j], base[j], s);
                            sc = fmaxf(sc, s);
                        }
                    }
                }
            }
            sc = fmaxf(sc, __shfl_xor(sc, 16));
            sc = fmaxf(sc, __shfl_xor(sc, 32));
            if (h == 0 && c < 2 * LSA_MAX_BEAM) keys[wid][c] = node >= 0 ? rank_key(sc, (uint32_t)node) : 0ull;
        }
        wave_sync();
        const int P = pow2_at_least(ncand);
        for (int j = ncand + l; j < P; j += 64) keys[wid][j] = 0ull;
        wave_sync();
        wave_sort_desc(keys[wid], P);
        int valid = 0;
        for (int j = l; j < P; j += 64) valid += keys[wid][j] != 0ull ? 1 : 0;
        valid = (int)wave_sum((float)valid);
        nf = valid < sa.beam ? valid : sa.beam;
        for (int j = l; j < nf; j += 64) front[wid][j] = rank_key_id(keys[wid][j]);
        wave_sync();
    }
    const int got = wave_walk_expand(keys[wid], nf, sel[wid], tk[wid], cv, bg, q, sa.k, out);
    write_pad(out, got, sa.k);
    if (l == 0) lr_cnt[u] = got;
}

}  // namespace

// ------------------------------------------------------------------ host launch

hipError_t launch_qlatent(const void* Q, const void* W, bool bf16, int d, int64_t rows, void* qhat, int* counters,
                          hipStream_t st) {
    int64_t need = (rows + 15) / 16;
    unsigned grid = (unsigned)(need < 2048 ? (need > 0 ? need : 1) : 2048);
    if (bf16)
        hipLaunchKernelGGL(qlatent_kernel<uint16_t>, dim3(grid), dim3(256), 0, st, static_cast<const uint16_t*>(Q),
                           static_cast<const uint16_t*>(W), d, rows, qhat, 1, counters);
    else
        hipLaunchKernelGGL(qlatent_kernel<float>, dim3(grid), dim3(256), 0, st, static_cast<const float*>(Q),
                           static_cast<const float*>(W), d, rows, qhat, 0, counters);
    return hipGetLastError();
}

hipError_t launch_select_fused(const CacheView& cv, bool bf16, const int64_t* q_pos, const SelArgs& sa, int B,
                               const SelectBuffers& sb, int32_t* lr_idx, int32_t* lr_cnt, hipStream_t st) {
    dim3 grid((unsigned)((sa.n_q + 63) / 64), (unsigned)sa.H_kv, (unsigned)B);
    if (bf16) {
        hipLaunchKernelGGL((fused_scan_kernel<true, 0>), grid, dim3(256), 0, st, cv, sb.qhat, q_pos, sa, sb.tau, sb.cnt,
                           sb.cand);
        hipLaunchKernelGGL((fused_scan_kernel<true, 1>), grid, dim3(256), 0, st, cv, sb.qhat, q_pos, sa, sb.tau, sb.cnt,
                           sb.cand);
    } else {
        hipLaunchKernelGGL((fused_scan_kernel<false, 0>), grid, dim3(256), 0, st, cv, sb.qhat, q_pos, sa, sb.tau,
                           sb.cnt, sb.cand);
        hipLaunchKernelGGL((fused_scan_kernel<false, 1>), grid, dim3(256), 0, st, cv, sb.qhat, q_pos, sa, sb.tau,
                           sb.cnt, sb.cand);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(fused_finalize_kernel, dim3((unsigned)((sa.n_units + 3) / 4)), dim3(256), 0, st, cv, q_pos, sa,
                       sb.cnt, sb.cand, sb.fb_list, sb.counters, lr_idx, lr_cnt);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (bf16)
        hipLaunchKernelGGL(exact_select_kernel<true>, dim3((unsigned)sb.fb_slots), dim3(256), 0, st, cv, sb.qhat, q_pos,
                           sa, sb.fb_list, sb.counters, sb.scores, sb.score_stride, lr_idx, lr_cnt);
    else
        hipLaunchKernelGGL(exact_select_kernel<false>, dim3((unsigned)sb.fb_slots), dim3(256), 0, st, cv, sb.qhat,
                           q_pos, sa, sb.fb_list, sb.counters, sb.scores, sb.score_stride, lr_idx, lr_cnt);
    return hipGetLastError();
}

hipError_t launch_select_materialized(const CacheView& cv, bool bf16, const int64_t* q_pos, const SelArgs& sa,
                                      const SelectBuffers& sb, int32_t* lr_idx, int32_t* lr_cnt, hipStream_t st) {
    const int64_t ntiles_max = (int64_t)cv.n_blocks * kLeavesPerBlock / 16;
    int splits = (int)((ntiles_max + 63) / 64);
    if (splits < 1) splits = 1;
    if (splits > 64) splits = 64;
    dim3 grid((unsigned)sa.n_units, (unsigned)splits);
    if (bf16)
        hipLaunchKernelGGL(score_all_kernel<true>, grid, dim3(256), 0, st, cv, sb.qhat, q_pos, sa, sb.scores,
                           sb.score_stride);
    else
        hipLaunchKernelGGL(score_all_kernel<false>, grid, dim3(256), 0, st, cv, sb.qhat, q_pos, sa, sb.scores,
                           sb.score_stride);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (bf16)
        hipLaunchKernelGGL(exact_select_kernel<true>, dim3((unsigned)sa.n_units), dim3(256), 0, st, cv, sb.qhat, q_pos,
                           sa, (const int*)nullptr, sb.counters, sb.scores, sb.score_stride, lr_idx, lr_cnt);
    else
        hipLaunchKernelGGL(exact_select_kernel<false>, dim3((unsigned)sa.n_units), dim3(256), 0, st, cv, sb.qhat,
                           q_pos, sa, (const int*)nullptr, sb.counters, sb.scores, sb.score_stride, lr_idx, lr_cnt);
    return hipGetLastError();
}

hipError_t launch_select_tree(const CacheView& cv, bool bf16, const int64_t* q_pos, const SelArgs& sa,
                              const SelectBuffers& sb, int32_t* lr_idx, int32_t* lr_cnt, hipStream_t st) {
    dim3 grid((unsigned)((sa.n_units + 3) / 4));
    if (bf16)
        hipLaunchKernelGGL(tree_kernel<true>, grid, dim3(256), 0, st, cv, sb.qhat, q_pos, sa, lr_idx, lr_cnt);
    else
        hipLaunchKernelGGL(tree_kernel<false>, grid, dim3(256), 0, st, cv, sb.qhat, q_pos, sa, lr_idx, lr_cnt);
    return hipGetLastError();
}

}  // namespace lsa
