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
//   fused (many queries): an MFMA scan of the centroids per KV head, 128
//     queries x 16-bucket tiles (bf16; fp32 in two passes of 64 queries).
//     Each query keeps a histogram of eligible token weight over score bins
//     and a floor: the bin where that weight, summed from the top, reaches
//     k.  Buckets at or above the floor are appended to the query's
//     candidate list and binned; the final crossing bin gives a bound tau
//     that the true boundary score cannot undercut.  A per-query wave then
//     keeps the candidates scoring >= tau (<= 512), sorts, walks and expands
//     them.  A query with more falls back to the exact path below.
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

// Grid-stride clear of zero_n 16-byte words (the per-call counters and
// histograms of the materialised path; a kernel rather than a memset node).
__device__ __forceinline__ void clear_words(uint4* zero, int64_t zero_n) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < zero_n; i += (int64_t)gridDim.x * blockDim.x)
        zero[i] = uint4{0u, 0u, 0u, 0u};
}

// ------------------------------------------------------------------ q latent
// q_hat = round(normalise(q W)) per (b, i, h) row; one wave handles 4 rows,
// lane c produces latent coordinate c.
template <typename TIN>
__global__ __launch_bounds__(256) void qlatent_kernel(const TIN* __restrict__ Q, const TIN* __restrict__ W, int d,
                                                      int64_t rows, void* qhat, int out_bf16, int* counters,
                                                      uint4* zero, int64_t zero_n) {
    __shared__ float Wsh[128 * kLatent];
    if (blockIdx.x == 0 && threadIdx.x < 4) counters[threadIdx.x] = 0;
    clear_words(zero, zero_n);
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

// bf16: 16 query rows per MFMA tile, Q [16 x d] . W [d x 64] as 4 column
// tiles; lane (r, h) feeds head dims [d/4 h, d/4 h + d/4) of row r, the W
// fragments use the same dim order.  The C layout gives lane (n, h) rows
// 4h..4h+3 of latent column n of each tile; row norms are reduced over the
// 16 lanes of a row group.  One code path for the latent kernel and for the
// decode scan (which computes its unit's rows itself), so both give the
// same q_hat bit for bit.
template <int D>
__device__ __forceinline__ void qlatent_w_frag(const uint16_t* __restrict__ W, int nt, bf16x8 (&wf)[D / 32]) {
    constexpr int DPL = D / 4, KS = DPL / 8;
    const int l = lane_id(), r = l & 15, h = l >> 4;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        uint16_t e[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) e[j] = W[(DPL * h + 8 * ks + j) * kLatent + 16 * nt + r];
        wf[ks] = as_bf16x8(uint4{(uint32_t)e[0] | ((uint32_t)e[1] << 16), (uint32_t)e[2] | ((uint32_t)e[3] << 16),
                                 (uint32_t)e[4] | ((uint32_t)e[5] << 16), (uint32_t)e[6] | ((uint32_t)e[7] << 16)});
    }
}

// Query rows row0 .. row0 + 15 (rows >= `rows` read as zero) as A fragments.
template <int D>
__device__ __forceinline__ void qlatent_q_frag(const uint16_t* __restrict__ Q, int64_t row0, int64_t rows,
                                               uint4 (&qa)[D / 32]) {
    constexpr int DPL = D / 4, KS = DPL / 8;
    const int l = lane_id(), r = l & 15, h = l >> 4;
    const int64_t row = row0 + r;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
        qa[ks] = row < rows ? *reinterpret_cast<const uint4*>(Q + row * D + DPL * h + 8 * ks) : uint4{0, 0, 0, 0};
}

// The rounded unit rows: out[nt][v] = q_hat[row0 + 4h + v][16 nt + n] for lane (n, h).
__device__ __forceinline__ void qlatent_normalise(const f32x4 (&c)[4], uint16_t (&out)[4][4]) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        float ss = c[0][v] * c[0][v] + c[1][v] * c[1][v] + c[2][v] * c[2][v] + c[3][v] * c[3][v];
        ss += __shfl_xor(ss, 1);
        ss += __shfl_xor(ss, 2);
        ss += __shfl_xor(ss, 4);
        ss += __shfl_xor(ss, 8);
        const float inv = ss > 0.f ? 1.0f / sqrtf(ss) : 0.f;
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) out[nt][v] = f32_to_bf16(c[nt][v] * inv);
    }
}

template <int D>
__global__ __launch_bounds__(256) void qlatent_bf16_kernel(const uint16_t* __restrict__ Q,
                                                           const uint16_t* __restrict__ W, int64_t rows,
                                                           uint16_t* __restrict__ qhat, int* counters,
                                                           uint4* zero, int64_t zero_n) {
    constexpr int KS = D / 32;
    if (blockIdx.x == 0 && threadIdx.x < 4) counters[threadIdx.x] = 0;
    clear_words(zero, zero_n);
    const int l = lane_id(), wid = threadIdx.x >> 6, r = l & 15, h = l >> 4;
    bf16x8 wf[4][KS];   // in registers for the whole (persistent) workgroup
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) qlatent_w_frag<D>(W, nt, wf[nt]);
    const int64_t ntile = (rows + 15) / 16;
    for (int64_t tile = (int64_t)blockIdx.x * 4 + wid; tile < ntile; tile += (int64_t)gridDim.x * 4) {
        uint4 qa[KS];
        qlatent_q_frag<D>(Q, tile * 16, rows, qa);
        f32x4 c[4];
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
            c[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                c[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(qa[ks]), wf[nt][ks], c[nt], 0, 0, 0);
        }
        uint16_t o[4][4];
        qlatent_normalise(c, o);
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int64_t orow = tile * 16 + 4 * h + v;
            if (orow < rows) {
#pragma unroll
                for (int nt = 0; nt < 4; ++nt) qhat[orow * kLatent + 16 * nt + r] = o[nt][v];
            }
        }
    }
}

// The decode scan's own q_hat rows of one unit (rows row0 .. row0 + G - 1): one
// MFMA tile per wave, the W fragments loaded one column tile at a time (few
// registers), the rows put in the wave's LDS area (16 x 64 bf16) for the
// query codes; with `out` set, the unit's G rows are also written there.
template <int D>
__device__ __forceinline__ void qlatent_unit_bf16(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ W,
                                                  int64_t row0, int64_t rows, int G, uint16_t* lds_rows,
                                                  uint16_t* __restrict__ out) {
    constexpr int KS = D / 32;
    const int l = lane_id(), r = l & 15, h = l >> 4;
    uint4 qa[KS];
    qlatent_q_frag<D>(Q, row0, rows, qa);
    f32x4 c[4];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
        bf16x8 wf[KS];
        qlatent_w_frag<D>(W, nt, wf);
        c[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            c[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(qa[ks]), wf[ks], c[nt], 0, 0, 0);
    }
    uint16_t o[4][4];
    qlatent_normalise(c, o);
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        const int rr = 4 * h + v;
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
            lds_rows[rr * kLatent + 16 * nt + r] = o[nt][v];
            if (out != nullptr && rr < G) out[(row0 + rr) * kLatent + 16 * nt + r] = o[nt][v];
        }
    }
    wave_sync();
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
    const int l = lane_id();
    const uint4* p = reinterpret_cast<const uint4*>(cent_bg) + (x0 >> 4) * 128 + l;   // tile-swizzled storage
    const bf16x8 a0 = as_bf16x8(p[0]), a1 = as_bf16x8(p[64]);
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
// of the tile; every wave scans all buckets visible to any of its queries,
// with the centroid fragments of the next 16 buckets in flight while the
// current ones are scored.
//
// The bound: a histogram over 256 score bins of width 1/128 accumulates
// token weights that are certainly eligible (4 x size for buckets of blocks
// inside [sink_end, l0), else 0).  While a wave sees at most
// kPerLeafMaxLeaves buckets every bucket is binned; beyond that the buckets
// of every other block.  The bin where the weight from the top reaches k
// gives tau = its lower edge minus 2^-16 (absorbs fp32 rounding of the
// binning): at least k eligible tokens lie in buckets scoring >= tau, so the
// k-th token's bucket does too.
constexpr int kPerLeafMaxLeaves = 96 * kLeavesPerBlock;
constexpr int kHistStride = 257;   // padded: neighbouring queries fall in different banks

// The A fragments of the tile of buckets x0..x0+15 (x0 a multiple of 16):
// lane (r, h) gets dims [16h, 16h+8) and [16h+8, 16h+16) of bucket x0 + r,
// one contiguous 1 KB read per fragment (tile-swizzled storage).
__device__ __forceinline__ void load_cent_bf16(const uint16_t* cent_bg, int64_t x0, uint4& a0, uint4& a1) {
    const uint4* p = reinterpret_cast<const uint4*>(cent_bg) + (x0 >> 4) * 128 + lane_id();
    a0 = p[0];
    a1 = p[64];
}

__device__ __forceinline__ f32x4 mfma_tile_bf16(uint4 u0, uint4 u1, const QFragBF16& qf, int G) {
    const bf16x8 a0 = as_bf16x8(u0), a1 = as_bf16x8(u1);
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

__device__ __forceinline__ int score_bin(float s) {
    int bin = (int)floorf((s + 1.0f) * 128.0f);
    return bin < 0 ? 0 : (bin > 255 ? 255 : bin);
}

template <bool BF16, int PASS>
__global__ __launch_bounds__(256) void fused_scan_kernel(CacheView cv, const void* __restrict__ qhat,
                                                         const int64_t* __restrict__ q_pos, SelArgs sa,
                                                         float* __restrict__ tau, int* __restrict__ cnt,
                                                         uint64_t* __restrict__ cand) {
    __shared__ uint32_t hist[PASS == 0 ? 4 * 16 * kHistStride : 1];
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
    const bool perleaf = maxNLv <= kPerLeafMaxLeaves;   // wave-uniform

    QFragBF16 qf;
    if constexpr (BF16) load_qfrag_bf16(qf, reinterpret_cast<const uint16_t*>(qhat) + (qv ? qrow : 0), qv, sa.G);
    const float* qf32 = reinterpret_cast<const float*>(qhat) + (qv ? qrow : 0);

    uint32_t* myhist = hist + (PASS == 0 ? (wid * 16 + n) * kHistStride : 0);
    float tau_n = 0.f;
    if constexpr (PASS == 0) {
        for (int j = l; j < 16 * kHistStride; j += 64) hist[wid * 16 * kHistStride + j] = 0u;
    } else {
        if (l < 16) lcnt[wid][l] = 0;
        tau_n = qv ? tau[u] : 0.f;
    }
    wave_sync();

    const uint16_t* cb16 = reinterpret_cast<const uint16_t*>(cv.cent) + bg * cv.s_cent;
    const float* cb32 = reinterpret_cast<const float*>(cv.cent) + bg * cv.s_cent;
    const uint32_t* meta = cv.meta + bg * cv.s_meta;

    // Tiles visited: all of them, or in pass 0 with many visible buckets only
    // those of every other block (a sample: its buckets above tau still hold
    // >= k eligible tokens, so tau stays a valid bound, for half the work).
    const bool sample = PASS == 0 && !perleaf;
    const int ntl_all = maxNLv / 16;
    const int ntl = sample ? 4 * ((ntl_all / 4 + 1) / 2) : ntl_all;
    auto tile_x = [&](int idx) -> int64_t {
        return sample ? (int64_t)(8 * (idx / 4) + (idx & 3)) * 16 : (int64_t)idx * 16;
    };
    // A ring of DEPTH tiles in flight: tile idx + DEPTH is loaded once tile idx is scored (loads are
    // unconditional: past the last tile they repeat it, so they never serialise on a branch)
    constexpr int DEPTH = 4;
    uint4 ra[DEPTH][2], rm[DEPTH];
    auto load_tile = [&](int idx, uint4 (&a)[2], uint4& m) {
        const int64_t x = tile_x(idx < ntl ? idx : (ntl > 0 ? ntl - 1 : 0));
        if constexpr (BF16) load_cent_bf16(cb16, x, a[0], a[1]);
        if constexpr (PASS == 0) m = *reinterpret_cast<const uint4*>(meta + x + 4 * h);
    };
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) {
        ra[d][0] = ra[d][1] = rm[d] = uint4{0, 0, 0, 0};
        if (ntl > 0) load_tile(d, ra[d], rm[d]);
    }
    for (int i0 = 0; i0 < ntl; i0 += DEPTH) {
#pragma unroll
        for (int d = 0; d < DEPTH; ++d) {
            const int idx = i0 + d;
            if (idx >= ntl) break;
            const int64_t x0 = tile_x(idx);
            f32x4 vals;
            if constexpr (BF16)
                vals = mfma_tile_bf16(ra[d][0], ra[d][1], qf, sa.G);
            else
                vals = score_tile_f32(cb32, x0, qf32, qv, sa.G);
            const uint4 m4 = rm[d];
            load_tile(idx + DEPTH, ra[d], rm[d]);
            const int64_t xb = x0 + 4 * h;
            const bool edge = x0 + 16 > minNLv;
            const int64_t lo = (x0 / kLeavesPerBlock) * (int64_t)kBlockTokens;
            if constexpr (PASS == 0) {
                const uint32_t mm[4] = {m4.x, m4.y, m4.z, m4.w};
                const bool elig = qv && lo >= q.sink_end && lo + kBlockTokens <= q.l0;
                if (elig) {
#pragma unroll
                    for (int v = 0; v < 4; ++v)
                        if (!edge || (xb + v < NLv))
                            atomicAdd(&myhist[score_bin(vals[v])], (uint32_t)kPool * (mm[v] & 0xFFu));
                }
            } else {
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const bool pred = (!edge || (xb + v < NLv)) && qv && vals[v] >= tau_n;
                    if (pred) {
                        const int pos = atomicAdd(&lcnt[wid][n], 1);   // slot pos % kSubCap of sub-list pos / kSubCap
                        if (pos < kCandStride) cand[u * kCandStride + pos] = rank_key(vals[v], (uint32_t)(xb + v));
                    }
                }
            }
        }
    }
    wave_sync();
    if constexpr (PASS == 0) {
        if (h == 0 && qv) {
            uint32_t cum = 0;
            float tv = kNegInf;
            for (int bin = 255; bin >= 1; --bin) {
                cum += myhist[bin];
                if (cum >= (uint32_t)sa.k) {
                    tv = (float)bin * (1.0f / 128.0f) - 1.0f - 1.52587890625e-05f;
                    break;
                }
            }
            tau[u] = tv;
        }
    } else {
        if (h == 0 && qv) {
            const int c = lcnt[wid][n];
#pragma unroll
            for (int j = 0; j < 4; ++j)
                cnt[4 * u + j] = j < 3 ? min(max(c - kSubCap * j, 0), kSubCap) : max(c - kSubCap * 3, 0);
        }
    }
}

// ------------------------------------------------------------------ single-pass scan, LDS-staged (bf16)
// The fused flat search's scan in one pass over the centroids, tiles shared
// through LDS: a workgroup owns 128 queries of one KV head (32 per wave, as
// two 16-query MFMA column groups), streams the visible tiles in chunks of 8
// (24 KB) with their buckets' meta words (the next chunk in registers while
// one is scored), and every wave reads its operand fragments from LDS (one
// fragment read feeds 2 x G x 2 MFMAs).
//
// Each query keeps a histogram of certainly eligible token weight (4 x size
// for buckets of blocks inside [sink_end, l0)) over score bins (one below 0,
// 64 of width 1/64 over [0, 1), the last open) and a floor bin fb: the
// highest bin at which the weight binned so far, summed from the top,
// reaches k (raised after every chunk).  A visible bucket in a bin >= fb is
// appended (rank key) to the query's candidate list and its weight binned;
// one below fb is skipped: fb only rises, so bins below it can never become
// the final crossing bin b*, and every bin >= b* holds all of its weight.
// Hence at the end tau = lower edge of b* (minus 2^-16; -inf if the weight
// never reaches k) bounds the k-th token's bucket score from below, and the
// list holds every visible bucket scoring >= tau (plus earlier ones below
// it, dropped by the finalize).  A query's list is 4 sub-lists of kSubCap
// slots filled in order (one running count per query; the counts are exact
// past the cap).  The floor rises by walking up from fb while the weight
// above the next bin still reaches k, with the weight at or above fb kept
// as a running sum (every binned bucket lies at or above the floor).
//
// Candidates are rare per lane (a query appends ~k(1 + ln(N/k)) of N
// buckets, mostly early) but present in nearly every tile of a wave, so
// appending them where they arise would run the wave's append code for one
// or two lanes per tile.  Instead a lane whose 4 scores of a column group
// reach the floor pushes them, as one group, into a per-wave LDS queue
// (compacted by a ballot; the other lanes write just past the compacted
// ones, which keeps the push free of branches), and the wave takes 64 groups
// at a time, one per lane: each score still at or above the floor gets a
// list slot from an LDS counter, its rank key stored, its weight binned.
// The queue is emptied before the floors rise, so the histogram is complete
// when they do.
//
// The tile loop is software-pipelined: the MFMAs of tile i + 1 are issued
// before tile i's scores are tested and pushed, so the matrix core runs
// while the same wave does the vector work of the previous tile.
constexpr int kSelCap = 256;        // buckets one finalize wave may take (more: the exact path)
constexpr int kScanQ = 128;         // queries per workgroup
constexpr int kScanChunk = 12;      // tiles per staged chunk (even)
constexpr int kQueueCap = 192;      // queued groups per wave: < 64 left + 2 column groups x 64
constexpr int kHBins = 65;          // score bins: s < 0, then 64 of width 1/64 over [0, 1) (the last open)
constexpr int kHStride = kHBins;    // odd: neighbouring queries' rows fall in different banks
constexpr int kMaxLeavesI = 0x7FFFFFFF;
constexpr float kFltMax = 3.402823466e38f;
constexpr float kPosInf = __builtin_huge_valf();

// multiplications by powers of two are exact, so for b >= 1: bin(s) >= b  <=>  s >= edge(b)
__device__ __forceinline__ int hbin(float s) { return s < 0.f ? 0 : min(1 + (int)(s * 64.0f), kHBins - 1); }
__device__ __forceinline__ float hedge(int b) { return (float)(b - 1) * (1.0f / 64.0f); }

// The 2 x G x 2 MFMAs of one tile (fragments a0, a1) for both column groups, and the max over heads.
template <int G>
__device__ __forceinline__ void scan_mfma(f32x4 (&acc)[2][G], const bf16x8& a0, const bf16x8& a1,
                                          const bf16x8 (&qf)[2][G][2]) {
#pragma unroll
    for (int cg = 0; cg < 2; ++cg)
#pragma unroll
        for (int hh = 0; hh < G; ++hh) {
            f32x4 c = {0.f, 0.f, 0.f, 0.f};
            c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, qf[cg][hh][0], c, 0, 0, 0);
            acc[cg][hh] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, qf[cg][hh][1], c, 0, 0, 0);
        }
}
template <int G>
__device__ __forceinline__ void head_max(const f32x4 (&acc)[2][G], f32x4 (&best)[2]) {
#pragma unroll
    for (int cg = 0; cg < 2; ++cg) {
        best[cg] = acc[cg][0];
#pragma unroll
        for (int hh = 1; hh < G; ++hh)
#pragma unroll
            for (int v = 0; v < 4; ++v) best[cg][v] = fmax_nc(best[cg][v], acc[cg][hh][v]);
    }
}

template <int G>
__global__ __launch_bounds__(256) void scan_fused_kernel(CacheView cv, const uint16_t* __restrict__ qhat,
                                                         const int64_t* __restrict__ q_pos, SelArgs sa,
                                                         float* __restrict__ tau, int* __restrict__ cnt,
                                                         uint64_t* __restrict__ cand) {
    __shared__ __align__(16) uint4 stage[kScanChunk * 128];     // 24 KB
    __shared__ __align__(16) uint32_t smeta[kScanChunk * 16];   // meta word of every bucket of the chunk
    __shared__ uint32_t hist[kScanQ * kHStride];
    __shared__ __align__(16) f32x4 qsc[4][kQueueCap];           // per wave: queued groups' 4 scores
    __shared__ uint16_t qhd[4][kQueueCap];                      //   and (tile << 7 | h << 5 | query slot)
    __shared__ int lcnt[kScanQ];                                // candidate list lengths
    __shared__ uint32_t wsum[kScanQ];                           // binned weight at or above the floor bin
    __shared__ int fbin[kScanQ];                                // floor bins
    __shared__ float fedge[kScanQ];                             // floor edges (+inf: no query)
    __shared__ int2 erng[kScanQ];                               // blocks [x, y) certainly eligible
    __shared__ int wmax[4], wmin[4];
    const int tid = threadIdx.x, l = lane_id(), wid = tid >> 6, n = l & 15, h = l >> 4;
    const int64_t b = blockIdx.z, g = blockIdx.y;
    const int64_t bg = b * sa.H_kv + g;
    // unit of the wave's query slot qs (0..31) = ubase + qs * H_kv
    const int64_t q0 = (int64_t)blockIdx.x * kScanQ + wid * 32;   // the wave's first query
    const int64_t ubase = (b * sa.n_q + q0) * sa.H_kv + g;
    // per column group cg: this lane's query (column n), query slot 16 cg + n
    int NLv[2];
    bool qv[2];
    bf16x8 qf[2][G][2];
#pragma unroll
    for (int cg = 0; cg < 2; ++cg) {
        const int64_t iq = q0 + cg * 16 + n;
        qv[cg] = iq < sa.n_q;
        const int64_t t = qv[cg] ? q_pos[b * sa.n_q + iq] : -1;
        const Geom q = query_geom(t < 0 ? 0 : t, cv.n_blocks, sa.n_sinks, sa.window);
        NLv[cg] = t < 0 ? 0 : kLeavesPerBlock * q.nvis;
        if (h == 0) {
            const int qw = wid * 32 + cg * 16 + n;
            lcnt[qw] = 0;
            wsum[qw] = 0u;
            fbin[qw] = 0;
            // every score is a candidate before the floor rises (-FLT_MAX: a masked -inf is not); a
            // column without a query never has one
            fedge[qw] = qv[cg] ? -kFltMax : kPosInf;
            // block j is eligible iff sink_end <= 2048 j and 2048 (j + 1) <= l0
            erng[qw] = int2{(int)((q.sink_end + kBlockTokens - 1) / kBlockTokens), (int)(q.l0 / kBlockTokens)};
        }
        const int64_t qrow = ((b * sa.n_q + (qv[cg] ? iq : 0)) * sa.H_q + g * sa.G) * kLatent;
#pragma unroll
        for (int hh = 0; hh < G; ++hh) {
            uint4 a = {0, 0, 0, 0}, c = {0, 0, 0, 0};
            if (qv[cg]) {
                const uint4* p = reinterpret_cast<const uint4*>(qhat + qrow + hh * kLatent + 16 * h);
                a = p[0];
                c = p[1];
            }
            qf[cg][hh][0] = as_bf16x8(a);
            qf[cg][hh][1] = as_bf16x8(c);
        }
    }
    // wait for the query fragments here: with them still in flight the compiler would wait for every
    // outstanding load before each chunk's tile loop (a loop holding stores and no loads), the chunk
    // prefetch included
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
    // queue header of this lane's group of column group cg in tile tt: (tt << 7) | (h << 5) | slot
    const uint32_t hb[2] = {((uint32_t)h << 5) | (uint32_t)n, ((uint32_t)h << 5) | (uint32_t)(16 + n)};
    for (int j = tid; j < kScanQ * kHStride; j += 256) hist[j] = 0u;
    // tiles visible to any query of the workgroup, and to all of them
    const int wm = wave_max_i(max(NLv[0], NLv[1]));
    const int wn = wave_min_i(min(qv[0] ? NLv[0] : kMaxLeavesI, qv[1] ? NLv[1] : kMaxLeavesI));
    if (l == 0) {
        wmax[wid] = wm;
        wmin[wid] = wn;
    }
    __syncthreads();
    const int maxNLv = max(max(wmax[0], wmax[1]), max(wmax[2], wmax[3]));
    const int minNLv = min(min(wmin[0], wmin[1]), min(wmin[2], wmin[3]));
    const int ntl = maxNLv / 16;
    const int ntlm = minNLv / 16;   // tiles visible to every query: no masking
    const int nch = (ntl + kScanChunk - 1) / kScanChunk;
    const u32x4* src = reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(cv.cent) + bg * cv.s_cent);
    const u32x4* msrc = reinterpret_cast<const u32x4*>(cv.meta + bg * cv.s_meta);
    float fe[2] = {qv[0] ? -kFltMax : kPosInf, qv[1] ? -kFltMax : kPosInf};
    f32x4* qs_w = qsc[wid];
    uint16_t* qh_w = qhd[wid];
    int qn = 0;   // queued groups of this wave (uniform)
    // One queued group per lane (slot e, chunk c): each of its scores at or above its query's floor edge
    // is appended to the query's list and, if its block is certainly eligible, binned.
    auto take = [&](int e, int c) {
        const f32x4 sv = qs_w[e];
        const uint32_t hd = qh_w[e];
        const int qs = (int)(hd & 31u);
        const int xl0 = (int)(hd >> 5) * 4;   // bucket of value 0 within the chunk: 16 tile + 4 h
        const int qw = wid * 32 + qs;
        const float fq = fedge[qw];
        const int x0 = c * kScanChunk * 16 + xl0;
        const int2 er = erng[qw];
        const int blk = x0 / kLeavesPerBlock;
        const bool el = (blk >= er.x) & (blk < er.y);
        bool p[4];
        int np = 0;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            p[v] = sv[v] >= fq;
            np += p[v] ? 1 : 0;
        }
        int pos = atomicAdd(&lcnt[qw], np);   // slot pos % kSubCap of sub-list pos / kSubCap
        uint64_t* dst = cand + (ubase + (int64_t)qs * sa.H_kv) * kCandStride;
        uint32_t wadd = 0;
        uint32_t* hr = hist + qw * kHStride;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            if (p[v]) {
                if (pos < kCandStride) dst[pos] = rank_key(sv[v], (uint32_t)(x0 + v));
                ++pos;
                if (el) {
                    const uint32_t w = (uint32_t)kPool * (smeta[xl0 + v] & 0xFFu);
                    atomicAdd(&hr[hbin(sv[v])], w);
                    wadd += w;
                }
            }
        }
        if (wadd) atomicAdd(&wsum[qw], wadd);
    };
    // A lane whose scores of column group cg reach the floor pushes them as a group (tile tt).  Compacted
    // slots from the ballot; the other lanes write the slots right after them, which later pushes
    // overwrite (every lane writes, so the push has no branch).
    auto push = [&](const f32x4 (&best)[2], int tt) {
        const uint32_t tb = (uint32_t)tt << 7;
#pragma unroll
        for (int cg = 0; cg < 2; ++cg) {
            const float lm = fmax_nc(fmax_nc(best[cg][0], best[cg][1]), fmax_nc(best[cg][2], best[cg][3]));
            const bool p = lm >= fe[cg];
            const uint64_t m = __ballot(p);
            const int cm = (int)__popcll(m);
            const uint32_t pre = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                           __builtin_amdgcn_mbcnt_lo((uint32_t)m, (uint32_t)qn));
            const uint32_t post = __builtin_amdgcn_mbcnt_hi(
                (uint32_t)(~m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)~m, (uint32_t)(qn + cm)));
            const int slot = (int)(p ? pre : post);
            qs_w[slot] = best[cg];
            qh_w[slot] = (uint16_t)(hb[cg] + tb);
            qn += cm;
        }
    };
    auto drain = [&](int c) {
        if (qn >= 64) {
            wave_sync();
            do {
                qn -= 64;
                take(qn + l, c);
            } while (qn >= 64);
            wave_sync();
        }
    };
    // staging: thread tid copies words tid + 256 j (j < kScanChunk / 2) of a chunk and, if tid <
    // 4 kScanChunk, meta word tid; tiles past the last one repeat it
    constexpr int kRW = kScanChunk / 2;
    u32x4 rw[kRW], rmt;
    auto load_chunk = [&](int c) {
#pragma unroll
        for (int j = 0; j < kRW; ++j)
            rw[j] = src[(int64_t)min(c * kScanChunk + (tid + 256 * j) / 128, ntl - 1) * 128 + (tid & 127)];
        if (tid < kScanChunk * 4) rmt = msrc[(int64_t)min(c * kScanChunk + tid / 4, ntl - 1) * 4 + (tid & 3)];
    };
    if (nch > 0) load_chunk(0);
    for (int c = 0; c < nch; ++c) {
        {
            u32x4* d4 = reinterpret_cast<u32x4*>(stage);
#pragma unroll
            for (int j = 0; j < kRW; ++j) d4[tid + 256 * j] = rw[j];
            if (tid < kScanChunk * 4) reinterpret_cast<u32x4*>(smeta)[tid] = rmt;
        }
        __syncthreads();
        if (c + 1 < nch) load_chunk(c + 1);
        const int tend = min(kScanChunk, ntl - c * kScanChunk);
        const int tmain = min(max(ntlm - c * kScanChunk, 0), tend);
        f32x4 acc[2][G], best[2];
        if (tmain > 0) {
            scan_mfma<G>(acc, as_bf16x8(stage[l]), as_bf16x8(stage[64 + l]), qf);
            for (int tt = 0; tt + 1 < tmain; ++tt) {
                const bf16x8 a0 = as_bf16x8(stage[(tt + 1) * 128 + l]), a1 = as_bf16x8(stage[(tt + 1) * 128 + 64 + l]);
                head_max<G>(acc, best);
                scan_mfma<G>(acc, a0, a1, qf);   // tile tt + 1 runs while tile tt is pushed
                push(best, tt);
                // one MFMA, then two vector instructions of the previous tile's work, in turn
                __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
                for (int i = 0; i < 2 * G * 2; ++i) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);
                }
                drain(c);
            }
            head_max<G>(acc, best);
            push(best, tmain - 1);
            drain(c);
        }
        // tiles past some query's visible leaves: those buckets never become candidates
        for (int tt = tmain; tt < tend; ++tt) {
            scan_mfma<G>(acc, as_bf16x8(stage[tt * 128 + l]), as_bf16x8(stage[tt * 128 + 64 + l]), qf);
            head_max<G>(acc, best);
            const int xb = (c * kScanChunk + tt) * 16 + 4 * h;
#pragma unroll
            for (int cg = 0; cg < 2; ++cg)
#pragma unroll
                for (int v = 0; v < 4; ++v)
                    best[cg][v] = (qv[cg] && xb + v < NLv[cg]) ? best[cg][v] : kNegInf;
            push(best, tt);
            drain(c);
        }
        // the chunk's last queued groups, then raise the floors (the rows are this wave's own)
        wave_sync();
        if (l < qn) take(l, c);
        qn = 0;
        wave_sync();
        if (l < 32) {
            // 8 bins read at once, walked in registers (the floor seldom rises further per chunk)
            const int qw = wid * 32 + l;
            int f = fbin[qw];
            uint32_t W = wsum[qw];
            const uint32_t* hr = hist + qw * kHStride;
            bool up = true;
            while (up) {
                uint32_t hv[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) hv[j] = hr[min(f + j, kHBins - 1)];
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    up = up && f < kHBins - 1 && W - hv[j] >= (uint32_t)sa.k;
                    if (up) {
                        W -= hv[j];
                        ++f;
                    }
                }
            }
            fbin[qw] = f;
            wsum[qw] = W;
            if (f >= 1 && q0 + l < sa.n_q) fedge[qw] = hedge(f);   // bin(s) >= f  <=>  s >= edge(f)
        }
        wave_sync();
        fe[0] = fedge[wid * 32 + n];
        fe[1] = fedge[wid * 32 + 16 + n];
        __syncthreads();   // the stage is rewritten next
    }
#pragma unroll
    for (int cg = 0; cg < 2; ++cg) {
        if (qv[cg]) {
            const int qw = wid * 32 + cg * 16 + n;
            const int64_t u = ubase + (int64_t)(cg * 16 + n) * sa.H_kv;
            const int c = lcnt[qw];
            if (h == 0) {
                const int f = fbin[qw];
                const bool crossed = wsum[qw] >= (uint32_t)sa.k;   // f is the crossing bin
                tau[u] = (crossed && f >= 1) ? hedge(f) - 1.52587890625e-05f : kNegInf;
            }
            cnt[4 * u + h] = h < 3 ? min(max(c - kSubCap * h, 0), kSubCap) : max(c - kSubCap * 3, 0);
        }
    }
}

// ------------------------------------------------------------------ wave-level finish
// Bitonic sort, descending, of 64 N 64-bit keys held in registers: element
// e = 64 i + lane is v[i].  Compare-exchanges across lanes use xor shuffles,
// those across registers stay in the lane.
template <int N>
__device__ __forceinline__ void reg_sort_desc(uint64_t (&v)[N]) {
    const int l = lane_id();
#pragma unroll
    for (int size = 2; size <= 64 * N; size <<= 1) {
#pragma unroll
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            if (stride >= 64) {
                const int rs = stride >> 6;
#pragma unroll
                for (int i = 0; i < N; ++i) {
                    if (i & rs) continue;
                    const bool desc = ((64 * i) & size) == 0;
                    const uint64_t x = v[i], y = v[i | rs];
                    const bool sw = desc ? (x < y) : (x > y);
                    v[i] = sw ? y : x;
                    v[i | rs] = sw ? x : y;
                }
            } else {
#pragma unroll
                for (int i = 0; i < N; ++i) {
                    const uint64_t y = shfl_xor_u64(v[i], stride);
                    const bool desc = ((64 * i + l) & size) == 0;
                    const bool lo = (l & stride) == 0;
                    const uint64_t mx = v[i] > y ? v[i] : y, mn = v[i] > y ? y : v[i];
                    v[i] = (lo == desc) ? mx : mn;
                }
            }
        }
    }
}

template <int N>
__device__ __forceinline__ void wave_sort_desc_n(uint64_t* a, int P) {
    const int l = lane_id();
    uint64_t v[N];
#pragma unroll
    for (int i = 0; i < N; ++i) v[i] = (64 * i + l < P) ? a[64 * i + l] : 0ull;
    reg_sort_desc<N>(v);
#pragma unroll
    for (int i = 0; i < N; ++i)
        if (64 * i + l < P) a[64 * i + l] = v[i];
    wave_sync();
}

template <int N>
__device__ __forceinline__ void reg_sort_desc_u32(uint32_t (&v)[N]) {
    const int l = lane_id();
#pragma unroll
    for (int size = 2; size <= 64 * N; size <<= 1) {
#pragma unroll
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            if (stride >= 64) {
                const int rs = stride >> 6;
#pragma unroll
                for (int i = 0; i < N; ++i) {
                    if (i & rs) continue;
                    const bool desc = ((64 * i) & size) == 0;
                    const uint32_t x = v[i], y = v[i | rs];
                    const bool sw = desc ? (x < y) : (x > y);
                    v[i] = sw ? y : x;
                    v[i | rs] = sw ? x : y;
                }
            } else {
#pragma unroll
                for (int i = 0; i < N; ++i) {
                    const uint32_t y = (uint32_t)__shfl_xor((int)v[i], stride);
                    const bool desc = ((64 * i + l) & size) == 0;
                    const bool lo = (l & stride) == 0;
                    const uint32_t mx = v[i] > y ? v[i] : y, mn = v[i] > y ? y : v[i];
                    v[i] = (lo == desc) ? mx : mn;
                }
            }
        }
    }
}

template <int N>
__device__ __forceinline__ void wave_sort_desc_u32_n(uint32_t* a, int P) {
    const int l = lane_id();
    uint32_t v[N];
#pragma unroll
    for (int i = 0; i < N; ++i) v[i] = (64 * i + l < P) ? a[64 * i + l] : 0u;
    reg_sort_desc_u32<N>(v);
#pragma unroll
    for (int i = 0; i < N; ++i)
        if (64 * i + l < P) a[64 * i + l] = v[i];
    wave_sync();
}

// Sorts a[0..P) (P a power of two, at most 1024) of 32-bit keys descending.
__device__ __forceinline__ void wave_sort_desc_u32(uint32_t* a, int P) {
    wave_sync();
    if (P <= 64)
        wave_sort_desc_u32_n<1>(a, P);
    else if (P <= 128)
        wave_sort_desc_u32_n<2>(a, P);
    else if (P <= 256)
        wave_sort_desc_u32_n<4>(a, P);
    else if (P <= 512)
        wave_sort_desc_u32_n<8>(a, P);
    else
        wave_sort_desc_u32_n<16>(a, P);
}

// Sorts a[0..P) (P a power of two, at most 512) descending in place.  Slots
// past P are treated as zero keys, which sort after every other key.
__device__ __forceinline__ void wave_sort_desc(uint64_t* a, int P) {
    wave_sync();
    if (P <= 64)
        wave_sort_desc_n<1>(a, P);
    else if (P <= 128)
        wave_sort_desc_n<2>(a, P);
    else if (P <= 256)
        wave_sort_desc_n<4>(a, P);
    else
        wave_sort_desc_n<8>(a, P);
}

__device__ __forceinline__ int pow2_at_least(int n) {
    int p = 2;
    while (p < n) p <<= 1;
    return p;
}

// A selected bucket: leaf id in bits 32..63, its member list (offset in the
// block's member array in bits 15..24, entry count in bits 25..29), its
// eligible tokens w in bits 8..14, bit 7 set when all of them are taken,
// else bits 0..6 = how many of its lowest eligible tokens are taken (only
// the boundary bucket).  Sorting the records ascending sorts them by leaf.
__device__ __forceinline__ uint64_t pack_sel(uint32_t leaf, uint32_t meta, int w, bool full, int take) {
    const uint64_t off = (meta >> 8) & 0x3FF, sz = meta & 0x1F;
    return ((uint64_t)leaf << 32) | (sz << 25) | (off << 15) | ((uint64_t)(w & 0x7F) << 8) |
           (full ? 0x80ull : (uint64_t)(take & 0x7F));
}
__device__ __forceinline__ int sel_off(uint64_t s) { return (int)((s >> 15) & 0x3FF); }
__device__ __forceinline__ int sel_size(uint64_t s) { return (int)((s >> 25) & 0x1F); }

__device__ __forceinline__ uint32_t sel_leaf(uint64_t s) { return (uint32_t)(s >> 32); }
__device__ __forceinline__ bool sel_full(uint64_t s) { return (s & 0x80ull) != 0; }
__device__ __forceinline__ int sel_count(uint64_t s) { return sel_full(s) ? (int)((s >> 8) & 0x7F) : (int)(s & 0x7F); }
__device__ __forceinline__ uint32_t sel_block(uint64_t s) { return sel_leaf(s) / kLeavesPerBlock; }

// Token-level expansion of one block (used when the block straddles the
// sink or window edge, or holds the partially taken boundary bucket): lane l
// owns entries l + 64 k (k = 0..7); for each k the 256 tokens are ordered by
// (lane, token in entry), so output positions follow from ballots and
// lane-prefix bit counts.  Writes the block's tokens ascending from out[0].
__device__ __forceinline__ void expand_block_scan(uint32_t blk, const uint64_t* sel, int a, int b, const CacheView& cv,
                                                  int64_t bg, const Geom& q, int32_t* out, int* tk) {
    const int l = lane_id();
    const uint64_t lt = (1ull << l) - 1ull;
    tk[l] = 0;
    wave_sync();
    for (int idx = a + l; idx < b; idx += 64) {
        const uint64_t sv = sel[idx];
        tk[sel_leaf(sv) % kLeavesPerBlock] = sel_full(sv) ? kFullTake : (int)(sv & 0x7F);
    }
    wave_sync();
    const int my = tk[l];
    const uint64_t pb = __ballot(my != 0 && my != kFullTake);
    const int quota = pb ? __shfl(my, __builtin_ctzll(pb)) : 0;
    const uint8_t* row = cv.eleaf + bg * cv.s_eleaf + (int64_t)blk * kBlockEntries + l;
    uint32_t rk[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) rk[k] = row[64 * k];
    const int64_t B0 = (int64_t)blk * kBlockTokens;
    int pseen = 0, count = 0;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const int take = tk[rk[k] & 0x3F];
        const int64_t t0 = B0 + (int64_t)kPool * (l + 64 * k);
        bool full[4], part[4], emit[4];
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            const int64_t tok = t0 + jj;
            const bool el = take != 0 && tok >= q.sink_end && tok < q.l0;
            full[jj] = el && take == kFullTake;
            part[jj] = el && take != kFullTake;
        }
        int before = pseen, mine = 0;
        uint64_t bp[4];
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            bp[jj] = __ballot(part[jj]);
            before += __popcll(bp[jj] & lt);
        }
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            emit[jj] = full[jj] || (part[jj] && before + mine < quota);
            mine += part[jj] ? 1 : 0;
            pseen += __popcll(bp[jj]);
        }
        uint64_t be[4];
        int pos = count;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            be[jj] = __ballot(emit[jj]);
            pos += __popcll(be[jj] & lt);
        }
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            if (emit[jj]) out[pos++] = (int32_t)(t0 + jj);
            count += __popcll(be[jj]);
        }
    }
    wave_sync();
}

// Sum over records [a, b) of their taken token counts (wave-wide).
__device__ __forceinline__ int records_tokens(const uint64_t* sel, int a, int b) {
    int acc = 0;
    for (int c0 = a; c0 < b; c0 += 64) {
        const int i = c0 + lane_id();
        acc += i < b ? sel_count(sel[i]) : 0;
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) acc += __shfl_xor(acc, o);
    return acc;
}

// Writes the tokens of the selected buckets (sel[0..nsel), sorted by leaf id)
// in ascending order and returns their number.  A block is "plain" when it
// lies inside [sink_end, l0) and every selected bucket of it is taken whole;
// the other (special) blocks, at most the two straddling an edge and the one
// holding the partially taken bucket, go through expand_block_scan.  The
// member entries of the plain buckets are listed as (block, entry) keys in
// record order, so grouped by block, each bucket's members ascending (as the
// build stores them).  An entry's place in (block, entry) order is then the
// start of its block's group plus the number of smaller entries in that
// group (its own index when the bucket is alone in the block), so the list
// is put in order in place, without a sort; entry p of the order lands at
// 4 p plus the tokens of the special blocks before its block.
// LDS scratch: ent[] of at least k/4 keys, tk[] of 256 ints (tk[0..64) is
// expand_block_scan's map, tk[64..) lists the special blocks).
__device__ __forceinline__ int wave_expand(const uint64_t* sel, int nsel, const CacheView& cv, int64_t bg,
                                           const Geom& q, int32_t* out, int* tk, uint32_t* ent) {
    const int l = lane_id();
    int* spec_first = tk + 64;    // [0] = count, then first record of each special block
    int* spec_tok = tk + 128;     // tokens of special block s
    int* spec_blk = tk + 192;     // block id of special block s
    // the block of the partially taken bucket (at most one), -1 if none
    int part_blk = -1;
    for (int c0 = 0; c0 < nsel; c0 += 64) {
        const int i = c0 + l;
        const uint64_t bal = __ballot(i < nsel && !sel_full(sel[i]));
        if (bal) {
            part_blk = (int)sel_block(sel[c0 + __builtin_ctzll(bal)]);
            break;
        }
    }
    if (l == 0) spec_first[0] = 0;
    wave_sync();
    const uint16_t* mem_bg = cv.members + bg * cv.s_members;
    int nent = 0;
    for (int c0 = 0; c0 < nsel; c0 += 64) {
        const int i = c0 + l;
        const bool live = i < nsel;
        const uint64_t sv = live ? sel[i] : 0ull;
        const int blk = (int)sel_block(sv);
        const int64_t lo = (int64_t)blk * kBlockTokens;
        const bool special = live && (!(lo >= q.sink_end && lo + kBlockTokens <= q.l0) || blk == part_blk);
        const bool first = live && (i == 0 || (int)sel_block(sel[i - 1]) != blk);
        if (special && first) {
            const int slot = atomicAdd(&spec_first[0], 1);
            if (slot < 63) spec_first[1 + slot] = i;
        }
        const int sz = (live && !special) ? sel_size(sv) : 0;
        const int incl = wave_incl_scan(sz);
        const int pos = nent + incl - sz;
        nent += __shfl(incl, 63);
        if (sz > 0) {
            uint16_t e[16];
            load_members(mem_bg + (int64_t)blk * kBlockEntries, sel_off(sv), e);
#pragma unroll
            for (int jm = 0; jm < 16; ++jm)
                if (jm < sz) ent[pos + jm] = ((uint32_t)blk << 9) | e[jm];
        }
    }
    wave_sync();
    const int nspec = spec_first[0] < 63 ? spec_first[0] : 63;
    // special blocks: their record ranges, token counts and output offsets
    for (int sidx = 0; sidx < nspec; ++sidx) {
        const int f = spec_first[1 + sidx];
        const uint32_t blk = sel_block(sel[f]);
        int g = f;
        while (true) {
            const int idx = g + l;
            const bool same = idx < nsel && sel_block(sel[idx]) == blk;
            const int r = __popcll(__ballot(same));
            g += r;
            if (r < 64) break;
        }
        const int tok = records_tokens(sel, f, g);
        if (l == 0) {
            spec_tok[sidx] = tok;
            spec_blk[sidx] = (int)blk;
        }
    }
    wave_sync();
    // plain entries into (block, entry) order, in place: an entry's place is the start of its block's
    // group plus the number of smaller entries in the group.  Records go in chunks of whole blocks
    // (a block has at most 64 buckets), so a group is permuted only after all its reads.
    int pbase = 0;
    for (int c0 = 0; c0 < nsel;) {
        const int i = c0 + l;
        const bool starts = i < nsel && (i == 0 || sel_block(sel[i - 1]) != sel_block(sel[i]));
        const uint64_t sb = __ballot(starts) & ~1ull;
        const bool cut_ok = c0 + 64 >= nsel || sel_block(sel[c0 + 64]) != sel_block(sel[c0 + 63]);
        const int width = (cut_ok || sb == 0ull) ? 64 : 63 - __builtin_clzll(sb);
        const bool live = l < width && i < nsel;
        c0 += width;
        const uint64_t sv = live ? sel[i] : 0ull;
        const int blk = (int)sel_block(sv);
        const int64_t lo = (int64_t)blk * kBlockTokens;
        const bool special = live && (!(lo >= q.sink_end && lo + kBlockTokens <= q.l0) || blk == part_blk);
        const int sz = (live && !special) ? sel_size(sv) : 0;
        const int incl = wave_incl_scan(sz);
        const int pos = pbase + incl - sz;
        pbase += __shfl(incl, 63);
        // the block's group of ent[]: from the place of its first record to that of the next block's
        // (or the chunk's end); the chunk holds whole blocks
        const uint64_t bs = __ballot(live && starts);
        const uint64_t upto = bs & ((2ull << l) - 1ull), after = bs & ~((2ull << l) - 1ull);
        const int ga_ = __shfl(pos, upto ? 63 - __builtin_clzll(upto) : 0);
        const int gz_ = __shfl(pos, after ? __builtin_ctzll(after) : 0);
        uint32_t e[16];
        int rank[16];
        int ga = 0;
        if (sz > 0) {
            ga = ga_;
            const int gz = after ? gz_ : pbase;
#pragma unroll
            for (int jm = 0; jm < 16; ++jm) {
                e[jm] = jm < sz ? ent[pos + jm] : 0u;
                rank[jm] = 0;
            }
            if (gz - ga == sz) {
#pragma unroll
                for (int jm = 0; jm < 16; ++jm) rank[jm] = jm;   // alone in its block: already ascending
            } else {
                for (int qq = ga; qq < gz; ++qq) {
                    const uint32_t v = ent[qq];
#pragma unroll
                    for (int jm = 0; jm < 16; ++jm) rank[jm] += v < e[jm] ? 1 : 0;
                }
            }
        }
        wave_sync();
        if (sz > 0) {
#pragma unroll
            for (int jm = 0; jm < 16; ++jm)
                if (jm < sz) ent[ga + rank[jm]] = e[jm];
        }
        wave_sync();
    }
    // entry p of that order lands at 4 p plus the tokens of the special blocks before its block
    for (int p = l; p < nent; p += 64) {
        const uint32_t key = ent[p];
        const int blk = (int)(key >> 9);
        int before = 0;
        for (int sidx = 0; sidx < nspec; ++sidx) before += spec_blk[sidx] < blk ? spec_tok[sidx] : 0;
        const int32_t t0 = (int32_t)((int64_t)blk * kBlockTokens + kPool * (int64_t)(key & 511u));
        int32_t* d = out + kPool * p + before;
        d[0] = t0;
        d[1] = t0 + 1;
        d[2] = t0 + 2;
        d[3] = t0 + 3;
    }
    // special blocks at their offsets: tokens of plain entries and special blocks before them
    const int total = records_tokens(sel, 0, nsel);
    for (int sidx = 0; sidx < nspec; ++sidx) {
        const int f = spec_first[1 + sidx];
        const int blk = spec_blk[sidx];
        int g = f;
        while (true) {
            const int idx = g + l;
            const bool same = idx < nsel && (int)sel_block(sel[idx]) == blk;
            const int r = __popcll(__ballot(same));
            g += r;
            if (r < 64) break;
        }
        const int off = records_tokens(sel, 0, f);
        expand_block_scan((uint32_t)blk, sel, f, g, cv, bg, q, out + off, tk);
    }
    wave_sync();
    return total;
}

// The selection as bucket records (sel[0..nsel), ascending leaf id): per
// bucket {leaf, key mask lo, hi, 0}, key j being token 4 members[j/4] + j%4
// of its block.  The mask holds the bucket's eligible keys (tokens in
// [sink_end, l0)); for the partially taken bucket, the lowest `take` of them,
// the same tokens expand_block_scan emits for it.
__device__ __forceinline__ void write_bucket_records(const uint64_t* sel, int nsel, const CacheView& cv, int64_t bg,
                                                     const Geom& q, u32x4* rec, int32_t* rcnt) {
    const int l = lane_id();
    for (int i = l; i < nsel; i += 64) {
        const uint64_t sv = sel[i];
        const uint32_t leaf = sel_leaf(sv);
        const int blk = (int)(leaf / kLeavesPerBlock), sz = sel_size(sv);
        const int64_t lo = (int64_t)blk * kBlockTokens;
        uint64_t m = 0ull;
        if (lo >= q.sink_end && lo + kBlockTokens <= q.l0) {
            m = sz >= 16 ? ~0ull : (1ull << (kPool * sz)) - 1ull;
        } else {
            uint16_t e[16];
            load_members(cv.members + bg * cv.s_members + (int64_t)blk * kBlockEntries, sel_off(sv), e);
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const int64_t t0 = lo + (int64_t)e[j] * kPool;
#pragma unroll
                for (int x = 0; x < kPool; ++x)
                    if (j < sz && t0 + x >= q.sink_end && t0 + x < q.l0) m |= 1ull << (kPool * j + x);
            }
        }
        if (!sel_full(sv))
            for (int drop = __popcll(m) - (int)(sv & 0x7F); drop > 0; --drop) m &= ~(1ull << (63 - __builtin_clzll(m)));
        rec[i] = u32x4{leaf, (uint32_t)m, (uint32_t)(m >> 32), 0u};
    }
    if (l == 0) *rcnt = nsel;
}

// Walk keys[0..n) (sorted by rank), pick the buckets until k eligible
// tokens, sort the picks by id into sel[] (room for sel_cap) and expand;
// with rec, also write the picks as bucket records (and with rec_only, no
// tokens).  Returns the count, or -1 with nothing written when more than
// sel_cap buckets are needed.
__device__ __forceinline__ int wave_walk_expand(uint64_t* keys, int n, uint64_t* sel, int sel_cap, int* tk,
                                                uint32_t* ent, const CacheView& cv, int64_t bg, const Geom& q, int k,
                                                int32_t* out, u32x4* rec, int32_t* rcnt, bool rec_only) {
    const int l = lane_id();
    int have = 0, nsel = 0;
    bool done = false;
    for (int c0 = 0; c0 < n && !done; c0 += 64) {
        const int r = c0 + l;
        const bool in = r < n && keys[r] != 0ull;
        const uint32_t leaf = in ? rank_key_id(keys[r]) : 0u;
        const int w = in ? leaf_weight(cv, bg, leaf, q) : 0;
        const uint32_t lmeta = in ? cv.meta[bg * cv.s_meta + leaf] : 0u;
        const int cum = wave_incl_scan(w) + have;
        const int before = cum - w;
        const bool take = w > 0 && before < k;
        const uint64_t bal = __ballot(take);
        const int pos = __popcll(bal & ((1ull << l) - 1ull));
        if (take && nsel + pos < sel_cap) sel[nsel + pos] = pack_sel(leaf, lmeta, w, cum <= k, k - before);
        nsel += __popcll(bal);
        have = __shfl(cum, 63);
        if (have >= k) done = true;
    }
    if (nsel > sel_cap) return -1;   // more buckets than sel holds: nothing written, the caller falls back
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
    if (rec != nullptr) {
        write_bucket_records(sel, nsel, cv, bg, q, rec, rcnt);
        if (rec_only) return records_tokens(sel, 0, nsel);
    }
    return wave_expand(sel, nsel, cv, bg, q, out, tk, ent);
}

__device__ __forceinline__ void write_pad(int32_t* out, int from, int k) {
    for (int j = from + lane_id(); j < k; j += 64) out[j] = -1;
}

// Handles the cases that need no ranking: invalid position (count -1), and
// a budget covering every eligible token (the whole range [sink_end, l0)).
__device__ __forceinline__ bool trivial_unit(int64_t t, const Geom& q, int k, int32_t* out, int32_t* cnt_out) {
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
                                                             const float* __restrict__ tau, const int* __restrict__ cnt,
                                                             const uint64_t* __restrict__ cand, int* fb_list,
                                                             int* counters, int32_t* lr_idx, int32_t* lr_cnt) {
    __shared__ __align__(16) uint64_t keys[4][kCandCap];
    __shared__ uint64_t sel[4][kSelCap];
    __shared__ int tk[4][256];
    const int l = lane_id(), wid = threadIdx.x >> 6;
    const int64_t u = (int64_t)blockIdx.x * 4 + wid;
    if (u >= sa.n_units) return;
    const Unit un = unit_of(u, sa);
    const int64_t t = q_pos[un.b * sa.n_q + un.i];
    const Geom q = query_geom(t < 0 ? 0 : t, cv.n_blocks, sa.n_sinks, sa.window);
    int32_t* out = lr_idx + u * sa.k;
    if (trivial_unit(t, q, sa.k, out, lr_cnt + u)) return;
    // the candidates scoring >= tau (the lists may also hold buckets below it), compacted; the
    // candidate list is 4 sub-lists of kSubCap slots with their own counts
    const int4 c4 = *reinterpret_cast<const int4*>(cnt + 4 * u);
    const int cs[4] = {c4.x, c4.y, c4.z, c4.w};
    const bool over = c4.x > kSubCap || c4.y > kSubCap || c4.z > kSubCap || c4.w > kSubCap;
    int f = 0;
    if (!over) {
        const uint64_t kmin = (uint64_t)ord_key(tau[u]) << 32;   // key >= kmin  <=>  score >= tau
        const uint64_t lt = (1ull << l) - 1ull;
#pragma unroll
        for (int sl = 0; sl < 4; ++sl) {
            const int c = cs[sl];
            const uint64_t* cl = cand + u * kCandStride + sl * kSubCap;
            uint64_t kk[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) kk[r] = 64 * r + l < c ? cl[64 * r + l] : 0ull;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const bool keep = 64 * r + l < c && kk[r] >= kmin;
                const uint64_t bal = __ballot(keep);
                const int pos = f + __popcll(bal & lt);
                if (keep && pos < kCandCap) keys[wid][pos] = kk[r];
                f += __popcll(bal);
            }
        }
    }
    if (over || f > kCandCap) {
        if (l == 0) {
            const int pos = atomicAdd(&counters[0], 1);
            fb_list[pos] = (int)u;
        }
        return;
    }
    const int P = pow2_at_least(f);
    for (int j = f + l; j < P; j += 64) keys[wid][j] = 0ull;
    wave_sync();
    wave_sort_desc(keys[wid], P);
    const int64_t bg = un.b * sa.H_kv + un.g;
    // the rank keys are dead once the walk is done: their space holds the entry keys (<= k / 4)
    const int got = wave_walk_expand(keys[wid], f, sel[wid], kSelCap, tk[wid], reinterpret_cast<uint32_t*>(keys[wid]),
                                     cv, bg, q, sa.k, out, sa.brec ? sa.brec + u * LSA_BUCKET_RECS : nullptr,
                                     sa.bcnt ? sa.bcnt + u : nullptr, sa.skip_lists != 0);
    if (got < 0) {   // many small buckets: the exact path takes the unit
        if (l == 0) {
            const int pos = atomicAdd(&counters[0], 1);
            fb_list[pos] = (int)u;
        }
        return;
    }
    if (!(sa.brec && sa.skip_lists)) write_pad(out, got, sa.k);
    if (l == 0) lr_cnt[u] = got;
}

// ------------------------------------------------------------------ materialised path
// Few queries against many buckets (decode).  Two kernels:
//
// score_all_kernel, grid (units x splits), unit-major: every visible bucket
// score of a (query, KV head) and the largest score of every 16-bucket tile,
// written to the workspace (fp32).  A pure stream over the tile-swizzled
// centroids, kScoreTiles tiles per workgroup.
//
// decode_finish_kernel, one workgroup per unit: bounds the candidates with
// the tile maxima, ranks and walks them, and writes the tokens in order
// (below).
// tiles (16 buckets each) per scoring workgroup: 256 (64 per wave) gives 1024 workgroups per 16 x 1M decode
// step, all resident at once, and half as many copies of each unit's query-latent setup as 128 (the decode
// step 2-4 us faster)
constexpr int kScoreTiles = 256;
constexpr int64_t kExactScanAbove = 2048;   // tiles per unit above which the bf16 decode scan writes exact scores

// Eligible tokens of a bucket whose block lies inside or outside [sink_end,
// l0); a block straddling an edge (at most two) needs its member lists.
__device__ __forceinline__ int leaf_weight_whole(uint32_t leaf, uint32_t m, const Geom& q) {
    const int64_t lo = (int64_t)(leaf / kLeavesPerBlock) * kBlockTokens;
    return (lo >= q.sink_end && lo + kBlockTokens <= q.l0) ? kPool * (int)(m & 0xFFu) : 0;
}

// The (at most two) blocks that straddle an edge of [sink_end, l0).
__device__ __forceinline__ void straddling_blocks(const Geom& q, int& b0, int& b1) {
    b0 = (q.sink_end % kBlockTokens) ? (int)(q.sink_end / kBlockTokens) : -1;
    b1 = (q.l0 % kBlockTokens) ? (int)(q.l0 / kBlockTokens) : -1;
    if (b1 == b0) b1 = -1;
}

// Needs no ranking: invalid position, k = 0, or k covering every eligible token.
__device__ __forceinline__ bool unit_is_trivial(int64_t t, const Geom& q, int k) {
    const int64_t total = q.l0 > q.sink_end ? q.l0 - q.sink_end : 0;
    return t < 0 || k == 0 || (int64_t)k >= total;
}

// int8 stage of the bf16 decode scan.  Lane (n, kg) of a wave holds query
// head n's latent dims [16 kg, 16 kg + 16) (zero past the group) as int8
// codes q = round(qhat / sq_n), sq_n = max |qhat_n| / 127.  With the leaf
// codes c = round(cent / sc_x) (the cache's int8 copy), the stage-1 score of
// leaf x is s~ = max_n D_nx sq_n sc_x (D the exact int32 code dot product),
// and |s~ - s| <= sc_x Qa + Qb for the bf16 score s of the same leaf:
//   Qa = 0.5001 max_n ||qhat_n||_1      (the leaf's rounding, |cent - sc c| <= 0.5001 sc),
//   Qb = 0.5001 * 8.3 max_n sq_n + 1e-5 (the query's rounding against ||sc c||_1 <= 8.3 for a
//        centroid of norm <= 1.002, plus fp32 rounding of both scores).
struct QCodes {
    i32x4 codes;     // this lane's 16 codes (B operand of the int8 MFMA)
    float sq;        // sq of this lane's head column (0 past the group)
    float qa, qb;    // the unit's bound constants
};
__device__ __forceinline__ QCodes query_codes(const uint16_t* qrow_h0, int G) {
    const int l = lane_id(), n = l & 15, kg = l >> 4;
    float v[16];
    if (n < G) {
        const uint4* p = reinterpret_cast<const uint4*>(qrow_h0 + n * kLatent + 16 * kg);
        const uint4 a = p[0], b = p[1];
        const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            v[2 * i] = __uint_as_float(w[i] << 16);
            v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
        }
    } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) v[i] = 0.f;
    }
    float amax = 0.f, l1 = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        amax = fmaxf(amax, fabsf(v[i]));
        l1 += fabsf(v[i]);
    }
    amax = fmaxf(amax, __shfl_xor(amax, 16));
    amax = fmaxf(amax, __shfl_xor(amax, 32));
    l1 += __shfl_xor(l1, 16);
    l1 += __shfl_xor(l1, 32);
    QCodes r;
    r.sq = amax / 127.0f;
    const float rq = r.sq > 0.f ? __builtin_amdgcn_rcpf(r.sq) : 0.f;   // 1 ulp: |code - q / sq| <= 0.50003
    uint32_t w4[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        uint32_t word = 0;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const float x = v[4 * e + b];
            const int c = (int)fminf(fmaxf(rintf(x * rq), -127.f), 127.f);
            word |= (uint32_t)(uint8_t)(int8_t)c << (8 * b);
        }
        w4[e] = word;
    }
    r.codes = i32x4{(int)w4[0], (int)w4[1], (int)w4[2], (int)w4[3]};
    float qa = l1 * 1.0001f, qs = r.sq;   // l1 of head n (every kg lane), its sq
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) {
        qa = fmaxf(qa, __shfl_xor(qa, o));
        qs = fmaxf(qs, __shfl_xor(qs, o));
    }
    r.qa = 0.5001f * qa;
    r.qb = 0.5001f * 8.3f * qs + 1e-5f;
    return r;
}

// Maximum over the 16 lanes of each row of the wave (in every lane of the row), by DPP moves: swaps
// inside quads (xor 1, xor 2), then the mirrored half row and the mirrored row.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, true));
}
static_assert(kMaxGroup <= 8, "the decode scan folds heads 4..7 in with one exchange");
__device__ __forceinline__ float row_max16(float x) {
    x = fmaxf(x, dpp_mov<0xB1>(x));    // quad_perm [1, 0, 3, 2]
    x = fmaxf(x, dpp_mov<0x4E>(x));    // quad_perm [2, 3, 0, 1]
    x = fmaxf(x, dpp_mov<0x141>(x));   // row_half_mirror
    return fmaxf(x, dpp_mov<0x140>(x));  // row_mirror
}

// Largest of the 16 scores of a tile held as 4 values in each of the lanes 0, 16, 32, 48 (in every
// lane on return).  Exact: the maximum does not depend on the order it is taken in.
__device__ __forceinline__ float tile_max(const f32x4& v) {
    float m = fmaxf(fmaxf(v[0], v[1]), fmaxf(v[2], v[3]));
    m = fmaxf(m, __shfl_xor(m, 16));
    return fmaxf(m, __shfl_xor(m, 32));
}

// bf16 (D > 0): the scan computes its unit's q_hat rows from Q and W itself
// (no separate latent kernel ahead of it in decode), and the workgroup of
// split 0 writes them to qhat for the finish.
template <bool BF16, int D>
__global__ __launch_bounds__(256) void score_all_kernel(CacheView cv, void* __restrict__ qhat,
                                                        const int64_t* __restrict__ q_pos, SelArgs sa, int splits,
                                                        float* __restrict__ scores, int64_t score_stride,
                                                        float* __restrict__ tmax, int64_t tmax_stride,
                                                        const uint16_t* __restrict__ Qin, const uint16_t* __restrict__ Win,
                                                        int64_t q_rows, int exact) {
    __shared__ __align__(16) uint16_t qrows_lds[BF16 ? 4 * 16 * kLatent : 1];
    __shared__ __align__(16) uint16_t w_lds[BF16 ? (D > 0 ? D : 1) * kLatent : 1];
    const int l = lane_id(), wid = threadIdx.x >> 6, n = l & 15, h = l >> 4;
    const int64_t u = (int64_t)blockIdx.x / splits;
    const int split = (int)((int64_t)blockIdx.x % splits);
    const Unit un = unit_of(u, sa);
    const int64_t t = q_pos[un.b * sa.n_q + un.i];
    const Geom q = query_geom(t < 0 ? 0 : t, cv.n_blocks, sa.n_sinks, sa.window);
    if (unit_is_trivial(t, q, sa.k)) return;
    const int ntiles = kLeavesPerBlock * q.nvis / 16;
    const int t0 = split * kScoreTiles, t1 = min(ntiles, t0 + kScoreTiles);
    const int w0 = t0 + (kScoreTiles / 4) * wid, w1 = min(t1, w0 + kScoreTiles / 4);   // this wave's tiles
    const int64_t bg = un.b * sa.H_kv + un.g;
    const int64_t qrow = ((un.b * sa.n_q + un.i) * sa.H_q + un.g * sa.G) * kLatent;
    float* sc = scores + u * score_stride;
    float* tmx = tmax + u * tmax_stride;
    if constexpr (BF16) {
        const uint4* cq = reinterpret_cast<const uint4*>(cv.cq + bg * cv.s_cq);
        const float* csc = cv.csc + bg * cv.s_csc;
        // batches of TPI tiles; the next batch's loads are in flight while one is scored
        // (loads are unconditional, past the last tile they repeat it, so they stay in flight together)
        constexpr int TPI = 4;
        uint4 a[2][TPI];
        float scl[2][TPI];
        auto issue = [&](int buf, int tb) {
#pragma unroll
            for (int j = 0; j < TPI; ++j) {
                const int64_t tt = min(tb + j, w1 - 1);
                a[buf][j] = cq[tt * 64 + l];
                scl[buf][j] = csc[tt * 16 + n];   // this lane's bucket
            }
        };
        // the first codes are in flight while W is staged in LDS (whole workgroup) and this unit's q_hat
        // rows are computed (the wave of split 0 that scores the first tiles also stores them for the finish)
        if (w0 < w1 && !exact) issue(0, w0);
        for (int x = threadIdx.x; x < D * kLatent / 8; x += 256)
            reinterpret_cast<uint4*>(w_lds)[x] = reinterpret_cast<const uint4*>(Win)[x];
        __syncthreads();
        if (w0 >= w1) return;
        uint16_t* myrows = qrows_lds + wid * 16 * kLatent;
        qlatent_unit_bf16<D>(Qin, w_lds, qrow / kLatent, q_rows, sa.G, myrows,
                             (split == 0 && wid == 0) ? reinterpret_cast<uint16_t*>(qhat) : nullptr);
        if (exact) {
            // exact bf16 scores and tile maxima (the exact path's own MFMA, so the same scores as the fused
            // strategy): the finish's first tile bound then holds without widening however many tiles
            QFragBF16 qf;
            load_qfrag_bf16(qf, myrows, n == 0, sa.G);
            const uint16_t* cent_bg = reinterpret_cast<const uint16_t*>(cv.cent) + bg * cv.s_cent;
            for (int tt = w0; tt < w1; ++tt) {
                const int64_t x0 = (int64_t)tt * 16;
                const f32x4 vals = score_tile_bf16(cent_bg, x0, qf, sa.G);
                if (n == 0) *reinterpret_cast<f32x4*>(sc + x0 + 4 * h) = vals;
                const float m = tile_max(vals);   // lanes 0, 16, 32, 48: query slot 0
                if (l == 0) tmx[tt] = m;
            }
            return;
        }
        // stage-1 scores from the int8 codes (query head n in column n); the tile maximum taken of the
        // upper bounds s~ + sc Qa + Qb
        const QCodes qc = query_codes(myrows, sa.G);
        // the MFMA takes the query heads as rows and the tile's buckets as columns (the operand layouts are
        // alike), so lane (bucket c, h) holds heads 4h..4h+3 of bucket c: the max over heads is 3 maxima in
        // the lane and 2 across its 4 lanes; sq of those heads, a negative factor past the group
        float sqh[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float sj = __shfl(qc.sq, 4 * h + j);   // lane 4h + j holds head 4h + j's sq
            sqh[j] = 4 * h + j < sa.G ? sj : -1.0f;
        }
        const float qa = qc.qa, qb = qc.qb;
        for (int tt0 = w0; tt0 < w1; tt0 += 2 * TPI) {
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                const int tb = tt0 + half * TPI;
                if (tb >= w1) break;
                issue(half ^ 1, tb + TPI);
#pragma unroll
                for (int j = 0; j < TPI; ++j) {
                    if (tb + j < w1) {
                        const uint4 av = a[half][j];
                        i32x4 acc = {0, 0, 0, 0};
                        acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(qc.codes, i32x4{(int)av.x, (int)av.y, (int)av.z,
                                                                                    (int)av.w}, acc, 0, 0, 0);
                        float x = kNegInf;
#pragma unroll
                        for (int v = 0; v < 4; ++v) x = fmaxf(x, sqh[v] >= 0.f ? (float)acc[v] * sqh[v] : kNegInf);
                        x = fmaxf(x, __shfl_xor(x, 16));   // heads 4..7 (a group has at most 8)
                        const float sv = scl[half][j];
                        const float val = x * sv;
                        const float ub = val + (sv * qa + qb);
                        if (h == 0) sc[(int64_t)(tb + j) * 16 + n] = val;
                        const float m = row_max16(ub);   // tile maximum over the 16 buckets (rows 0 and 1)
                        if (l == 0) tmx[tb + j] = m;
                    }
                }
            }
        }
    } else {
        if (w0 >= w1) return;
        const float* qf32 = reinterpret_cast<const float*>(qhat) + qrow;
        for (int tt = w0; tt < w1; ++tt) {
            const int64_t x0 = (int64_t)tt * 16;
            const f32x4 vals =
                score_tile_f32(reinterpret_cast<const float*>(cv.cent) + bg * cv.s_cent, x0, qf32, n == 0, sa.G);
            if (n == 0) *reinterpret_cast<f32x4*>(sc + x0 + 4 * h) = vals;
            const float m = tile_max(vals);   // lanes past column 0 hold -inf
            if (l == 0) tmx[tt] = m;
        }
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

// LDS the exact path of one unit works in: hist[256], sel[kExactSel],
// ebase[kExactSel] (entry keys of the expansion, >= k / 4), tk[256], sh4[4], bc[4].
struct ExactLds {
    uint32_t* hist;
    uint64_t* sel;
    uint32_t* ebase;
    int* tk;
    int* sh4;
    uint32_t* bc;
};

// The exact path for unit u by one 256-thread workgroup: a weighted radix
// select over the unit's scores sc (computed here first when rescore), then
// the selected buckets in id order and their expansion.
template <bool BF16>
__device__ void exact_select_unit(const CacheView& cv, const void* __restrict__ qhat, const int64_t* __restrict__ q_pos,
                                  const SelArgs& sa, int64_t u, float* sc, bool rescore, int32_t* lr_idx,
                                  int32_t* lr_cnt, const ExactLds& m) {
    uint32_t* hist = m.hist;
    uint64_t* sel = m.sel;
    uint32_t* ebase = m.ebase;
    int* tk = m.tk;
    int* sh4 = m.sh4;
    uint32_t* bc = m.bc;
    const int tid = threadIdx.x, l = lane_id(), wid = tid >> 6, n = l & 15, h = l >> 4;
    const Unit un = unit_of(u, sa);
    const int64_t t = q_pos[un.b * sa.n_q + un.i];
    const Geom q = query_geom(t < 0 ? 0 : t, cv.n_blocks, sa.n_sinks, sa.window);
    int32_t* out = lr_idx + u * sa.k;
    if (wid == 0) trivial_unit(t, q, sa.k, out, lr_cnt + u);
    const int64_t total = q.l0 > q.sink_end ? q.l0 - q.sink_end : 0;
    if (t < 0 || sa.k == 0 || (int64_t)sa.k >= total) {
        __syncthreads();
        return;
    }
    const int NLv = kLeavesPerBlock * q.nvis;
    const int64_t bg = un.b * sa.H_kv + un.g;
    if (rescore) {
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
        const bool take_all = gt || (eq && eb + w <= (int)target);
        const bool take_part = !take_all && eq && eb < (int)target;
        int s_tot;
        const int pos = wg_excl_scan((take_all || take_part) ? 1 : 0, sh4, s_tot);
        if ((take_all || take_part) && nsel + pos < kExactSel)
            sel[nsel + pos] = pack_sel((uint32_t)x, cv.meta[bg * cv.s_meta + x], w, take_all, (int)target - eb);
        nsel += s_tot;
        eq_have += eq_tot;
    }
    __syncthreads();
    if (wid == 0) {
        const int ns = nsel < kExactSel ? nsel : kExactSel;
        const int got = wave_expand(sel, ns, cv, bg, q, out, tk, ebase);
        write_pad(out, got, sa.k);
        if (l == 0) lr_cnt[u] = got;
    }
    __syncthreads();
}

// Bin of a score for the decode finish: 4096 bins of width 2^-11 over [-1, 1), monotone
// non-decreasing in the score (scores outside the range land in the end bins).
constexpr int kFinBins = 4096;
constexpr int kFinTiles = 512;     // tiles whose scores one finish reads (more: the exact path)
constexpr int kFinMinTiles = 16;
__device__ __forceinline__ int fin_bin(float s) {
    return (int)fminf(fmaxf((s + 1.0f) * 2048.0f, 0.0f), 4095.0f);
}

// The bin where a histogram's count from the top first reaches `target`
// (thread tid holding bins [16 tid, 16 tid + 16) in hb, `above` the count
// of the higher threads' bins): written to *out by the one thread holding
// it; nothing is written when the whole histogram holds less than target.
__device__ __forceinline__ void crossing_bin(const uint32_t (&hb)[16], int above, int target, int* out) {
#pragma unroll
    for (int j = 15; j >= 0; --j) {
        const int hv = (int)hb[j];
        if (above < target && target <= above + hv) *out = 16 * (int)threadIdx.x + j;
        above += hv;
    }
}

// This thread's 16 bins of an LDS histogram of kFinBins, their sum, and the
// sum over the bins of higher threads (256 threads).
__device__ __forceinline__ int load_bins(const uint32_t* hist, uint32_t (&hb)[16], int* sh4) {
    const uint4* h4 = reinterpret_cast<const uint4*>(hist);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const uint4 v = h4[4 * threadIdx.x + j];
        hb[4 * j] = v.x;
        hb[4 * j + 1] = v.y;
        hb[4 * j + 2] = v.z;
        hb[4 * j + 3] = v.w;
    }
    int mine = 0;
#pragma unroll
    for (int j = 0; j < 16; ++j) mine += (int)hb[j];
    int tot;
    const int pre = wg_excl_scan(mine, sh4, tot);
    return tot - pre - mine;
}

__device__ __forceinline__ void clear_bins(uint32_t* hist) {
    uint4* h4 = reinterpret_cast<uint4*>(hist);
#pragma unroll
    for (int j = 0; j < kFinBins / 1024; ++j) h4[threadIdx.x + 256 * j] = uint4{0u, 0u, 0u, 0u};
}

// Candidate keys of the decode finish: ordered like rank_key (score desc,
// bucket id asc), carrying the candidate's slot in the finish's candidate
// arrays (< kFinC) in the low 10 bits; bucket ids below 2^22.
constexpr int kFinC = 1024;   // buckets at or above the tile bound a finish keeps in LDS
constexpr uint32_t kFinIdMax = (1u << 22) - 1u;
__device__ __forceinline__ uint64_t fin_key(float s, uint32_t id, int slot) {
    return ((uint64_t)ord_key(s) << 32) | ((uint64_t)(kFinIdMax - id) << 10) | (uint64_t)slot;
}
__device__ __forceinline__ uint32_t fin_key_id(uint64_t k) { return kFinIdMax - ((uint32_t)k >> 10); }
__device__ __forceinline__ int fin_key_slot(uint64_t k) { return (int)(k & 0x3FFu); }
__device__ __forceinline__ float fin_key_score(uint64_t k) { return ord_key_inv((uint32_t)(k >> 32)); }

// Exclusive prefix over the wave's lanes of c (0 <= c < 16), and the wave's total, by four ballots.
__device__ __forceinline__ int wave_excl_count16(int c, int& tot) {
    const uint64_t lt = (1ull << lane_id()) - 1ull;
    int pre = 0;
    tot = 0;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        const uint64_t m = __ballot((c >> b) & 1);
        pre += __popcll(m & lt) << b;
        tot += __popcll(m) << b;
    }
    return pre;
}

// Position of the j-th (from 0) set bit of x, which has more than j set bits.
__device__ __forceinline__ int nth_set_bit(uint64_t x, int j) {
    int b = 0;
    uint32_t v = (uint32_t)x;
    int c = __popc(v);
    if (j >= c) {
        j -= c;
        b = 32;
        v = (uint32_t)(x >> 32);
    }
#pragma unroll
    for (int w = 16; w >= 1; w >>= 1) {
        c = __popc(v & ((1u << w) - 1u));
        if (j >= c) {
            j -= c;
            b += w;
            v >>= w;
        }
    }
    return b;
}

constexpr int kFinTmRegs = 8;    // tile maxima a thread holds (2048 tiles; more are read again)
constexpr int kFinSlots = 128;   // blocks among the taken buckets (more: the exact path)
constexpr int kFinOutPer = 8;    // output positions a thread places together

// One workgroup per (query, KV head) after score_all_kernel.  Any bucket
// whose score bin is >= b lies in a tile whose maximum's bin is >= b, so a
// histogram of the tile maxima names a bin b0 with at least M tiles at or
// above it (M = max(16, k / 16), grown while too few tokens turn up; M = all
// tiles means b0 = 0); the buckets of those tiles with a bin >= b0 (the set
// C, kept in LDS) hold every bucket that scores at least as high as any of
// them.  A weighted histogram of C (eligible tokens per bucket) names the bin
// b1 where the tokens from the top first reach k: the buckets of C with a bin
// >= b1 form the candidate set S, and every other bucket scores below every
// bucket in S, so the walk over all buckets in rank order (score desc, id
// asc) ends inside S.  S is ranked (each candidate counts the candidates
// above it), walked to k tokens (the last bucket giving its lowest eligible
// tokens), and the taken buckets are put in id order; their blocks get slots
// in block order, each taken token sets its bit in its slot's 2048-bit mask,
// and prefix counts over the mask words place every output position's token.
// The member lists of S are fetched as soon as S is known, so their latency
// hides behind the ranking.  More than kFinTiles tiles, S larger than
// kCandCap, more than kSelCap taken buckets or kFinSlots blocks: the workgroup
// runs the exact radix path for the unit instead.
__global__ __launch_bounds__(256) void decode_finish_kernel(CacheView cv, const void* __restrict__ qhat,
                                                            const int64_t* __restrict__ q_pos,
                                                            SelArgs sa, const float* __restrict__ scores,
                                                            int64_t score_stride, const float* __restrict__ tmax,
                                                            int64_t tmax_stride, int32_t* lr_idx, int32_t* lr_cnt,
                                                            int int8_scores) {
    __shared__ __align__(16) uint32_t hist[kFinBins];   // histograms, then the mask words' prefix counts
    __shared__ __align__(16) uint64_t keys[kCandCap];   // S
    __shared__ __align__(16) uint64_t mask[kFinSlots * 32 > kExactSel ? kFinSlots * 32 : kExactSel];
    __shared__ __align__(16) uint64_t ckey[kFinC];      // C (or S's own entries when C overflows)
    __shared__ uint32_t cmeta[kFinC];
    __shared__ int cw[kFinC];
    __shared__ int cp[kFinC];      // bounded scores: the candidates of C whose upper bound reaches the bound
    __shared__ float cex[kFinC];   // their bf16 scores
    __shared__ __align__(16) uint4 cmem[kCandCap * 3];  // per S position: 24 member entries from off & ~7
    __shared__ int rk[kCandCap];                         // rank -> S position
    __shared__ uint64_t rmask[kSelCap];
    __shared__ uint32_t tleaf[kSelCap], sleaf[kSelCap], smeta[kSelCap];
    __shared__ int stake[kSelCap], sw[kSelCap], sslot[kSelCap], spos[kSelCap];
    __shared__ int tiles[kFinTiles];
    __shared__ int slot_blk[kFinSlots];
    __shared__ int stk[2 * kLeavesPerBlock];   // eligible tokens of the straddling blocks' buckets
    __shared__ int sh4[4];
    __shared__ int ntl, nc, nk, wsum, bsel, need_stk, fin[3];
    __shared__ uint32_t ebc[4];
    const int tid = threadIdx.x, l = lane_id(), wid = tid >> 6;
    const uint64_t lt = (1ull << l) - 1ull;
    const int64_t u = blockIdx.x;
    const Unit un = unit_of(u, sa);
    // scores are the int8 stage's s~, bounded by +-(sc Qa + Qb); else exact
    const bool filter = cv.bf16 != 0 && int8_scores != 0;
    const int64_t bg = un.b * sa.H_kv + un.g;
    const float* sc = scores + u * score_stride;
    const float* tm = tmax + u * tmax_stride;
    const uint32_t* meta = cv.meta + bg * cv.s_meta;
    const uint16_t* mem_bg = cv.members + bg * cv.s_members;
    const int64_t qrow = ((un.b * sa.n_q + un.i) * sa.H_q + un.g * sa.G) * kLatent;
    // the tile maxima of every bucketed tile and the query rows are loaded before the position (and so
    // the visible tile count NT <= NTmax) is known: their loads are in flight together
    const int NTmax = (int)min((int64_t)kLeavesPerBlock * cv.n_blocks / 16, tmax_stride);
    float tmr[kFinTmRegs];
#pragma unroll
    for (int r = 0; r < kFinTmRegs; ++r) tmr[r] = tid + 256 * r < NTmax ? tm[tid + 256 * r] : 0.f;
    const int64_t t = q_pos[un.b * sa.n_q + un.i];
    float Qa = 0.f, Qb = 0.f;
    if (filter) {   // the bound constants of the scan (the same arithmetic on the same query)
        const QCodes qc = query_codes(reinterpret_cast<const uint16_t*>(qhat) + qrow, sa.G);
        Qa = qc.qa;
        Qb = qc.qb;
    }
    const Geom q = query_geom(t < 0 ? 0 : t, cv.n_blocks, sa.n_sinks, sa.window);
    int32_t* out = lr_idx + u * sa.k;
    if (unit_is_trivial(t, q, sa.k)) {
        if (wid == 0) trivial_unit(t, q, sa.k, out, lr_cnt + u);
        return;
    }
    const int NT = kLeavesPerBlock * q.nvis / 16;
    // the exact radix path, in this workgroup, over the unit's scores (its LDS in arrays that are
    // free whenever it runs)
    auto to_exact = [&]() {
        const ExactLds m{hist, mask, reinterpret_cast<uint32_t*>(cmem), rk, sh4, ebc};
        exact_select_unit<true>(cv, qhat, q_pos, sa, u, const_cast<float*>(scores + u * score_stride), filter,
                                lr_idx, lr_cnt, m);
    };
    static_assert(kCandCap * 3 * 4 >= kExactSel && kCandCap >= 256, "the exact path's LDS fits the finish's arrays");
    // the bounded path; true: the unit needs the exact path instead (one copy of its code, below: the
    // kernel runs once per CU, so its instruction fetch is part of its latency)
    const bool exact = [&]() -> bool {
        if ((int64_t)NT * 16 > (int64_t)kFinIdMax + 1) {
            return true;
        }
        const float* csc = filter ? cv.csc + bg * cv.s_csc : nullptr;
        int sb0, sb1;
        straddling_blocks(q, sb0, sb1);
        // the entry -> bucket map of the straddling blocks (threads 0..127: sb0, 128..255: sb1; 4 entries
        // each), loaded now and turned into eligible tokens per bucket when a listed tile needs them
        const int eblk = tid < 128 ? sb0 : sb1;
        const bool ehave = eblk >= 0 && eblk < q.nvis;
        const uint32_t ecodes =
            ehave ? reinterpret_cast<const uint32_t*>(cv.eleaf + bg * cv.s_eleaf + (int64_t)eblk * kBlockEntries)[tid & 127]
                  : 0u;
        clear_bins(hist);
        if (tid == 0) need_stk = 0;
        __syncthreads();
    #pragma unroll
        for (int r = 0; r < kFinTmRegs; ++r)
            if (tid + 256 * r < NT) atomicAdd(&hist[fin_bin(tmr[r])], 1u);
        for (int x = tid + 256 * kFinTmRegs; x < NT; x += 256) atomicAdd(&hist[fin_bin(tm[x])], 1u);
        __syncthreads();
        uint32_t tb[16];   // this thread's bins of the tile-maximum histogram
        const int tabove = load_bins(hist, tb, sh4);
        // scores, metas and eligible tokens of buckets 4 c .. 4 c + 3 of tile x (0 tokens: not eligible)
        // quarter tile c of tile x: the raw loads (scores, metas, scales), then the per-bucket values:
        // scores, half-widths of their bounds (0 for exact scores), metas and eligible tokens
        struct QuadRaw {
            float4 sv;
            uint4 mv;
            float4 cs;
        };
        auto quad_load = [&](int x, int c) {
            QuadRaw r;
            r.sv = reinterpret_cast<const float4*>(sc + (int64_t)x * 16)[c];
            r.mv = reinterpret_cast<const uint4*>(meta + (int64_t)x * 16)[c];
            r.cs = filter ? reinterpret_cast<const float4*>(csc + (int64_t)x * 16)[c] : float4{0.f, 0.f, 0.f, 0.f};
            return r;
        };
        auto quad_eval = [&](const QuadRaw& r, int x, int c, float (&s4)[4], float (&e4)[4], uint32_t (&m4)[4],
                             int (&w4)[4]) {
            s4[0] = r.sv.x;
            s4[1] = r.sv.y;
            s4[2] = r.sv.z;
            s4[3] = r.sv.w;
            e4[0] = filter ? r.cs.x * Qa + Qb : 0.f;
            e4[1] = filter ? r.cs.y * Qa + Qb : 0.f;
            e4[2] = filter ? r.cs.z * Qa + Qb : 0.f;
            e4[3] = filter ? r.cs.w * Qa + Qb : 0.f;
            m4[0] = r.mv.x;
            m4[1] = r.mv.y;
            m4[2] = r.mv.z;
            m4[3] = r.mv.w;
            const int blk = x / (kLeavesPerBlock / 16);   // a tile lies in one block
            const int so = blk == sb0 ? 0 : (blk == sb1 ? kLeavesPerBlock : -1);
    #pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint32_t leaf = (uint32_t)(16 * x + 4 * c + i);
                w4[i] = so >= 0 ? stk[so + leaf % kLeavesPerBlock] : leaf_weight_whole(leaf, m4[i], q);
            }
        };
        auto quad_buckets = [&](int x, int c, float (&s4)[4], float (&e4)[4], uint32_t (&m4)[4], int (&w4)[4]) {
            quad_eval(quad_load(x, c), x, c, s4, e4, m4, w4);
        };
        // bounded scores need more tiles: the lower bounds of the top buckets must clear the bin of the
        // M-th tile maximum of the upper bounds
        int M = min(NT, filter ? max(4 * kFinMinTiles, sa.k / 8) : max(kFinMinTiles, sa.k / 16));
        int b1 = 0, nt = 0;
        bool have_stk = false;
        for (;;) {
            if (tid == 0) {
                bsel = 0;
                ntl = 0;
                nc = 0;
                wsum = 0;
            }
            clear_bins(hist);   // the tile histogram is in tb[]
            __syncthreads();
            crossing_bin(tb, tabove, M, &bsel);
            __syncthreads();
            const int b0 = M < NT ? bsel : 0;   // M = NT: every bucket of every tile
            auto list = [&](int x, float v) {
                const bool qual = x < NT && fin_bin(v) >= b0;
                const uint64_t bal = __ballot(qual);
                int base = 0;
                if (l == 0 && bal) base = atomicAdd(&ntl, __popcll(bal));
                base = __shfl(base, 0);
                const int pos = base + __popcll(bal & lt);
                if (qual && pos < kFinTiles) tiles[pos] = x;
                const int blk = x / (kLeavesPerBlock / 16);
                if (qual && (blk == sb0 || blk == sb1)) need_stk = 1;
            };
            {   // the tiles held in registers: one slot reservation per wave
                uint32_t qm = 0;
                bool stk_hit = false;
    #pragma unroll
                for (int r = 0; r < kFinTmRegs; ++r) {
                    const int x = tid + 256 * r;
                    if (x < NT && fin_bin(tmr[r]) >= b0) {
                        qm |= 1u << r;
                        const int blk = x / (kLeavesPerBlock / 16);
                        stk_hit = stk_hit || blk == sb0 || blk == sb1;
                    }
                }
                const int c = __popc(qm);
                int tot;
                const int pre = wave_excl_count16(c, tot);
                int base = 0;
                if (l == 0 && tot) base = atomicAdd(&ntl, tot);
                int pos = __shfl(base, 0) + pre;
    #pragma unroll
                for (int r = 0; r < kFinTmRegs; ++r) {
                    if ((qm >> r) & 1u) {
                        if (pos < kFinTiles) tiles[pos] = tid + 256 * r;
                        ++pos;
                    }
                }
                if (stk_hit) need_stk = 1;
            }
            for (int x0 = 256 * kFinTmRegs; x0 < NT; x0 += 256) list(x0 + tid, x0 + tid < NT ? tm[x0 + tid] : 0.f);
            __syncthreads();
            nt = ntl;
            if (nt > kFinTiles) break;   // the exact path (b1 = 0 marks it)
            if (need_stk && !have_stk) {   // a listed tile lies in a block straddling an edge
                // eligible tokens of each bucket of the block: the sum over its entries (entry e holds
                // tokens [4 e, 4 e + 4) of the block) of their tokens inside [sink_end, l0)
                if (tid < 2 * kLeavesPerBlock) stk[tid] = 0;
                __syncthreads();
                if (ehave) {
                    const int so = tid < 128 ? 0 : kLeavesPerBlock;
                    const int64_t tb = (int64_t)eblk * kBlockTokens + (int64_t)kPool * 4 * (tid & 127);
    #pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const uint32_t lf = (ecodes >> (8 * i)) & 0xFFu;
                        int w = 0;
    #pragma unroll
                        for (int jj = 0; jj < kPool; ++jj) {
                            const int64_t tk = tb + kPool * i + jj;
                            w += (tk >= q.sink_end && tk < q.l0) ? 1 : 0;
                        }
                        if (w > 0 && lf < (uint32_t)kLeavesPerBlock) atomicAdd(&stk[so + lf], w);
                    }
                }
                have_stk = true;
                __syncthreads();
            }
            // The weighted histogram of the lower bounds s~ - e (bins >= b0) and C: the buckets of the listed
            // tiles whose upper bound s~ + e has a bin >= b0 (e = 0 for exact scores; a quarter tile per thread)
            int wl = 0;
            constexpr int QPT = 6;   // quarter tiles per thread whose loads are in flight together (384 tiles)
            for (int i0 = 0; i0 < 4 * nt; i0 += 256 * QPT) {
                QuadRaw raw[QPT];   // every load first, then the evaluation
                int xq[QPT];
    #pragma unroll
                for (int qq = 0; qq < QPT; ++qq) {
                    const int idx = min(i0 + 256 * qq + tid, 4 * nt - 1);
                    xq[qq] = tiles[idx >> 2];
                    if (i0 + 256 * qq < 4 * nt) raw[qq] = quad_load(xq[qq], idx & 3);   // uniform
                }
    #pragma unroll
                for (int qq = 0; qq < QPT; ++qq) {
                    if (i0 + 256 * qq >= 4 * nt) break;   // uniform: the wave goes on while any lane has a quarter
                    const int idx = i0 + 256 * qq + tid;
                    const bool valid = idx < 4 * nt;
                    const int x = xq[qq], c4 = idx & 3;
                    float s4[QPT][4], e4[QPT][4];
                    uint32_t m4[QPT][4];
                    int w4[QPT][4];
                    quad_eval(raw[qq], x, c4, s4[qq], e4[qq], m4[qq], w4[qq]);
                    if (!valid) {
    #pragma unroll
                        for (int i = 0; i < 4; ++i) w4[qq][i] = 0;
                    }
                    bool inc[4];
                    int c = 0;
    #pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int bin = fin_bin(s4[qq][i] - e4[qq][i]);
                        if (w4[qq][i] > 0 && bin >= b0) {
                            atomicAdd(&hist[bin], (uint32_t)w4[qq][i]);
                            wl += w4[qq][i];
                        }
                        inc[i] = w4[qq][i] > 0 && fin_bin(s4[qq][i] + e4[qq][i]) >= b0;
                        c += inc[i] ? 1 : 0;
                    }
                    int tot;
                    const int pre = wave_excl_count16(c, tot);   // one slot reservation per wave
                    int base = 0;
                    if (l == 0 && tot) base = atomicAdd(&nc, tot);
                    int pos = __shfl(base, 0) + pre;
    #pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        if (inc[i]) {
                            if (pos < kFinC) {
                                ckey[pos] = fin_key(s4[qq][i] + e4[qq][i], (uint32_t)(16 * x + 4 * c4 + i), pos);
                                cmeta[pos] = m4[qq][i];
                                cw[pos] = w4[qq][i];
                            }
                            ++pos;
                        }
                    }
                }
            }
    #pragma unroll
            for (int o = 32; o >= 1; o >>= 1) wl += __shfl_xor(wl, o);
            if (l == 0 && wl) atomicAdd(&wsum, wl);
            __syncthreads();
            if (wsum >= sa.k) {
                uint32_t wb[16];
                const int wabove = load_bins(hist, wb, sh4);
                if (tid == 0) bsel = -1;
                __syncthreads();
                crossing_bin(wb, wabove, sa.k, &bsel);
                __syncthreads();
                b1 = bsel;   // >= b0: the buckets below b0 were not counted
                break;
            }
            if (M >= NT) break;   // cannot happen: the visible buckets hold more than k eligible tokens (b1 = 0)
            M = min(NT, 4 * M);
            __syncthreads();   // every thread has read wsum before it is reset
        }
        if (b1 <= 0) {   // b1 = 0 would take every bucket: leave the unit to the exact path
            return true;
        }
        // b1: the bin where the lower bounds' tokens reach k, so at least k tokens score >= its edge and
        // every bucket scoring that high has its upper bound in a bin >= b1.  Exact scores (e = 0): S = the
        // buckets of C with a bin >= b1.  Bounded scores: C' = the buckets of C whose upper bound has a
        // bin >= b1, their bf16 scores computed here (the same MFMA as the exact scan), and S = those of C'
        // at or above the bin b where their tokens reach k.
        if (tid == 0) {
            nk = 0;
            fin[0] = 0;
            fin[2] = -1;
        }
        __syncthreads();
        const int ncc = nc;
        if (filter && ncc > kFinC) {
            return true;
        }
        if (filter) {
            if (tid == 0) ntl = 0;
            clear_bins(hist);
            __syncthreads();
            for (int j0 = 0; j0 < ncc; j0 += 256) {   // C'
                const int j = j0 + tid;
                const bool in = j < ncc && fin_bin(fin_key_score(ckey[j])) >= b1;
                const uint64_t bal = __ballot(in);
                int base = 0;
                if (l == 0 && bal) base = atomicAdd(&ntl, __popcll(bal));
                base = __shfl(base, 0);
                if (in) cp[base + __popcll(bal & lt)] = j;
            }
            __syncthreads();
            const int ncp = ntl;
            {   // bf16 scores of C': groups of 16 candidates (MFMA rows), kGrp consecutive groups per wave with
                // their loads in flight together (128 candidates per round)
                constexpr int kGrp = 2;
                const int n = l & 15, h = l >> 4;
                uint4 qa4 = {0, 0, 0, 0}, qc4 = {0, 0, 0, 0};
                if (n < sa.G) {
                    const uint4* pq = reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(qhat) + qrow +
                                                                     n * kLatent + 16 * h);
                    qa4 = pq[0];
                    qc4 = pq[1];
                }
                const bf16x8 q0 = as_bf16x8(qa4), q1 = as_bf16x8(qc4);
                const uint4* cw4 = reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(cv.cent) + bg * cv.s_cent);
                for (int g0 = 16 * kGrp * wid; g0 < ncp; g0 += 64 * kGrp) {
                    uint4 a[kGrp][2];
    #pragma unroll
                    for (int gg = 0; gg < kGrp; ++gg) {
                        if (g0 + 16 * gg < ncp) {   // uniform
                            const int e = min(g0 + 16 * gg + n, ncp - 1);
                            const uint32_t leaf = fin_key_id(ckey[cp[e]]);
                            a[gg][0] = cw4[cent_tile_word(leaf, h, 0)];
                            a[gg][1] = cw4[cent_tile_word(leaf, h, 1)];
                        }
                    }
    #pragma unroll
                    for (int gg = 0; gg < kGrp; ++gg) {
                        if (g0 + 16 * gg >= ncp) break;   // uniform
                        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
                        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a[gg][0]), q0, acc, 0, 0, 0);
                        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a[gg][1]), q1, acc, 0, 0, 0);
    #pragma unroll
                        for (int v = 0; v < 4; ++v) {
                            float x = n < sa.G ? acc[v] : kNegInf;
                            x = fmaxf(x, __shfl_xor(x, 1));
                            x = fmaxf(x, __shfl_xor(x, 2));
                            x = fmaxf(x, __shfl_xor(x, 4));
                            x = fmaxf(x, __shfl_xor(x, 8));
                            const int idx = g0 + 16 * gg + 4 * h + v;
                            if (n == 0 && idx < ncp) cex[idx] = x;
                        }
                    }
                }
            }
            __syncthreads();
            for (int j = tid; j < ncp; j += 256) atomicAdd(&hist[fin_bin(cex[j])], (uint32_t)cw[cp[j]]);
            __syncthreads();
            uint32_t eb[16];
            const int eabove = load_bins(hist, eb, sh4);
            if (tid == 0) bsel = -1;
            __syncthreads();
            crossing_bin(eb, eabove, sa.k, &bsel);
            __syncthreads();
            const int be = bsel;   // >= b1: C' holds every bucket scoring >= the edge of b1
            for (int j0 = 0; j0 < ncp; j0 += 256) {   // S
                const int j = j0 + tid;
                const bool in = j < ncp && be >= 0 && fin_bin(cex[j]) >= be;
                const uint64_t bal = __ballot(in);
                int base = 0;
                if (l == 0 && bal) base = atomicAdd(&nk, __popcll(bal));
                base = __shfl(base, 0);
                const int pos = base + __popcll(bal & lt);
                if (in && pos < kCandCap) keys[pos] = fin_key(cex[j], fin_key_id(ckey[cp[j]]), cp[j]);
            }
        } else if (ncc <= kFinC) {
            for (int j0 = 0; j0 < ncc; j0 += 256) {
                const int j = j0 + tid;
                const uint64_t kc = j < ncc ? ckey[j] : 0ull;
                const bool in = j < ncc && fin_bin(fin_key_score(kc)) >= b1;
                const uint64_t bal = __ballot(in);
                int base = 0;
                if (l == 0 && bal) base = atomicAdd(&nk, __popcll(bal));
                base = __shfl(base, 0);
                const int pos = base + __popcll(bal & lt);
                if (in && pos < kCandCap) keys[pos] = kc;
            }
        } else {   // C overflowed: S from the listed tiles again, its own entries in the C arrays
            for (int idx = tid; idx < 4 * nt; idx += 256) {
                const int x = tiles[idx >> 2], c4 = idx & 3;
                float s4[4], e4[4];
                uint32_t m4[4];
                int w4[4];
                quad_buckets(x, c4, s4, e4, m4, w4);
                bool in[4];
                int c = 0;
    #pragma unroll
                for (int i = 0; i < 4; ++i) {
                    in[i] = w4[i] > 0 && fin_bin(s4[i]) >= b1;
                    c += in[i] ? 1 : 0;
                }
                int pos = c > 0 ? atomicAdd(&nk, c) : 0;
    #pragma unroll
                for (int i = 0; i < 4; ++i) {
                    if (in[i]) {
                        if (pos < kCandCap) {
                            keys[pos] = fin_key(s4[i], (uint32_t)(16 * x + 4 * c4 + i), pos);
                            cmeta[pos] = m4[i];
                            cw[pos] = w4[i];
                        }
                        ++pos;
                    }
                }
            }
        }
        __syncthreads();
        const int f = nk;
        if (f > kCandCap) {
            return true;
        }
        // the member lists of S: 24 entries from off & ~7 per candidate, in flight during the ranking
        uint4 pmv[2][3];
    #pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
            const int j = tid + 256 * h2;
            pmv[h2][0] = pmv[h2][1] = pmv[h2][2] = uint4{0u, 0u, 0u, 0u};
            if (j < f) {
                const uint64_t kj = keys[j];
                const uint32_t m = cmeta[fin_key_slot(kj)];
                const int a = (int)((m >> 8) & 0x3F8u);
                const uint4* p = reinterpret_cast<const uint4*>(mem_bg + (int64_t)(fin_key_id(kj) / kLeavesPerBlock) *
                                                                             kBlockEntries + a);
                pmv[h2][0] = p[0];
                if (a + 8 < kBlockEntries) pmv[h2][1] = p[1];
                if (a + 16 < kBlockEntries) pmv[h2][2] = p[2];
            }
        }
        // rank of each candidate: the number of candidates above it (keys are distinct)
        for (int j = tid; j < f; j += 256) {
            const uint64_t kj = keys[j];
            int r = 0;
            for (int i = 0; i < f; ++i) r += keys[i] > kj ? 1 : 0;
            rk[r] = j;
        }
        __syncthreads();
        // the walk: thread tid holds ranks 2 tid and 2 tid + 1; the rank where the tokens reach k
        {
            const int j0 = 2 * tid, j1 = j0 + 1;
            const int w0 = j0 < f ? cw[fin_key_slot(keys[rk[j0]])] : 0;
            const int w1 = j1 < f ? cw[fin_key_slot(keys[rk[j1]])] : 0;
            int tot;
            const int ex = wg_excl_scan(w0 + w1, sh4, tot);
            if (w0 > 0 && ex < sa.k && sa.k <= ex + w0) {
                fin[0] = j0 + 1;
                fin[1] = sa.k - ex;
            }
            if (w1 > 0 && ex + w0 < sa.k && sa.k <= ex + w0 + w1) {
                fin[0] = j1 + 1;
                fin[1] = sa.k - ex - w0;
            }
        }
        __syncthreads();
        const int ntake = fin[0], last = fin[1];
        if (ntake == 0 || ntake > kSelCap) {   // more buckets than one record row holds
            return true;
        }
        if (tid < ntake) tleaf[tid] = fin_key_id(keys[rk[tid]]);
        __syncthreads();
        // the taken buckets in id order (ids are distinct: a bucket's place is the count of smaller ids)
        if (tid < ntake) {
            const int j = rk[tid];
            const uint32_t leaf = tleaf[tid];
            int r = 0;
            for (int i = 0; i < ntake; ++i) r += tleaf[i] < leaf ? 1 : 0;
            const int slot = fin_key_slot(keys[j]);
            const int w = cw[slot], take = tid == ntake - 1 ? last : w;
            sleaf[r] = leaf;
            smeta[r] = cmeta[slot];
            stake[r] = take;
            sw[r] = w;
            spos[r] = j;
            rmask[r] = 0ull;
        }
        __syncthreads();
        // block slots in block order
        {
            int first = 0, blk = 0;
            if (tid < ntake) {
                blk = (int)(sleaf[tid] / kLeavesPerBlock);
                first = (tid == 0 || (int)(sleaf[tid - 1] / kLeavesPerBlock) != blk) ? 1 : 0;
                if (stake[tid] < sw[tid]) fin[2] = tid;   // the partially taken bucket
            }
            int ns;
            const int ex = wg_excl_scan(first, sh4, ns);
            if (tid < ntake) {
                sslot[tid] = ex + first - 1;
                if (first && ex < kFinSlots) slot_blk[ex] = blk;
            }
            if (tid == 0) fin[1] = ns;
        }
    #pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
            const int j = tid + 256 * h2;
            if (j < f) {
                cmem[3 * j] = pmv[h2][0];
                cmem[3 * j + 1] = pmv[h2][1];
                cmem[3 * j + 2] = pmv[h2][2];
            }
        }
        __syncthreads();
        const int ns = fin[1], rp = fin[2];
        if (ns > kFinSlots) {
            return true;
        }
        for (int w = tid; w < ns * 32; w += 256) mask[w] = 0ull;
        __syncthreads();
        const uint16_t* cm16 = reinterpret_cast<const uint16_t*>(cmem);
        // entry e of taken bucket r (in id order) by thread (16 r + e) mod 256
        for (int idx = tid; idx < ntake * 16; idx += 256) {
            const int r = idx >> 4, e = idx & 15;
            const uint32_t m = smeta[r];
            if (r == rp || e >= (int)(m & 0xFFu)) continue;
            const int mbr = cm16[24 * spos[r] + ((m >> 8) & 7u) + e];
            const int tb0 = kPool * mbr;   // token offset in the block
            const int64_t t0 = (int64_t)(sleaf[r] / kLeavesPerBlock) * kBlockTokens + tb0;
            uint32_t bits = 0;
    #pragma unroll
            for (int jj = 0; jj < kPool; ++jj) bits |= (t0 + jj >= q.sink_end && t0 + jj < q.l0) ? 1u << jj : 0u;
            if (bits) {
                atomicOr(&mask[sslot[r] * 32 + tb0 / 64], (uint64_t)bits << (tb0 % 64));
                atomicOr(&rmask[r], (uint64_t)bits << (kPool * e));
            }
        }
        if (wid == 0 && rp >= 0) {   // the partial bucket: its lowest `take` eligible keys (key l = lane l)
            const uint32_t m = smeta[rp];
            const int e = l >> 2, jj = l & 3, blk = (int)(sleaf[rp] / kLeavesPerBlock);
            const bool in = e < (int)(m & 0xFFu);
            const int tb = in ? kPool * (int)cm16[24 * spos[rp] + ((m >> 8) & 7u) + e] + jj : 0;
            const int64_t t0 = (int64_t)blk * kBlockTokens + tb;
            const bool el = in && t0 >= q.sink_end && t0 < q.l0;
            const uint64_t bal = __ballot(el);
            const bool tk = el && __popcll(bal & lt) < stake[rp];
            const uint64_t bt = __ballot(tk);
            if (tk) atomicOr(&mask[sslot[rp] * 32 + tb / 64], 1ull << (tb % 64));
            if (l == 0) rmask[rp] = bt;
        }
        __syncthreads();
        if (sa.brec) {
            u32x4* rec = sa.brec + u * LSA_BUCKET_RECS;
            if (tid < ntake) rec[tid] = u32x4{sleaf[tid], (uint32_t)rmask[tid], (uint32_t)(rmask[tid] >> 32), 0u};
            if (tid == 0) sa.bcnt[u] = ntake;
        }
        if (!(sa.brec && sa.skip_lists)) {
            // prefix counts of the mask words (thread tid owns words [per tid, per tid + per)), then the
            // token of each output position: its word (the last one whose prefix is <= the position, found
            // by kFinOutPer interleaved binary searches) and the matching set bit in it
            const int nw = ns * 32, per = (nw + 255) / 256, w0 = per * tid;
            int pc = 0;
            for (int w = w0; w < w0 + per && w < nw; ++w) pc += __popcll(mask[w]);
            int tot;
            int run = wg_excl_scan(pc, sh4, tot);
            for (int w = w0; w < w0 + per && w < nw; ++w) {
                hist[w] = (uint32_t)run;
                run += __popcll(mask[w]);
            }
            for (int w = nw + tid; w < kFinBins; w += 256) hist[w] = 0x7FFFFFFFu;   // past the last word
            __syncthreads();
            for (int p0 = 0; p0 < tot; p0 += 256 * kFinOutPer) {
                int lo[kFinOutPer];
    #pragma unroll
                for (int i = 0; i < kFinOutPer; ++i) lo[i] = 0;
    #pragma unroll
                for (int step = kFinBins / 2; step >= 1; step >>= 1) {
    #pragma unroll
                    for (int i = 0; i < kFinOutPer; ++i) {   // lo + step < kFinBins: the read is in bounds
                        const int c = lo[i] + step, p = p0 + 256 * i + tid;
                        lo[i] = (int)hist[c] <= p ? c : lo[i];
                    }
                }
    #pragma unroll
                for (int i = 0; i < kFinOutPer; ++i) {
                    const int p = p0 + 256 * i + tid;
                    if (p < tot)
                        out[p] = slot_blk[lo[i] / 32] * kBlockTokens + (lo[i] % 32) * 64 +
                                 nth_set_bit(mask[lo[i]], p - (int)hist[lo[i]]);
                }
            }
            for (int j = tot + tid; j < sa.k; j += 256) out[j] = -1;
        }
        if (tid == 0) lr_cnt[u] = sa.k;
        return false;
    }();
    if (exact) to_exact();
}



// One workgroup per (query, KV head): weighted radix select of the boundary
// key over materialised scores, then the selected buckets in id order.
// With unit_list, loops over the fallback list; with rescore, it scores each
// unit itself into the row of its workgroup, else reads the unit's own row.
template <bool BF16>
__global__ __launch_bounds__(256) void exact_select_kernel(CacheView cv, const void* __restrict__ qhat,
                                                           const int64_t* __restrict__ q_pos, SelArgs sa,
                                                           const int* unit_list, const int* counters,
                                                           float* scores, int64_t score_stride, int rescore,
                                                           int32_t* lr_idx, int32_t* lr_cnt) {
    __shared__ uint32_t hist[256];
    __shared__ uint64_t sel[kExactSel];
    __shared__ uint32_t ebase[kExactSel];
    __shared__ int tk[256];
    __shared__ int sh4[4];
    __shared__ uint32_t bc[4];
    const ExactLds m{hist, sel, ebase, tk, sh4, bc};
    const int n_items = unit_list ? counters[0] : (int)sa.n_units;
    for (int slot = blockIdx.x; slot < n_items; slot += gridDim.x) {
        const int64_t u = unit_list ? unit_list[slot] : slot;
        exact_select_unit<BF16>(cv, qhat, q_pos, sa, u, scores + (rescore ? (int64_t)blockIdx.x : u) * score_stride,
                                rescore != 0, lr_idx, lr_cnt, m);
    }
}

// ------------------------------------------------------------------ tree beam descent
// One wave per (query, KV head).  A = the group's query latents (heads as
// rows), B = 16 candidate node centroids per MFMA, so lane l ends with the
// scores of heads 4*(l/16)..+3 for candidate l % 16.
// Occupancy: the expansion's entry scratch is dynamic LDS sized by k (ent_cap
// = ceil(k / 4) keys per wave, 8.4 KB per workgroup at k = 2048 instead of
// 16 KB for the largest k), and the register budget is 85 VGPRs, so six
// workgroups share a CU at k = 2048 (a level waits on its centroid loads;
// more waves fill those waits: 8.70 -> 8.35 ms per 65,536-query chunk of the
// 1M layer with its tree).
template <bool BF16>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(6, 6))) void tree_kernel(
    CacheView cv, const void* __restrict__ qhat, const int64_t* __restrict__ q_pos, SelArgs sa, int32_t* lr_idx,
    int32_t* lr_cnt, int ent_cap) {
    __shared__ uint64_t keys[4][2 * LSA_MAX_BEAM];
    __shared__ uint32_t front[4][LSA_MAX_BEAM];
    __shared__ uint64_t sel[4][2 * LSA_MAX_BEAM];
    __shared__ int tk[4][256];
    extern __shared__ __align__(16) uint32_t tree_ent[];   // [4][ent_cap]
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
        const int64_t n_lev = tree_level_size(cv.n_leaves, lev);
        const int64_t lev_off = tree_level_off(cv.n_leaves_cap, lev);
        const int64_t span = (int64_t)1 << lev;
        const int ncand = 2 * nf;
        const int ntiles = (ncand + 15) / 16;
        if (lev > 0 && ncand <= sa.beam) {
            // every visible child is kept whatever its score (only the leaves are ranked): no scoring
            for (int c = l; c < ncand; c += 64) {
                int64_t node = 2 * (int64_t)front[wid][c >> 1] + (c & 1);
                if (node >= n_lev || node * span >= NLv) node = -1;
                keys[wid][c] = node >= 0 ? rank_key(0.f, (uint32_t)node) : 0ull;
            }
        } else if constexpr (BF16) {
            // the candidate tiles' centroid fragments are loaded kTiles at a time before they are
            // scored (a level waits for memory once per batch; fewer registers than one batch of
            // all eight, so more waves per SIMD: measured faster)
            constexpr int kTiles = 2;
            for (int t0 = 0; t0 < 2 * LSA_MAX_BEAM / 16; t0 += kTiles) {
            if (t0 >= ntiles) break;
            uint4 b0[kTiles], b1[kTiles];
            int64_t nodes[kTiles];
#pragma unroll
            for (int tt = 0; tt < kTiles; ++tt) {
                const int c = 16 * (t0 + tt) + n;
                int64_t node = -1;
                if (t0 + tt < ntiles && c < ncand) {
                    node = 2 * (int64_t)front[wid][c >> 1] + (c & 1);
                    if (node >= n_lev || node * span >= NLv) node = -1;
                }
                nodes[tt] = node;
                b0[tt] = b1[tt] = uint4{0, 0, 0, 0};
                if (node >= 0) {
                    if (lev == 0) {   // leaves: tile-swizzled storage
                        const uint4* p =
                            reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(cv.cent) + bg * cv.s_cent);
                        b0[tt] = p[cent_tile_word(node, h, 0)];
                        b1[tt] = p[cent_tile_word(node, h, 1)];
                    } else {
                        // a node straddling the visible leaves: its visible part's centroid (causal mode)
                        const bool edge = sa.causal_tree && (node + 1) * span > NLv;
                        const uint16_t* src =
                            edge ? reinterpret_cast<const uint16_t*>(cv.edge) + bg * cv.s_edge +
                                       ((int64_t)q.nvis * cv.n_lev_cap + lev) * kLatent
                                 : reinterpret_cast<const uint16_t*>(cv.tcent) + bg * cv.s_tcent + (lev_off + node) * kLatent;
                        const uint4* p = reinterpret_cast<const uint4*>(src + 16 * h);
                        b0[tt] = p[0];
                        b1[tt] = p[1];
                    }
                }
            }
#pragma unroll
            for (int tt = 0; tt < kTiles; ++tt) {
                if (t0 + tt < ntiles) {
                    const int c = 16 * (t0 + tt) + n;
                    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa0, as_bf16x8(b0[tt]), acc, 0, 0, 0);
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa1, as_bf16x8(b1[tt]), acc, 0, 0, 0);
                    float sc = kNegInf;
#pragma unroll
                    for (int v = 0; v < 4; ++v)
                        if (4 * h + v < G) sc = fmaxf(sc, acc[v]);
                    sc = fmaxf(sc, __shfl_xor(sc, 16));
                    sc = fmaxf(sc, __shfl_xor(sc, 32));
                    if (h == 0 && c < 2 * LSA_MAX_BEAM)
                        keys[wid][c] = nodes[tt] >= 0 ? rank_key(sc, (uint32_t)nodes[tt]) : 0ull;
                }
            }
            }
        } else {
            for (int tt = 0; tt < ntiles; ++tt) {
                const int c = 16 * tt + n;
                int64_t node = -1;
                if (c < ncand) {
                    node = 2 * (int64_t)front[wid][c >> 1] + (c & 1);
                    if (node >= n_lev || node * span >= NLv) node = -1;
                }
                float sc = kNegInf;
                if (node >= 0) {
                    const bool edge = lev > 0 && sa.causal_tree && (node + 1) * span > NLv;
                    const float* base = lev == 0 ? reinterpret_cast<const float*>(cv.cent) + bg * cv.s_cent +
                                                       node * kLatent
                                        : edge ? reinterpret_cast<const float*>(cv.edge) + bg * cv.s_edge +
                                                     ((int64_t)q.nvis * cv.n_lev_cap + lev) * kLatent
                                               : reinterpret_cast<const float*>(cv.tcent) + bg * cv.s_tcent +
                                                     (lev_off + node) * kLatent;
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
                sc = fmaxf(sc, __shfl_xor(sc, 16));
                sc = fmaxf(sc, __shfl_xor(sc, 32));
                if (h == 0 && c < 2 * LSA_MAX_BEAM) keys[wid][c] = node >= 0 ? rank_key(sc, (uint32_t)node) : 0ull;
            }
        }
        wave_sync();
        const int P = pow2_at_least(ncand);
        for (int j = ncand + l; j < P; j += 64) keys[wid][j] = 0ull;
        wave_sync();
        // the next front is the set of the top `beam` candidates by key (key 0: no candidate),
        // found exactly by a threshold: the beam-th largest high word (the ordered score) by a
        // binary search on ballot counts, then among the keys equal to it the low word (the
        // inverted id) likewise; only the leaves need their rank order, for the walk
        {
            const uint64_t ka = l < P ? keys[wid][l] : 0ull, kb = 64 + l < P ? keys[wid][64 + l] : 0ull;
            const int nvalid = __popcll(__ballot(ka != 0ull)) + __popcll(__ballot(kb != 0ull));
            bool sel_a = ka != 0ull, sel_b = kb != 0ull;
            if (nvalid > sa.beam) {
                const uint32_t ah = (uint32_t)(ka >> 32), bh = (uint32_t)(kb >> 32);
                const uint32_t al = (uint32_t)ka, bl = (uint32_t)kb;
                uint32_t xh = 0;
                for (int bit = 31; bit >= 0; --bit) {
                    const uint32_t c = xh | (1u << bit);
                    if (__popcll(__ballot(ah >= c)) + __popcll(__ballot(bh >= c)) >= sa.beam) xh = c;
                }
                const int need = sa.beam - (__popcll(__ballot(ah > xh)) + __popcll(__ballot(bh > xh)));
                const bool ea = ah == xh, eb = bh == xh;
                uint32_t yl = 0;
                if (__popcll(__ballot(ea)) + __popcll(__ballot(eb)) > need) {
                    for (int bit = 31; bit >= 0; --bit) {
                        const uint32_t c = yl | (1u << bit);
                        if (__popcll(__ballot(ea && al >= c)) + __popcll(__ballot(eb && bl >= c)) >= need) yl = c;
                    }
                }
                sel_a = ah > xh || (ea && al >= yl);
                sel_b = bh > xh || (eb && bl >= yl);
            }
            const uint64_t ba = __ballot(sel_a), bb = __ballot(sel_b);
            const uint64_t lt = (1ull << l) - 1ull;
            const int pa = __popcll(ba & lt), pb = __popcll(ba) + __popcll(bb & lt);
            nf = __popcll(ba) + __popcll(bb);   // min(valid candidates, beam)
            if (lev > 0) {
                if (sel_a) front[wid][pa] = rank_key_id(ka);
                if (sel_b) front[wid][pb] = rank_key_id(kb);
            } else {   // leaves: the nf <= 64 selected keys, sorted descending, for the walk
                wave_sync();
                if (sel_a) keys[wid][pa] = ka;
                if (sel_b) keys[wid][pb] = kb;
                wave_sync();
                uint64_t v[1] = {l < nf ? keys[wid][l] : 0ull};
                reg_sort_desc<1>(v);
                keys[wid][l] = v[0];
            }
        }
        wave_sync();
    }
    // nf <= beam buckets: never more than sel holds
    const int got = wave_walk_expand(keys[wid], nf, sel[wid], 2 * LSA_MAX_BEAM, tk[wid], tree_ent + wid * ent_cap, cv,
                                     bg, q, sa.k,
                                     out, sa.brec ? sa.brec + u * LSA_BUCKET_RECS : nullptr,
                                     sa.bcnt ? sa.bcnt + u : nullptr, sa.skip_lists != 0);
    if (!(sa.brec && sa.skip_lists)) write_pad(out, got, sa.k);
    if (l == 0) lr_cnt[u] = got;
}

// p[0..n) = v (grid-stride)
__global__ __launch_bounds__(256) void fill_i32_kernel(int32_t* __restrict__ p, int64_t n, int32_t v) {
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) p[i] = v;
}

}  // namespace

// ------------------------------------------------------------------ host launch

hipError_t launch_qlatent(const void* Q, const void* W, bool bf16, int d, int64_t rows, void* qhat, int* counters,
                          void* zero, size_t zero_bytes, hipStream_t st) {
    const int64_t zero_n = (int64_t)(zero_bytes / 16);
    // enough workgroups that each thread clears at most ~8 words
    const int64_t zg = (zero_n + 2047) / 2048;
    const unsigned zgrid = (unsigned)(zg < 1024 ? zg : 1024);
    int64_t need = (rows + 15) / 16;
    unsigned grid = (unsigned)(need < 2048 ? (need > 0 ? need : 1) : 2048);
    if (grid < zgrid) grid = zgrid;
    uint4* z = static_cast<uint4*>(zero);
    if (bf16) {
        const int64_t tiles = (rows + 15) / 16;
        unsigned g2 = (unsigned)((tiles + 3) / 4 < 1024 ? ((tiles + 3) / 4 > 0 ? (tiles + 3) / 4 : 1) : 1024);
        if (g2 < zgrid) g2 = zgrid;
        if (d == 128)
            hipLaunchKernelGGL(qlatent_bf16_kernel<128>, dim3(g2), dim3(256), 0, st, static_cast<const uint16_t*>(Q),
                               static_cast<const uint16_t*>(W), rows, static_cast<uint16_t*>(qhat), counters, z, zero_n);
        else
            hipLaunchKernelGGL(qlatent_bf16_kernel<64>, dim3(g2), dim3(256), 0, st, static_cast<const uint16_t*>(Q),
                               static_cast<const uint16_t*>(W), rows, static_cast<uint16_t*>(qhat), counters, z, zero_n);
    } else
        hipLaunchKernelGGL(qlatent_kernel<float>, dim3(grid), dim3(256), 0, st, static_cast<const float*>(Q),
                           static_cast<const float*>(W), d, rows, qhat, 0, counters, z, zero_n);
    return hipGetLastError();
}

hipError_t launch_fill_i32(int32_t* p, int64_t n, int32_t v, hipStream_t st) {
    if (n <= 0) return hipSuccess;
    const unsigned g = (unsigned)((n + 255) / 256 < 4096 ? (n + 255) / 256 : 4096);
    hipLaunchKernelGGL(fill_i32_kernel, dim3(g), dim3(256), 0, st, p, n, v);
    return hipGetLastError();
}

hipError_t launch_select_fused(const CacheView& cv, bool bf16, const int64_t* q_pos, const SelArgs& sa, int B,
                               const SelectBuffers& sb, int32_t* lr_idx, int32_t* lr_cnt, hipStream_t st) {
    dim3 grid((unsigned)((sa.n_q + 63) / 64), (unsigned)sa.H_kv, (unsigned)B);
    if (bf16) {
        const dim3 g2((unsigned)((sa.n_q + kScanQ - 1) / kScanQ), (unsigned)sa.H_kv, (unsigned)B);
        const uint16_t* qh = static_cast<const uint16_t*>(sb.qhat);
        switch (sa.G) {
#define LSA_SCAN_G(GG)                                                                                           \
    case GG:                                                                                                     \
        hipLaunchKernelGGL(scan_fused_kernel<GG>, g2, dim3(256), 0, st, cv, qh, q_pos, sa, sb.tau, sb.cnt, sb.cand); \
        break;
            LSA_SCAN_G(1) LSA_SCAN_G(2) LSA_SCAN_G(3) LSA_SCAN_G(4) LSA_SCAN_G(5) LSA_SCAN_G(6) LSA_SCAN_G(7)
            LSA_SCAN_G(8)
#undef LSA_SCAN_G
            default: return hipErrorInvalidValue;
        }
    } else {
        hipLaunchKernelGGL((fused_scan_kernel<false, 0>), grid, dim3(256), 0, st, cv, sb.qhat, q_pos, sa, sb.tau,
                           sb.cnt, sb.cand);
        hipLaunchKernelGGL((fused_scan_kernel<false, 1>), grid, dim3(256), 0, st, cv, sb.qhat, q_pos, sa, sb.tau,
                           sb.cnt, sb.cand);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(fused_finalize_kernel, dim3((unsigned)((sa.n_units + 3) / 4)), dim3(256), 0, st, cv, q_pos, sa,
                       sb.tau, sb.cnt, sb.cand, sb.fb_list, sb.counters, lr_idx, lr_cnt);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (bf16)
        hipLaunchKernelGGL(exact_select_kernel<true>, dim3((unsigned)sb.fb_slots), dim3(256), 0, st, cv, sb.qhat, q_pos,
                           sa, sb.fb_list, sb.counters, sb.scores, sb.score_stride, 1, lr_idx, lr_cnt);
    else
        hipLaunchKernelGGL(exact_select_kernel<false>, dim3((unsigned)sb.fb_slots), dim3(256), 0, st, cv, sb.qhat,
                           q_pos, sa, sb.fb_list, sb.counters, sb.scores, sb.score_stride, 1, lr_idx, lr_cnt);
    return hipGetLastError();
}

hipError_t launch_select_materialized(const CacheView& cv, bool bf16, const int64_t* q_pos, const SelArgs& sa,
                                      const SelectBuffers& sb, int32_t* lr_idx, int32_t* lr_cnt, const void* Q,
                                      const void* W, int d, int64_t q_rows, hipStream_t st) {
    const int64_t ntiles_max = (int64_t)cv.n_blocks * kLeavesPerBlock / 16;
    const int splits = (int)((ntiles_max + kScoreTiles - 1) / kScoreTiles > 0 ? (ntiles_max + kScoreTiles - 1) / kScoreTiles : 1);
    const dim3 grid((unsigned)(sa.n_units * splits));
    const uint16_t* Qb = static_cast<const uint16_t*>(Q);
    const uint16_t* Wb = static_cast<const uint16_t*>(W);
    // bf16 caches of more than 2048 tiles (1M tokens) are scanned with exact bf16 scores: the int8 bounds'
    // half-width (about 0.016) leaves too few certainly-eligible tokens in the top tiles once there are many
    // tiles near the top, so the finish would widen past its tile capacity and rescore every bucket on the
    // exact path (16 x 2M decode 1.2 ms, 10M 6.8 ms per select); exact scores need no widening
    const int exact = (bf16 && ntiles_max > kExactScanAbove) ? 1 : 0;
    if (bf16 && d == 128)
        hipLaunchKernelGGL((score_all_kernel<true, 128>), grid, dim3(256), 0, st, cv, sb.qhat, q_pos, sa, splits,
                           sb.scores, sb.score_stride, sb.tmax, sb.tmax_stride, Qb, Wb, q_rows, exact);
    else if (bf16)
        hipLaunchKernelGGL((score_all_kernel<true, 64>), grid, dim3(256), 0, st, cv, sb.qhat, q_pos, sa, splits,
                           sb.scores, sb.score_stride, sb.tmax, sb.tmax_stride, Qb, Wb, q_rows, exact);
    else
        hipLaunchKernelGGL((score_all_kernel<false, 0>), grid, dim3(256), 0, st, cv, sb.qhat, q_pos, sa, splits,
                           sb.scores, sb.score_stride, sb.tmax, sb.tmax_stride, Qb, Wb, q_rows, 0);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(decode_finish_kernel, dim3((unsigned)sa.n_units), dim3(256), 0, st, cv, sb.qhat, q_pos, sa,
                       sb.scores,
                       sb.score_stride, sb.tmax, sb.tmax_stride, lr_idx, lr_cnt, exact ? 0 : 1);
    return hipGetLastError();
}

hipError_t launch_select_tree(const CacheView& cv, bool bf16, const int64_t* q_pos, const SelArgs& sa,
                              const SelectBuffers& sb, int32_t* lr_idx, int32_t* lr_cnt, hipStream_t st) {
    dim3 grid((unsigned)((sa.n_units + 3) / 4));
    // the expansion scratch: at least k / 4 entry keys per wave, rounded to 16 bytes (a k above LSA_MAX_K is
    // only accepted when it covers every bucketed token, and then every unit is trivial: no expansion)
    const int k_exp = sa.k < LSA_MAX_K ? sa.k : LSA_MAX_K;
    const int ent_cap = ((k_exp + kPool - 1) / kPool + 3) & ~3;
    const size_t dyn = (size_t)4 * ent_cap * sizeof(uint32_t);
    if (bf16)
        hipLaunchKernelGGL(tree_kernel<true>, grid, dim3(256), dyn, st, cv, sb.qhat, q_pos, sa, lr_idx, lr_cnt,
                           ent_cap);
    else
        hipLaunchKernelGGL(tree_kernel<false>, grid, dim3(256), dyn, st, cv, sb.qhat, q_pos, sa, lr_idx, lr_cnt,
                           ent_cap);
    return hipGetLastError();
}

}  // namespace lsa
