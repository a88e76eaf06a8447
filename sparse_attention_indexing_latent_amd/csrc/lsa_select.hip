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
// fragments use the same dim order and stay in registers for the whole
// (persistent) workgroup.  The C layout gives lane (n, h) rows 4h..4h+3 of
// latent column n of each tile; row norms are reduced over the 16 lanes of
// a row group.
template <int D>
__global__ __launch_bounds__(256) void qlatent_bf16_kernel(const uint16_t* __restrict__ Q,
                                                           const uint16_t* __restrict__ W, int64_t rows,
                                                           uint16_t* __restrict__ qhat, int* counters,
                                                           uint4* zero, int64_t zero_n) {
    constexpr int DPL = D / 4, KS = DPL / 8;
    if (blockIdx.x == 0 && threadIdx.x < 4) counters[threadIdx.x] = 0;
    clear_words(zero, zero_n);
    const int l = lane_id(), wid = threadIdx.x >> 6, r = l & 15, h = l >> 4;
    bf16x8 wf[4][KS];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            uint16_t e[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) e[j] = W[(DPL * h + 8 * ks + j) * kLatent + 16 * nt + r];
            wf[nt][ks] = as_bf16x8(uint4{(uint32_t)e[0] | ((uint32_t)e[1] << 16), (uint32_t)e[2] | ((uint32_t)e[3] << 16),
                                         (uint32_t)e[4] | ((uint32_t)e[5] << 16), (uint32_t)e[6] | ((uint32_t)e[7] << 16)});
        }
    const int64_t ntile = (rows + 15) / 16;
    for (int64_t tile = (int64_t)blockIdx.x * 4 + wid; tile < ntile; tile += (int64_t)gridDim.x * 4) {
        const int64_t row = tile * 16 + r;
        uint4 qa[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            qa[ks] = row < rows ? *reinterpret_cast<const uint4*>(Q + row * D + DPL * h + 8 * ks) : uint4{0, 0, 0, 0};
        f32x4 c[4];
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
            c[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                c[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(qa[ks]), wf[nt][ks], c[nt], 0, 0, 0);
        }
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            float ss = c[0][v] * c[0][v] + c[1][v] * c[1][v] + c[2][v] * c[2][v] + c[3][v] * c[3][v];
            ss += __shfl_xor(ss, 1);
            ss += __shfl_xor(ss, 2);
            ss += __shfl_xor(ss, 4);
            ss += __shfl_xor(ss, 8);
            const float inv = ss > 0.f ? 1.0f / sqrtf(ss) : 0.f;
            const int64_t orow = tile * 16 + 4 * h + v;
            if (orow < rows) {
#pragma unroll
                for (int nt = 0; nt < 4; ++nt) qhat[orow * kLatent + 16 * nt + r] = f32_to_bf16(c[nt][v] * inv);
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
// (16 KB) with their buckets' meta words, double-buffered, and every wave
// reads its operand fragments from LDS (one fragment read feeds 2 x G x 2
// MFMAs).
//
// Each query keeps a histogram of certainly eligible token weight (4 x size
// for buckets of blocks inside [sink_end, l0)) over score bins (8 of width
// 1/8 below 0, 64 of width 1/64 over [0, 1), the end bins open) and a floor
// bin fb: the highest bin at which the weight binned so far, summed from the
// top, reaches k (raised after every chunk).  A visible bucket in a bin >= fb
// is appended (rank key) to the query's candidate list and its weight binned;
// one below fb is skipped: fb only rises, so bins below it can never become
// the final crossing bin b*, and every bin >= b* holds all of its weight.
// Hence at the end tau = lower edge of b* (minus 2^-16; -inf if the weight
// never reaches k) is the bound of the two-pass scan, and the list holds
// every visible bucket scoring >= tau (plus earlier ones below it, dropped
// by the finalize).  A query's list is 4 sub-lists of kSubCap slots, one per
// lane of its MFMA column (no cross-lane step per append); their counts are
// exact even past the cap.
constexpr int kSelCap = 256;        // buckets one finalize wave may take (more: the exact path)
constexpr int kScanQ = 128;         // queries per workgroup
constexpr int kScanChunk = 8;       // tiles per staged chunk
constexpr int kFNeg = 8;
constexpr int kFBins = kFNeg + 64;
constexpr int kFStride = kFBins + 1;   // odd: neighbouring queries fall in different banks

// multiplications by powers of two are exact, so bin(s) >= b  <=>  s >= edge(b)
__device__ __forceinline__ int fscan_bin(float s) {
    const int bp = min(kFNeg + (int)(s * 64.0f), kFBins - 1);
    const int bn = max(kFNeg + (int)floorf(s * 8.0f), 0);
    return s >= 0.f ? bp : bn;
}

__device__ __forceinline__ float fscan_edge(int bin) {
    return bin >= kFNeg ? (float)(bin - kFNeg) * (1.0f / 64.0f) : (float)(bin - kFNeg) * (1.0f / 8.0f);
}

// The highest bin at which one query's histogram, summed from the top,
// reaches k (-1 if it never does).  The query's 4 lanes (h = 0..3, the same
// n) each take a quarter of the bins into registers, the top quarter on
// h = 0; the lane whose quarter holds the crossing walks it down.  All 64
// lanes call it (it shuffles across the wave); the result is on all 4.
__device__ __forceinline__ int fscan_cross_bin(const uint32_t* row, int h, uint32_t k) {
    constexpr int Q4 = kFBins / 4;
    const int lo = kFBins - Q4 * (h + 1);   // this lane's bins: [lo, lo + Q4)
    uint32_t w[Q4];
    uint32_t sq = 0;
#pragma unroll
    for (int j = 0; j < Q4; ++j) w[j] = row[lo + j];
#pragma unroll
    for (int j = 0; j < Q4; ++j) sq += w[j];
    const int n = lane_id() & 15;
    const uint32_t s0 = (uint32_t)__shfl((int)sq, n), s1 = (uint32_t)__shfl((int)sq, n + 16),
                   s2 = (uint32_t)__shfl((int)sq, n + 32);
    uint32_t cum = (h > 0 ? s0 : 0u) + (h > 1 ? s1 : 0u) + (h > 2 ? s2 : 0u);
    int bin = -1;
    if (cum < k) {
#pragma unroll
        for (int j = Q4 - 1; j >= 0; --j) {
            cum += w[j];
            bin = (bin < 0 && cum >= k) ? lo + j : bin;
        }
    }
    bin = max(bin, __shfl_xor(bin, 16));
    bin = max(bin, __shfl_xor(bin, 32));
    return bin;
}

template <int G>
__global__ __launch_bounds__(256) void scan_fused_kernel(CacheView cv, const uint16_t* __restrict__ qhat,
                                                         const int64_t* __restrict__ q_pos, SelArgs sa,
                                                         float* __restrict__ tau, int* __restrict__ cnt,
                                                         uint64_t* __restrict__ cand) {
    __shared__ __align__(16) uint4 stage[2][kScanChunk * 128];   // 2 x 16 KB
    __shared__ __align__(16) uint4 smeta[2][kScanChunk * 4];     // 16 meta words per tile
    __shared__ uint32_t hist[kScanQ * kFStride];
    __shared__ int wmax[4];
    const int tid = threadIdx.x, l = lane_id(), wid = tid >> 6, n = l & 15, h = l >> 4;
    const int64_t b = blockIdx.z, g = blockIdx.y;
    const int64_t bg = b * sa.H_kv + g;
    // per column group cg: this lane's query (column n)
    int64_t u[2], lo_ok[2], hi_ok[2];
    int NLv[2];
    bool qv[2];
    bf16x8 qf[2][G][2];
#pragma unroll
    for (int cg = 0; cg < 2; ++cg) {
        const int64_t iq = (int64_t)blockIdx.x * kScanQ + wid * 32 + cg * 16 + n;
        qv[cg] = iq < sa.n_q;
        const int64_t t = qv[cg] ? q_pos[b * sa.n_q + iq] : -1;
        const Geom q = query_geom(t < 0 ? 0 : t, cv.n_blocks, sa.n_sinks, sa.window);
        NLv[cg] = t < 0 ? 0 : kLeavesPerBlock * q.nvis;
        lo_ok[cg] = q.sink_end;
        hi_ok[cg] = q.l0;
        u[cg] = (b * sa.n_q + (qv[cg] ? iq : 0)) * sa.H_kv + g;
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
    uint32_t* hrow[2] = {hist + (wid * 32 + n) * kFStride, hist + (wid * 32 + 16 + n) * kFStride};
    for (int j = tid; j < kScanQ * kFStride; j += 256) hist[j] = 0u;
    // tiles visible to any query of the workgroup
    const int wm = wave_max_i(max(NLv[0], NLv[1]));
    if (l == 0) wmax[wid] = wm;
    __syncthreads();
    const int maxNLv = max(max(wmax[0], wmax[1]), max(wmax[2], wmax[3]));
    const int ntl = maxNLv / 16;
    const int nch = (ntl + kScanChunk - 1) / kScanChunk;
    const u32x4* src = reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(cv.cent) + bg * cv.s_cent);
    const u32x4* msrc = reinterpret_cast<const u32x4*>(cv.meta + bg * cv.s_meta);
    int fb[2] = {0, 0};
    float fe[2] = {kNegInf, kNegInf};
    int base[2] = {0, 0};   // length of this lane's sub-list (h) of its query's candidate list
    // staging: thread tid copies words tid + 256 j (j < 4) of a chunk and, if tid < 32, meta word tid;
    // tiles past the last one repeat it
    u32x4 r0, r1, r2, r3, rmt;
#define LSA_LOAD_CHUNK(c)                                                                               \
    {                                                                                                   \
        r0 = src[(int64_t)min((c) * kScanChunk + (tid) / 128, ntl - 1) * 128 + (tid & 127)];            \
        r1 = src[(int64_t)min((c) * kScanChunk + (tid + 256) / 128, ntl - 1) * 128 + (tid & 127)];      \
        r2 = src[(int64_t)min((c) * kScanChunk + (tid + 512) / 128, ntl - 1) * 128 + (tid & 127)];      \
        r3 = src[(int64_t)min((c) * kScanChunk + (tid + 768) / 128, ntl - 1) * 128 + (tid & 127)];      \
        if (tid < kScanChunk * 4) rmt = msrc[(int64_t)min((c) * kScanChunk + tid / 4, ntl - 1) * 4 + (tid & 3)]; \
    }
#define LSA_STORE_CHUNK(bf)                                                                             \
    {                                                                                                   \
        u32x4* d4 = reinterpret_cast<u32x4*>(stage[bf]);                                                \
        d4[tid] = r0;                                                                                   \
        d4[tid + 256] = r1;                                                                             \
        d4[tid + 512] = r2;                                                                             \
        d4[tid + 768] = r3;                                                                             \
        if (tid < kScanChunk * 4) reinterpret_cast<u32x4*>(smeta[bf])[tid] = rmt;                       \
    }
    if (nch > 0) {
        LSA_LOAD_CHUNK(0)
        LSA_STORE_CHUNK(0)
    }
    __syncthreads();
    for (int c = 0; c < nch; ++c) {
        if (c + 1 < nch) LSA_LOAD_CHUNK(c + 1)
        const uint4* sb = stage[c & 1];
        const uint4* sm = smeta[c & 1];
        const int tend = min(kScanChunk, ntl - c * kScanChunk);
        bf16x8 a0 = as_bf16x8(sb[l]), a1 = as_bf16x8(sb[64 + l]);
        for (int tt = 0; tt < tend; ++tt) {
            const int x0 = (c * kScanChunk + tt) * 16;
            const int xb = x0 + 4 * h;
            f32x4 best[2];
#pragma unroll
            for (int cg = 0; cg < 2; ++cg) {
#pragma unroll
                for (int hh = 0; hh < G; ++hh) {
                    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, qf[cg][hh][0], acc, 0, 0, 0);
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, qf[cg][hh][1], acc, 0, 0, 0);
                    if (hh == 0) {
                        best[cg] = acc;
                    } else {
                        best[cg][0] = fmaxf(best[cg][0], acc[0]);
                        best[cg][1] = fmaxf(best[cg][1], acc[1]);
                        best[cg][2] = fmaxf(best[cg][2], acc[2]);
                        best[cg][3] = fmaxf(best[cg][3], acc[3]);
                    }
                }
            }
            // next tile's fragments (the last tile of a chunk re-reads itself)
            const int tn = tt + 1 < tend ? tt + 1 : tt;
            a0 = as_bf16x8(sb[tn * 128 + l]);
            a1 = as_bf16x8(sb[tn * 128 + 64 + l]);
            // visible buckets of each query scoring at or above its floor's edge (few once it has risen)
            uint32_t m[2];
#pragma unroll
            for (int cg = 0; cg < 2; ++cg) {
                const int lim = qv[cg] ? NLv[cg] - xb : 0;   // buckets xb + v with v < lim are visible
                m[cg] = (best[cg][0] >= fe[cg] && 0 < lim ? 1u : 0u) | (best[cg][1] >= fe[cg] && 1 < lim ? 2u : 0u) |
                        (best[cg][2] >= fe[cg] && 2 < lim ? 4u : 0u) | (best[cg][3] >= fe[cg] && 3 < lim ? 8u : 0u);
            }
            if (m[0] | m[1]) {
                const int64_t lo = (int64_t)(x0 / kLeavesPerBlock) * kBlockTokens;
                const uint4 m4 = sm[tt * 4 + h];
                const uint32_t mm[4] = {m4.x, m4.y, m4.z, m4.w};
#pragma unroll
                for (int cg = 0; cg < 2; ++cg) {
                    if (m[cg]) {
                        // this lane's sub-list h of its query's candidate list
                        const bool elig = lo >= lo_ok[cg] && lo + kBlockTokens <= hi_ok[cg];
                        uint64_t* sub = cand + u[cg] * kCandStride + h * kSubCap;
#pragma unroll
                        for (int v = 0; v < 4; ++v) {
                            if (m[cg] & (1u << v)) {
                                if (base[cg] < kSubCap) sub[base[cg]] = rank_key(best[cg][v], (uint32_t)(xb + v));
                                ++base[cg];
                                if (elig)
                                    atomicAdd(&hrow[cg][fscan_bin(best[cg][v])], (uint32_t)kPool * (mm[v] & 0xFFu));
                            }
                        }
                    }
                }
            }
        }
        if (c + 1 < nch) LSA_STORE_CHUNK((c + 1) & 1)
        // raise the floors (the histogram rows are this wave's own)
        wave_sync();
#pragma unroll
        for (int cg = 0; cg < 2; ++cg) {
            fb[cg] = max(fb[cg], fscan_cross_bin(hrow[cg], h, (uint32_t)sa.k));
            fe[cg] = fb[cg] >= 1 ? fscan_edge(fb[cg]) : kNegInf;   // bin(s) >= fb  <=>  s >= fe
        }
        __syncthreads();
    }
#undef LSA_LOAD_CHUNK
#undef LSA_STORE_CHUNK
    wave_sync();
#pragma unroll
    for (int cg = 0; cg < 2; ++cg) {
        const int bin = fscan_cross_bin(hrow[cg], h, (uint32_t)sa.k);
        if (qv[cg]) {
            if (h == 0) tau[u[cg]] = bin >= 1 ? fscan_edge(bin) - 1.52587890625e-05f : kNegInf;
            cnt[4 * u[cg] + h] = base[cg];
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
// score of a (query, KV head), written to the workspace (fp32).  A pure
// stream over the tile-swizzled centroids, up to 128 tiles per workgroup.
//
// score_select_kernel, one 1024-thread workgroup per unit, records held in
// registers: packed record = offset key << 7 | eligible tokens per bucket
// (the key is monotone in the score).  Finds a key bound L such that the
// buckets keyed >= L hold at least k eligible tokens while those above L's
// bin hold fewer, with at most kCandCap buckets at or above L (weighted
// histograms of 3072, 2048 and 4 bins, each refining the boundary bin of the
// one before), collects those buckets, and wave 0 ranks them by (score
// desc, id asc), walks them to k tokens and expands.  Every bucket keyed
// below L ranks after every collected one, so the walk ends exactly where a
// walk over all buckets would.  Too many ties at L send the unit to the
// exact radix path.
constexpr int kScoreTiles = 16;   // tiles (16 buckets each) per scoring workgroup: small workgroups overlap best
constexpr int kThrThreads = 1024;
constexpr int kThrBins = 3072;    // level 0: key >> 13
constexpr int kThrGoal = 128;     // refine the bound while more buckets than this sit at or above it
constexpr int kThrRegs = 32;      // records per thread (one chunk = 32768 buckets)
constexpr int kMaxBlockWords = 1024;   // blocks a unit may see: 64 x 1024 (2^27 tokens)
constexpr int kMaskSlots = 384;        // distinct blocks among the taken buckets

// Workgroup-wide exclusive scan over 1024 threads; tot = the sum.  scratch: 16 ints.
__device__ __forceinline__ int wg1024_excl_scan(int v, int* scratch, int& tot) {
    const int l = lane_id(), wid = threadIdx.x >> 6;
    const int inc = wave_incl_scan(v);
    if (l == 63) scratch[wid] = inc;
    __syncthreads();
    int base = 0;
    tot = 0;
    for (int w = 0; w < 16; ++w) {
        const int s = scratch[w];
        base += w < wid ? s : 0;
        tot += s;
    }
    __syncthreads();
    return base + inc - v;
}

// Offset key of a score: monotone non-decreasing in the score and in
// [0, 3 * 2^23) (s + 2 clamped to [0.5, 4)).  Equal keys need not mean equal
// scores, so the key only bounds the candidate set; ranking uses the score.
__device__ __forceinline__ uint32_t thr_key(float s) {
    const float v = fminf(fmaxf(s + 2.0f, 0.5f), 3.99999976f);
    return __float_as_uint(v) - 0x3F000000u;
}

__device__ __forceinline__ unsigned long long shfl_down_u64(unsigned long long v, int o) {
    uint32_t lo = (uint32_t)v, hi = (uint32_t)(v >> 32);
    lo = __shfl_down(lo, o);
    hi = __shfl_down(hi, o);
    return ((unsigned long long)hi << 32) | lo;
}

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

template <bool BF16>
__global__ __launch_bounds__(256) void score_all_kernel(CacheView cv, const void* __restrict__ qhat,
                                                        const int64_t* __restrict__ q_pos, SelArgs sa, int splits,
                                                        float* __restrict__ scores, int64_t score_stride) {
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
    if (w0 >= w1) return;
    const int64_t bg = un.b * sa.H_kv + un.g;
    const int64_t qrow = ((un.b * sa.n_q + un.i) * sa.H_q + un.g * sa.G) * kLatent;
    float* sc = scores + u * score_stride;
    if constexpr (BF16) {
        // B operand: query head n of the group in column n (zero columns past G);
        // the group max is taken across the 16 lanes of each row group
        uint4 qa = {0, 0, 0, 0}, qc = {0, 0, 0, 0};
        if (n < sa.G) {
            const uint4* p = reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(qhat) + qrow +
                                                            n * kLatent + 16 * h);
            qa = p[0];
            qc = p[1];
        }
        const bf16x8 q0 = as_bf16x8(qa), q1 = as_bf16x8(qc);
        const uint16_t* cb = reinterpret_cast<const uint16_t*>(cv.cent) + bg * cv.s_cent;
        // batches of TPI tiles; the next batch's loads are in flight while one is scored
        // (loads are unconditional, past the last tile they repeat it, so they stay in flight together)
        constexpr int TPI = 4;
        uint4 a[2][TPI][2];
#pragma unroll
        for (int j = 0; j < TPI; ++j)
            load_cent_bf16(cb, (int64_t)min(w0 + j, w1 - 1) * 16, a[0][j][0], a[0][j][1]);
        for (int tt0 = w0; tt0 < w1; tt0 += 2 * TPI) {
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                const int tb = tt0 + half * TPI;
                if (tb >= w1) break;
#pragma unroll
                for (int j = 0; j < TPI; ++j)
                    load_cent_bf16(cb, (int64_t)min(tb + TPI + j, w1 - 1) * 16, a[half ^ 1][j][0], a[half ^ 1][j][1]);
#pragma unroll
                for (int j = 0; j < TPI; ++j) {
                    if (tb + j < w1) {
                        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
                        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a[half][j][0]), q0, acc, 0, 0, 0);
                        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a[half][j][1]), q1, acc, 0, 0, 0);
                        f32x4 vals;
#pragma unroll
                        for (int v = 0; v < 4; ++v) {
                            float x = n < sa.G ? acc[v] : kNegInf;
                            x = fmaxf(x, __shfl_xor(x, 1));
                            x = fmaxf(x, __shfl_xor(x, 2));
                            x = fmaxf(x, __shfl_xor(x, 4));
                            x = fmaxf(x, __shfl_xor(x, 8));
                            vals[v] = x;
                        }
                        if (n == 0) *reinterpret_cast<f32x4*>(sc + (int64_t)(tb + j) * 16 + 4 * h) = vals;
                    }
                }
            }
        }
    } else {
        const float* qf32 = reinterpret_cast<const float*>(qhat) + qrow;
        for (int tt = w0; tt < w1; ++tt) {
            const int64_t x0 = (int64_t)tt * 16;
            const f32x4 vals =
                score_tile_f32(reinterpret_cast<const float*>(cv.cent) + bg * cv.s_cent, x0, qf32, n == 0, sa.G);
            if (n == 0) *reinterpret_cast<f32x4*>(sc + x0 + 4 * h) = vals;
        }
    }
}

template <bool BF16>
__global__ __launch_bounds__(kThrThreads) void score_select_kernel(CacheView cv, const int64_t* __restrict__ q_pos,
                                                                    SelArgs sa, const float* __restrict__ scores,
                                                                    int64_t score_stride, int* fb_list, int* counters,
                                                                    int32_t* lr_idx, int32_t* lr_cnt) {
    // LDS (153 KB): the packed records of up to 32768 buckets, the histogram
    // (count << 32 | weight), and small scratch.  Once the candidates are
    // collected, the record space holds the ranking scratch and the tokens.
    __shared__ __align__(16) uint32_t rec[kThrRegs * kThrThreads];
    __shared__ unsigned long long hist[kThrBins];
    __shared__ unsigned long long wtot[kThrThreads / 64];
    __shared__ int wtot32[kThrThreads / 64];
    __shared__ uint32_t bc[4];
    __shared__ int ncand, fin[3];
    __shared__ int tk[2 * kLeavesPerBlock];   // eligible tokens of the straddling blocks' buckets
    const int tid = threadIdx.x, l = lane_id(), wid = tid >> 6;
    const int64_t u = blockIdx.x;
    const Unit un = unit_of(u, sa);
    const int64_t t = q_pos[un.b * sa.n_q + un.i];
    const Geom q = query_geom(t < 0 ? 0 : t, cv.n_blocks, sa.n_sinks, sa.window);
    int32_t* out = lr_idx + u * sa.k;
    if (unit_is_trivial(t, q, sa.k)) {
        if (wid == 0) trivial_unit(t, q, sa.k, out, lr_cnt + u);
        return;
    }
    const int64_t bg = un.b * sa.H_kv + un.g;
    const float* sc = scores + u * score_stride;
    const uint32_t* meta = cv.meta + bg * cv.s_meta;
    const int NLv = kLeavesPerBlock * q.nvis;
    constexpr int kChunk = kThrRegs * kThrThreads;
    const int nchunks = (NLv + kChunk - 1) / kChunk;
    // Eligible tokens of the buckets of the (at most two) blocks straddling an
    // edge of [sink_end, l0), from their member lists, once.
    int sb0, sb1;
    straddling_blocks(q, sb0, sb1);
    if (tid < 2 * kLeavesPerBlock) {
        const int blk = tid < kLeavesPerBlock ? sb0 : sb1;
        const int64_t x = (int64_t)blk * kLeavesPerBlock + tid % kLeavesPerBlock;
        tk[tid] = (blk >= 0 && x < NLv) ? leaf_weight(cv, bg, (uint32_t)x, q) : 0;
    }
    __syncthreads();
    // Records of one chunk into LDS, 16 at a time per thread with their
    // score and meta loads in flight together (unconditional, clamped index).
    auto load_chunk = [&](int c0) {
        for (int j0 = 0; j0 < kThrRegs; j0 += 16) {
            float s8[16];
            uint32_t m8[16];
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const int x = c0 + (j0 + j) * kThrThreads + tid;
                const int xc = x < NLv ? x : NLv - 1;
                s8[j] = sc[xc];
                m8[j] = meta[xc];
            }
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const int x = c0 + (j0 + j) * kThrThreads + tid;
                const int blk = x / kLeavesPerBlock;
                const int w = blk == sb0   ? tk[x % kLeavesPerBlock]
                              : blk == sb1 ? tk[kLeavesPerBlock + x % kLeavesPerBlock]
                                           : leaf_weight_whole((uint32_t)x, m8[j], q);
                rec[(j0 + j) * kThrThreads + tid] = x < NLv ? (thr_key(s8[j]) << 7) | (uint32_t)w : 0u;
            }
        }
        __syncthreads();
    };
    const bool resident = nchunks == 1;
    if (resident) load_chunk(0);
    uint32_t lo = 0, target = (uint32_t)sa.k, cabove = 0, lower = 0, flo = 0;
    int shift = 13, nb = kThrBins;
    bool overflow = false;
    // Level -1 histograms only each thread's best bucket.  Those are a subset
    // of all buckets, so if the ones at or above bin F hold >= k tokens then so
    // do all buckets at or above F, and the boundary bin is >= F: level 0 may
    // skip every bucket below F (far fewer LDS atomics).
    for (int level = -1; level < 3; ++level) {
        for (int j = tid; j < nb; j += kThrThreads) hist[j] = 0ull;
        __syncthreads();
        const uint32_t hi = lo + ((uint32_t)nb << shift);
        uint32_t best = 0;   // best record with a nonzero weight (records compare by key first)
        for (int c = 0; c < nchunks; ++c) {
            if (!resident) load_chunk(c * kChunk);
            for (int j = 0; j < kThrRegs; ++j) {
                const uint32_t r = rec[j * kThrThreads + tid];
                const uint32_t key = r >> 7, w = r & 0x7Fu;
                if (level < 0) {
                    if (w > 0 && r > best) best = r;
                } else if (w > 0 && key >= lo && key < hi && key >= flo) {
                    atomicAdd(&hist[(key - lo) >> shift], (1ull << 32) | (unsigned long long)w);
                }
            }
            if (!resident) __syncthreads();   // the chunk's records are overwritten next
        }
        if (level < 0 && best != 0u)
            atomicAdd(&hist[(best >> 7) >> shift], (1ull << 32) | (unsigned long long)(best & 0x7Fu));
        if (level < 0 && tid == 0) bc[0] = 0xFFFFFFFFu;   // stays so if the best buckets hold < k tokens
        __syncthreads();
        // thread tid owns bins [per * tid, per * tid + per); suffix sums run from the top bin down
        const int per = (nb + kThrThreads - 1) / kThrThreads;
        const int b0 = per * tid;
        unsigned long long mine = 0ull;
        for (int j = 0; j < per; ++j)
            if (b0 + j < nb) mine += hist[b0 + j];
        unsigned long long suf = mine;   // inclusive suffix within the wave (lanes >= l)
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const unsigned long long v = shfl_down_u64(suf, o);
            if (l + o < 64) suf += v;
        }
        if (l == 0) wtot[wid] = suf;
        __syncthreads();
        unsigned long long above = suf - mine;   // bins of higher threads in this wave
        for (int w2 = wid + 1; w2 < kThrThreads / 64; ++w2) above += wtot[w2];
        // the boundary bin: weight above it < target <= weight above it + its own
        for (int j = per - 1; j >= 0; --j) {
            const int bin = b0 + j;
            if (bin >= nb) continue;
            const unsigned long long hv = hist[bin];
            const uint32_t wa = (uint32_t)above, wb = (uint32_t)hv;
            if (wa < target && target <= wa + wb) {
                bc[0] = (uint32_t)bin;
                bc[1] = target - wa;
                bc[2] = (uint32_t)(above >> 32);
                bc[3] = (uint32_t)(hv >> 32);
            }
            above += hv;
        }
        __syncthreads();
        const uint32_t B = bc[0], rem = bc[1], cab = cabove + bc[2], cB = bc[3];
        __syncthreads();
        if (level < 0) {
            flo = B == 0xFFFFFFFFu ? 0u : (B << shift);
            continue;
        }
        if (B == 0xFFFFFFFFu) {   // cannot happen: the visible buckets hold every eligible token (> k)
            overflow = true;
            break;
        }
        if (cab + cB <= (uint32_t)(level == 2 ? kCandCap : kThrGoal)) {
            lower = lo + (B << shift);
            break;
        }
        if (level == 2) {
            overflow = true;
            break;
        }
        lo += B << shift;
        target = rem;
        cabove = cab;
        shift = level == 0 ? 2 : 0;
        nb = level == 0 ? 2048 : 4;
    }
    if (overflow) {   // too many buckets tie at the boundary key: the exact radix path takes the unit
        if (tid == 0) {
            const int pos = atomicAdd(&counters[0], 1);
            fb_list[pos] = (int)u;
        }
        return;
    }
    uint32_t* cid = reinterpret_cast<uint32_t*>(hist);   // [kCandCap] candidate ids (the histogram is dead)
    if (tid == 0) ncand = 0;
    __syncthreads();
    for (int c = 0; c < nchunks; ++c) {
        if (!resident) load_chunk(c * kChunk);
        for (int j = 0; j < kThrRegs; ++j) {
            const int x = c * kChunk + j * kThrThreads + tid;
            const uint32_t r = rec[j * kThrThreads + tid];
            const bool take = (r & 0x7Fu) != 0u && (r >> 7) >= lower;
            const uint64_t bal = __ballot(take);
            int base = 0;
            if (l == 0 && bal) base = atomicAdd(&ncand, __popcll(bal));
            base = __shfl(base, 0);
            if (take) {
                const int pos = base + __popcll(bal & ((1ull << l) - 1ull));
                if (pos < kCandCap) cid[pos] = (uint32_t)x;
            }
        }
        if (!resident) __syncthreads();
    }
    __syncthreads();
    // the record space is dead: ranking scratch and the tokens
    uint64_t* keys = reinterpret_cast<uint64_t*>(rec);         // [kCandCap]
    uint64_t* used = keys + kCandCap;                           // [kMaxBlockWords] blocks holding taken buckets
    uint64_t* mask = used + kMaxBlockWords;                     // [kMaskSlots][32] token masks
    uint32_t* cmeta = reinterpret_cast<uint32_t*>(mask + kMaskSlots * 32);   // [kCandCap]
    int* cw = reinterpret_cast<int*>(cmeta + kCandCap);         // [kCandCap]
    int* coff = cw + kCandCap;                                  // [kCandCap]
    int* upre = coff + kCandCap;                                // [kMaxBlockWords]
    int* slot_blk = upre + kMaxBlockWords;                      // [kMaskSlots]
    static_assert(kCandCap * (8 + 12) + kMaxBlockWords * 12 + kMaskSlots * (256 + 4) <= kThrRegs * kThrThreads * 4,
                  "ranking scratch fits the records' space");
    // ---- rank the candidates (score desc, id asc)
    const int nc = ncand < kCandCap ? ncand : kCandCap;
    const int P = pow2_at_least(nc);
    for (int j = tid; j < P; j += kThrThreads) keys[j] = j < nc ? rank_key(sc[cid[j]], cid[j]) : 0ull;
    __syncthreads();
    if (wid == 0) wave_sort_desc(keys, P);
    __syncthreads();
    // ---- eligible tokens of each ranked candidate, then the buckets taken until k tokens
    if (tid < nc) {
        const uint32_t x = rank_key_id(keys[tid]);
        const uint32_t m = meta[x];
        const int blk = (int)(x / kLeavesPerBlock);
        cmeta[tid] = m;
        cw[tid] = blk == sb0 ? tk[x % kLeavesPerBlock]
                  : blk == sb1 ? tk[kLeavesPerBlock + x % kLeavesPerBlock]
                               : leaf_weight_whole(x, m, q);
    }
    __syncthreads();
    if (wid == 0) {
        int run = 0, ntake = nc, last = 0;
        for (int c0 = 0; c0 < nc; c0 += 64) {
            const int j = c0 + l;
            const int w = j < nc ? cw[j] : 0;
            const int incl = wave_incl_scan(w) + run;
            if (j < nc) coff[j] = incl - w;
            const uint64_t hit = __ballot(j < nc && w > 0 && incl >= sa.k && incl - w < sa.k);
            if (hit) {
                const int hl = __builtin_ctzll(hit);
                ntake = c0 + hl + 1;
                last = sa.k - __shfl(incl - w, hl);   // tokens the boundary bucket gives
                break;
            }
            run = __shfl(incl, 63);
        }
        if (l == 0) {
            fin[0] = ntake;
            // total: k when the boundary was reached (always, the candidates hold >= k tokens)
            fin[1] = ntake < nc || last > 0 ? sa.k : run;
            fin[2] = last;
        }
    }
    __syncthreads();
    const int ntake = fin[0], total = fin[1], last = fin[2];
    // ---- tokens in ascending order through per-block token masks: the blocks of the taken buckets
    // get slots in block order (a bitmap of used blocks and its prefix counts), every emitted token
    // sets its bit in its block's 2048-bit mask, and a prefix count over the mask words places it.
    const int nbw = (cv.n_blocks + 63) / 64;
    if (nbw > kMaxBlockWords) {   // beyond the masks' reach: the exact radix path takes the unit
        if (tid == 0) fb_list[atomicAdd(&counters[0], 1)] = (int)u;
        return;
    }
    for (int w = tid; w < nbw; w += kThrThreads) used[w] = 0ull;
    __syncthreads();
    for (int j = tid; j < ntake; j += kThrThreads) {
        const uint32_t blk = rank_key_id(keys[j]) / kLeavesPerBlock;
        atomicOr(&used[blk / 64], 1ull << (blk % 64));
    }
    __syncthreads();
    {
        const int pc = tid < nbw ? __popcll(used[tid]) : 0;   // nbw <= kThrThreads
        int tot;
        const int ex = wg1024_excl_scan(pc, wtot32, tot);
        if (tid < nbw) {
            upre[tid] = ex;
            uint64_t m = used[tid];
            int r = ex;
            while (m) {   // slot -> block
                const int b = __builtin_ctzll(m);
                m &= m - 1;
                if (r < kMaskSlots) slot_blk[r] = tid * 64 + b;
                ++r;
            }
        }
        if (tid == 0) fin[0] = tot;
    }
    __syncthreads();
    const int nslots = fin[0];
    if (nslots > kMaskSlots) {
        if (tid == 0) fb_list[atomicAdd(&counters[0], 1)] = (int)u;
        return;
    }
    for (int w = tid; w < nslots * 32; w += kThrThreads) mask[w] = 0ull;
    __syncthreads();
    // emit: bucket j by wave j % 16, lane l = member l / 4, token l % 4 (members ascending, so the
    // lanes' eligible tokens are in ascending order and the boundary bucket keeps its lowest ones)
    {
        constexpr int NW = kThrThreads / 64, GB = 4;   // waves; buckets per wave whose member loads fly together
        const uint16_t* mem_bg = cv.members + bg * cv.s_members;
        const int e = l >> 2, jj = l & 3;
        for (int j0 = wid; j0 < ntake; j0 += NW * GB) {
            uint16_t mv[GB];
#pragma unroll
            for (int g = 0; g < GB; ++g) {
                const int j = min(j0 + g * NW, ntake - 1);
                const uint32_t m = cmeta[j];
                const int sz = (int)(m & 0xFFu), off = (int)((m >> 8) & 0x3FFu);
                const int64_t blk = rank_key_id(keys[j]) / kLeavesPerBlock;
                mv[g] = mem_bg[blk * kBlockEntries + off + (e < sz ? e : 0)];
            }
#pragma unroll
            for (int g = 0; g < GB; ++g) {
                const int j = j0 + g * NW;
                if (j >= ntake) break;
                const uint32_t m = cmeta[j];
                const int sz = (int)(m & 0xFFu);
                const int blk = (int)(rank_key_id(keys[j]) / kLeavesPerBlock);
                const int tb = kPool * mv[g] + jj;   // token offset in the block
                const int64_t t0 = (int64_t)blk * kBlockTokens + tb;
                const bool el = e < sz && t0 >= q.sink_end && t0 < q.l0;
                const uint64_t bal = __ballot(el);
                const int pos = __popcll(bal & ((1ull << l) - 1ull));
                const int quota = (j == ntake - 1 && last > 0) ? last : 64;
                if (el && pos < quota) {
                    const int slot = upre[blk / 64] + __popcll(used[blk / 64] & ((1ull << (blk % 64)) - 1ull));
                    atomicOr(&mask[slot * 32 + tb / 64], 1ull << (tb % 64));
                }
            }
        }
    }
    __syncthreads();
    // thread tid owns mask words [per * tid, per * tid + per): its tokens follow those of lower words
    {
        const int nw = nslots * 32, per = (nw + kThrThreads - 1) / kThrThreads, w0 = per * tid;
        int pc = 0;
        for (int w = w0; w < w0 + per && w < nw; ++w) pc += __popcll(mask[w]);
        int tot;
        int pos = wg1024_excl_scan(pc, wtot32, tot);
        for (int w = w0; w < w0 + per && w < nw; ++w) {
            uint64_t m = mask[w];
            const int32_t base = slot_blk[w / 32] * kBlockTokens + (w % 32) * 64;
            while (m) {
                const int b = __builtin_ctzll(m);
                m &= m - 1;
                out[pos++] = base + b;
            }
        }
    }
    for (int j = total + tid; j < sa.k; j += kThrThreads) out[j] = -1;
    if (tid == 0) lr_cnt[u] = total;
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
    __shared__ uint32_t ebase[kExactSel];   // entry keys of the expansion (>= k / 4)
    __shared__ int tk[256];
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
        float* sc = scores + (rescore ? (int64_t)blockIdx.x : u) * score_stride;
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
    __shared__ int tk[4][256];
    __shared__ uint32_t ent[4][LSA_MAX_K / kPool];
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
    const int got = wave_walk_expand(keys[wid], nf, sel[wid], 2 * LSA_MAX_BEAM, tk[wid], ent[wid], cv, bg, q, sa.k,
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
                                      const SelectBuffers& sb, int32_t* lr_idx, int32_t* lr_cnt, hipStream_t st) {
    const int64_t ntiles_max = (int64_t)cv.n_blocks * kLeavesPerBlock / 16;
    const int splits = (int)((ntiles_max + kScoreTiles - 1) / kScoreTiles > 0 ? (ntiles_max + kScoreTiles - 1) / kScoreTiles : 1);
    const dim3 grid((unsigned)(sa.n_units * splits));
    if (bf16)
        hipLaunchKernelGGL(score_all_kernel<true>, grid, dim3(256), 0, st, cv, sb.qhat, q_pos, sa, splits, sb.scores,
                           sb.score_stride);
    else
        hipLaunchKernelGGL(score_all_kernel<false>, grid, dim3(256), 0, st, cv, sb.qhat, q_pos, sa, splits, sb.scores,
                           sb.score_stride);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (bf16)
        hipLaunchKernelGGL(score_select_kernel<true>, dim3((unsigned)sa.n_units), dim3(kThrThreads), 0, st, cv, q_pos,
                           sa, sb.scores, sb.score_stride, sb.fb_list, sb.counters, lr_idx, lr_cnt);
    else
        hipLaunchKernelGGL(score_select_kernel<false>, dim3((unsigned)sa.n_units), dim3(kThrThreads), 0, st, cv, q_pos,
                           sa, sb.scores, sb.score_stride, sb.fb_list, sb.counters, lr_idx, lr_cnt);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    // the fallback list is almost always empty: a few workgroups loop over it (cheaper to launch)
    const unsigned fb_grid = (unsigned)(sb.fb_slots < 8 ? sb.fb_slots : 8);
    if (bf16)
        hipLaunchKernelGGL(exact_select_kernel<true>, dim3(fb_grid), dim3(256), 0, st, cv, sb.qhat, q_pos, sa,
                           sb.fb_list, sb.counters, sb.scores, sb.score_stride, 0, lr_idx, lr_cnt);
    else
        hipLaunchKernelGGL(exact_select_kernel<false>, dim3(fb_grid), dim3(256), 0, st, cv, sb.qhat, q_pos, sa,
                           sb.fb_list, sb.counters, sb.scores, sb.score_stride, 0, lr_idx, lr_cnt);
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
