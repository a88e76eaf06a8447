// Bucket-major (inverted) attention over the long-range keys on gfx950.
//
// Method: diosapp.com.cn LSA tutorial, section 二 (the attention itself is
// plain softmax(q K[keys]^T / sqrt(d)) V[keys]); zhichai.net explainer
// "卡片柜", ch.3 (the long-range keys of a query are whole buckets, the last
// one cut to its lowest-index keys).
//
// In a prefill pass every bucket is picked by many queries, so instead of
// gathering each query's keys (about 1 MiB of K/V per query and KV head),
// the (query, bucket) pairs are grouped by bucket: a workgroup stages one
// bucket's keys and values in LDS once and runs the MFMAs for every query
// that picked it, leaving one partial (fp32 max and denominator, the
// unnormalised output per head as fp16 times an fp32 scale) per pair.  The gather kernel then attends sinks + window
// and merges the unit's partials with a log-sum-exp combine.  The result is
// the same attention; only the order of the softmax sums differs.
//
// Steps of one pass (queries [q0, q0 + nqp) of every sequence):
//   pairs    one wave per unit: its sorted long-range list -> (bucket, 64-bit
//            key mask) pairs, a slot range from the pool, a rank per bin
//   scan     exclusive scan of the per-bin pair counts
//   scatter  pair slots grouped by bin
//   leaf     one workgroup per bucket: keys and values in LDS, 16 query heads
//            (whole GQA groups of 16 / G pairs) per MFMA column tile
// A unit whose list the pairs step cannot take (not strictly ascending, a key
// outside [sink end, window start), more than kBmUnitCap buckets, or a full
// pool) keeps np = -1 and is gathered whole by the gather kernel instead.

#include "lsa_launch.hpp"

namespace lsa {

namespace {

constexpr float kNegInf = -__builtin_huge_valf();

__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__global__ __launch_bounds__(256) void bm_clear_kernel(uint32_t* __restrict__ p, int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) p[i] = 0u;
}

// Pairs of the current block: lane r turns the mask gathered for bucket
// rank r into one pair (if any key of it was listed) and clears it.
__device__ __forceinline__ int bm_flush(unsigned long long* mk, uint32_t* pl, unsigned long long* pm, int blk,
                                        int np) {
    const int l = lane_id();
    wave_lds_sync();
    const unsigned long long m = mk[l];
    const uint64_t nz = __ballot(m != 0ull);
    const int idx = np + __popcll(nz & ((1ull << l) - 1ull));
    if (m != 0ull && idx < kBmUnitCap) {
        pl[idx] = (uint32_t)(blk * kLeavesPerBlock + l);
        pm[idx] = m;
    }
    mk[l] = 0ull;
    wave_lds_sync();
    return np + __popcll(nz);
}

// One wave per local unit ul = (b * nqp + i - q0) * H_kv + g.  A listed
// token tk lies in block tk / 2048, entry e = (tk / 4) % 512 of it, bucket
// rank entry_leaf[e] and key number 4 entry_pos[e] + tk % 4 of that bucket.
// The list is ascending, so the tokens of one block are consecutive: their
// keys are OR-ed into 64 per-rank masks in LDS and flushed when the block
// changes.
__global__ __launch_bounds__(256) void bm_pairs_kernel(CacheView cv, const int64_t* __restrict__ q_pos,
                                                       const int32_t* __restrict__ lr_idx,
                                                       const int32_t* __restrict__ lr_cnt, AttArgs aa, BmBuffers bm) {
    __shared__ unsigned long long mk[4][64];
    __shared__ uint32_t pl[4][kBmUnitCap];
    __shared__ unsigned long long pm[4][kBmUnitCap];
    const int l = lane_id(), wid = threadIdx.x >> 6;
    const int64_t ul = (int64_t)blockIdx.x * 4 + wid;
    if (ul >= aa.n_units) return;
    const int g = (int)(ul % aa.H_kv);
    const int64_t rr = ul / aa.H_kv;
    const int64_t b = rr / aa.nqp, i = aa.q0 + rr % aa.nqp;
    const int64_t u = (b * aa.n_q + i) * aa.H_kv + g;
    const int64_t t = q_pos[b * aa.n_q + i];
    int32_t cnt = lr_cnt[u];
    cnt = cnt < aa.k ? cnt : aa.k;
    mk[wid][l] = 0ull;
    wave_lds_sync();
    int np = 0;
    bool bad = false;
    const int64_t bg = b * aa.H_kv + g;
    if (t >= 0 && cnt > 0) {
        const Geom q = query_geom(t, aa.n_blocks, aa.n_sinks, aa.window);
        const int32_t* lr = lr_idx + u * aa.k;
        const uint8_t* el = cv.eleaf + bg * cv.s_eleaf;
        const uint8_t* ep = cv.epos + bg * cv.s_epos;
        int32_t prev = -1;
        int cur = -1;
        // rounds of 16 groups of 64 listed tokens: every load of a round is
        // issued before the groups are walked in order
        constexpr int RG = 16;
        for (int r0 = 0; r0 < cnt && !bad; r0 += 64 * RG) {
            int32_t tkr[RG];
            uint32_t inf[RG];   // bucket rank | key number << 8
#pragma unroll
            for (int m = 0; m < RG; ++m) {
                const int j = r0 + 64 * m + l;
                tkr[m] = j < cnt ? lr[j] : 0;
            }
#pragma unroll
            for (int m = 0; m < RG; ++m) {
                const int j = r0 + 64 * m + l;
                const int32_t tk = tkr[m];
                // a token outside the bucketed blocks is caught by the range check below; clamp the lookup
                const int64_t tc = tk >= 0 && (int64_t)tk < (int64_t)aa.n_blocks * kBlockTokens ? tk : 0;
                const int64_t e = (tc / kBlockTokens) * kBlockEntries + ((tc / kPool) % kBlockEntries);
                inf[m] = 0u;
                if (j < cnt) inf[m] = (uint32_t)(el[e] & (kLeavesPerBlock - 1)) | ((uint32_t)(kPool * ep[e] + (tc % kPool)) << 8);
            }
#pragma unroll
            for (int m = 0; m < RG; ++m) {
                const int j0 = r0 + 64 * m;
                if (j0 >= cnt || bad) break;
                const bool valid = j0 + l < cnt;
                const int32_t tk = tkr[m];
                int32_t before = __shfl_up(tk, 1);
                if (l == 0) before = prev;
                // [sink end, window start) lies inside the bucketed blocks
                const bool ok = !valid || (tk > before && (int64_t)tk >= q.sink_end && (int64_t)tk < q.l0);
                if (__ballot(!ok) != 0ull) {
                    bad = true;
                    break;
                }
                prev = __shfl(tk, 63);   // read only when lane 63 was valid (a further group exists)
                const int blk = tk / kBlockTokens;
                const int rank = (int)(inf[m] & 0xFFu), bit = (int)(inf[m] >> 8);
                uint64_t pending = __ballot(valid);
                while (pending != 0ull) {
                    const int cb = __shfl(blk, __builtin_ctzll(pending));
                    if (cb != cur) {
                        if (cur >= 0) np = bm_flush(mk[wid], pl[wid], pm[wid], cur, np);
                        cur = cb;
                    }
                    const uint64_t mine = __ballot(valid && blk == cb) & pending;
                    if ((mine >> l) & 1ull) atomicOr(&mk[wid][rank], 1ull << bit);
                    pending &= ~mine;
                }
            }
        }
        if (!bad && cur >= 0) np = bm_flush(mk[wid], pl[wid], pm[wid], cur, np);
    }
    if (bad || np > kBmUnitCap) np = -1;
    uint32_t base = 0;
    if (np > 0) {
        if (l == 0) base = atomicAdd(bm.lcnt + bm.nbins_pad, (uint32_t)np);
        base = __shfl(base, 0);
        if ((uint64_t)base + (uint64_t)np > (uint64_t)bm.pool_cap) np = -1;
    }
    if (np > 0) {
        wave_lds_sync();
        for (int idx = l; idx < np; idx += 64) {
            const uint32_t bin = (uint32_t)(bg * bm.leaves_max + pl[wid][idx]);
            const uint32_t rk = atomicAdd(bm.lcnt + bin, 1u);
            const unsigned long long m = pm[wid][idx];
            bm.rec[base + (uint32_t)idx] = u32x4{bin, rk, (uint32_t)m, (uint32_t)(m >> 32)};
        }
    }
    if (l == 0) {
        bm.unit_off[ul] = base;
        bm.unit_np[ul] = np;
    }
}

// Exclusive scan of the pair counts inside each chunk of kBmScanChunk bins
// (16 per thread), and the chunk's total.
__global__ __launch_bounds__(256) void bm_scan_kernel(BmBuffers bm) {
    __shared__ uint32_t ws[4];
    const int tid = threadIdx.x, l = lane_id(), wid = tid >> 6;
    const int64_t b0 = (int64_t)blockIdx.x * kBmScanChunk + tid * 16;
    const u32x4* src = reinterpret_cast<const u32x4*>(bm.lcnt + b0);
    u32x4 v[4];
    uint32_t s = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        v[j] = src[j];
        s += v[j][0] + v[j][1] + v[j][2] + v[j][3];
    }
    const uint32_t incl = (uint32_t)wave_incl_scan((int)s);
    if (l == 63) ws[wid] = incl;
    __syncthreads();
    uint32_t wpre = 0;
    for (int w = 0; w < wid; ++w) wpre += ws[w];
    uint32_t run = wpre + incl - s;
    u32x4* dst = reinterpret_cast<u32x4*>(bm.loff + b0);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        u32x4 o;
#pragma unroll
        for (int x = 0; x < 4; ++x) {
            o[x] = run;
            run += v[j][x];
        }
        dst[j] = o;
    }
    if (tid == 255) bm.ctot[blockIdx.x] = wpre + incl;
}

// Exclusive scan of the chunk totals: one workgroup, 1024 chunks per step.
__global__ __launch_bounds__(1024) void bm_scan_top_kernel(BmBuffers bm, int64_t nch) {
    __shared__ uint32_t ws[16];
    const int tid = threadIdx.x, l = lane_id(), wid = tid >> 6;
    uint32_t carry = 0;
    for (int64_t c0 = 0; c0 < nch; c0 += 1024) {
        const int64_t c = c0 + tid;
        const uint32_t v = c < nch ? bm.ctot[c] : 0u;
        const uint32_t incl = (uint32_t)wave_incl_scan((int)v);
        if (l == 63) ws[wid] = incl;
        __syncthreads();
        uint32_t wpre = 0, tot = 0;
        for (int w = 0; w < 16; ++w) {
            wpre += w < wid ? ws[w] : 0u;
            tot += ws[w];
        }
        if (c < nch) bm.csum[c] = carry + wpre + incl - v;
        carry += tot;
        __syncthreads();
    }
}

__device__ __forceinline__ uint32_t bm_bin_start(const BmBuffers& bm, uint32_t bin) {
    return bm.csum[bin / kBmScanChunk] + bm.loff[bin];
}

// One wave per local unit: its pair records go to their bin's place as
// (unit, pair slot, key mask).
__global__ __launch_bounds__(256) void bm_scatter_kernel(AttArgs aa, BmBuffers bm) {
    const int l = lane_id(), wid = threadIdx.x >> 6;
    const int64_t ul = (int64_t)blockIdx.x * 4 + wid;
    if (ul >= aa.n_units) return;
    const int np = bm.unit_np[ul];
    if (np <= 0) return;
    const uint32_t base = bm.unit_off[ul];
    for (int idx = l; idx < np; idx += 64) {
        const uint32_t p = base + (uint32_t)idx;
        const u32x4 r = bm.rec[p];
        bm.srec[bm_bin_start(bm, r[0]) + r[1]] = u32x4{(uint32_t)ul, p, r[2], r[3]};
    }
}

// LDS of one bucket (up to 64 keys, kept in member order: key j is token
// 4 members[j / 4] + j % 4 of the block).
//   K   [64 keys][D]: 16-byte chunk c of key j at chunk c ^ (j % CPR) of its
//       row, so the MFMA A-operand reads (16 keys x one chunk) and the
//       row-wise writes are free of bank conflicts;
//   V^T [D][64 slots]: slot s of k-step kk holds key 32 kk + 16 (s%8/4) +
//       4 (s/8 % 4) + s % 4, i.e. the 8 keys lane (n, h) of the score tiles
//       2 kk and 2 kk + 1 owns, so P needs no shuffle; chunk c of row d is
//       stored at c ^ (d % 8) ^ (d / 8 % 8): the MFMA reads (rows 16 dt + n)
//       and the transposing writes (rows 8 c' + 2x for 16 chunks c') both
//       spread over all banks.
template <int D>
struct LeafLds {
    static constexpr int CPR = D / 8;
    static constexpr int K_BYTES = 64 * D * 2;
    static constexpr int BYTES = 2 * K_BYTES;
    __device__ static __forceinline__ int k_off(int j, int c) { return (j * CPR + (c ^ (j % CPR))) * 16; }
    __device__ static __forceinline__ int vt_chunk(int d, int c) { return c ^ (d % 8) ^ ((d / 8) % 8); }
    __device__ static __forceinline__ int vt_word(int d, int slot) {   // 32-bit word holding slots 2w, 2w+1
        return K_BYTES / 4 + d * 32 + vt_chunk(d, slot / 8) * 4 + (slot % 8) / 2;
    }
    __device__ static __forceinline__ int vt_off(int d, int c) { return K_BYTES + (d * 8 + vt_chunk(d, c)) * 16; }
};

// slot of key j inside the V^T rows
__device__ __forceinline__ int vt_slot(int j) {
    const int kk = j / 32, r = j % 32;
    return 32 * kk + 8 * ((r % 16) / 4) + 4 * (r / 16) + r % 4;
}

// One workgroup per bin (grid-stride): a bucket's keys/values in LDS, then
// groups of GP = 16 / G pairs (G query heads each) per wave.  Lane (n, h):
// column n = pair n / G, head n % G; S^T tiles are 16 keys x 16 columns
// (rows 4h + v), O^T tiles 16 dims x 16 columns.
template <int D>
__global__ __launch_bounds__(256) void bm_leaf_kernel(CacheView cv, const uint16_t* __restrict__ Q,
                                                      const uint16_t* __restrict__ K,
                                                      const uint16_t* __restrict__ V, AttArgs aa, BmBuffers bm) {
    using LL = LeafLds<D>;
    constexpr int KS = D / 32, NDT = D / 16, CPR = D / 8;
    __shared__ __align__(16) uint8_t lds[LL::BYTES];
    __shared__ int32_t toks[64];
    const int tid = threadIdx.x, l = lane_id(), wid = tid >> 6, n = l & 15, h = l >> 4;
    const int G = aa.G, GP = 16 / G;
    const float sl2 = aa.scale;
    for (int64_t bin = blockIdx.x; bin < bm.nbins; bin += gridDim.x) {
        const uint32_t npairs = bm.lcnt[bin];
        if (npairs == 0u) continue;
        const uint32_t start = bm_bin_start(bm, (uint32_t)bin);
        const int64_t bg = bin / bm.leaves_max, leaf = bin % bm.leaves_max;
        const int blk = (int)(leaf / kLeavesPerBlock);
        const uint32_t meta = cv.meta[bg * cv.s_meta + leaf];
        const int ntok = kPool * (int)(meta & 0xFF);
        const int nrow = (ntok + 31) & ~31;   // keys staged: whole 32-key k-steps
        __syncthreads();   // the previous bucket's LDS is no longer read
        if (tid < 64) {
            int32_t tk = -1;
            if (tid < ntok) {
                const int off = (int)((meta >> 8) & 0x3FF);
                const int e = cv.members[bg * cv.s_members + (int64_t)blk * kBlockEntries + off + tid / kPool];
                tk = blk * kBlockTokens + kPool * e + tid % kPool;
            }
            toks[tid] = tk;
        }
        __syncthreads();
        const uint16_t* Kbg = K + bg * aa.t_cap * D;
        const uint16_t* Vbg = V + bg * aa.t_cap * D;
        // staging: item = (key pair jp, chunk c); keys past the bucket repeat key 0 (finite, weight 0)
        for (int it = tid; it < (nrow / 2) * CPR; it += 256) {
            const int jp = it / CPR, c = it % CPR;
            const int j0 = 2 * jp;
            const int32_t t0 = toks[j0] >= 0 ? toks[j0] : toks[0];
            const int32_t t1 = toks[j0 + 1] >= 0 ? toks[j0 + 1] : toks[0];
            const u32x4 k0 = *reinterpret_cast<const u32x4*>(Kbg + (int64_t)t0 * D + 8 * c);
            const u32x4 k1 = *reinterpret_cast<const u32x4*>(Kbg + (int64_t)t1 * D + 8 * c);
            const u32x4 v0 = *reinterpret_cast<const u32x4*>(Vbg + (int64_t)t0 * D + 8 * c);
            const u32x4 v1 = *reinterpret_cast<const u32x4*>(Vbg + (int64_t)t1 * D + 8 * c);
            *reinterpret_cast<u32x4*>(lds + LL::k_off(j0, c)) = k0;
            *reinterpret_cast<u32x4*>(lds + LL::k_off(j0 + 1, c)) = k1;
            uint32_t* w = reinterpret_cast<uint32_t*>(lds);
            const int s0 = vt_slot(j0);   // even; key j0 + 1 sits in slot s0 + 1
#pragma unroll
            for (int x = 0; x < 4; ++x) {
                w[LL::vt_word(8 * c + 2 * x, s0)] = (v0[x] & 0xFFFFu) | (v1[x] << 16);
                w[LL::vt_word(8 * c + 2 * x + 1, s0)] = (v0[x] >> 16) | (v1[x] & 0xFFFF0000u);
            }
        }
        __syncthreads();
        const int NT = (ntok + 15) / 16, NK = nrow / 32;
        const uint32_t ngroups = (npairs + GP - 1) / GP;
        const int pi = n / G, hh = n % G;
        // software pipeline over this wave's groups: the records two groups
        // ahead and the Q rows one group ahead are in flight while a group
        // is computed (a record with unit ~0: no pair in this column)
#define LSA_BM_REC(GRP, R)                                                                  \
    {                                                                                        \
        const uint32_t pidx_ = (GRP) * GP + pi;                                              \
        R = u32x4{~0u, 0u, 0u, 0u};                                                          \
        if ((GRP) < ngroups && pi < GP && pidx_ < npairs) R = bm.srec[start + pidx_];        \
    }
#define LSA_BM_Q(R, QV)                                                                     \
    {                                                                                        \
        _Pragma("unroll") for (int ks = 0; ks < KS; ++ks) QV[ks] = u32x4{0u, 0u, 0u, 0u};    \
        if (R[0] != ~0u) {                                                                   \
            const int64_t ul_ = R[0];                                                        \
            const int64_t gq_ = ul_ % aa.H_kv, rq_ = ul_ / aa.H_kv;                          \
            const int64_t bq_ = rq_ / aa.nqp, iq_ = aa.q0 + rq_ % aa.nqp;                    \
            const uint16_t* qrow_ = Q + ((bq_ * aa.n_q + iq_) * aa.H_q + gq_ * G + hh) * D;  \
            _Pragma("unroll") for (int ks = 0; ks < KS; ++ks) QV[ks] =                       \
                *reinterpret_cast<const u32x4*>(qrow_ + 32 * ks + 8 * h);                    \
        }                                                                                    \
    }
        u32x4 rc, rn, qf[KS], qn[KS];
        LSA_BM_REC(wid, rc)
        LSA_BM_Q(rc, qf)
        LSA_BM_REC(wid + 4, rn)
        for (uint32_t grp = wid; grp < ngroups; grp += 4) {
            LSA_BM_Q(rn, qn)
            u32x4 rnn;
            LSA_BM_REC(grp + 8, rnn)
            const bool col = rc[0] != ~0u;
            const uint32_t p = rc[1];
            const unsigned long long mask = col ? ((unsigned long long)rc[3] << 32) | rc[2] : 0ull;
            // S^T = K Q^T over the bucket's keys
            f32x4 s[4];
            float mx = kNegInf;
#pragma unroll
            for (int tt = 0; tt < 4; ++tt) {
                s[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
                if (tt < NT) {
#pragma unroll
                    for (int ks = 0; ks < KS; ++ks) {
                        const bf16x8 ka = *reinterpret_cast<const bf16x8*>(lds + LL::k_off(16 * tt + n, 4 * ks + h));
                        s[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, __builtin_bit_cast(bf16x8, qf[ks]), s[tt],
                                                                        0, 0, 0);
                    }
                }
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const int j = 16 * tt + 4 * h + v;
                    s[tt][v] = ((mask >> j) & 1ull) ? s[tt][v] * sl2 : kNegInf;
                    mx = fmaxf(mx, s[tt][v]);
                }
            }
            mx = fmaxf(mx, __shfl_xor(mx, 16));
            mx = fmaxf(mx, __shfl_xor(mx, 32));
            // P (bf16, as the PV MFMA uses it) and its sum
            uint32_t pk[4][2];
            float psum = 0.f;
#pragma unroll
            for (int tt = 0; tt < 4; ++tt) {
                uint16_t q4[4];
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const float e = mx > kNegInf && s[tt][v] > kNegInf ? __expf(s[tt][v] - mx) : 0.f;
                    q4[v] = f32_to_bf16(e);
                    psum += bf16_to_f32(q4[v]);
                }
                pk[tt][0] = (uint32_t)q4[0] | ((uint32_t)q4[1] << 16);
                pk[tt][1] = (uint32_t)q4[2] | ((uint32_t)q4[3] << 16);
            }
            psum += __shfl_xor(psum, 16);
            psum += __shfl_xor(psum, 32);
            // O^T = V^T P^T
            f32x4 acc[NDT];
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt) acc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                if (kk < NK) {
                    const bf16x8 pf = __builtin_bit_cast(
                        bf16x8, u32x4{pk[2 * kk][0], pk[2 * kk][1], pk[2 * kk + 1][0], pk[2 * kk + 1][1]});
#pragma unroll
                    for (int dt = 0; dt < NDT; ++dt) {
                        const bf16x8 va = *reinterpret_cast<const bf16x8*>(lds + LL::vt_off(16 * dt + n, 4 * kk + h));
                        acc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pf, acc[dt], 0, 0, 0);
                    }
                }
            }
            // the row's scale: its largest magnitude over the D dims (4 lanes of the column)
            float amax = 0.f;
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
                for (int v = 0; v < 4; ++v) amax = fmaxf(amax, fabsf(acc[dt][v]));
            amax = fmaxf(amax, __shfl_xor(amax, 16));
            amax = fmaxf(amax, __shfl_xor(amax, 32));
            if (col) {
                const int64_t slot = (int64_t)p * G + hh;
                const float inv = amax > 0.f ? 1.0f / amax : 0.f;
                uint16_t* po = bm.po + slot * D;
#pragma unroll
                for (int dt = 0; dt < NDT; ++dt) {
                    uint32_t w2[2];
#pragma unroll
                    for (int v = 0; v < 4; v += 2)
                        w2[v / 2] = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)(acc[dt][v] * inv)) |
                                    ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)(acc[dt][v + 1] * inv)) << 16);
                    *reinterpret_cast<u32x2*>(po + 16 * dt + 4 * h) = u32x2{w2[0], w2[1]};
                }
                if (h == 0) *reinterpret_cast<f32x4*>(bm.pml + slot * 4) = f32x4{mx, psum, amax, 0.f};
            }
            rc = rn;
            rn = rnn;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) qf[ks] = qn[ks];
        }
#undef LSA_BM_REC
#undef LSA_BM_Q
    }
}

}  // namespace

hipError_t launch_bucket_partials(const CacheView& cv, const void* Q, const void* K, const void* V,
                                  const int64_t* q_pos, const int32_t* lr_idx, const int32_t* lr_cnt,
                                  const AttArgs& aa, const BmBuffers& bm, int D, hipStream_t st) {
    const int64_t nclear = bm.nbins_pad + 1;
    const unsigned cg = (unsigned)((nclear + 2047) / 2048 < 1024 ? (nclear + 2047) / 2048 : 1024);
    hipLaunchKernelGGL(bm_clear_kernel, dim3(cg), dim3(256), 0, st, bm.lcnt, nclear);
    if (aa.n_units == 0) return hipGetLastError();
    const unsigned ug = (unsigned)((aa.n_units + 3) / 4);
    hipLaunchKernelGGL(bm_pairs_kernel, dim3(ug), dim3(256), 0, st, cv, q_pos, lr_idx, lr_cnt, aa, bm);
    const int64_t nch = bm.nbins_pad / kBmScanChunk;
    hipLaunchKernelGGL(bm_scan_kernel, dim3((unsigned)nch), dim3(256), 0, st, bm);
    hipLaunchKernelGGL(bm_scan_top_kernel, dim3(1), dim3(1024), 0, st, bm, nch);
    hipLaunchKernelGGL(bm_scatter_kernel, dim3(ug), dim3(256), 0, st, aa, bm);
    const unsigned lg = (unsigned)(bm.nbins < 8192 ? bm.nbins : 8192);
    if (D == 128)
        hipLaunchKernelGGL(bm_leaf_kernel<128>, dim3(lg), dim3(256), 0, st, cv, static_cast<const uint16_t*>(Q),
                           static_cast<const uint16_t*>(K), static_cast<const uint16_t*>(V), aa, bm);
    else
        hipLaunchKernelGGL(bm_leaf_kernel<64>, dim3(lg), dim3(256), 0, st, cv, static_cast<const uint16_t*>(Q),
                           static_cast<const uint16_t*>(K), static_cast<const uint16_t*>(V), aa, bm);
    return hipGetLastError();
}

}  // namespace lsa
