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
// unnormalised output per head as fp16 values times a power-of-two scale)
// per pair.  The gather kernel then attends sinks + window and merges the
// unit's partials with a log-sum-exp combine.  The result is the same
// attention up to the order of the softmax sums and the fp16 rounding of each
// partial value (relative 2^-11 of that value; the scale is exact).
//
// Steps of one pass (queries [q0, q0 + nqp) of every sequence):
//   pairs    one wave per unit: its bucket records, or its sorted long-range
//            list, -> (bucket, 64-bit key mask) pairs in the unit's staging row
//   uscan    exclusive scan of the units' pair counts, in unit order: each
//            unit's range of partial slots in the pool
//   rank     a rank per pair in its bin (units past the pool: gathered whole)
//   scan     exclusive scan of the per-bin pair counts
//   scatter  pair slots grouped by bin
//   leaf     one workgroup per bucket: keys and values in LDS, 16 query heads
//            (whole GQA groups of 16 / G pairs) per MFMA column tile
// A unit whose list the pairs step cannot take (not strictly ascending, a key
// outside [sink end, window start), more than kBmUnitCap buckets) keeps
// np = -1 and its list is gathered whole by the window kernel instead; so is
// a unit whose pairs do not fit in the pool, from its list (np = -1) or from
// the keys its bucket records name (np = -2).

#include "lsa_launch.hpp"

namespace lsa {

namespace {

constexpr float kNegInf = -__builtin_huge_valf();

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kSwap16 = 0x401F;   // ds_swizzle pattern: lane ^ 16 inside each half-wave

// two values rounded to nearest-even fp16 / bf16 (one gfx950 conversion each), as the halves of a word
__device__ __forceinline__ uint32_t cvt_pk_f16(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, f16x2));
}
__device__ __forceinline__ uint32_t cvt_pk_bf16(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
}
// acc + both bf16 halves of a word (exact products by 1.0, fp32 sum)
__device__ __forceinline__ float sum2_bf16(uint32_t w, float acc) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w), __builtin_bit_cast(bf16x2, 0x3F803F80u), acc,
                                           false);
}

__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// A value from another lane of the same quad (DPP quad_perm; every lane of
// the wave must be active).
template <int CTRL>
__device__ __forceinline__ uint32_t quad_dpp(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ uint64_t quad_dpp64(uint64_t v) {
    return ((uint64_t)quad_dpp<CTRL>((uint32_t)(v >> 32)) << 32) | quad_dpp<CTRL>((uint32_t)v);
}

__global__ __launch_bounds__(256) void bm_clear_kernel(uint32_t* __restrict__ p, int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) p[i] = 0u;
}

constexpr int kBmTableBlocks = 8;   // blocks whose bucket masks a pairs wave holds at once

// Pairs of the blocks in the wave's table: for slot s (block tb[s]), lane r
// turns the mask gathered for bucket rank r into one pair (if any key of it
// was listed) and clears it.
__device__ __forceinline__ int bm_flush(unsigned long long (*tab)[64], const int* tb, int used, uint32_t* pl,
                                        unsigned long long* pm, int np) {
    const int l = lane_id();
    wave_lds_sync();
    for (int s = 0; s < used; ++s) {
        const unsigned long long m = tab[s][l];
        const uint64_t nz = __ballot(m != 0ull);
        const int idx = np + __popcll(nz & ((1ull << l) - 1ull));
        if (m != 0ull) {
            if (idx < kBmUnitCap) {
                pl[idx] = (uint32_t)(tb[s] * kLeavesPerBlock + l);
                pm[idx] = m;
            }
            tab[s][l] = 0ull;
        }
        np += __popcll(nz);
    }
    wave_lds_sync();
    return np;
}

// One wave per local unit ul = (b * nqp + i - q0) * H_kv + g.  A listed
// token tk lies in block tk / 2048, entry e = (tk / 4) % 512 of it, bucket
// rank entry_leaf[e] and key number 4 entry_pos[e] + tk % 4 of that bucket.
// The list is ascending, so the tokens of one block are consecutive: the
// wave gives each new block the next slot of a table of kBmTableBlocks
// blocks x 64 bucket masks in LDS, ORs every token's key bit into its slot
// (one LDS atomic per token, a whole group of 64 tokens at once) and turns
// the table into pairs when it is full and at the end.  A bucket whose
// tokens straddle a flush gives two pairs with disjoint key masks, each
// merged as its own partial: the same attention.
__global__ __launch_bounds__(256) void bm_pairs_kernel(CacheView cv, const int64_t* __restrict__ q_pos,
                                                       const int32_t* __restrict__ lr_idx,
                                                       const int32_t* __restrict__ lr_cnt, AttArgs aa, BmBuffers bm) {
    __shared__ unsigned long long tab[4][kBmTableBlocks][64];
    __shared__ int tbl[4][kBmTableBlocks];
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
#pragma unroll
    for (int x = 0; x < kBmTableBlocks; ++x) tab[wid][x][l] = 0ull;
    wave_lds_sync();
    int np = 0;
    bool bad = false;
    const int64_t bg = b * aa.H_kv + g;
    const int32_t nrec = (aa.bm_bcnt != nullptr && t >= 0 && cnt > 0) ? aa.bm_bcnt[u] : -1;
    if (nrec >= 0) {
        // the selection's bucket records: one pair per record, in the order the list gives them
        // (ascending leaf), checked against the query's long-range blocks and the row's count
        const Geom q = query_geom(t, aa.n_blocks, aa.n_sinks, aa.window);
        const u32x4* rr = aa.bm_brec + u * LSA_BUCKET_RECS;
        int keys = 0;
        bool fine = nrec <= kBmUnitCap;   // wave-uniform, as every quantity below
        for (int c0 = 0; fine && c0 < nrec; c0 += 64) {
            const int i = c0 + l;
            const bool live = i < nrec;
            const u32x4 r = live ? rr[i] : u32x4{0u, 0u, 0u, 0u};
            const int blk = (int)(r[0] / kLeavesPerBlock);
            const unsigned long long m = ((unsigned long long)r[2] << 32) | r[1];
            const bool good = blk < aa.n_blocks && (int64_t)blk * kBlockTokens < q.l0 &&
                              (int64_t)(blk + 1) * kBlockTokens > q.sink_end && m != 0ull;
            if (live && good) {
                pl[wid][i] = r[0];
                pm[wid][i] = m;
            }
            keys += live && good ? __popcll(m) : 0;
            if (__ballot(live && !good) != 0ull) fine = false;
        }
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) keys += __shfl_xor(keys, o);
        bad = !fine || keys != cnt;
        np = nrec;
    } else if (t >= 0 && cnt > 0) {
        const Geom q = query_geom(t, aa.n_blocks, aa.n_sinks, aa.window);
        const int32_t* lr = lr_idx + u * aa.k;
        const uint8_t* el = cv.eleaf + bg * cv.s_eleaf;
        const uint8_t* ep = cv.epos + bg * cv.s_epos;
        int32_t prev = -1;
        int used = 0, lastb = -1;   // table slots in use; block of the last one
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
                // pending lanes are a contiguous run; each takes slot used - 1 + (new blocks up to it)
                uint64_t pending = __ballot(valid);
                while (pending != 0ull) {
                    const bool pend = (pending >> l) & 1ull;
                    int pb = __shfl_up(blk, 1);
                    if (l == __builtin_ctzll(pending)) pb = lastb;
                    const uint64_t newm = __ballot(pend && blk != pb);
                    const int slot = used - 1 + __popcll(newm & ((2ull << l) - 1ull));
                    const uint64_t take = __ballot(pend && slot < kBmTableBlocks);
                    if (take == 0ull) {   // table full: turn it into pairs
                        np = bm_flush(tab[wid], tbl[wid], used, pl[wid], pm[wid], np);
                        used = 0;
                        lastb = -1;
                        continue;
                    }
                    // the key bits of a run of lanes with the same (slot, bucket) inside a lane quad (an
                    // entry's 4 tokens, usually) are ORed first: one LDS atomic per run
                    const bool tl = (take >> l) & 1ull;
                    const uint32_t key = tl ? ((uint32_t)slot << 8) | (uint32_t)rank : 0xFFFFFFFFu;
                    const uint64_t bits = tl ? 1ull << bit : 0ull;
                    const int qi = l & 3;
                    // (every DPP read runs with the whole wave active: a read from an inactive lane
                    // would return the reader's own value)
                    const uint32_t k1 = quad_dpp<0xF9>(key), k2 = quad_dpp<0xFE>(key), k3 = quad_dpp<0xFF>(key),
                                   k0 = quad_dpp<0x90>(key);   // lanes + 1, + 2, + 3, - 1
                    const uint64_t b1 = quad_dpp64<0xF9>(bits), b2 = quad_dpp64<0xFE>(bits), b3 = quad_dpp64<0xFF>(bits);
                    const bool s1 = qi <= 2 && k1 == key, s2 = s1 && qi <= 1 && k2 == key, s3 = s2 && qi == 0 && k3 == key;
                    const uint64_t comb = bits | (s1 ? b1 : 0ull) | (s2 ? b2 : 0ull) | (s3 ? b3 : 0ull);
                    const bool head = qi == 0 || k0 != key;   // lane - 1 is another run
                    if (tl) {
                        if ((newm >> l) & 1ull) tbl[wid][slot] = blk;
                        if (head) atomicOr(&tab[wid][slot][rank], comb);
                    }
                    const int last = 63 - __builtin_clzll(take);
                    used = __shfl(slot, last) + 1;
                    lastb = __shfl(blk, last);
                    pending &= ~take;
                }
            }
        }
        if (!bad && used > 0) np = bm_flush(tab[wid], tbl[wid], used, pl[wid], pm[wid], np);
    }
    if (bad || np > kBmUnitCap) np = -1;
    // the unit's pairs go to its own staging row; pool slots and bin ranks come later (bm_rank_kernel)
    if (np > 0) {
        wave_lds_sync();
        u32x4* st = bm.stage + ul * kBmUnitCap;
        for (int idx = l; idx < np; idx += 64) {
            const unsigned long long m = pm[wid][idx];
            st[idx] = u32x4{(uint32_t)(bg * bm.leaves_max + pl[wid][idx]), 0u, (uint32_t)m, (uint32_t)(m >> 32)};
        }
    }
    if (l == 0) bm.unit_np[ul] = np;
}

// Exclusive scan of the units' pair counts (negative counts as 0) inside each
// chunk of kBmScanChunk units, 16 per thread, and the chunk's total.
__global__ __launch_bounds__(256) void bm_uscan_kernel(int64_t n_units, BmBuffers bm) {
    __shared__ uint32_t ws[4];
    const int tid = threadIdx.x, l = lane_id(), wid = tid >> 6;
    const int64_t u0 = (int64_t)blockIdx.x * kBmScanChunk + tid * 16;
    uint32_t v[16], s = 0;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        const int np = u0 + j < n_units ? bm.unit_np[u0 + j] : 0;
        v[j] = np > 0 ? (uint32_t)np : 0u;
        s += v[j];
    }
    const uint32_t incl = (uint32_t)wave_incl_scan((int)s);
    if (l == 63) ws[wid] = incl;
    __syncthreads();
    uint32_t wpre = 0;
    for (int w = 0; w < wid; ++w) wpre += ws[w];
    uint32_t run = wpre + incl - s;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        if (u0 + j < n_units) bm.unit_off[u0 + j] = run;
        run += v[j];
    }
    if (tid == 255) bm.utot[blockIdx.x] = wpre + incl;
}

// Exclusive scan of n words by one 1024-thread workgroup, 1024 per step;
// returns the total to every thread.
__device__ uint32_t wg_exclusive_scan(const uint32_t* in, uint32_t* out, int64_t n, uint32_t* ws) {
    const int tid = threadIdx.x, l = lane_id(), wid = tid >> 6;
    uint32_t carry = 0;
    for (int64_t c0 = 0; c0 < n; c0 += 1024) {
        const int64_t c = c0 + tid;
        const uint32_t v = c < n ? in[c] : 0u;
        const uint32_t incl = (uint32_t)wave_incl_scan((int)v);
        if (l == 63) ws[wid] = incl;
        __syncthreads();
        uint32_t wpre = 0, tot = 0;
        for (int w = 0; w < 16; ++w) {
            wpre += w < wid ? ws[w] : 0u;
            tot += ws[w];
        }
        if (c < n) out[c] = carry + wpre + incl - v;
        carry += tot;
        __syncthreads();
    }
    return carry;
}

__global__ __launch_bounds__(1024) void bm_uscan_top_kernel(BmBuffers bm) {
    __shared__ uint32_t ws[16];
    wg_exclusive_scan(bm.utot, bm.ucsum, bm.nuch, ws);
}

// One wave per local unit: its first pool slot is the scan of the pair counts
// before it; a unit whose pairs would run past the pool is gathered whole
// instead (its token list, or, for a records row, the keys its records name),
// and counted.  Every other unit takes a rank in each of its pairs' bins.
__global__ __launch_bounds__(256) void bm_rank_kernel(AttArgs aa, BmBuffers bm) {
    const int l = lane_id(), wid = threadIdx.x >> 6;
    const int64_t ul = (int64_t)blockIdx.x * 4 + wid;
    if (ul >= aa.n_units) return;
    int np = bm.unit_np[ul];
    const uint32_t off = bm.ucsum[ul / kBmScanChunk] + bm.unit_off[ul];
    bool full = false;
    if (np > 0 && (uint64_t)off + (uint64_t)np > (uint64_t)bm.pool_cap) {
        full = true;
        const int64_t rr = ul / aa.H_kv, b = rr / aa.nqp, i = aa.q0 + rr % aa.nqp;
        const int64_t u = (b * aa.n_q + i) * aa.H_kv + ul % aa.H_kv;
        // np > 0 with records means they passed the checks (else np would be -1)
        np = (aa.bm_bcnt != nullptr && aa.bm_bcnt[u] >= 0) ? -2 : -1;
    }
    if (np > 0) {
        u32x4* st = bm.stage + ul * kBmUnitCap;
        for (int idx = l; idx < np; idx += 64) {
            uint32_t* w = reinterpret_cast<uint32_t*>(st + idx);
            w[1] = atomicAdd(bm.lcnt + w[0], 1u);
        }
    }
    if (l == 0) {
        bm.unit_off[ul] = off;
        bm.unit_np[ul] = np;
        if (bm.fallback != nullptr && np < 0) {
            atomicAdd(bm.fallback, 1u);
            if (full) atomicAdd(bm.fallback + 1, 1u);
        }
    }
}

// Exclusive scan of the pair counts inside each chunk of kBmScanChunk bins
// (16 per thread), and the chunk's total; likewise for the number of bins
// that have pairs (per 64-bin group, for the work records in bin order).
__global__ __launch_bounds__(256) void bm_scan_kernel(BmBuffers bm) {
    __shared__ uint32_t ws[4], wz[4];
    const int tid = threadIdx.x, l = lane_id(), wid = tid >> 6;
    const int64_t b0 = (int64_t)blockIdx.x * kBmScanChunk + tid * 16;
    const u32x4* src = reinterpret_cast<const u32x4*>(bm.lcnt + b0);
    u32x4 v[4];
    uint32_t s = 0, z = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        v[j] = src[j];
        s += v[j][0] + v[j][1] + v[j][2] + v[j][3];
#pragma unroll
        for (int x = 0; x < 4; ++x) z += v[j][x] != 0u ? 1u : 0u;
    }
    const uint32_t zincl = (uint32_t)wave_incl_scan((int)z);
    if (l == 63) wz[wid] = zincl;
    const uint32_t incl = (uint32_t)wave_incl_scan((int)s);
    if (l == 63) ws[wid] = incl;
    __syncthreads();
    uint32_t wpre = 0, zpre = 0;
    for (int w = 0; w < wid; ++w) {
        wpre += ws[w];
        zpre += wz[w];
    }
    if ((tid & 3) == 0) bm.gpre[b0 / 64] = zpre + zincl - z;
    if (tid == 255) bm.ctot[gridDim.x + blockIdx.x] = zpre + zincl;
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

// Exclusive scans of the chunk totals (pairs, then bins with pairs): one
// workgroup; the number of bins with pairs (work records) goes to
// lcnt[nbins_pad + 1].
__global__ __launch_bounds__(1024) void bm_scan_top_kernel(BmBuffers bm, int64_t nch) {
    __shared__ uint32_t ws[16];
    wg_exclusive_scan(bm.ctot, bm.csum, nch, ws);
    const uint32_t nwork = wg_exclusive_scan(bm.ctot + nch, bm.csum + nch, nch, ws);
    if (threadIdx.x == 0) bm.lcnt[bm.nbins_pad + 1] = nwork;
}

__device__ __forceinline__ uint32_t bm_bin_start(const BmBuffers& bm, uint32_t bin) {
    return bm.csum[bin / kBmScanChunk] + bm.loff[bin];
}

// One wave per local unit: its staged pairs go to their bin's place as
// (query row of the unit's first head, pair slot, key mask).
__global__ __launch_bounds__(256) void bm_scatter_kernel(AttArgs aa, BmBuffers bm) {
    const int l = lane_id(), wid = threadIdx.x >> 6;
    const int64_t ul = (int64_t)blockIdx.x * 4 + wid;
    if (ul >= aa.n_units) return;
    const int np = bm.unit_np[ul];
    if (np <= 0) return;
    const uint32_t base = bm.unit_off[ul];
    // the row of the group's first query head in Q [B, n_q, H_q, d] (fits 32 bits: checked on the host)
    const int64_t rr = ul / aa.H_kv, b = rr / aa.nqp, i = aa.q0 + rr % aa.nqp;
    const uint32_t qrow = (uint32_t)((b * aa.n_q + i) * aa.H_q + (ul % aa.H_kv) * aa.G);
    const u32x4* st = bm.stage + ul * kBmUnitCap;
    for (int idx = l; idx < np; idx += 64) {
        const u32x4 r = st[idx];
        bm.srec[bm_bin_start(bm, r[0]) + r[1]] = u32x4{qrow, base + (uint32_t)idx, r[2], r[3]};
    }
}

// Work records of the bins that received pairs: one wave per 64 bins; for
// each such bin the wave writes (pair start, pairs, keys, b * H_kv + g) and
// the bucket's key tokens in member order (key j = token 4 members[j / 4] +
// j % 4 of its block; keys past the bucket repeat its first).  Records are
// in bin order, so workgroups running together take neighbouring buckets,
// which share many of their queries (rows then found in the caches).
__global__ __launch_bounds__(256) void bm_prep_kernel(CacheView cv, BmBuffers bm) {
    __shared__ uint16_t memb[4][64][16];
    const int l = lane_id(), wid = threadIdx.x >> 6;
    const int64_t b0 = ((int64_t)blockIdx.x * 4 + wid) * 64;
    if (b0 >= bm.nbins) return;
    const int64_t bin = b0 + l;
    const uint32_t np = bin < bm.nbins ? bm.lcnt[bin] : 0u;
    uint64_t nz = __ballot(np > 0u);
    if (nz == 0ull) return;
    // every lane with pairs fetches its bucket's meta and members at once
    const int64_t bg = bin / bm.leaves_max, leaf = bin % bm.leaves_max;
    const int blk = (int)(leaf / kLeavesPerBlock);
    uint32_t meta = 0;
    if (np > 0u) {
        meta = cv.meta[bg * cv.s_meta + leaf];
        uint16_t e[16];
        load_members(cv.members + bg * cv.s_members + (int64_t)blk * kBlockEntries, (int)((meta >> 8) & 0x3FF), e);
#pragma unroll
        for (int j = 0; j < 16; ++j) memb[wid][l][j] = e[j];
    }
    // records in bin order: bins with pairs before this 64-bin group, then inside it
    const uint32_t base = bm.csum[bm.nbins_pad / kBmScanChunk + b0 / kBmScanChunk] + bm.gpre[b0 / 64];
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    for (uint32_t idx = 0; nz != 0ull; ++idx) {
        const int src = __builtin_ctzll(nz);
        nz &= nz - 1ull;
        const uint32_t npairs = __shfl(np, src);
        const uint32_t m = __shfl(meta, src);
        const int64_t bgs = (b0 + src) / bm.leaves_max;
        const int blks = (int)(((b0 + src) % bm.leaves_max) / kLeavesPerBlock);
        const int ntok = kPool * (int)(m & 0xFF);
        const int j = l < ntok ? l : 0;
        const int32_t tk = blks * kBlockTokens + kPool * (int)memb[wid][src][j / kPool] + j % kPool;
        u32x4* rec = bm.work + (int64_t)(base + idx) * 17;
        if (l == 0) rec[0] = u32x4{bm_bin_start(bm, (uint32_t)(b0 + src)), npairs, (uint32_t)ntok, (uint32_t)bgs};
        reinterpret_cast<int32_t*>(rec + 1)[l] = tk;
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

// One workgroup per work record (grid-stride): a bucket's keys/values in LDS, then
// groups of GP = 16 / G pairs (G query heads each) per wave.  Lane (n, h):
// column n = pair n / G, head n % G; S^T tiles are 16 keys x 16 columns
// (rows 4h + v), O^T tiles 16 dims x 16 columns.
template <int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4, 4))) void bm_leaf_kernel(CacheView cv, const uint16_t* __restrict__ Q,
                                                      const uint16_t* __restrict__ K,
                                                      const uint16_t* __restrict__ V, AttArgs aa, BmBuffers bm) {
    using LL = LeafLds<D>;
    constexpr int KS = D / 32, NDT = D / 16, CPR = D / 8;
    __shared__ __align__(16) uint8_t lds[LL::BYTES];
    const int tid = threadIdx.x, l = lane_id(), wid = tid >> 6, n = l & 15, h = l >> 4;
    const int G = aa.G, GP = 16 / G;
    const float sl2 = aa.scale * kLog2e;   // scores in log2 units
    const uint32_t n_work = bm.lcnt[bm.nbins_pad + 1];
    for (uint32_t wk = blockIdx.x; wk < n_work; wk += gridDim.x) {
        const u32x4* rec = bm.work + (int64_t)wk * 17;
        const u32x4 hdr = rec[0];
        const uint32_t start = hdr[0], npairs = hdr[1];
        const int ntok = (int)hdr[2];
        const int64_t bg = hdr[3];
        const int32_t* tokr = reinterpret_cast<const int32_t*>(rec + 1);
        const int nrow = (ntok + 31) & ~31;   // keys staged: whole 32-key k-steps
        __syncthreads();   // the previous bucket's LDS is no longer read
        const uint16_t* Kbg = K + bg * aa.t_cap * D;
        const uint16_t* Vbg = V + bg * aa.t_cap * D;
        // staging: item = (key pair jp, chunk c); keys past the bucket repeat its first (finite, weight 0)
        for (int it = tid; it < (nrow / 2) * CPR; it += 256) {
            const int jp = it / CPR, c = it % CPR;
            const int j0 = 2 * jp;
            const u32x2 tp = *reinterpret_cast<const u32x2*>(tokr + j0);
            const int32_t t0 = (int32_t)tp[0], t1 = (int32_t)tp[1];
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
        // is computed (a record with query row ~0: no pair in this column)
#define LSA_BM_REC(GRP, R)                                                                  \
    {                                                                                        \
        const uint32_t pidx_ = (GRP) * GP + pi;                                              \
        R = u32x4{~0u, 0u, 0u, 0u};                                                          \
        if ((GRP) < ngroups && pi < GP && pidx_ < npairs) R = bm.srec[start + pidx_];        \
    }
#define LSA_BM_Q(R, QV)                                                                     \
    {                                                                                        \
        /* a column without a pair reads Q row 0 (always present; its results are dropped) */ \
        const uint16_t* qrow_ = Q + ((int64_t)(R[0] != ~0u ? R[0] : 0u) + hh) * D;          \
        _Pragma("unroll") for (int ks = 0; ks < KS; ++ks) QV[ks] =                           \
            *reinterpret_cast<const u32x4*>(qrow_ + 32 * ks + 8 * h);                        \
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
            // this lane's 16 mask bits: key 16 tt + 4 h + v of the bucket is bit 4 tt + v of mk
            const uint32_t mlo = col ? rc[2] : 0u, mhi = col ? rc[3] : 0u;
            const uint32_t mk = ((mlo >> (4 * h)) & 0xFu) | (((mlo >> (16 + 4 * h)) & 0xFu) << 4) |
                                (((mhi >> (4 * h)) & 0xFu) << 8) | (((mhi >> (16 + 4 * h)) & 0xFu) << 12);
            // S^T = K Q^T over the bucket's keys, in log2 units (scale * log2 e): p = 2^(s - max)
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
                    // a key the pair does not list: min with -inf (with +inf it stays)
                    const float bias = __uint_as_float((((~mk >> (4 * tt + v)) & 1u) << 31) | 0x7F800000u);
                    s[tt][v] = __builtin_elementwise_minimum(s[tt][v] * sl2, bias);
                }
                mx = fmax_nc(mx, fmax_nc(fmax_nc(s[tt][0], s[tt][1]), fmax_nc(s[tt][2], s[tt][3])));
            }
            mx = fmax_nc(mx, __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(mx), kSwap16)));
            mx = fmax_nc(mx, __shfl_xor(mx, 32));
            // P (bf16, as the PV MFMA uses it) and its sum over the same rounded values
            uint32_t pk[4][2];
            float psum = 0.f;
#pragma unroll
            for (int tt = 0; tt < 4; ++tt) {
                pk[tt][0] = cvt_pk_bf16(exp2_hw(s[tt][0] - mx), exp2_hw(s[tt][1] - mx));
                pk[tt][1] = cvt_pk_bf16(exp2_hw(s[tt][2] - mx), exp2_hw(s[tt][3] - mx));
                psum = sum2_bf16(pk[tt][0], psum);
                psum = sum2_bf16(pk[tt][1], psum);
            }
            psum += __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(psum), kSwap16));
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
            // the fp16 row is stored unscaled when every value of the wave's pairs fits (a lane's largest
            // magnitude below 2^15 and, unless zero, at least 2^-8); otherwise each row gets a power-of-two
            // scale 2^e with its largest magnitude times 2^-e in [2^14, 2^15): no value overflows, and every
            // value down to 2^-10 of the largest keeps fp16's relative precision
            float lmax = 0.f;
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt)
                lmax = fmax_nc(lmax, fmax_nc(fmax_nc(fabsf(acc[dt][0]), fabsf(acc[dt][1])),
                                             fmax_nc(fabsf(acc[dt][2]), fabsf(acc[dt][3]))));
            const bool plain = lmax < 32768.f && (lmax >= 0.00390625f || lmax == 0.f);
            float osc = 1.f;
            if (__ballot(col && !plain) != 0ull) {
                float amax = fmax_nc(lmax, __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(lmax), kSwap16)));
                amax = fmax_nc(amax, __shfl_xor(amax, 32));
                int e = amax > 0.f ? __builtin_amdgcn_frexp_expf(amax) - 15 : 0;
                e = e > -100 ? e : -100;
                const float q = ldexpf(1.0f, -e);
                osc = ldexpf(1.0f, e);
#pragma unroll
                for (int dt = 0; dt < NDT; ++dt) acc[dt] *= q;
            }
            if (col) {
                const int64_t slot = (int64_t)p * G + hh;
                constexpr int MW = D / 32;
                // partial layout [pair][m][head][reading lane], 16 bytes each: one store instruction writes
                // every head of a pair's group m as one contiguous run (G x 64 bytes)
                uint32_t* pw = bm.po + ((int64_t)p * MW * G + hh) * 16;
#pragma unroll
                for (int m = 0; m < NDT / 2; ++m) {
                    // lane h holds dims 32m + 4h + [0,4) (A) and 32m + 16 + 4h + [0,4) (B); lanes h, h^1
                    // swap one of them so that each holds the 8 dims 32m + 8r + [0,8) of one reading lane r
                    const u32x2 A = u32x2{cvt_pk_f16(acc[2 * m][0], acc[2 * m][1]), cvt_pk_f16(acc[2 * m][2], acc[2 * m][3])};
                    const u32x2 Bv = u32x2{cvt_pk_f16(acc[2 * m + 1][0], acc[2 * m + 1][1]),
                                           cvt_pk_f16(acc[2 * m + 1][2], acc[2 * m + 1][3])};
                    const bool even = (h & 1) == 0;
                    const u32x2 send = even ? Bv : A;
                    const u32x2 got = u32x2{(uint32_t)__builtin_amdgcn_ds_swizzle((int)send[0], kSwap16),
                                            (uint32_t)__builtin_amdgcn_ds_swizzle((int)send[1], kSwap16)};
                    const u32x4 v8 = even ? u32x4{A[0], A[1], got[0], got[1]} : u32x4{got[0], got[1], Bv[0], Bv[1]};
                    const int r = (h >> 1) + 2 * (h & 1);   // the reading lane whose dims this lane holds
                    // streaming stores: the pass's partials (tens of GB) never stay in the caches, and
                    // bypassing them keeps the Q rows and K/V there
                    __builtin_nontemporal_store(v8, reinterpret_cast<u32x4*>(pw + (int64_t)m * G * 16 + r * 4));
                }
                // the max back in natural units (the merge and the window part use e^x)
                if (h == 0)
                    __builtin_nontemporal_store(f32x4{mx * kLn2, psum, osc, 0.f},
                                                reinterpret_cast<f32x4*>(bm.pml + slot * 4));
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
    const int64_t nclear = bm.nbins_pad + 4;
    const unsigned cg = (unsigned)((nclear + 2047) / 2048 < 1024 ? (nclear + 2047) / 2048 : 1024);
    hipLaunchKernelGGL(bm_clear_kernel, dim3(cg), dim3(256), 0, st, bm.lcnt, nclear);
    if (aa.n_units == 0) return hipGetLastError();
    const unsigned ug = (unsigned)((aa.n_units + 3) / 4);
    hipLaunchKernelGGL(bm_pairs_kernel, dim3(ug), dim3(256), 0, st, cv, q_pos, lr_idx, lr_cnt, aa, bm);
    hipLaunchKernelGGL(bm_uscan_kernel, dim3((unsigned)bm.nuch), dim3(256), 0, st, aa.n_units, bm);
    hipLaunchKernelGGL(bm_uscan_top_kernel, dim3(1), dim3(1024), 0, st, bm);
    hipLaunchKernelGGL(bm_rank_kernel, dim3(ug), dim3(256), 0, st, aa, bm);
    const int64_t nch = bm.nbins_pad / kBmScanChunk;
    hipLaunchKernelGGL(bm_scan_kernel, dim3((unsigned)nch), dim3(256), 0, st, bm);
    hipLaunchKernelGGL(bm_scan_top_kernel, dim3(1), dim3(1024), 0, st, bm, nch);
    hipLaunchKernelGGL(bm_scatter_kernel, dim3(ug), dim3(256), 0, st, aa, bm);
    hipLaunchKernelGGL(bm_prep_kernel, dim3((unsigned)((bm.nbins + 255) / 256)), dim3(256), 0, st, cv, bm);
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
