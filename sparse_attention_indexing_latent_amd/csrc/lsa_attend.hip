// Exact softmax attention over the selected keys on gfx950.
//
// Method: diosapp.com.cn LSA tutorial, section 二 (pseudocode: output =
// softmax(q K[keys]^T / sqrt(d)) V[keys]); zhichai.net explainer "卡片柜",
// ch.3 (keys = sinks + recent window + the selected long-range tokens; the
// attention itself is unchanged, only the keys it reads).
//
// One wave per (query, KV head) — or per slice of its key list when few
// queries must fill the chip (decode), followed by a log-sum-exp combine.
// The G query heads of the group share the key list, so they form the N = 16
// columns of the MFMAs.  Per 32 gathered keys:
//   S^T = K Q^T        two 16x16x32 bf16 MFMA tiles per 8-dim k-step,
//   online softmax     fp32, max subtracted, per head,
//   V^T                V rows pass through a 16x16x16 MFMA with the
//                      identity as B, which hands each lane 4 consecutive
//                      keys of one head dimension (the k-layout PV needs),
//   O^T += V^T P^T     16x16x32 bf16 MFMAs, P rounded to bf16.
// Every lane loads contiguous 64-byte pieces of K/V rows (4 lanes per
// 256-byte row), so each gathered row is one fully used 256-byte segment.

#include "lsa_launch.hpp"

namespace lsa {

namespace {

constexpr float kNegInf = -__builtin_huge_valf();

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

// Unit order inside the kernel: KV head slowest, then sequence, then query,
// so neighbouring waves (and, after the XCD remap, one XCD) handle
// neighbouring queries of one head and share their local windows in L2.
// u indexes the call's [B, n_q, H_kv] arrays, l the launch's own [B, nqp,
// H_kv] ones (the same when a launch covers every query).
struct AUnit {
    int64_t b, i, g, u, l;
};
__device__ __forceinline__ AUnit aunit_of(int64_t uu, const AttArgs& aa) {
    AUnit r;
    const int64_t per_g = (int64_t)aa.B * aa.nqp;
    r.g = uu / per_g;
    const int64_t rem = uu % per_g;
    r.b = rem / aa.nqp;
    const int64_t il = rem % aa.nqp;
    r.i = aa.q0 + il;
    r.u = (r.b * aa.n_q + r.i) * aa.H_kv + r.g;
    r.l = (r.b * aa.nqp + il) * aa.H_kv + r.g;
    return r;
}

// Log-sum-exp merge of a unit's bucket partials of head hh (of its group)
// into this lane's running state (lane (n, h) holds dims 32 (c/2) + 8h +
// 4 (c%2) + [0, 4) of acc[c]), in two passes: the largest partial maximum M
// first (the running state is rescaled to it once), then every partial's
// values weighted by exp(m_j - M) times its scale, one fp16-source FMA per
// value (v_fma_mix) with no rescaling of the accumulator per partial.
// Partials are read four at a time, a missing one (past the unit's count)
// reads the first slot again with weight 0.
template <int D>
__device__ __forceinline__ void merge_bucket_partials(const AttArgs& aa, int64_t ul, int npl, int hh, int h,
                                                      float& m_run, float& l_run, f32x4* acc) {
    constexpr int NC = D / 16;
    constexpr int MW = D / 32;
    constexpr int MN = 4;   // partials in flight
    constexpr int MX = 8;   // maxima in flight
    const int64_t s0 = aa.bm_off[ul];
    float M = m_run;
    for (int s = 0; s < npl; s += MX) {
        float mx[MX];
#pragma unroll
        for (int j = 0; j < MX; ++j) {
            const int64_t pp = s0 + (s + j < npl ? s + j : 0);
            mx[j] = aa.bm_ml[(pp * aa.G + hh) * 4];
        }
#pragma unroll
        for (int j = 0; j < MX; ++j) M = fmaxf(M, mx[j]);   // the repeated first slot changes nothing
    }
    const float a = m_run > kNegInf ? __expf(m_run - M) : 0.f;
#pragma unroll
    for (int c = 0; c < NC; ++c) acc[c] *= a;
    l_run *= a;
    m_run = M;
    for (int s = 0; s < npl; s += MN) {
        f32x4 ml[MN];
        u32x4 w[MN][MW];
#pragma unroll
        for (int j = 0; j < MN; ++j) {
            const int64_t pp = s0 + (s + j < npl ? s + j : 0);
            ml[j] = *reinterpret_cast<const f32x4*>(aa.bm_ml + (pp * aa.G + hh) * 4);
            // this lane's dims 32m + 8h + [0,8) for every m, fp16 (layout [pair][m][head][lane])
            const u32x4* pw = reinterpret_cast<const u32x4*>(aa.bm_po + (pp * MW * aa.G + hh) * 16 + h * 4);
#pragma unroll
            for (int m = 0; m < MW; ++m) w[j][m] = pw[(int64_t)m * aa.G * 4];
        }
#pragma unroll
        for (int j = 0; j < MN; ++j) {
            const float b = s + j < npl ? __expf(ml[j][0] - M) : 0.f;
            const float bs = b * ml[j][2];
#pragma unroll
            for (int c = 0; c < NC; ++c) {
                // acc[c] holds dims 32 (c/2) + 8h + 4 (c%2) + [0,4): words 2 (c%2), +1 of chunk c/2
                const uint32_t w0 = w[j][c / 2][2 * (c % 2)], w1 = w[j][c / 2][2 * (c % 2) + 1];
                acc[c][0] = fmaf((float)__builtin_bit_cast(_Float16, (uint16_t)(w0 & 0xFFFFu)), bs, acc[c][0]);
                acc[c][1] = fmaf((float)__builtin_bit_cast(_Float16, (uint16_t)(w0 >> 16)), bs, acc[c][1]);
                acc[c][2] = fmaf((float)__builtin_bit_cast(_Float16, (uint16_t)(w1 & 0xFFFFu)), bs, acc[c][2]);
                acc[c][3] = fmaf((float)__builtin_bit_cast(_Float16, (uint16_t)(w1 >> 16)), bs, acc[c][3]);
            }
            l_run = fmaf(ml[j][1], b, l_run);
        }
    }
}

// Map the hardware workgroup id (dispatched round-robin over the 8 XCDs) to a
// logical id so that consecutive logical ids run on the same XCD.
__device__ __forceinline__ int64_t xcd_logical(int64_t bid, int64_t nwg_padded) {
    const int64_t per = nwg_padded / 8;
    return (bid % 8) * per + bid / 8;
}

struct KeyList {
    int64_t ns, nl, l0, nS;
    const int32_t* lr;
    __device__ __forceinline__ int64_t at(int64_t j) const {
        if (j < ns) return j;
        if (j < ns + nl) return l0 + (j - ns);
        return (int64_t)lr[j - ns - nl];
    }
};

__device__ __forceinline__ KeyList key_list(int64_t t, const AttArgs& aa, const int32_t* lr_row, int32_t cnt) {
    const Geom q = query_geom(t, aa.n_blocks, aa.n_sinks, aa.window);
    KeyList kl;
    kl.ns = q.sink_end < q.l0 ? q.sink_end : q.l0;
    kl.l0 = q.l0;
    kl.nl = t - q.l0 + 1;
    kl.lr = lr_row;
    kl.nS = kl.ns + kl.nl + (cnt > 0 ? cnt : 0);
    return kl;
}

// Token of position jr of the key list, or -1 past the end or when the
// list holds an index outside [0, t] (never read, never scored).
__device__ __forceinline__ int32_t tok_of(const KeyList& kl, int64_t jr, int64_t j1, int64_t t) {
    if (jr >= j1) return -1;
    const int64_t tk = kl.at(jr);
    return (tk >= 0 && tk <= t) ? (int32_t)tk : -1;
}

// Log-sum-exp combine of the split partials of one unit (all G heads), by
// one wave.  Lane s (< splits <= 64) holds split s's max and denominator of
// every head; lane l then sums dims 2l, 2l + 1 over the splits in split
// order.  The partials come from other waves, so they are read with
// coherent loads; those of 8 splits of every head are in flight at once,
// the first 8 together with the maxima.
constexpr int kCombSplits = 8;
__device__ __forceinline__ void combine_unit(const float* __restrict__ part, const AttArgs& aa, int D, int out_bf16,
                                             void* O, int64_t u) {
    const int l = lane_id();
    const int G = aa.G, S = aa.splits;
    const int64_t rec = D + 2;   // floats per (split, head): max, denominator, D values
    const float* base = part + u * (int64_t)S * G * rec;
    const bool active = 2 * l < D;
    uint64_t ml[kMaxGroup];
#pragma unroll
    for (int hh = 0; hh < kMaxGroup; ++hh)
        ml[hh] = (hh < G && l < S) ? load_coherent_u64(base + ((int64_t)l * G + hh) * rec)
                                   : pack_f32x2(kNegInf, 0.f);
    uint64_t v[kMaxGroup][kCombSplits];
    auto load_chunk = [&](int s0) {
#pragma unroll
        for (int hh = 0; hh < kMaxGroup; ++hh)
#pragma unroll
            for (int j = 0; j < kCombSplits; ++j)
                v[hh][j] = (hh < G && s0 + j < S && active)
                               ? load_coherent_u64(base + ((int64_t)(s0 + j) * G + hh) * rec + 2 + 2 * l)
                               : 0ull;
    };
    load_chunk(0);
    float e[kMaxGroup], inv[kMaxGroup], o0[kMaxGroup], o1[kMaxGroup];
#pragma unroll
    for (int hh = 0; hh < kMaxGroup; ++hh) {
        const float ms = __uint_as_float((uint32_t)ml[hh]), ls = __uint_as_float((uint32_t)(ml[hh] >> 32));
        const float m = wave_max(ms);
        e[hh] = ms > kNegInf ? __expf(ms - m) : 0.f;
        const float lsum = wave_sum(ls * e[hh]);
        inv[hh] = lsum > 0.f ? 1.0f / lsum : 0.f;
        o0[hh] = 0.f;
        o1[hh] = 0.f;
    }
    for (int s0 = 0; s0 < S; s0 += kCombSplits) {
        if (s0 > 0) load_chunk(s0);
#pragma unroll
        for (int hh = 0; hh < kMaxGroup; ++hh) {
#pragma unroll
            for (int j = 0; j < kCombSplits; ++j) {
                const float es = __shfl(e[hh], (s0 + j) & 63);
                if (hh < G && s0 + j < S && es != 0.f) {   // a split that saw no key holds no partial output
                    o0[hh] += __uint_as_float((uint32_t)v[hh][j]) * es;
                    o1[hh] += __uint_as_float((uint32_t)(v[hh][j] >> 32)) * es;
                }
            }
        }
    }
    const int64_t g = u % aa.H_kv, bi = u / aa.H_kv;
#pragma unroll
    for (int hh = 0; hh < kMaxGroup; ++hh) {
        const int64_t orow = (bi * aa.H_q + g * G + hh) * D;
        if (hh < G && active) {
            if (out_bf16) {
                uint16_t* o = reinterpret_cast<uint16_t*>(O);
                *reinterpret_cast<uint32_t*>(o + orow + 2 * l) =
                    (uint32_t)f32_to_bf16(o0[hh] * inv[hh]) | ((uint32_t)f32_to_bf16(o1[hh] * inv[hh]) << 16);
            } else {
                float* o = reinterpret_cast<float*>(O);
                *reinterpret_cast<uint64_t*>(o + orow + 2 * l) = pack_f32x2(o0[hh] * inv[hh], o1[hh] * inv[hh]);
            }
        }
    }
}

// Arrival of one split of a unit: returns true for the split that arrives
// last.  The word holds (call tag << 32 | splits arrived so far).  A word
// that carries another call's tag (an earlier call, or junk in fresh memory)
// is claimed by this call's first arrival with one compare-and-swap to
// (tag, 1); every other arrival adds 1 with one fetch-add, so the last
// arrival waits for at most two device-scope atomics however many splits
// arrive together (a compare-and-swap loop for every arrival serialises the
// splits' round trips: 8 splits per unit cost 49.6 instead of 41.9 us per
// 16 x 1M decode step).  The only writers of the word during a call are that
// call's splits, so the claim loop ends as soon as one claim succeeds.
__device__ __forceinline__ bool split_arrive(unsigned long long* word, uint32_t tag, int splits) {
    unsigned long long cur = __hip_atomic_load(word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    while ((uint32_t)(cur >> 32) != tag) {
        if (__hip_atomic_compare_exchange_strong(word, &cur, ((unsigned long long)tag << 32) | 1ull,
                                                 __ATOMIC_RELAXED, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT))
            return splits == 1;
    }
    const unsigned long long old = __hip_atomic_fetch_add(word, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return (uint32_t)old + 1u == (uint32_t)splits;
}

// After a split wave has written its partials (coherent stores): the last
// split of the unit combines all of the unit's heads.
__device__ __forceinline__ void finish_split(const AttArgs& aa, const float* part, int D, int out_bf16, void* O,
                                             int64_t u) {
    wait_all_memory();   // this wave's partials are complete before it arrives
    int last = 0;
    if (lane_id() == 0) last = split_arrive(aa.arrive + u, aa.tag, aa.splits) ? 1 : 0;
    last = __shfl(last, 0);
    if (!last) return;
    combine_unit(part, aa, D, out_bf16, O, u);
}

// One 32-key tile of K and V rows staged in LDS (per wave).  Rows are
// loaded with whole-row coalescing: load instruction i brings rows RPI i ..
// RPI i + RPI - 1 of the tile, lane l taking row RPI i + l / CPR, 16-byte
// column l % CPR (each instruction covers RPI complete rows, 1 KB); the rows
// are written to LDS in a swizzled layout and read back in the MFMA operand
// layout (lane (r, h): row r, column 4 ks + h, i.e. head dims 32 ks + 8 h +
// [0, 8)).  The swizzle (slot (j CPR/RPI + col) mod CPR inside the row, 16
// bytes of padding per instruction group) keeps both the writes and the
// 16-row reads free of bank conflicts for D = 128.
template <int D>
struct TileLds {
    static constexpr int RPI = 512 / D;   // rows per load instruction
    static constexpr int CPR = D / 8;     // 16-byte columns per row
    static constexpr int NI = 32 / RPI;   // load instructions per tile and array
    static constexpr int GB = 1024 + 16;  // bytes per instruction group, padded
    static constexpr int ARR = NI * GB;   // bytes per array (K or V)
    static constexpr int BYTES = 2 * ARR;
    __device__ static __forceinline__ int off(int row, int col) {
        const int i = row / RPI, j = row % RPI;
        return i * GB + 16 * (CPR * j + ((j * (CPR / RPI) + col) % CPR));
    }
};

// Global loads of one tile: lane l's row of instruction i is tile row
// RPI i + l / CPR, whose token lane (row & 31) holds in `tok` (-1: masked; a
// masked row reads row 0, always present, and gets probability exactly 0).
// (native vector type: arrays of it stay in registers)
template <int D>
__device__ __forceinline__ void load_tile(const uint16_t* Kbg, const uint16_t* Vbg, int32_t tok, u32x4 (&kr)[TileLds<D>::NI],
                                          u32x4 (&vr)[TileLds<D>::NI]) {
    using TL = TileLds<D>;
    const int l = lane_id();
#pragma unroll
    for (int i = 0; i < TL::NI; ++i) {
        const int32_t tk = __shfl(tok, TL::RPI * i + l / TL::CPR);
        const size_t row = tk >= 0 ? (size_t)tk : 0;
        kr[i] = *reinterpret_cast<const u32x4*>(Kbg + row * D + 8 * (l % TL::CPR));
        vr[i] = *reinterpret_cast<const u32x4*>(Vbg + row * D + 8 * (l % TL::CPR));
    }
}

template <int D>
__device__ __forceinline__ void store_tile(const u32x4 (&kr)[TileLds<D>::NI], const u32x4 (&vr)[TileLds<D>::NI],
                                           uint8_t* buf) {
    using TL = TileLds<D>;
    const int l = lane_id();
#pragma unroll
    for (int i = 0; i < TL::NI; ++i) {
        const int o = TL::off(TL::RPI * i + l / TL::CPR, l % TL::CPR);
        *reinterpret_cast<u32x4*>(buf + o) = kr[i];
        *reinterpret_cast<u32x4*>(buf + TL::ARR + o) = vr[i];
    }
}

// One tile of 32 keys: S^T = K Q^T, online softmax, V^T via the identity
// MFMA, O^T += V^T P^T.  Bit v of ok_a (ok_b): key row 4h + v (16 + 4h + v)
// of the tile counts for this lane's column; a column that has seen no key
// yet keeps m = -inf and l = 0.
template <int D>
__device__ __forceinline__ void attend_tile(uint32_t ok_a, uint32_t ok_b, const uint8_t* buf, int r, const uint4* qf,
                                            const s16x4& ident, int h, float scale, float& m_run, float& l_run,
                                            f32x4* acc) {
    using TL = TileLds<D>;
    constexpr int KS = D / 32, NC = D / 16;
    f32x4 sa = {0.f, 0.f, 0.f, 0.f}, sb = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {   // K fragments: rows r and 16 + r, column 4 ks + h
        const bf16x8 ka = *reinterpret_cast<const bf16x8*>(buf + TL::off(r, 4 * ks + h));
        const bf16x8 kb = *reinterpret_cast<const bf16x8*>(buf + TL::off(16 + r, 4 * ks + h));
        sa = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, as_bf16x8(qf[ks]), sa, 0, 0, 0);
        sb = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kb, as_bf16x8(qf[ks]), sb, 0, 0, 0);
    }
    // rows of sa: keys 4h + v of the tile; rows of sb: keys 16 + 4h + v
    float pa[4], pb[4];
    float mx = kNegInf;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        pa[v] = ((ok_a >> v) & 1u) ? sa[v] * scale : kNegInf;
        pb[v] = ((ok_b >> v) & 1u) ? sb[v] * scale : kNegInf;
        mx = fmaxf(mx, fmaxf(pa[v], pb[v]));
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    const float alpha = m_run > kNegInf ? __expf(m_run - m_new) : 0.f;
    m_run = m_new;
    uint32_t pk[4];
    float psum = 0.f;
    auto pexp = [m_new](float x) { return x > kNegInf ? __expf(x - m_new) : 0.f; };
#pragma unroll
    for (int v = 0; v < 4; v += 2) {
        const uint16_t a0 = f32_to_bf16(pexp(pa[v])), a1 = f32_to_bf16(pexp(pa[v + 1]));
        const uint16_t b0 = f32_to_bf16(pexp(pb[v])), b1 = f32_to_bf16(pexp(pb[v + 1]));
        psum += bf16_to_f32(a0) + bf16_to_f32(a1) + bf16_to_f32(b0) + bf16_to_f32(b1);
        pk[v / 2] = (uint32_t)a0 | ((uint32_t)a1 << 16);
        pk[2 + v / 2] = (uint32_t)b0 | ((uint32_t)b1 << 16);
    }
    l_run = l_run * alpha + psum;
    const bf16x8 pfrag = as_bf16x8(uint4{pk[0], pk[1], pk[2], pk[3]});
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        // chunk c: lane (r, h) contributes V[key r][32 (c/2) + 8h + 4 (c%2) + 0..3]: 8 bytes of the
        // V fragments of rows r and 16 + r, column 4 (c/2) + h
        const int vo = TL::ARR + 8 * (c & 1);
        const s16x4 va4 = *reinterpret_cast<const s16x4*>(buf + vo + TL::off(r, 4 * (c / 2) + h));
        const s16x4 vb4 = *reinterpret_cast<const s16x4*>(buf + vo + TL::off(16 + r, 4 * (c / 2) + h));
        f32x4 z = {0.f, 0.f, 0.f, 0.f};
        const f32x4 ta4 = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va4, ident, z, 0, 0, 0);
        const f32x4 tb4 = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vb4, ident, z, 0, 0, 0);
        // lane (n, h): V[key 4h+v][dim(c, n)] and V[key 16+4h+v][dim(c, n)], exact in fp32
        uint32_t vt[4];
        vt[0] = (__float_as_uint(ta4[0]) >> 16) | (__float_as_uint(ta4[1]) & 0xFFFF0000u);
        vt[1] = (__float_as_uint(ta4[2]) >> 16) | (__float_as_uint(ta4[3]) & 0xFFFF0000u);
        vt[2] = (__float_as_uint(tb4[0]) >> 16) | (__float_as_uint(tb4[1]) & 0xFFFF0000u);
        vt[3] = (__float_as_uint(tb4[2]) >> 16) | (__float_as_uint(tb4[3]) & 0xFFFF0000u);
        acc[c] *= alpha;
        acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(uint4{vt[0], vt[1], vt[2], vt[3]}), pfrag, acc[c],
                                                         0, 0, 0);
    }
}

template <int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void attend_bf16_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                                                          const uint16_t* __restrict__ V,
                                                          const int64_t* __restrict__ q_pos,
                                                          const int32_t* __restrict__ lr_idx,
                                                          const int32_t* __restrict__ lr_cnt, AttArgs aa,
                                                          uint16_t* __restrict__ O, float* __restrict__ part,
                                                          int64_t nwg_padded) {
    __shared__ __align__(16) uint8_t tile_lds[4 * TileLds<D>::BYTES];
    // lane (r, h) owns head dims 32 ks + 8 h + [0, 8), ks < KS (see TileLds)
    constexpr int KS = D / 32;   // 8-element k-steps per lane for QK
    constexpr int NC = 2 * KS;   // 4-dim chunks for the transpose and PV: chunk c = dims 32 (c/2) + 8h + 4 (c%2) + [0, 4)
    const int l = lane_id(), wid = threadIdx.x >> 6, r = l & 15, h = l >> 4;
    const int64_t logical = xcd_logical(blockIdx.x, nwg_padded);
    const int64_t w_id = logical * 4 + wid;
    if (w_id >= aa.n_units * aa.splits) return;
    const int64_t uu = w_id / aa.splits;
    const int s = (int)(w_id % aa.splits);
    const AUnit un = aunit_of(uu, aa);
    const int64_t t = q_pos[un.b * aa.n_q + un.i];
    // a count above k (never written by the selection) is clamped: the list row holds k entries
    const int32_t cnt = min(lr_cnt[un.u], aa.k);
    const int n = r;  // head column of the C layouts
    const int64_t orow = ((un.b * aa.n_q + un.i) * aa.H_q + un.g * aa.G + n) * D;

    f32x4 acc[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = kNegInf, l_run = 0.f;

    if (t >= 0 && cnt >= 0) {
        const KeyList kl = key_list(t, aa, lr_idx + un.u * aa.k, cnt);
        int64_t chunk = (kl.nS + aa.splits - 1) / aa.splits;
        chunk = (chunk + 31) & ~(int64_t)31;
        const int64_t j0 = (int64_t)s * chunk;
        const int64_t j1 = j0 + chunk < kl.nS ? j0 + chunk : kl.nS;

        // B operand of S^T = K Q^T: head n, dims 32 ks + 8 h + [0, 8)
        uint4 qf[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            qf[ks] = uint4{0, 0, 0, 0};
            if (n < aa.G) qf[ks] = *reinterpret_cast<const uint4*>(Q + orow + 32 * ks + 8 * h);
        }
        // identity B for the transposing MFMA: lane (col n, k-group h) holds I[4h + j][n]
        s16x4 ident;
#pragma unroll
        for (int j = 0; j < 4; ++j) ident[j] = (4 * h + j == n) ? (short)0x3F80 : (short)0;

        const int64_t bg = un.b * aa.H_kv + un.g;
        const uint16_t* Kbg = K + bg * aa.t_cap * D;
        const uint16_t* Vbg = V + bg * aa.t_cap * D;

        // Software pipeline over 32-key tiles: the rows of the next tile are in
        // flight (registers) while the current one, staged through LDS, is
        // computed, and the indices of the tile after it are fetched then, so
        // a row load never waits for its index load.  A key outside [0, t]
        // (malformed list) is never read nor scored.
        uint8_t* buf = tile_lds + wid * TileLds<D>::BYTES;
        constexpr int NI = TileLds<D>::NI;
        int32_t tok = tok_of(kl, j0 + (l & 31), j1, t);
        int32_t nxt = tok_of(kl, j0 + 32 + (l & 31), j1, t);
        u32x4 kR[NI], vR[NI];
        load_tile<D>(Kbg, Vbg, tok, kR, vR);
        for (int64_t j = j0; j < j1; j += 32) {
            const int32_t nn = tok_of(kl, j + 64 + (l & 31), j1, t);
            const uint64_t vm = __ballot(tok >= 0);   // bit r: tile row r valid (lanes 32..63 repeat 0..31)
            store_tile<D>(kR, vR, buf);
            load_tile<D>(Kbg, Vbg, nxt, kR, vR);   // past the end: masked rows (row 0), never used
            if ((vm & 0xFFFFFFFFull) != 0ull)
                attend_tile<D>((uint32_t)(vm >> (4 * h)) & 0xFu, (uint32_t)(vm >> (16 + 4 * h)) & 0xFu, buf, r, qf,
                               ident, h, aa.scale, m_run, l_run, acc);
            tok = nxt;
            nxt = nn;
        }
    }
    // acc[c][v] = unnormalised O[head n][32 (c/2) + 8h + 4 (c%2) + v]
    l_run += __shfl_xor(l_run, 16);
    l_run += __shfl_xor(l_run, 32);
    if (aa.splits == 1) {
        if (n < aa.G) {
            const float inv = l_run > 0.f ? 1.0f / l_run : 0.f;
            uint32_t w[2 * NC];
#pragma unroll
            for (int c = 0; c < NC; ++c) {
                w[2 * c] = (uint32_t)f32_to_bf16(acc[c][0] * inv) | ((uint32_t)f32_to_bf16(acc[c][1] * inv) << 16);
                w[2 * c + 1] = (uint32_t)f32_to_bf16(acc[c][2] * inv) | ((uint32_t)f32_to_bf16(acc[c][3] * inv) << 16);
            }
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)   // dims 32 ks + 8h + [0, 8)
                *reinterpret_cast<uint4*>(O + orow + 32 * ks + 8 * h) =
                    uint4{w[4 * ks], w[4 * ks + 1], w[4 * ks + 2], w[4 * ks + 3]};
        }
    } else {
        if (n < aa.G) {
            float* pp = part + ((un.u * aa.splits + s) * aa.G + n) * (D + 2);
            if (h == 0) store_coherent_u64(pp, pack_f32x2(m_run, l_run));
#pragma unroll
            for (int c = 0; c < NC; ++c) {
                const int d0 = 32 * (c / 2) + 8 * h + 4 * (c % 2);
                store_coherent_u64(pp + 2 + d0, pack_f32x2(acc[c][0], acc[c][1]));
                store_coherent_u64(pp + 4 + d0, pack_f32x2(acc[c][2], acc[c][3]));
            }
        }
        finish_split(aa, part, D, 1, O, un.u);
    }
}

// Rows [RPI i, RPI i + RPI) of a tile, for the NI / 4 load instructions i
// of wave `wid` (the four waves of a workgroup stage one tile together); the
// tile holds keys k0 .. k0 + 31, a key past `kend` reads row 0 (weight 0).
template <int D>
__device__ __forceinline__ void load_tile_part(const uint16_t* Kbg, const uint16_t* Vbg, int64_t k0, int64_t kend,
                                               int wid, u32x4 (&kr)[TileLds<D>::NI / 4],
                                               u32x4 (&vr)[TileLds<D>::NI / 4]) {
    using TL = TileLds<D>;
    const int l = lane_id();
#pragma unroll
    for (int i = 0; i < TL::NI / 4; ++i) {
        const int row = TL::RPI * (wid * (TL::NI / 4) + i) + l / TL::CPR;
        const int64_t key = k0 + row < kend ? k0 + row : 0;
        kr[i] = *reinterpret_cast<const u32x4*>(Kbg + key * D + 8 * (l % TL::CPR));
        vr[i] = *reinterpret_cast<const u32x4*>(Vbg + key * D + 8 * (l % TL::CPR));
    }
}
template <int D>
__device__ __forceinline__ void store_tile_part(const u32x4 (&kr)[TileLds<D>::NI / 4],
                                                const u32x4 (&vr)[TileLds<D>::NI / 4], int wid, uint8_t* buf) {
    using TL = TileLds<D>;
    const int l = lane_id();
#pragma unroll
    for (int i = 0; i < TL::NI / 4; ++i) {
        const int o = TL::off(TL::RPI * (wid * (TL::NI / 4) + i) + l / TL::CPR, l % TL::CPR);
        *reinterpret_cast<u32x4*>(buf + o) = kr[i];
        *reinterpret_cast<u32x4*>(buf + TL::ARR + o) = vr[i];
    }
}

// Sinks + local window of the bucket-major path, then the merge of the
// unit's bucket partials.  One workgroup per 4 QW consecutive queries of a
// KV head (QW = 16 / G per wave): column n of a wave's MFMAs is query n / G,
// head n % G, and the four waves share every 32-key tile, staged once in LDS
// (double-buffered), so the window keys the queries have in common are read
// once per workgroup.  The keys are walked in 32-key tiles aligned to
// multiples of 32 — those covering [0, S1), S1 the largest sink end, then
// those covering the rest of [kmin, kmax], the union of the windows — and a
// key counts for a column when it is one of that query's sinks or inside its
// window, so no key is counted twice; a column's keys fall in the same tiles
// whichever queries share the workgroup, and a tile holding none of them
// leaves its state exactly as it was.  A unit whose list the bucket pass
// could not take (np = -1) has that list gathered afterwards by its wave,
// for its own columns only.
template <int D>
// 3 waves per SIMD (168 VGPRs, some spilled; 33 KB of LDS): three workgroups per CU keep more partial
// reads in flight than two without spills (1M layer: the attention call 3-4% faster)
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3, 3))) void bm_local_kernel(
    CacheView cv, const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const int64_t* __restrict__ q_pos, const int32_t* __restrict__ lr_idx, const int32_t* __restrict__ lr_cnt,
    AttArgs aa, uint16_t* __restrict__ O, int64_t nwg_padded) {
    using TL = TileLds<D>;
    // window: two shared tiles; afterwards the private tiles of two waves at a time
    __shared__ __align__(16) uint8_t tile_lds[2 * TL::BYTES];
    __shared__ int64_t red[3][4];
    constexpr int KS = D / 32, NC = 2 * KS, NI = TL::NI, NIW = NI / 4;
    const int l = lane_id(), wid = threadIdx.x >> 6, r = l & 15, h = l >> 4, n = r;
    const int G = aa.G, QW = 16 / G, TQ = 4 * QW;
    const int64_t ntq = (aa.nqp + TQ - 1) / TQ;
    const int64_t per_g = (int64_t)aa.B * ntq;
    const int64_t wg = xcd_logical(blockIdx.x, nwg_padded);
    if (wg >= (int64_t)aa.H_kv * per_g) return;   // whole workgroup
    const int64_t g = wg / per_g, rem = wg % per_g, b = rem / ntq, tq = rem % ntq;
    const int qi = n / G, hh = n % G;
    const int64_t il = tq * TQ + wid * QW + qi;
    const bool colq = qi < QW && il < aa.nqp;
    const int64_t i = aa.q0 + (colq ? il : 0);
    const int64_t t = colq ? q_pos[b * aa.n_q + i] : -1;
    const int64_t u = (b * aa.n_q + i) * aa.H_kv + g, ul = (b * aa.nqp + (colq ? il : 0)) * aa.H_kv + g;
    const int32_t cnt = colq ? min(lr_cnt[u], aa.k) : -1;
    const bool live = colq && t >= 0 && cnt >= 0;
    const int32_t npl = live ? aa.bm_np[ul] : 0;
    int64_t se = 0, l0 = INT64_MAX, te = -1;   // this column's sinks [0, se) and window [l0, te]
    if (live) {
        const Geom q = query_geom(t, aa.n_blocks, aa.n_sinks, aa.window);
        se = q.sink_end < q.l0 ? q.sink_end : q.l0;
        l0 = q.l0;
        te = t;
    }
    const int64_t orow = ((b * aa.n_q + i) * aa.H_q + g * G + hh) * D;
    uint4 qf[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        qf[ks] = uint4{0, 0, 0, 0};
        if (live) qf[ks] = *reinterpret_cast<const uint4*>(Q + orow + 32 * ks + 8 * h);
    }
    s16x4 ident;
#pragma unroll
    for (int j = 0; j < 4; ++j) ident[j] = (4 * h + j == n) ? (short)0x3F80 : (short)0;
    f32x4 acc[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = kNegInf, l_run = 0.f;

    int64_t S1 = se, kmin = l0, kmax = te;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
        S1 = max(S1, (int64_t)__shfl_xor(S1, o));
        kmin = min(kmin, (int64_t)__shfl_xor(kmin, o));
        kmax = max(kmax, (int64_t)__shfl_xor(kmax, o));
    }
    if (l == 0) {
        red[0][wid] = S1;
        red[1][wid] = kmin;
        red[2][wid] = kmax;
    }
    __syncthreads();
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        S1 = max(S1, red[0][w]);
        kmin = min(kmin, red[1][w]);
        kmax = max(kmax, red[2][w]);
    }
    const int64_t bg = b * aa.H_kv + g;
    const uint16_t* Kbg = K + bg * aa.t_cap * D;
    const uint16_t* Vbg = V + bg * aa.t_cap * D;
    const int64_t nt1 = (S1 + 31) / 32;
    const int64_t kmin_al = kmin == INT64_MAX ? kmin : (kmin / 32) * 32;
    const int64_t a2 = 32 * nt1 > kmin_al ? 32 * nt1 : kmin_al;
    const int64_t nt2 = kmax >= a2 ? (kmax - a2 + 32) / 32 : 0;
    const int64_t ntiles = nt1 + nt2;
    const int64_t kend = kmax + 1;   // no row past the last window is read
    if (ntiles > 0) {
        u32x4 kr[NIW], vr[NIW];
        int64_t k0 = 0 < nt1 ? 0 : a2;
        load_tile_part<D>(Kbg, Vbg, k0, kend, wid, kr, vr);
        for (int64_t x = 0; x < ntiles; ++x) {
            uint8_t* buf = tile_lds + (x & 1) * TL::BYTES;
            store_tile_part<D>(kr, vr, wid, buf);
            __syncthreads();
            const int64_t kn = x + 1 < nt1 ? 32 * (x + 1) : a2 + 32 * (x + 1 - nt1);
            if (x + 1 < ntiles) load_tile_part<D>(Kbg, Vbg, kn, kend, wid, kr, vr);
            uint32_t va4 = 0, vb4 = 0;
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int64_t ka = k0 + 4 * h + v, kb = k0 + 16 + 4 * h + v;
                va4 |= (ka < se || (ka >= l0 && ka <= te)) ? (1u << v) : 0u;
                vb4 |= (kb < se || (kb >= l0 && kb <= te)) ? (1u << v) : 0u;
            }
            if (__ballot((va4 | vb4) != 0u) != 0ull)
                attend_tile<D>(va4, vb4, buf, r, qf, ident, h, aa.scale, m_run, l_run, acc);
            k0 = kn;
        }
    }
    __syncthreads();   // the shared tiles are read no more: they become private tiles, one per wave of a pair
    // long-range keys of the units the bucket pass left to the gather: their token lists (np = -1), or
    // the keys their bucket records name (np = -2: records rows whose pairs did not fit in the pool; such
    // rows may have no token list).  Waves 0 and 1 gather first, then waves 2 and 3 in the same two tiles
    // (the LDS holds two tiles, not four: three workgroups then share a CU)
    const uint64_t fb = __ballot(npl < 0);
    for (int rnd = 0; rnd < 2; ++rnd) {
        if ((wid >> 1) == rnd && fb != 0ull) {
            uint8_t* buf = tile_lds + (wid & 1) * TL::BYTES;
            u32x4 kR[NI], vR[NI];
            for (int q2 = 0; q2 < QW; ++q2) {
                if (((fb >> (q2 * G)) & 1ull) == 0ull) continue;   // column q2 * G stands for its query
                const int lane0 = q2 * G;
                const int64_t u2 = __shfl(u, lane0);
                const int64_t t2 = __shfl(t, lane0);
                const int32_t c2 = __shfl(cnt, lane0);
                const int32_t np2 = __shfl(npl, lane0);
                const bool mine = qi == q2;
                if (np2 == -2) {
                    // bucket by bucket: key j = 32 half + (l % 32) of the record's bucket, if its mask bit is set
                    const Geom q = query_geom(t2, aa.n_blocks, aa.n_sinks, aa.window);
                    const int32_t nr = aa.bm_bcnt[u2];
                    const u32x4* recs = aa.bm_brec + u2 * LSA_BUCKET_RECS;
                    for (int x = 0; x < nr; ++x) {
                        const u32x4 rec = recs[x];
                        const int64_t leaf = rec[0], blk = leaf / kLeavesPerBlock;
                        const unsigned long long mask = ((unsigned long long)rec[2] << 32) | rec[1];
                        const uint32_t meta = cv.meta[bg * cv.s_meta + leaf];
                        const int sz = (int)(meta & 0xFF), off = (int)((meta >> 8) & 0x3FF);
                        const uint16_t* mem = cv.members + bg * cv.s_members + blk * kBlockEntries + off;
                        for (int half = 0; half < 2; ++half) {
                            const int j = 32 * half + (l & 31);
                            int32_t tok = -1;
                            if (((mask >> j) & 1ull) && j < kPool * sz) {
                                const int64_t tk = blk * kBlockTokens + kPool * (int64_t)mem[j / kPool] + j % kPool;
                                if (tk >= q.sink_end && tk < q.l0 && tk <= t2) tok = (int32_t)tk;
                            }
                            const uint64_t vm = __ballot(tok >= 0);
                            if ((vm & 0xFFFFFFFFull) == 0ull) continue;
                            load_tile<D>(Kbg, Vbg, tok, kR, vR);
                            store_tile<D>(kR, vR, buf);
                            attend_tile<D>(mine ? (uint32_t)(vm >> (4 * h)) & 0xFu : 0u,
                                           mine ? (uint32_t)(vm >> (16 + 4 * h)) & 0xFu : 0u, buf, r, qf, ident, h,
                                           aa.scale, m_run, l_run, acc);
                        }
                    }
                    continue;
                }
                const int32_t* lr = lr_idx + u2 * aa.k;
                auto tok_at = [&](int64_t j) -> int32_t {
                    if (j >= c2) return -1;
                    const int32_t tk = lr[j];
                    return (tk >= 0 && tk <= t2) ? tk : -1;
                };
                int32_t tok = tok_at(l & 31);
                load_tile<D>(Kbg, Vbg, tok, kR, vR);
                for (int64_t j = 0; j < c2; j += 32) {
                    const int32_t nxt = tok_at(j + 32 + (l & 31));
                    const uint64_t vm = __ballot(tok >= 0);
                    store_tile<D>(kR, vR, buf);
                    load_tile<D>(Kbg, Vbg, nxt, kR, vR);
                    if ((vm & 0xFFFFFFFFull) != 0ull) {
                        attend_tile<D>(mine ? (uint32_t)(vm >> (4 * h)) & 0xFu : 0u,
                                       mine ? (uint32_t)(vm >> (16 + 4 * h)) & 0xFu : 0u, buf, r, qf, ident, h, aa.scale,
                                       m_run, l_run, acc);
                    }
                    tok = nxt;
                }
            }
        }
        if (rnd == 0) __syncthreads();   // the second pair reuses the first pair's tiles
    }
    l_run += __shfl_xor(l_run, 16);
    l_run += __shfl_xor(l_run, 32);
    if (npl > 0) merge_bucket_partials<D>(aa, ul, npl, hh, h, m_run, l_run, acc);
    if (colq) {
        const float inv = l_run > 0.f ? 1.0f / l_run : 0.f;
        uint32_t w[2 * NC];
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            w[2 * c] = (uint32_t)f32_to_bf16(acc[c][0] * inv) | ((uint32_t)f32_to_bf16(acc[c][1] * inv) << 16);
            w[2 * c + 1] = (uint32_t)f32_to_bf16(acc[c][2] * inv) | ((uint32_t)f32_to_bf16(acc[c][3] * inv) << 16);
        }
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            *reinterpret_cast<uint4*>(O + orow + 32 * ks + 8 * h) =
                uint4{w[4 * ks], w[4 * ks + 1], w[4 * ks + 2], w[4 * ks + 3]};
    }
}

// fp32 path: plain fp32 arithmetic (lanes over keys for the scores, lanes
// over head dims for PV).
__global__ __launch_bounds__(256) void attend_f32_kernel(const float* __restrict__ Q, const float* __restrict__ K,
                                                         const float* __restrict__ V,
                                                         const int64_t* __restrict__ q_pos,
                                                         const int32_t* __restrict__ lr_idx,
                                                         const int32_t* __restrict__ lr_cnt, AttArgs aa, int D,
                                                         float* __restrict__ O, float* __restrict__ part,
                                                         int64_t nwg_padded) {
    __shared__ float qs[4][kMaxGroup][128];
    __shared__ float ps[4][64][kMaxGroup];
    __shared__ int64_t ts[4][64];
    const int l = lane_id(), wid = threadIdx.x >> 6;
    const int64_t logical = xcd_logical(blockIdx.x, nwg_padded);
    const int64_t w_id = logical * 4 + wid;
    if (w_id >= aa.n_units * aa.splits) return;
    const int64_t uu = w_id / aa.splits;
    const int s = (int)(w_id % aa.splits);
    const AUnit un = aunit_of(uu, aa);
    const int64_t t = q_pos[un.b * aa.n_q + un.i];
    // a count above k (never written by the selection) is clamped: the list row holds k entries
    const int32_t cnt = min(lr_cnt[un.u], aa.k);
    const int G = aa.G;
    const int64_t qrow0 = ((un.b * aa.n_q + un.i) * aa.H_q + un.g * G) * D;
    float m_run[kMaxGroup], l_run[kMaxGroup], acc[kMaxGroup][2];
#pragma unroll
    for (int hh = 0; hh < kMaxGroup; ++hh) {
        m_run[hh] = kNegInf;
        l_run[hh] = 0.f;
        acc[hh][0] = acc[hh][1] = 0.f;
    }
    if (t >= 0 && cnt >= 0) {
        for (int hh = 0; hh < G; ++hh)
            for (int dd = l; dd < D; dd += 64) qs[wid][hh][dd] = Q[qrow0 + (int64_t)hh * D + dd];
        __builtin_amdgcn_wave_barrier();
        const KeyList kl = key_list(t, aa, lr_idx + un.u * aa.k, cnt);
        int64_t chunk = (kl.nS + aa.splits - 1) / aa.splits;
        chunk = (chunk + 31) & ~(int64_t)31;
        const int64_t j0 = (int64_t)s * chunk;
        const int64_t j1 = j0 + chunk < kl.nS ? j0 + chunk : kl.nS;
        const int64_t bg = un.b * aa.H_kv + un.g;
        const float* Kbg = K + bg * aa.t_cap * D;
        const float* Vbg = V + bg * aa.t_cap * D;
        for (int64_t j = j0; j < j1; j += 64) {
            int64_t tk = j + l < j1 ? kl.at(j + l) : -1;
            const bool ok = tk >= 0 && tk <= t;
            tk = ok ? tk : 0;
            ts[wid][l] = tk;
            float sc[kMaxGroup];
            for (int hh = 0; hh < G; ++hh) {
                float a = 0.f;
                for (int dd = 0; dd < D; ++dd) a = fmaf(qs[wid][hh][dd], Kbg[tk * D + dd], a);
                sc[hh] = ok ? a * aa.scale : kNegInf;
            }
            for (int hh = 0; hh < G; ++hh) {
                const float m_new = fmaxf(m_run[hh], wave_max(sc[hh]));
                const float alpha = m_new == kNegInf ? 1.f : expf(m_run[hh] - m_new);
                const float p = (ok && m_new > kNegInf) ? expf(sc[hh] - m_new) : 0.f;
                l_run[hh] = l_run[hh] * alpha + wave_sum(p);
                m_run[hh] = m_new;
                acc[hh][0] *= alpha;
                acc[hh][1] *= alpha;
                ps[wid][l][hh] = p;
            }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            const int nk = (int)((j1 - j) < 64 ? (j1 - j) : 64);
            for (int jj = 0; jj < nk; ++jj) {
                const int64_t tt = ts[wid][jj];
                const float v0 = l < D ? Vbg[tt * D + l] : 0.f;
                const float v1 = l + 64 < D ? Vbg[tt * D + l + 64] : 0.f;
                for (int hh = 0; hh < G; ++hh) {
                    const float p = ps[wid][jj][hh];
                    acc[hh][0] = fmaf(p, v0, acc[hh][0]);
                    acc[hh][1] = fmaf(p, v1, acc[hh][1]);
                }
            }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        }
    }
    for (int hh = 0; hh < G; ++hh) {
        if (aa.splits == 1) {
            const float inv = l_run[hh] > 0.f ? 1.0f / l_run[hh] : 0.f;
            if (l < D) O[qrow0 + (int64_t)hh * D + l] = acc[hh][0] * inv;
            if (l + 64 < D) O[qrow0 + (int64_t)hh * D + l + 64] = acc[hh][1] * inv;
        } else {
            float* pp = part + ((un.u * aa.splits + s) * G + hh) * (D + 2);
            if (l == 0) store_coherent_u64(pp, pack_f32x2(m_run[hh], l_run[hh]));
            if (l < D) store_coherent_u32(pp + 2 + l, __float_as_uint(acc[hh][0]));
            if (l + 64 < D) store_coherent_u32(pp + 2 + l + 64, __float_as_uint(acc[hh][1]));
        }
    }
    if (aa.splits > 1) finish_split(aa, part, D, 0, O, un.u);
}

}  // namespace

// Key-list splits per (query, KV head): few units are spread over about one
// wave per SIMD (1024 SIMDs), at least 128 keys each; more splits cost more
// in arrivals and combining than they gain in parallel gathers.
int attend_splits(int64_t n_units, int window, int k) {
    if (n_units >= 1024) return 1;
    const int64_t keys = (int64_t)window + kBlockTokens + k + 64;
    int64_t want = 1024 / n_units;
    const int64_t maxs = (keys + 127) / 128;
    if (want > maxs) want = maxs;
    if (want < 1) want = 1;
    if (want > 64) want = 64;
    return (int)want;
}

hipError_t launch_attend_local(const CacheView& cv, const void* Q, const void* K, const void* V,
                               const int64_t* q_pos, const int32_t* lr_idx, const int32_t* lr_cnt, const AttArgs& aa,
                               int D, void* O, hipStream_t st) {
    const int TQ = 4 * (16 / aa.G);
    int64_t nwg = (int64_t)aa.H_kv * aa.B * ((aa.nqp + TQ - 1) / TQ);
    nwg = (nwg + 7) & ~(int64_t)7;
    if (D == 128)
        hipLaunchKernelGGL(bm_local_kernel<128>, dim3((unsigned)nwg), dim3(256), 0, st, cv,
                           static_cast<const uint16_t*>(Q), static_cast<const uint16_t*>(K),
                           static_cast<const uint16_t*>(V), q_pos, lr_idx, lr_cnt, aa, static_cast<uint16_t*>(O), nwg);
    else
        hipLaunchKernelGGL(bm_local_kernel<64>, dim3((unsigned)nwg), dim3(256), 0, st, cv,
                           static_cast<const uint16_t*>(Q), static_cast<const uint16_t*>(K),
                           static_cast<const uint16_t*>(V), q_pos, lr_idx, lr_cnt, aa, static_cast<uint16_t*>(O), nwg);
    return hipGetLastError();
}

hipError_t launch_attend(const void* Q, const void* K, const void* V, const int64_t* q_pos, const int32_t* lr_idx,
                         const int32_t* lr_cnt, const AttArgs& aa, int D, bool bf16, void* O, float* part,
                         hipStream_t st) {
    const int64_t waves = aa.n_units * aa.splits;
    int64_t nwg = (waves + 3) / 4;
    nwg = (nwg + 7) & ~(int64_t)7;
    if (bf16) {
        if (D == 128)
            hipLaunchKernelGGL(attend_bf16_kernel<128>, dim3((unsigned)nwg), dim3(256), 0, st,
                               static_cast<const uint16_t*>(Q), static_cast<const uint16_t*>(K),
                               static_cast<const uint16_t*>(V), q_pos, lr_idx, lr_cnt, aa, static_cast<uint16_t*>(O),
                               part, nwg);
        else
            hipLaunchKernelGGL(attend_bf16_kernel<64>, dim3((unsigned)nwg), dim3(256), 0, st,
                               static_cast<const uint16_t*>(Q), static_cast<const uint16_t*>(K),
                               static_cast<const uint16_t*>(V), q_pos, lr_idx, lr_cnt, aa, static_cast<uint16_t*>(O),
                               part, nwg);
    } else {
        hipLaunchKernelGGL(attend_f32_kernel, dim3((unsigned)nwg), dim3(256), 0, st, static_cast<const float*>(Q),
                           static_cast<const float*>(K), static_cast<const float*>(V), q_pos, lr_idx, lr_cnt, aa, D,
                           static_cast<float*>(O), part, nwg);
    }
    return hipGetLastError();
}

}  // namespace lsa
