// Training-free projection on gfx950: the 64 leading principal directions of
// the keys (zhichai.net explainer "卡片柜", ch.5: the D-LSA variant that needs
// no training takes its projection straight from a principal component
// analysis of the keys).
//
//   moments   512 workgroups: S = sum (k - r)(k - r)^T and m = sum (k - r)
//             over every key of every (sequence, KV head), fp32 per
//             workgroup (each thread an 8 x 8 tile of S), r = the first key
//             (a shift leaves the covariance unchanged and keeps the sums
//             small)
//   reduce    the workgroups' partials summed in fp64
//   eig       one 1024-thread workgroup: C = S/N - m m^T / N^2, cyclic
//             Jacobi in LDS (fp32, round-robin pairing: d/2 disjoint
//             rotations per round, d - 1 rounds per sweep) until the
//             off-diagonal mass is negligible; eigenvalues ranked
//             descending (ties to the lower index); W = the leading 64
//             eigenvectors, each with its largest-magnitude component
//             positive.

#include "lsa_launch.hpp"

namespace lsa {

namespace {

constexpr int kPcaWgs = 512;
constexpr int kPcaMaxD = 128;

template <typename T, int D>
__global__ __launch_bounds__(256) void pca_moments_kernel(const T* __restrict__ K, int64_t t_cap, int64_t Tn,
                                                          int64_t N, float* __restrict__ part) {
    constexpr int TL = D / 16;   // outputs per thread: a TL x TL tile of S
    __shared__ float rows[64][D + 4];
    __shared__ float ref[D];
    const int tid = threadIdx.x, ti = tid / 16, tj = tid % 16;
    if (tid < D) ref[tid] = load_f32(K + tid);
    __syncthreads();
    float acc[TL][TL];
#pragma unroll
    for (int x = 0; x < TL; ++x)
#pragma unroll
        for (int y = 0; y < TL; ++y) acc[x][y] = 0.f;
    float ms = 0.f;
    for (int64_t r0 = (int64_t)blockIdx.x * 64; r0 < N; r0 += (int64_t)gridDim.x * 64) {
        for (int e = tid; e < 64 * D; e += 256) {
            const int rr = e / D, c = e % D;
            const int64_t n = r0 + rr;
            float v = 0.f;   // rows past the end add nothing
            if (n < N) {
                const int64_t bh = n / Tn, t = n % Tn;
                v = load_f32(K + (bh * t_cap + t) * D + c) - ref[c];
            }
            rows[rr][c] = v;
        }
        __syncthreads();
        for (int rr = 0; rr < 64; ++rr) {
            float a[TL], b[TL];
#pragma unroll
            for (int x = 0; x < TL; ++x) {
                a[x] = rows[rr][ti * TL + x];
                b[x] = rows[rr][tj * TL + x];
            }
#pragma unroll
            for (int x = 0; x < TL; ++x)
#pragma unroll
                for (int y = 0; y < TL; ++y) acc[x][y] = fmaf(a[x], b[y], acc[x][y]);
        }
        if (tid < D)
            for (int rr = 0; rr < 64; ++rr) ms += rows[rr][tid];
        __syncthreads();
    }
    float* out = part + (int64_t)blockIdx.x * (D * D + D);
#pragma unroll
    for (int x = 0; x < TL; ++x)
#pragma unroll
        for (int y = 0; y < TL; ++y) out[(ti * TL + x) * D + tj * TL + y] = acc[x][y];
    if (tid < D) out[D * D + tid] = ms;
}

__global__ __launch_bounds__(256) void pca_reduce_kernel(const float* __restrict__ part, int nwg, int D,
                                                         double* __restrict__ sums) {
    const int e = blockIdx.x * 256 + threadIdx.x;
    if (e >= D * D + D) return;
    double s = 0.0;
    for (int w = 0; w < nwg; ++w) s += (double)part[(int64_t)w * (D * D + D) + e];
    sums[e] = s;
}

// players of the round-robin schedule: position 0 keeps player 0, position i
// (1..n-1) holds player (i - 1 + r) mod (n - 1) + 1 in round r; pair k of a
// round is positions (k, n - 1 - k)
__device__ __forceinline__ int rr_player(int pos, int r, int n) {
    return pos == 0 ? 0 : (pos - 1 + r) % (n - 1) + 1;
}

template <typename T>
__global__ __launch_bounds__(1024) void pca_eig_kernel(const double* __restrict__ sums, int D, int64_t N,
                                                       T* __restrict__ W, float* __restrict__ eig, int n_dir) {
    __shared__ float A[kPcaMaxD][kPcaMaxD + 1];
    __shared__ float Vm[kPcaMaxD][kPcaMaxD + 1];
    __shared__ float rc[kPcaMaxD / 2], rs[kPcaMaxD / 2];
    __shared__ int rp[kPcaMaxD / 2], rq[kPcaMaxD / 2];
    __shared__ float red[16];
    __shared__ int order[kPcaMaxD];
    const int tid = threadIdx.x, l = lane_id(), wid = tid >> 6;
    const double inv = 1.0 / (double)N;
    for (int e = tid; e < D * D; e += 1024) {
        const int i = e / D, j = e % D;
        const double mi = sums[D * D + i] * inv, mj = sums[D * D + j] * inv;
        A[i][j] = (float)(sums[e] * inv - mi * mj);
        Vm[i][j] = i == j ? 1.f : 0.f;
    }
    __syncthreads();
    const int half = D / 2;
    for (int sweep = 0; sweep < 30; ++sweep) {
        // off-diagonal and diagonal mass
        float off = 0.f, dia = 0.f;
        for (int e = tid; e < D * D; e += 1024) {
            const int i = e / D, j = e % D;
            const float v = A[i][j] * A[i][j];
            if (i != j) off += v; else dia += v;
        }
        off = wave_sum(off);
        dia = wave_sum(dia);
        if (l == 0) {
            red[wid] = off;
        }
        __syncthreads();
        float offt = 0.f;
        for (int w = 0; w < 16; ++w) offt += red[w];
        __syncthreads();
        if (l == 0) red[wid] = dia;
        __syncthreads();
        float diat = 0.f;
        for (int w = 0; w < 16; ++w) diat += red[w];
        __syncthreads();
        if (offt <= 1e-14f * diat || offt == 0.f) break;
        for (int r = 0; r < D - 1; ++r) {
            if (tid < half) {
                const int p0 = rr_player(tid, r, D), q0 = rr_player(D - 1 - tid, r, D);
                const int p = p0 < q0 ? p0 : q0, q = p0 < q0 ? q0 : p0;
                const float apq = A[p][q], app = A[p][p], aqq = A[q][q];
                float c = 1.f, s = 0.f;
                if (fabsf(apq) > 1e-30f) {
                    const float tau = (aqq - app) / (2.f * apq);
                    const float t = tau >= 0.f ? 1.f / (tau + sqrtf(1.f + tau * tau))
                                               : -1.f / (-tau + sqrtf(1.f + tau * tau));
                    c = 1.f / sqrtf(1.f + t * t);
                    s = t * c;
                }
                rc[tid] = c;
                rs[tid] = s;
                rp[tid] = p;
                rq[tid] = q;
            }
            __syncthreads();
            // A <- J^T A (rows p, q of every pair)
            for (int e = tid; e < half * D; e += 1024) {
                const int k = e / D, j = e % D;
                const int p = rp[k], q = rq[k];
                const float c = rc[k], s = rs[k];
                const float ap = A[p][j], aq = A[q][j];
                A[p][j] = c * ap - s * aq;
                A[q][j] = s * ap + c * aq;
            }
            __syncthreads();
            // A <- A J and V <- V J (columns p, q of every pair)
            for (int e = tid; e < half * D; e += 1024) {
                const int k = e / D, i = e % D;
                const int p = rp[k], q = rq[k];
                const float c = rc[k], s = rs[k];
                const float ap = A[i][p], aq = A[i][q];
                A[i][p] = c * ap - s * aq;
                A[i][q] = s * ap + c * aq;
                const float vp = Vm[i][p], vq = Vm[i][q];
                Vm[i][p] = c * vp - s * vq;
                Vm[i][q] = s * vp + c * vq;
            }
            __syncthreads();
        }
    }
    // eigenvalues ranked descending, ties to the lower index
    if (tid < D) {
        const float li = A[tid][tid];
        int rank = 0;
        for (int j = 0; j < D; ++j) {
            const float lj = A[j][j];
            rank += (lj > li || (lj == li && j < tid)) ? 1 : 0;
        }
        order[rank] = tid;
    }
    __syncthreads();
    if (tid < D && eig != nullptr) eig[tid] = A[order[tid]][order[tid]];
    // W[:, r] = eigenvector order[r], its largest-magnitude component positive
    if (tid < n_dir) {
        const int c = order[tid];
        int best = 0;
        float bv = -1.f;
        for (int i = 0; i < D; ++i) {
            const float a = fabsf(Vm[i][c]);
            if (a > bv) {
                bv = a;
                best = i;
            }
        }
        const float sg = Vm[best][c] < 0.f ? -1.f : 1.f;
        for (int i = 0; i < D; ++i) {
            const float v = sg * Vm[i][c];
            if constexpr (sizeof(T) == 2)
                W[i * n_dir + tid] = f32_to_bf16(v);
            else
                W[i * n_dir + tid] = v;
        }
    }
}

}  // namespace

size_t pca_workspace_bytes(int D) {
    const size_t part = (size_t)kPcaWgs * (D * D + D) * 4;
    return ((part + 255) & ~(size_t)255) + (size_t)(D * D + D) * 8;
}

hipError_t launch_pca(const void* K, bool bf16, int D, int64_t t_cap, int64_t T, int BH, void* W, float* eig,
                      void* workspace, hipStream_t st) {
    const int64_t N = (int64_t)BH * T;
    float* part = static_cast<float*>(workspace);
    double* sums = reinterpret_cast<double*>(static_cast<char*>(workspace) +
                                             (((size_t)kPcaWgs * (D * D + D) * 4 + 255) & ~(size_t)255));
    const int64_t need = (N + 63) / 64;
    const int nwg = (int)(need < kPcaWgs ? (need > 0 ? need : 1) : kPcaWgs);
    if (bf16) {
        if (D == 128)
            hipLaunchKernelGGL((pca_moments_kernel<uint16_t, 128>), dim3(nwg), dim3(256), 0, st,
                               static_cast<const uint16_t*>(K), t_cap, T, N, part);
        else
            hipLaunchKernelGGL((pca_moments_kernel<uint16_t, 64>), dim3(nwg), dim3(256), 0, st,
                               static_cast<const uint16_t*>(K), t_cap, T, N, part);
    } else {
        if (D == 128)
            hipLaunchKernelGGL((pca_moments_kernel<float, 128>), dim3(nwg), dim3(256), 0, st,
                               static_cast<const float*>(K), t_cap, T, N, part);
        else
            hipLaunchKernelGGL((pca_moments_kernel<float, 64>), dim3(nwg), dim3(256), 0, st,
                               static_cast<const float*>(K), t_cap, T, N, part);
    }
    hipLaunchKernelGGL(pca_reduce_kernel, dim3((unsigned)((D * D + D + 255) / 256)), dim3(256), 0, st, part, nwg, D,
                       sums);
    if (bf16)
        hipLaunchKernelGGL(pca_eig_kernel<uint16_t>, dim3(1), dim3(1024), 0, st, sums, D, N,
                           static_cast<uint16_t*>(W), eig, kLatent);
    else
        hipLaunchKernelGGL(pca_eig_kernel<float>, dim3(1), dim3(1024), 0, st, sums, D, N, static_cast<float*>(W),
                           eig, kLatent);
    return hipGetLastError();
}

}  // namespace lsa
