// Compactness diagnostics of a clustering for gfx950 (AdaCluster paper,
// section 3.2.1 for the reconstruction error and the layer score Comp, Fig. 10
// for the average intra-cluster distance and the Davies-Bouldin index).
//
// The rows arrive in cluster-contiguous order (the K' copy the key clustering
// writes, with its offsets), so each cluster's members are one contiguous run
// and no labels or atomics are needed:
//   pass 1  one wave per cluster: sum ||x - c||^2 and sum ||x - c|| over the run
//           (f32 inside a row, f64 across rows, fixed lane order);
//   pass 2  one thread per cluster a: max over clusters b != a with members and
//           c_b != c_a of (s_a + s_b) / ||c_a - c_b||, the centres streamed
//           through LDS in tiles of 64 (direct differences, not the Gram form,
//           so close centres keep their accuracy);
//   pass 3  one workgroup per head: fixed-order f64 sums into MSE, the mean
//           distance and DB; then Comp = 1 / mean over heads of MSE.
#include <math.h>
#include "common.hpp"
#include "kernels.hpp"

namespace adc {

template <typename T, int D>
__global__ __launch_bounds__(256) void cluster_dist_kernel(int N, int M, const T* __restrict__ x,
                                                           const int32_t* __restrict__ offsets,
                                                           const float* __restrict__ cent,
                                                           double* __restrict__ csq,
                                                           double* __restrict__ cdist,
                                                           float* __restrict__ smean) {
    constexpr int E = 16 / sizeof(T);        // elements per 16-byte chunk
    constexpr int LPR = D / E;               // lanes per row
    constexpr int RPW = 64 / LPR;            // rows per wave step
    const int bh = blockIdx.y;
    const int b = blockIdx.x * 4 + (threadIdx.x >> 6), l = threadIdx.x & 63;
    if (b >= M) return;
    const int64_t slot = (int64_t)bh * M + b;
    const int r0 = offsets[(int64_t)bh * (M + 1) + b], r1 = offsets[(int64_t)bh * (M + 1) + b + 1];
    const int col = (l % LPR) * E, sub = l / LPR;
    float c[E];
#pragma unroll
    for (int i = 0; i < E; ++i) c[i] = cent[slot * D + col + i];
    double sq = 0.0, dist = 0.0;
    for (int r = r0 + sub; r < r1; r += RPW) {
        float v[E];
        const T* p = x + ((int64_t)bh * N + r) * D + col;
        if constexpr (sizeof(T) == 2) {
            load8<T>(p, v);
        } else {
            const float4 f = *reinterpret_cast<const float4*>(p);
            v[0] = f.x; v[1] = f.y; v[2] = f.z; v[3] = f.w;
        }
        float part = 0.0f;
#pragma unroll
        for (int i = 0; i < E; ++i) {
            const float d = v[i] - c[i];
            part = fmaf(d, d, part);
        }
#pragma unroll
        for (int o = LPR / 2; o > 0; o >>= 1) part += __shfl_xor(part, o);
        if (l % LPR == 0) {
            sq += (double)part;
            dist += (double)sqrtf(part);
        }
    }
    sq = wave_sum_d(sq);
    dist = wave_sum_d(dist);
    if (l == 0) {
        const int n = r1 - r0;
        csq[slot] = sq;
        cdist[slot] = dist;
        smean[slot] = n > 0 ? (float)(dist / (double)n) : 0.0f;
    }
}

template <int D>
__global__ __launch_bounds__(256) void db_kernel(int M, const int32_t* __restrict__ offsets,
                                                 const float* __restrict__ cent,
                                                 const float* __restrict__ smean,
                                                 float* __restrict__ dbmax) {
    __shared__ __attribute__((aligned(16))) float tc[64 * D];
    __shared__ float ts[64];
    __shared__ int tn[64];
    const int bh = blockIdx.y;
    const int a = blockIdx.x * 256 + threadIdx.x;
    const int32_t* off = offsets + (int64_t)bh * (M + 1);
    const bool live = a < M && off[a + 1] > off[a];
    float ca[D];
    const float* cp = cent + ((int64_t)bh * M + (a < M ? a : 0)) * D;
#pragma unroll
    for (int i = 0; i < D; i += 4) {
        const float4 f = *reinterpret_cast<const float4*>(cp + i);
        ca[i] = f.x; ca[i + 1] = f.y; ca[i + 2] = f.z; ca[i + 3] = f.w;
    }
    const float sa = live ? smean[(int64_t)bh * M + a] : 0.0f;
    float mx = 0.0f;
    for (int j0 = 0; j0 < M; j0 += 64) {
        __syncthreads();
        for (int e = threadIdx.x; e < 64 * D / 4; e += 256) {
            const int row = e / (D / 4), c4 = e % (D / 4);
            float4 f = make_float4(0.f, 0.f, 0.f, 0.f);
            if (j0 + row < M) f = *reinterpret_cast<const float4*>(cent + ((int64_t)bh * M + j0 + row) * D + c4 * 4);
            *reinterpret_cast<float4*>(&tc[row * D + c4 * 4]) = f;
        }
        if (threadIdx.x < 64) {
            const int j = j0 + threadIdx.x;
            const bool ok = j < M && off[j + 1] > off[j];
            tn[threadIdx.x] = ok ? 1 : 0;
            ts[threadIdx.x] = ok ? smean[(int64_t)bh * M + j] : 0.0f;
        }
        __syncthreads();
        if (!live) continue;
        const int jn = min(64, M - j0);
        for (int jj = 0; jj < jn; ++jj) {
            float d2 = 0.0f;
#pragma unroll
            for (int i = 0; i < D; i += 4) {
                const float4 f = *reinterpret_cast<const float4*>(&tc[jj * D + i]);
                const float d0 = ca[i] - f.x, d1 = ca[i + 1] - f.y, e2 = ca[i + 2] - f.z, d3 = ca[i + 3] - f.w;
                d2 = fmaf(d0, d0, d2);
                d2 = fmaf(d1, d1, d2);
                d2 = fmaf(e2, e2, d2);
                d2 = fmaf(d3, d3, d2);
            }
            if (tn[jj] && j0 + jj != a && d2 > 0.0f) mx = fmaxf(mx, (sa + ts[jj]) / sqrtf(d2));
        }
    }
    if (a < M) dbmax[(int64_t)bh * M + a] = live ? mx : 0.0f;
}

__global__ __launch_bounds__(256) void compact_head_kernel(int N, int M, const int32_t* __restrict__ offsets,
                                                           const double* __restrict__ csq,
                                                           const double* __restrict__ cdist,
                                                           const float* __restrict__ dbmax,
                                                           double* __restrict__ mse,
                                                           double* __restrict__ mean_dist,
                                                           double* __restrict__ db) {
    __shared__ double red[3][4];
    __shared__ int redk[4];
    const int bh = blockIdx.x;
    const int32_t* off = offsets + (int64_t)bh * (M + 1);
    double s0 = 0.0, s1 = 0.0, s2 = 0.0;
    int k = 0;
    for (int b = threadIdx.x; b < M; b += 256) {
        const int64_t i = (int64_t)bh * M + b;
        s0 += csq[i];
        s1 += cdist[i];
        s2 += (double)dbmax[i];
        k += off[b + 1] > off[b] ? 1 : 0;
    }
    s0 = wave_sum_d(s0);
    s1 = wave_sum_d(s1);
    s2 = wave_sum_d(s2);
    k = wave_sum_i(k);
    const int w = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) {
        red[0][w] = s0;
        red[1][w] = s1;
        red[2][w] = s2;
        redk[w] = k;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        const double t0 = (red[0][0] + red[0][1]) + (red[0][2] + red[0][3]);
        const double t1 = (red[1][0] + red[1][1]) + (red[1][2] + red[1][3]);
        const double t2 = (red[2][0] + red[2][1]) + (red[2][2] + red[2][3]);
        const int kk = redk[0] + redk[1] + redk[2] + redk[3];
        mse[bh] = t0 / (double)N;
        mean_dist[bh] = t1 / (double)N;
        db[bh] = kk >= 2 ? t2 / (double)kk : 0.0;
    }
}

__global__ void comp_kernel(int B, int H, const double* __restrict__ mse, double* __restrict__ comp) {
    const int b = blockIdx.x * blockDim.x + threadIdx.x;
    if (b >= B) return;
    double s = 0.0;
    for (int h = 0; h < H; ++h) s += mse[(int64_t)b * H + h];
    comp[b] = (double)H / s;
}

hipError_t launch_compactness(const Prob& p, int M, const void* x_perm, const int32_t* offsets,
                              const float* cent, double* csq, double* cdist, float* smean,
                              float* dbmax, double* mse, double* mean_dist, double* db,
                              double* comp, hipStream_t s) {
    const dim3 g1((unsigned)((M + 3) / 4), (unsigned)p.BH);
    if (p.bf16) {
        auto k = p.D == 64 ? cluster_dist_kernel<u16, 64> : cluster_dist_kernel<u16, 128>;
        hipLaunchKernelGGL(k, g1, dim3(256), 0, s, p.N, M, (const u16*)x_perm, offsets, cent, csq,
                           cdist, smean);
    } else {
        auto k = p.D == 64 ? cluster_dist_kernel<float, 64> : cluster_dist_kernel<float, 128>;
        hipLaunchKernelGGL(k, g1, dim3(256), 0, s, p.N, M, (const float*)x_perm, offsets, cent, csq,
                           cdist, smean);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const dim3 g2((unsigned)((M + 255) / 256), (unsigned)p.BH);
    if (p.D == 64)
        hipLaunchKernelGGL(db_kernel<64>, g2, dim3(256), 0, s, M, offsets, cent, smean, dbmax);
    else
        hipLaunchKernelGGL(db_kernel<128>, g2, dim3(256), 0, s, M, offsets, cent, smean, dbmax);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(compact_head_kernel, dim3((unsigned)p.BH), dim3(256), 0, s, p.N, M, offsets,
                       csq, cdist, dbmax, mse, mean_dist, db);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (comp) {
        const int B = p.BH / p.H;
        hipLaunchKernelGGL(comp_kernel, dim3((unsigned)((B + 63) / 64)), dim3(64), 0, s, B, p.H,
                           mse, comp);
        e = hipGetLastError();
    }
    return e;
}

}  // namespace adc
