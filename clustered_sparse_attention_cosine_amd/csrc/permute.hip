// Cluster-contiguous layout for gfx950: member counts, offsets, a stable
// permutation (ascending id inside a cluster) and a gather that writes the
// permuted K/V copies together with per-cluster means and per-dimension
// max/min. This is the "K* <- K[Index], V* <- V[Index]" gather of Algorithm 3
// (AdaCluster paper, section 3.3) laid out once per layer instead of per query.
#include <math.h>
#include "common.hpp"
#include "kernels.hpp"

namespace adc {

hipError_t fill_i32(int32_t* p, int64_t n, int32_t v, hipStream_t s);

// Exclusive scan of the counts (one workgroup per head, M <= 8192).
__global__ __launch_bounds__(1024) void scan_offsets_kernel(const int32_t* __restrict__ cnt, int M,
                                                            int32_t* __restrict__ sizes_out,
                                                            int32_t* __restrict__ offsets,
                                                            const uint8_t* __restrict__ active) {
    __shared__ int wsum[16];
    const int bh = blockIdx.x;
    if (active && !active[bh]) return;
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
    const int per = (M + 1023) / 1024;
    const int beg = tid * per;
    const int32_t* c = cnt + (int64_t)bh * M;
    int local = 0;
    for (int i = 0; i < per; ++i)
        if (beg + i < M) local += c[beg + i];
    int incl = local;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        int v = __shfl_up(incl, o);
        if (l >= o) incl += v;
    }
    if (l == 63) wsum[w] = incl;
    __syncthreads();
    int before = 0;
    for (int i = 0; i < w; ++i) before += wsum[i];
    int run = before + incl - local;
    int32_t* off = offsets + (int64_t)bh * (M + 1);
    for (int i = 0; i < per; ++i) {
        const int j = beg + i;
        if (j < M) {
            off[j] = run;
            run += c[j];
            if (sizes_out) sizes_out[(int64_t)bh * M + j] = c[j];
        }
    }
    if (tid == 1023) off[M] = run;
}

hipError_t launch_scan_offsets(const Prob& p, const int32_t* cnt, int M, int32_t* sizes_out,
                               int32_t* offsets, hipStream_t s, const uint8_t* active) {
    hipLaunchKernelGGL(scan_offsets_kernel, dim3(p.BH), dim3(1024), 0, s, cnt, M, sizes_out, offsets,
                       active);
    return hipGetLastError();
}

// Stable counting sort over segments: the rows of a head are cut into
// segments of SORT_SEG rows; (1) each segment counts its labels in LDS,
// (2) for every label a column scan over the segments gives each segment's
// start inside the label's range and the label's total, (3) the totals are
// scanned into offsets, (4) each segment ranks its rows as the one-workgroup
// sweep above does, starting every label's counter at offsets[label] plus the
// rows of that label in the earlier segments. Same permutation, with
// BH x segments workgroups instead of BH.
__global__ __launch_bounds__(1024) void seg_hist_kernel(const int32_t* __restrict__ labels, int N, int M,
                                                        int nseg, int32_t* __restrict__ seg_cnt,
                                                        const int32_t* __restrict__ nrows,
                                                        const uint8_t* __restrict__ active) {
    __shared__ int h[8192];
    const int sg = blockIdx.x, bh = blockIdx.y, tid = threadIdx.x;
    if (active && !active[bh]) return;
    const int n = nrows ? nrows[bh] : N;
    for (int j = tid; j < M; j += 1024) h[j] = 0;
    __syncthreads();
    const int beg = sg * SORT_SEG, end = min(n, beg + SORT_SEG);
    const int32_t* lab = labels + (int64_t)bh * N;
    for (int i = beg + tid; i < end; i += 1024) {
        const int v = lab[i];
        if (v >= 0 && v < M) atomicAdd(&h[v], 1);
    }
    __syncthreads();
    int32_t* out = seg_cnt + ((int64_t)bh * nseg + sg) * M;
    for (int j = tid; j < M; j += 1024) out[j] = h[j];
}

// In place: seg_cnt[s][j] <- rows of label j in segments before s; total[j].
__global__ __launch_bounds__(256) void seg_scan_kernel(int M, int nseg, int32_t* __restrict__ seg_cnt,
                                                       int32_t* __restrict__ total,
                                                       const uint8_t* __restrict__ active) {
    const int bh = blockIdx.y;
    const int j = blockIdx.x * 256 + threadIdx.x;
    if (j >= M || (active && !active[bh])) return;
    int32_t* c = seg_cnt + (int64_t)bh * nseg * M + j;
    int run = 0;
    // eight segments' counts loaded at once (clamped reads, so the loads are
    // unconditional and in flight together), then scanned
    for (int s0 = 0; s0 < nseg; s0 += 8) {
        int v[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) v[k] = c[(int64_t)min(s0 + k, nseg - 1) * M];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            if (s0 + k < nseg) {
                c[(int64_t)(s0 + k) * M] = run;
                run += v[k];
            }
        }
    }
    total[(int64_t)bh * M + j] = run;
}

__global__ __launch_bounds__(1024) void seg_rank_kernel(const int32_t* __restrict__ labels, int N, int M,
                                                        int nseg, const int32_t* __restrict__ offsets,
                                                        const int32_t* __restrict__ seg_cnt,
                                                        int32_t* __restrict__ perm,
                                                        const int32_t* __restrict__ nrows,
                                                        const uint8_t* __restrict__ active) {
    __shared__ int running[8192];
    __shared__ int grp_lab[16][64], grp_size[16][64], grp_base[16][64];
    __shared__ int ngrp[16];
    const int sg = blockIdx.x, bh = blockIdx.y;
    if (active && !active[bh]) return;
    const int n = nrows ? nrows[bh] : N;
    if (sg * SORT_SEG >= n) return;
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
    const int32_t* off = offsets + (int64_t)bh * (M + 1);
    const int32_t* before = seg_cnt + ((int64_t)bh * nseg + sg) * M;
    for (int j = tid; j < M; j += 1024) running[j] = off[j] + before[j];
    int nbits = 0;
    while ((1 << nbits) < M) ++nbits;
    const int32_t* lab_h = labels + (int64_t)bh * N;
    const uint64_t lt = (l == 0) ? 0ull : (~0ull >> (64 - l));
    __syncthreads();
    const int beg = sg * SORT_SEG, end = min(n, beg + SORT_SEG);
    // the segment's labels, all loads issued at once (clamped to the segment)
    constexpr int IT = SORT_SEG / 1024;
    int raws[IT];
#pragma unroll
    for (int it = 0; it < IT; ++it) raws[it] = lab_h[min(beg + it * 1024 + tid, end - 1)];
#pragma unroll
    for (int it = 0; it < IT; ++it) {
        const int base = beg + it * 1024;
        if (base >= end) break;
        const int i = base + tid;
        const int raw = i < end ? raws[it] : -1;
        const bool ok = raw >= 0 && raw < M;   // rows with out-of-range labels are left out
        const int lab = ok ? raw : 0;
        uint64_t m = __ballot(ok);
        for (int bit = 0; bit < nbits; ++bit) {
            const bool set = (lab >> bit) & 1;
            const uint64_t b = __ballot(ok && set);
            m &= set ? b : ~b;
        }
        const int rank = __popcll(m & lt);
        const int gsize = __popcll(m);
        const int leader = m ? __ffsll((unsigned long long)m) - 1 : 0;
        // each wave lists its groups (label, size) in lane order of their leaders;
        // one wave then walks the 16 lists in wave order, one lane per group (the
        // labels of one list are distinct), advancing the counters and writing
        // back every group's base
        const bool is_leader = ok && l == leader;
        const uint64_t lm = __ballot(is_leader);
        if (is_leader) {
            const int slot = __popcll(lm & lt);
            grp_lab[w][slot] = lab;
            grp_size[w][slot] = gsize;
        }
        if (l == 0) ngrp[w] = __popcll(lm);
        __syncthreads();
        if (w == 0) {
            for (int ww = 0; ww < 16; ++ww) {
                if (l < ngrp[ww]) {
                    const int lb = grp_lab[ww][l];
                    const int b = running[lb];
                    grp_base[ww][l] = b;
                    running[lb] = b + grp_size[ww][l];
                }
            }
        }
        __syncthreads();
        if (ok) {
            const int slot = __popcll(lm & ((leader == 0) ? 0ull : (~0ull >> (64 - leader))));
            perm[(int64_t)bh * N + grp_base[w][slot] + rank] = i;
        }
    }
}

int sort_segments(int N) { return (N + SORT_SEG - 1) / SORT_SEG; }

hipError_t launch_counting_sort(const Prob& p, const int32_t* labels, int M, int32_t* seg_cnt,
                                int32_t* total, int32_t* sizes, int32_t* offsets, int32_t* perm,
                                hipStream_t s, const int32_t* nrows, const uint8_t* active) {
    const int nseg = sort_segments(p.N);
    hipLaunchKernelGGL(seg_hist_kernel, dim3(nseg, p.BH), dim3(1024), 0, s, labels, p.N, M, nseg, seg_cnt,
                       nrows, active);
    hipLaunchKernelGGL(seg_scan_kernel, dim3((M + 255) / 256, p.BH), dim3(256), 0, s, M, nseg, seg_cnt, total,
                       active);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if ((e = launch_scan_offsets(p, total, M, sizes, offsets, s, active)) != hipSuccess) return e;
    hipLaunchKernelGGL(seg_rank_kernel, dim3(nseg, p.BH), dim3(1024), 0, s, labels, p.N, M, nseg, offsets,
                       seg_cnt, perm, nrows, active);
    return hipGetLastError();
}

// The f32 rounding of a quotient v / n (v exact in f64) formed as p = v * r,
// r = RN64(1 / n): p lies within 3 f64 units in the last place of RN64(v / n)
// (relative errors 2^-53 of r and of the product, 2^-53 of the exact
// quotient), so both round to the same f32 unless an f32 rounding midpoint
// (the 29 bits below f32 precision equal to 2^28) lies that close, or the
// value is below the normal f32 range. Returns true when p is more than 16
// units from any midpoint and normal (or zero): then RN32(p) = RN32(RN64(v / n)).
__device__ __forceinline__ bool f32_rounding_settled(double p) {
    const uint64_t b = (uint64_t)__double_as_longlong(p);
    const uint32_t low = (uint32_t)b & 0x1FFFFFFFu;
    const uint32_t hi = (uint32_t)(b >> 32) & 0x7FFFFFFFu;
    const bool normal = hi >= (898u << 20) || (hi | (uint32_t)b) == 0u;  // |p| >= 2^-125, or p = 0
    return normal && (low - (0x10000000u - 16u)) > 32u;
}

// One wave per cluster walks its members in permuted order, RS rows at a
// time: the rows are copied to x_perm / v_perm and staged in LDS with
// coalesced 16-byte accesses (all loads of a batch in flight at once), and the
// statistics are accumulated with one lane per dimension in member order (f64
// sums, as the definition).
//
// NORM (queries; sums of the normalized and of the raw rows, no max/min): lane
// q first takes the norm of staged row q (f64, index order) and its
// reciprocal; then, QB rows at a time, every lane forms its dimension of the
// QB normalized values, each rounded to f32 as the definition has it, before
// the member-order adds, so only the adds form a dependent chain (the last
// nb mod QB rows of a cluster one by one). A quotient
// is taken as a product with the reciprocal when that provably rounds to the
// same f32 (f32_rounding_settled), else by division for the whole block. With
// a division per member on the chain this pass ran at under a fifth of the key
// pass's bandwidth.
template <typename T, int D, bool NORM>
__global__ __launch_bounds__(256) void gather_stats_kernel(int N, int M,
                                                           const int32_t* __restrict__ offsets,
                                                           const int32_t* __restrict__ perm,
                                                           const T* __restrict__ x,
                                                           const T* __restrict__ v,
                                                           float* __restrict__ means,
                                                           float* __restrict__ raw_means,
                                                           T* __restrict__ xmax, T* __restrict__ xmin,
                                                           T* __restrict__ x_perm,
                                                           T* __restrict__ v_perm) {
#pragma clang fp contract(off)
    constexpr int E = D / 64;
    // rows staged at once: 32 for the copies (half the LDS of 64 rows, twice
    // the workgroups per CU); 64 for bf16 D = 64 queries, one row per lane
    // for the norms
    constexpr int RS = (NORM && sizeof(T) == 2 && D == 64) ? 64 : 32;
    constexpr int LDX = D + 16 / (int)sizeof(T);   // padded row stride (elements)
    constexpr int CPR = D / 8;                     // 8-element chunks per row
    constexpr int RPI = 64 / CPR;                  // rows per wave instruction
    constexpr int W8 = 8 * (int)sizeof(T) / 16;    // 16-byte words per chunk
    constexpr int QB = D == 64 ? 16 : 8;           // rows per block of quotients (NORM)
    __shared__ __attribute__((aligned(16))) T xs[4][RS * LDX];
    __shared__ double nrm_s[NORM ? 4 : 1][NORM ? RS : 1];
    __shared__ double rcp_s[NORM ? 4 : 1][NORM ? RS : 1];
    const int bh = blockIdx.y;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), l = threadIdx.x & 63;
    const int j = blockIdx.x * 4 + w;
    if (j >= M) return;
    const int32_t* off = offsets + (int64_t)bh * (M + 1);
    const int beg = off[j], end = off[j + 1];
    T* xw = xs[w];
    double sum[E], rsum[E];
    float mx[E], mn[E];
#pragma unroll
    for (int e = 0; e < E; ++e) { sum[e] = 0.0; rsum[e] = 0.0; mx[e] = -INFINITY; mn[e] = INFINITY; }
    for (int h0 = beg; h0 < end; h0 += RS) {
        const int nb = min(RS, end - h0);
        const int tok_l = perm[(int64_t)bh * N + h0 + min(l, nb - 1)];
        // every load of the batch (x, and v when it is permuted too) is issued
        // before the first store; rows past the cluster repeat its last row
        constexpr int IT = RS / RPI;
        constexpr int EW = 16 / (int)sizeof(T);  // elements per 16-byte word
        u32x4 xv[IT][W8], vv[IT][W8];
#pragma unroll
        for (int it = 0; it < IT; ++it) {
            const int q = it * RPI + l / CPR, c = l % CPR;
            const int64_t src = ((int64_t)bh * N + __shfl(tok_l, q)) * D + c * 8;
#pragma unroll
            for (int k = 0; k < W8; ++k) xv[it][k] = *reinterpret_cast<const u32x4*>(x + src + k * EW);
            if (!NORM && v_perm) {
#pragma unroll
                for (int k = 0; k < W8; ++k) vv[it][k] = *reinterpret_cast<const u32x4*>(v + src + k * EW);
            }
        }
#pragma unroll
        for (int it = 0; it < IT; ++it) {
            const int q = it * RPI + l / CPR, c = l % CPR;
            const int64_t dst = ((int64_t)bh * N + h0 + q) * D + c * 8;
#pragma unroll
            for (int k = 0; k < W8; ++k) *reinterpret_cast<u32x4*>(&xw[q * LDX + c * 8 + k * EW]) = xv[it][k];
            if (q < nb) {
                if (x_perm) {
#pragma unroll
                    for (int k = 0; k < W8; ++k) *reinterpret_cast<u32x4*>(x_perm + dst + k * EW) = xv[it][k];
                }
                if (!NORM && v_perm) {
#pragma unroll
                    for (int k = 0; k < W8; ++k) *reinterpret_cast<u32x4*>(v_perm + dst + k * EW) = vv[it][k];
                }
            }
        }
        // lanes read rows other lanes wrote
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        if constexpr (NORM) {
            for (int q = l; q < RS; q += 64) {
                double nrm = 1.0;
                if (q < nb) {
                    double ss = 0.0;
                    for (int d = 0; d < D; ++d) {
                        const double vd = (double)elem<T>::load(xw, q * LDX + d);
                        ss += vd * vd;
                    }
                    nrm = sqrt(ss);
                    if (nrm < 1e-12) nrm = 1e-12;
                }
                nrm_s[w][q] = nrm;
                rcp_s[w][q] = 1.0 / nrm;
            }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            // full blocks of QB rows, then the cluster's last rows one by one
            const int nfull = nb / QB * QB;
            for (int q0 = 0; q0 < nfull; q0 += QB) {
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    float val[QB], nv[QB];
#pragma unroll
                    for (int i = 0; i < QB; ++i) val[i] = elem<T>::load(xw, (q0 + i) * LDX + l + 64 * e);
                    bool exact = true;
#pragma unroll
                    for (int i = 0; i < QB; ++i) {
                        const double qd = (double)val[i] * rcp_s[w][q0 + i];
                        nv[i] = (float)qd;
                        exact = exact && f32_rounding_settled(qd);
                    }
                    if (__builtin_expect(__ballot(!exact) != 0, 0)) {
#pragma unroll
                        for (int i = 0; i < QB; ++i) nv[i] = (float)((double)val[i] / nrm_s[w][q0 + i]);
                    }
#pragma unroll
                    for (int i = 0; i < QB; ++i) {
                        sum[e] += (double)nv[i];
                        rsum[e] += (double)val[i];
                    }
                }
            }
            for (int q = nfull; q < nb; ++q) {
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    const float val = elem<T>::load(xw, q * LDX + l + 64 * e);
                    sum[e] += (double)(float)((double)val / nrm_s[w][q]);
                    rsum[e] += (double)val;
                }
            }
        } else {
            for (int q = 0; q < nb; ++q) {
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    const float val = elem<T>::load(xw, q * LDX + l + 64 * e);
                    sum[e] += (double)val;
                    mx[e] = fmaxf(mx[e], val);
                    mn[e] = fminf(mn[e], val);
                }
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
    const int cnt = end - beg;
    const int64_t slot = ((int64_t)bh * M + j) * D;
#pragma unroll
    for (int e = 0; e < E; ++e) {
        const int d = l + 64 * e;
        if (cnt > 0 && means) means[slot + d] = (float)(sum[e] / (double)cnt);
        if (raw_means) raw_means[slot + d] = cnt > 0 ? (float)(rsum[e] / (double)cnt) : 0.0f;
        if (xmax) elem<T>::store(xmax, slot + d, cnt > 0 ? mx[e] : 0.0f);
        if (xmin) elem<T>::store(xmin, slot + d, cnt > 0 ? mn[e] : 0.0f);
    }
}

hipError_t launch_gather_stats(const Prob& p, int M, const int32_t* offsets, const int32_t* perm,
                               const void* x, const void* v, int normalize, float* means,
                               float* raw_means, void* xmax, void* xmin, void* x_perm, void* v_perm,
                               hipStream_t s) {
    dim3 grid((unsigned)((M + 3) / 4), (unsigned)p.BH);
    // the normalized pass copies one tensor and takes no max/min
    if (normalize && (v_perm || xmax || xmin)) return hipErrorInvalidValue;
    if (p.bf16) {
        auto k = normalize ? (p.D == 64 ? gather_stats_kernel<u16, 64, true> : gather_stats_kernel<u16, 128, true>)
                           : (p.D == 64 ? gather_stats_kernel<u16, 64, false> : gather_stats_kernel<u16, 128, false>);
        hipLaunchKernelGGL(k, grid, dim3(256), 0, s, p.N, M, offsets, perm, (const u16*)x,
                           (const u16*)v, means, raw_means, (u16*)xmax, (u16*)xmin,
                           (u16*)x_perm, (u16*)v_perm);
    } else {
        auto k = normalize ? (p.D == 64 ? gather_stats_kernel<float, 64, true> : gather_stats_kernel<float, 128, true>)
                           : (p.D == 64 ? gather_stats_kernel<float, 64, false> : gather_stats_kernel<float, 128, false>);
        hipLaunchKernelGGL(k, grid, dim3(256), 0, s, p.N, M, offsets, perm, (const float*)x,
                           (const float*)v, means, raw_means, (float*)xmax,
                           (float*)xmin, (float*)x_perm, (float*)v_perm);
    }
    return hipGetLastError();
}

}  // namespace adc
