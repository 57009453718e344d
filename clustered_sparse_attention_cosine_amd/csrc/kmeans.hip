// k-means kernels for gfx950: query normalisation, cold initialisation, the
// assignment step as a bf16 matrix-core contraction with a certified argmin,
// an exact f64 recheck of uncertain rows, the centroid update, and the
// bookkeeping of the multi-stage key clustering.
//
// Method: "AdaCluster: Adaptive Query-Key Clustering for Sparse Attention in
// Video Generation" (arXiv 2604.18348v1), section 3.1 (queries are clustered
// on the unit sphere), section 3.2.2 / Algorithm 1 (keys: stages of k-means on
// the still-unassigned keys, threshold tau) and section 4.1 (tau = 1.5 x mean
// distance).
#include <math.h>
#include "common.hpp"
#include "kernels.hpp"

namespace adc {

// ------------------------------------------------------------------ helpers
template <typename T>
__device__ __forceinline__ const T* row_ptr(const T* x, int N, int D, int bh, int64_t tok) {
    return x + ((int64_t)bh * N + tok) * D;
}

// ||x||, summed in index order in f64, floored at 1e-12 (query normalisation).
template <typename T>
__device__ double seq_norm(const T* r, int D) {
#pragma clang fp contract(off)
    double s = 0.0;
    for (int j = 0; j < D; ++j) {
        double v = (double)elem<T>::load(r, j);
        s += v * v;
    }
    double n = sqrt(s);
    return n < 1e-12 ? 1e-12 : n;
}

__global__ void fill_i32_kernel(int32_t* p, int64_t n, int32_t v) {
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = v;
}

hipError_t fill_i32(int32_t* p, int64_t n, int32_t v, hipStream_t s) {
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(fill_i32_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, p, n, v);
    return hipGetLastError();
}

__global__ void zero2_i32_kernel(int32_t* a, int32_t* b, int n) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) {
        a[i] = 0;
        b[i] = 0;
    }
}

__global__ void fill_u8_kernel(uint8_t* p, int64_t n, uint8_t v) {
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = v;
}

hipError_t fill_u8(uint8_t* p, int64_t n, uint8_t v, hipStream_t s) {
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(fill_u8_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, p, n, v);
    return hipGetLastError();
}

// Fixed-count key clustering: n_clusters = m, F = 0, tau = 0, stage sizes [N].
__global__ void fixed_info_kernel(int BH, int N, int m, int32_t* n_clusters, uint8_t* full,
                                  float* tau, int32_t* stage_sizes) {
    int bh = blockIdx.x * blockDim.x + threadIdx.x;
    if (bh >= BH) return;
    n_clusters[bh] = m;
    full[bh] = 0;
    tau[bh] = 0.0f;
    if (stage_sizes) {
        stage_sizes[bh * 8] = N;
        for (int i = 1; i < 8; ++i) stage_sizes[bh * 8 + i] = -1;
    }
}

hipError_t launch_fixed_info(int BH, int N, int m, int32_t* n_clusters, uint8_t* full, float* tau,
                             int32_t* stage_sizes, hipStream_t s) {
    hipLaunchKernelGGL(fixed_info_kernel, dim3((BH + 63) / 64), dim3(64), 0, s, BH, N, m, n_clusters,
                       full, tau, stage_sizes);
    return hipGetLastError();
}

// Warm start (section 3.2.2): the per-head count from an earlier multi-stage
// call is clamped to [1, cap] in place, and the fixed-path stage record (N,
// then -1) is written.
__global__ void warm_info_kernel(int BH, int N, int cap, int32_t* n_clusters, int32_t* stage_sizes) {
    int bh = blockIdx.x * blockDim.x + threadIdx.x;
    if (bh >= BH) return;
    n_clusters[bh] = min(max(n_clusters[bh], 1), cap);
    if (stage_sizes) {
        stage_sizes[bh * 8] = N;
        for (int i = 1; i < 8; ++i) stage_sizes[bh * 8 + i] = -1;
    }
}

hipError_t launch_warm_info(int BH, int N, int cap, int32_t* n_clusters, int32_t* stage_sizes,
                            hipStream_t s) {
    hipLaunchKernelGGL(warm_info_kernel, dim3((BH + 63) / 64), dim3(64), 0, s, BH, N, cap,
                       n_clusters, stage_sizes);
    return hipGetLastError();
}

// Slots [0, count) of each head take the caller's centres and hold a centre;
// the rest hold none (their centre rows were cleared beforehand). One wave per
// slot.
template <int D>
__global__ __launch_bounds__(256) void warm_init_kernel(const float* __restrict__ init,
                                                        const int32_t* __restrict__ count,
                                                        CentView cv) {
    const int bh = blockIdx.y;
    const int j = blockIdx.x * 4 + (threadIdx.x >> 6), l = threadIdx.x & 63;
    if (j >= cv.cap) return;
    const int64_t slot = (int64_t)bh * cv.cap + j;
    const bool used = j < count[bh];
    if (used) {
#pragma unroll
        for (int e = 0; e < D / 64; ++e) cv.cent[slot * D + l + 64 * e] = init[slot * D + l + 64 * e];
    }
    if (l == 0) cv.valid[slot] = used ? 1 : 0;
}

hipError_t launch_warm_init(const Prob& p, const float* init, const int32_t* count, CentView cv,
                            hipStream_t s) {
    dim3 grid((unsigned)((cv.cap + 3) / 4), (unsigned)p.BH);
    if (p.D == 64)
        hipLaunchKernelGGL(warm_init_kernel<64>, grid, dim3(256), 0, s, init, count, cv);
    else
        hipLaunchKernelGGL(warm_init_kernel<128>, grid, dim3(256), 0, s, init, count, cv);
    return hipGetLastError();
}

// Caller-supplied centres ([BH][m][D], m = cv.m) copied into slots
// [base, base + m) of every head, each marked as holding a centre. One wave
// per slot.
template <int D>
__global__ __launch_bounds__(256) void caller_init_kernel(const float* __restrict__ init, CentView cv) {
    const int bh = blockIdx.y;
    const int j = blockIdx.x * 4 + (threadIdx.x >> 6), l = threadIdx.x & 63;
    if (j >= cv.m) return;
    const int64_t slot = (int64_t)bh * cv.cap + cv.base + j;
    const int64_t src = ((int64_t)bh * cv.m + j) * D;
#pragma unroll
    for (int e = 0; e < D / 64; ++e) cv.cent[slot * D + l + 64 * e] = init[src + l + 64 * e];
    if (l == 0) cv.valid[slot] = 1;
}

hipError_t launch_caller_init(const Prob& p, const float* init, CentView cv, hipStream_t s) {
    dim3 grid((unsigned)((cv.m + 3) / 4), (unsigned)p.BH);
    if (p.D == 64)
        hipLaunchKernelGGL(caller_init_kernel<64>, grid, dim3(256), 0, s, init, cv);
    else
        hipLaunchKernelGGL(caller_init_kernel<128>, grid, dim3(256), 0, s, init, cv);
    return hipGetLastError();
}

// Slots past the last one holding a centre cannot win an assignment: m_eff =
// min(mcount, last valid slot + 1), one workgroup per head.
__global__ __launch_bounds__(256) void last_valid_kernel(int cap, int m, const uint8_t* __restrict__ valid,
                                                         const int32_t* __restrict__ mcount,
                                                         int32_t* __restrict__ m_eff) {
    __shared__ int red[4];
    const int bh = blockIdx.x;
    const int lim = mcount ? min(mcount[bh], m) : m;
    int last = -1;
    for (int j = threadIdx.x; j < lim; j += 256)
        if (valid[(int64_t)bh * cap + j]) last = j;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) last = max(last, __shfl_xor(last, o));
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = last;
    __syncthreads();
    if (threadIdx.x == 0) m_eff[bh] = max(max(red[0], red[1]), max(red[2], red[3])) + 1;
}

hipError_t launch_last_valid(const Prob& p, CentView cv, const int32_t* mcount, int32_t* m_eff,
                             hipStream_t s) {
    hipLaunchKernelGGL(last_valid_kernel, dim3((unsigned)p.BH), dim3(256), 0, s, cv.cap, cv.m,
                       cv.valid + cv.base, mcount, m_eff);
    return hipGetLastError();
}

// ------------------------------------------------------------------ norms
// 8 lanes per row, each reading 8-element chunks with 16-byte loads; a
// workgroup takes 8 rows per group of 8 lanes (256 rows), every load issued
// before the first product so enough bytes are in flight. Squares summed in
// f64 over each lane's chunks, then over the 8 lanes.
template <typename T>
__global__ __launch_bounds__(256) void inv_norm_kernel(const T* __restrict__ x, int64_t rows,
                                                       int D, float* __restrict__ inv) {
    constexpr int RPG = 8;  // rows per lane group
    const int grp = threadIdx.x >> 3, sub = threadIdx.x & 7;
    const int64_t row0 = (int64_t)blockIdx.x * (32 * RPG) + grp;  // rows row0 + 32 r
    double s[RPG];
#pragma unroll
    for (int r = 0; r < RPG; ++r) s[r] = 0.0;
    for (int j = sub * 8; j < D; j += 64) {
        // rows past the end read the last row (unconditional loads stay in flight
        // together; their sums are not stored)
        float v[RPG][8];
#pragma unroll
        for (int r = 0; r < RPG; ++r) load8<T>(x + min(row0 + 32 * r, rows - 1) * D + j, v[r]);
#pragma unroll
        for (int r = 0; r < RPG; ++r)
#pragma unroll
            for (int i = 0; i < 8; ++i) s[r] += (double)v[r][i] * (double)v[r][i];
    }
#pragma unroll
    for (int r = 0; r < RPG; ++r) {
#pragma unroll
        for (int o = 4; o > 0; o >>= 1) s[r] += __shfl_xor(s[r], o);
        const int64_t row = row0 + 32 * r;
        if (sub == 0 && row < rows) {
            double n = sqrt(s[r]);
            if (n < 1e-12) n = 1e-12;
            inv[row] = (float)(1.0 / n);
        }
    }
}

hipError_t launch_inv_norm(const Prob& p, const void* x, float* inv, hipStream_t s) {
    int64_t rows = (int64_t)p.BH * p.N;
    dim3 grid((unsigned)((rows + 255) / 256));
    if (p.bf16)
        hipLaunchKernelGGL(inv_norm_kernel<u16>, grid, dim3(256), 0, s, (const u16*)x, rows, p.D, inv);
    else
        hipLaunchKernelGGL(inv_norm_kernel<float>, grid, dim3(256), 0, s, (const float*)x, rows, p.D, inv);
    return hipGetLastError();
}

template <typename T>
__global__ __launch_bounds__(256) void normalize_kernel(const T* __restrict__ x, int64_t rows,
                                                        int D, float* __restrict__ out) {
#pragma clang fp contract(off)
    int64_t row = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (row >= rows) return;
    const T* r = x + row * D;
    double n = seq_norm(r, D);
    for (int j = 0; j < D; ++j) out[row * D + j] = (float)((double)elem<T>::load(r, j) / n);
}

hipError_t launch_normalize(const Prob& p, const void* x, float* xhat, hipStream_t s) {
    int64_t rows = (int64_t)p.BH * p.N;
    dim3 grid((unsigned)((rows + 255) / 256));
    if (p.bf16)
        hipLaunchKernelGGL(normalize_kernel<u16>, grid, dim3(256), 0, s, (const u16*)x, rows, p.D, xhat);
    else
        hipLaunchKernelGGL(normalize_kernel<float>, grid, dim3(256), 0, s, (const float*)x, rows, p.D, xhat);
    return hipGetLastError();
}

// ------------------------------------------------------------------ SAMPLE init
// Slot j < min(m, n) takes row floor((j n + r) / m) of the clustered rows (row j
// when n < m), r = draw 0 mod n; slots beyond hold no centre.
template <typename T>
__global__ __launch_bounds__(256) void init_sample_kernel(const T* __restrict__ x, int N, int D,
                                                          int H, int normalize, RowSet rs,
                                                          CentView cv, uint64_t seed,
                                                          uint32_t tensor, uint32_t stage) {
#pragma clang fp contract(off)
    const int bh = blockIdx.y;
    const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
    const int j = blockIdx.x * 4 + w;
    if (rs.active && !rs.active[bh]) return;
    if (j >= cv.m) return;
    const int n = rs.nrows ? rs.nrows[bh] : N;
    const int cm = n < cv.m ? n : cv.m;
    const int64_t slot = (int64_t)bh * cv.cap + cv.base + j;
    float* c = cv.cent + slot * D;
    if (j >= cm) {
        for (int d = l; d < D; d += 64) c[d] = 0.0f;
        if (l == 0) cv.valid[slot] = 0;
        return;
    }
    uint64_t strm = draw_stream(seed, tensor, stage, (uint32_t)(bh / H), (uint32_t)(bh % H));
    uint64_t r = sm64_at(strm, 0) % (uint64_t)n;
    int64_t idx = (n >= cv.m) ? (int64_t)(((uint64_t)j * (uint64_t)n + r) / (uint64_t)cv.m) : j;
    int64_t tok = rs.rows ? rs.rows[(int64_t)bh * N + idx] : idx;
    const T* xr = row_ptr(x, N, D, bh, tok);
    // one coalesced load per lane and 64 elements; the norm as seq_norm (squares
    // summed in index order in f64, floored at 1e-12) from the lanes in order
    float xv[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) xv[e] = l + 64 * e < D ? elem<T>::load(xr, l + 64 * e) : 0.0f;
    double nrm = 1.0;
    if (normalize) {
        double q = 0.0;
        for (int d = 0; d < D; ++d) {
            const double v = (double)__shfl(xv[d >> 6], d & 63);
            q += v * v;
        }
        nrm = sqrt(q);
        nrm = nrm < 1e-12 ? 1e-12 : nrm;
    }
#pragma unroll
    for (int e = 0; e < 2; ++e)
        if (l + 64 * e < D) c[l + 64 * e] = normalize ? (float)((double)xv[e] / nrm) : xv[e];
    if (l == 0) cv.valid[slot] = 1;
}

hipError_t launch_init_sample(const Prob& p, const void* x, int normalize, RowSet rs, CentView cv,
                              uint64_t seed, uint32_t tensor, uint32_t stage, hipStream_t s) {
    dim3 grid((unsigned)((cv.m + 3) / 4), (unsigned)p.BH);
    if (p.bf16)
        hipLaunchKernelGGL(init_sample_kernel<u16>, grid, dim3(256), 0, s, (const u16*)x, p.N, p.D,
                           p.H, normalize, rs, cv, seed, tensor, stage);
    else
        hipLaunchKernelGGL(init_sample_kernel<float>, grid, dim3(256), 0, s, (const float*)x, p.N,
                           p.D, p.H, normalize, rs, cv, seed, tensor, stage);
    return hipGetLastError();
}

// ------------------------------------------------------------------ KMEANSPP init
// D^2 sampling (Arthur and Vassilvitskii 2007), one workgroup per head. The
// chosen rows must follow from the draws exactly, so the running sums of D^2
// are formed by one thread in row order, in f64, as the definition states;
// everything around that chain is parallel. Per round: the workgroup stages
// D^2 through LDS in chunks while thread 0 adds them up, keeping the running
// sum at each chunk start; with u = draw * S the crossing chunk is found from
// those starts and only that chunk is added up again to find the row. The
// D^2 update of every row (index-order f64 sums of squared differences) is
// spread over the workgroup.
constexpr int KPP_THREADS = 1024;
constexpr int KPP_CH = 2048;                 // f64 values per LDS chunk
constexpr int KPP_MAXCH = (1 << 21) / KPP_CH;  // chunks for the largest N
constexpr int KPP_FAST = 4096;  // up to this many rows D^2 and its running sums stay in LDS

template <typename T>
__device__ __forceinline__ void kpp_row(const T* x, const float* xf, int N, int D, int bh, int64_t tok,
                                        float (&v)[8], int d0) {
    if (xf) {
        load8<float>(xf + ((int64_t)bh * N + tok) * D + d0, v);
    } else {
        load8<T>(row_ptr(x, N, D, bh, tok) + d0, v);
    }
}

template <typename T>
__global__ __launch_bounds__(KPP_THREADS) void init_kmeanspp_kernel(const T* __restrict__ x,
                                                                    const float* __restrict__ xf, int N,
                                                                    int D, int H, RowSet rs, CentView cv,
                                                                    uint64_t seed, uint32_t tensor,
                                                                    uint32_t stage, double* __restrict__ d2g,
                                                                    uint8_t* __restrict__ chosen_g) {
#pragma clang fp contract(off)
    __shared__ double chunk[KPP_CH];
    __shared__ double cstart[KPP_MAXCH + 1];
    // n <= KPP_FAST: D^2 of every row and the running sums, in LDS for the whole init
    __shared__ double d2f[KPP_FAST], pre[KPP_FAST];
    __shared__ float cvec[128];
    __shared__ int64_t sh_idx;
    __shared__ int sh_first;
    __shared__ double sh_S;
    const int bh = blockIdx.x;
    const int tid = threadIdx.x;
    if (rs.active && !rs.active[bh]) return;
    const int n = rs.nrows ? rs.nrows[bh] : N;
    const bool fast = n <= KPP_FAST;
    const int cm = n < cv.m ? n : cv.m;
    double* d2 = d2g + (int64_t)bh * N;
    uint8_t* chosen = chosen_g + (int64_t)bh * N;
    for (int i = tid; i < n; i += KPP_THREADS) chosen[i] = 0;
    const uint64_t strm = draw_stream(seed, tensor, stage, (uint32_t)(bh / H), (uint32_t)(bh % H));
    const int nch = (n + KPP_CH - 1) / KPP_CH;
    __syncthreads();
    for (int t = 0; t < cm; ++t) {
        if (t == 0) {
            if (tid == 0) sh_idx = (int64_t)(sm64_at(strm, 0) % (uint64_t)n);
        } else if (fast) {
            // running sums in row order (thread 0, the LDS reads 16 ahead of the
            // adds), each kept; the sums never decrease (D^2 >= 0), so the first
            // row whose sum exceeds u is the number of sums <= u
            if (tid == 0) {
                double run = 0.0;
                int i = 0;
                for (; i + 16 <= n; i += 16) {
                    double v[16];
#pragma unroll
                    for (int j = 0; j < 16; ++j) v[j] = d2f[i + j];
#pragma unroll
                    for (int j = 0; j < 16; ++j) {
                        run += v[j];
                        pre[i + j] = run;
                    }
                }
                for (; i < n; ++i) {
                    run += d2f[i];
                    pre[i] = run;
                }
                sh_S = run;
                sh_first = n;
            }
            __syncthreads();
            const double S = sh_S;
            if (S == 0.0) {
                // the smallest row not chosen yet
                int first = n;
                for (int i = tid; i < n; i += KPP_THREADS)
                    if (!chosen[i]) { first = i; break; }
                atomicMin(&sh_first, first);
                __syncthreads();
                if (tid == 0) sh_idx = sh_first < n ? sh_first : -1;
            } else {
                const double u = (double)(sm64_at(strm, (uint64_t)t) >> 11) * 0x1.0p-53 * S;
                int cnt = 0;
                for (int i = tid; i < n; i += KPP_THREADS) cnt += pre[i] <= u ? 1 : 0;
#pragma unroll
                for (int o = 32; o > 0; o >>= 1) cnt += __shfl_xor(cnt, o);
                __syncthreads();  // every thread has read sh_first above
                if (tid == 0) sh_first = 0;
                __syncthreads();
                if ((tid & 63) == 0) atomicAdd(&sh_first, cnt);
                __syncthreads();
                if (tid == 0) sh_idx = min(sh_first, n - 1);
            }
        } else {
            // running sums in row order, chunk by chunk through LDS
            double run = 0.0;
            for (int c = 0; c < nch; ++c) {
                const int c0 = c * KPP_CH, cn = min(KPP_CH, n - c0);
                for (int i = tid; i < cn; i += KPP_THREADS) chunk[i] = d2[c0 + i];
                __syncthreads();
                if (tid == 0) {
                    cstart[c] = run;
                    // in row order; the LDS reads go out 16 at a time ahead of the adds
                    int i = 0;
                    for (; i + 16 <= cn; i += 16) {
                        double v[16];
#pragma unroll
                        for (int j = 0; j < 16; ++j) v[j] = chunk[i + j];
#pragma unroll
                        for (int j = 0; j < 16; ++j) run += v[j];
                    }
                    for (; i < cn; ++i) run += chunk[i];
                }
                __syncthreads();
            }
            if (tid == 0) cstart[nch] = run;
            __syncthreads();
            const double S = cstart[nch];
            if (S == 0.0) {
                // the smallest row not chosen yet
                if (tid == 0) sh_first = n;
                __syncthreads();
                int first = n;
                for (int i = tid; i < n; i += KPP_THREADS)
                    if (!chosen[i]) { first = i; break; }
                atomicMin(&sh_first, first);
                __syncthreads();
                if (tid == 0) sh_idx = sh_first < n ? sh_first : -1;
            } else {
                const double u = (double)(sm64_at(strm, (uint64_t)t) >> 11) * 0x1.0p-53 * S;
                // the running sum first exceeds u inside the first chunk whose end exceeds u
                int cc = -1;
                if (tid == 0)
                    for (int c = 0; c < nch; ++c)
                        if (cstart[c + 1] > u) { cc = c; break; }
                if (tid == 0) sh_first = cc;
                __syncthreads();
                cc = sh_first;
                if (cc < 0) {
                    if (tid == 0) sh_idx = n - 1;
                } else {
                    const int c0 = cc * KPP_CH, cn = min(KPP_CH, n - c0);
                    for (int i = tid; i < cn; i += KPP_THREADS) chunk[i] = d2[c0 + i];
                    __syncthreads();
                    if (tid == 0) {
                        double r = cstart[cc];
                        int64_t idx = n - 1;
                        bool found = false;
                        int i = 0;
                        // blocks of 16: the running sums of the block (the same
                        // additions in the same order), then its first one above u
                        for (; i + 16 <= cn; i += 16) {
                            double v[16], pr[16];
#pragma unroll
                            for (int j = 0; j < 16; ++j) v[j] = chunk[i + j];
#pragma unroll
                            for (int j = 0; j < 16; ++j) {
                                r += v[j];
                                pr[j] = r;
                            }
                            int hit = -1;
#pragma unroll
                            for (int j = 15; j >= 0; --j)
                                if (pr[j] > u) hit = j;
                            if (hit >= 0) {
                                idx = c0 + i + hit;
                                found = true;
                                break;
                            }
                        }
                        for (; i < cn && !found; ++i) {
                            r += chunk[i];
                            if (r > u) {
                                idx = c0 + i;
                                found = true;
                            }
                        }
                        sh_idx = idx;
                    }
                }
            }
        }
        __syncthreads();
        const int64_t idx = sh_idx;
        if (tid == 0) chosen[idx] = 1;
        const int64_t tok_c = rs.rows ? rs.rows[(int64_t)bh * N + idx] : idx;
        const int64_t slot = (int64_t)bh * cv.cap + cv.base + t;
        for (int d = tid; d < D; d += KPP_THREADS) {
            const float v = xf ? xf[((int64_t)bh * N + tok_c) * D + d]
                               : elem<T>::load(row_ptr(x, N, D, bh, tok_c), d);
            cvec[d] = v;
            cv.cent[slot * D + d] = v;
        }
        if (tid == 0) cv.valid[slot] = 1;
        __syncthreads();
        for (int i = tid; i < n; i += KPP_THREADS) {
            const int64_t tok = rs.rows ? rs.rows[(int64_t)bh * N + i] : i;
            double sacc = 0.0;
            for (int d0 = 0; d0 < D; d0 += 8) {
                float v[8];
                kpp_row<T>(x, xf, N, D, bh, tok, v, d0);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const double df = (double)v[e] - (double)cvec[d0 + e];
                    sacc += df * df;
                }
            }
            if (fast) {
                if (t == 0 || sacc < d2f[i]) d2f[i] = sacc;
            } else if (t == 0 || sacc < d2[i]) {
                d2[i] = sacc;
            }
        }
        __syncthreads();
    }
    for (int j = cm; j < cv.m; ++j) {
        const int64_t slot = (int64_t)bh * cv.cap + cv.base + j;
        for (int d = tid; d < D; d += KPP_THREADS) cv.cent[slot * D + d] = 0.0f;
        if (tid == 0) cv.valid[slot] = 0;
    }
}

hipError_t launch_init_kmeanspp(const Prob& p, const void* x, const float* xf, RowSet rs,
                                CentView cv, uint64_t seed, uint32_t tensor, uint32_t stage,
                                double* d2, uint8_t* chosen, hipStream_t s) {
    if (p.bf16)
        hipLaunchKernelGGL(init_kmeanspp_kernel<u16>, dim3(p.BH), dim3(KPP_THREADS), 0, s, (const u16*)x,
                           xf, p.N, p.D, p.H, rs, cv, seed, tensor, stage, d2, chosen);
    else
        hipLaunchKernelGGL(init_kmeanspp_kernel<float>, dim3(p.BH), dim3(KPP_THREADS), 0, s,
                           (const float*)x, xf, p.N, p.D, p.H, rs, cv, seed, tensor, stage, d2,
                           chosen);
    return hipGetLastError();
}

// ------------------------------------------------------------------ finalize / prep
// Sixteen lanes per slot, four slots per wave (lane L of a group holds
// dimensions 4L .. 4L + 3, and 64 + 4L .. 67 + 4L at D = 128, as 16-byte
// accesses): optional move to the member mean, then bf16 hi/lo split and the
// squared norm (+inf where the slot holds no centre). The members of slot j
// are the sorted rows [soff[j], soff[j + 1]); their sum is in sums[j] when one
// wave of the update covered them all, else it is the end part of the first
// wave plus the start parts of the later ones, added in wave order. The f64
// norms and drifts are summed in a fixed order (each lane's dimensions, then
// the group's lanes by a butterfly).
constexpr int FIN_LANES = 16;
template <int D>
__global__ __launch_bounds__(256) void finalize_kernel(CentView cv, const uint8_t* active,
                                                       const int32_t* __restrict__ soff, float* drift,
                                                       int32_t* zero_a, int32_t* zero_b, int32_t* zero_c,
                                                       float* __restrict__ rad,
                                                       const float* __restrict__ part_rad) {
    constexpr int E = D / 64;  // float4 chunks per lane
    const int bh = blockIdx.y;
    const int l = threadIdx.x & (FIN_LANES - 1);
    const int j = blockIdx.x * (256 / FIN_LANES) + (threadIdx.x / FIN_LANES);
    if (active && !active[bh]) return;
    if (j >= cv.m) return;
    if (j == 0 && l == 0) {
        // per-head counters of the next round (flag lists, rows to redo), so that
        // no separate clearing launch sits between the rounds
        if (zero_a) zero_a[bh] = 0;
        if (zero_b) zero_b[bh] = 0;
        if (zero_c) zero_c[bh] = 0;
    }
    const int64_t slot = (int64_t)bh * cv.cap + cv.base + j;
    float* c = cv.cent + slot * D;
    auto group_sum = [](double v) {
#pragma unroll
        for (int o = 1; o < FIN_LANES; o <<= 1) v += __shfl_xor(v, o);
        return v;
    };
    float4 cur[E];
#pragma unroll
    for (int e = 0; e < E; ++e) cur[e] = *reinterpret_cast<const float4*>(c + 64 * e + 4 * l);
    if (soff) {
        const int32_t* so = soff + (int64_t)bh * (cv.m + 1);
        const int s0 = so[j], s1 = so[j + 1];
        const int n = s1 - s0;
        double dd = 0.0;
        if (n > 0) {
            const int w1 = s0 >> 6, w2 = (s1 - 1) >> 6;
            float4 acc[E];
            if (w1 == w2) {
#pragma unroll
                for (int e = 0; e < E; ++e)
                    acc[e] = *reinterpret_cast<const float4*>(cv.sums + slot * D + 64 * e + 4 * l);
            } else {
                const float* pb = cv.part + (int64_t)bh * cv.nwav * 2 * D;
#pragma unroll
                for (int e = 0; e < E; ++e)
                    acc[e] = *reinterpret_cast<const float4*>(pb + ((int64_t)w1 * 2 + 1) * D + 64 * e + 4 * l);
                for (int ww = w1 + 1; ww <= w2; ++ww)
#pragma unroll
                    for (int e = 0; e < E; ++e) {
                        const float4 q = *reinterpret_cast<const float4*>(pb + ((int64_t)ww * 2) * D + 64 * e + 4 * l);
                        acc[e].x += q.x;
                        acc[e].y += q.y;
                        acc[e].z += q.z;
                        acc[e].w += q.w;
                    }
                if (rad && l == 0) {
                    // the radius of a cluster over several update waves: the largest part
                    const float* pr = part_rad + (int64_t)bh * cv.nwav * 2;
                    float r = pr[(int64_t)w1 * 2 + 1];
                    for (int ww = w1 + 1; ww <= w2; ++ww) r = fmaxf(r, pr[(int64_t)ww * 2]);
                    rad[slot] = r;
                }
            }
            const float fn = (float)n;
#pragma unroll
            for (int e = 0; e < E; ++e) {
                const float nv[4] = {acc[e].x / fn, acc[e].y / fn, acc[e].z / fn, acc[e].w / fn};
                const float ov[4] = {cur[e].x, cur[e].y, cur[e].z, cur[e].w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const double df = (double)(nv[i] - ov[i]);
                    dd += df * df;
                }
                cur[e] = make_float4(nv[0], nv[1], nv[2], nv[3]);
                *reinterpret_cast<float4*>(c + 64 * e + 4 * l) = cur[e];
            }
        } else if (rad && l == 0) {
            rad[slot] = 0.0f;
        }
        if (drift) {
            // ||new - old|| from the f32 differences (each within 2^-24 of
            // itself), rounded up by a margin
            dd = group_sum(dd);
            if (l == 0) drift[slot] = cv.valid[slot] ? (float)sqrt(dd) * (1.0f + 0x1.0p-20f) : 0.0f;
        }
    }
    double ss = 0.0;
#pragma unroll
    for (int e = 0; e < E; ++e) {
        const float v[4] = {cur[e].x, cur[e].y, cur[e].z, cur[e].w};
        u16 h[4], lo[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            h[i] = f2bf_bits(v[i]);
            lo[i] = f2bf_bits(v[i] - bf_bits2f(h[i]));
            ss += (double)v[i] * (double)v[i];
        }
        *reinterpret_cast<uint2*>(cv.c_hi + slot * D + 64 * e + 4 * l) =
            make_uint2((uint32_t)h[0] | ((uint32_t)h[1] << 16), (uint32_t)h[2] | ((uint32_t)h[3] << 16));
        *reinterpret_cast<uint2*>(cv.c_lo + slot * D + 64 * e + 4 * l) =
            make_uint2((uint32_t)lo[0] | ((uint32_t)lo[1] << 16), (uint32_t)lo[2] | ((uint32_t)lo[3] << 16));
    }
    ss = group_sum(ss);
    if (l == 0) cv.cn2[slot] = cv.valid[slot] ? (float)ss : INFINITY;
}

hipError_t launch_finalize(const Prob& p, CentView cv, const uint8_t* active, const int32_t* soff,
                           hipStream_t s, float* drift, int32_t* zero_a, int32_t* zero_b,
                           int32_t* zero_c, float* rad, const float* part_rad) {
    constexpr int SPB = 256 / FIN_LANES;  // slots per workgroup
    dim3 grid((unsigned)((cv.m + SPB - 1) / SPB), (unsigned)p.BH);
    if (p.D == 64)
        hipLaunchKernelGGL(finalize_kernel<64>, grid, dim3(256), 0, s, cv, active, soff, drift,
                           zero_a, zero_b, zero_c, rad, part_rad);
    else
        hipLaunchKernelGGL(finalize_kernel<128>, grid, dim3(256), 0, s, cv, active, soff, drift,
                           zero_a, zero_b, zero_c, rad, part_rad);
    return hipGetLastError();
}

// ------------------------------------------------------------------ pruned assignment
// Pairwise centre distances on the matrix cores: a workgroup takes 64 slots
// a (16 per wave, as the B operand) against every tile of 64 slots j (the A
// operand, staged in LDS), with the bf16 hi/lo parts finalize keeps:
// G = hi_j.hi_a + lo_j.hi_a + hi_j.lo_a, ||c_j - c_a||^2 = ||c_j||^2 +
// ||c_a||^2 - 2 G. The dropped lo.lo term, the hi/lo residuals and the f32
// accumulation stay below 2^-15 ||c_a|| ||c_j||, the roundings of the sum
// below 2^-21 (||c_a||^2 + ||c_j||^2), so subtracting 2^-13 (||c_a||^2 +
// ||c_j||^2) gives a lower bound: j joins a's set when that bound is at most
// (2 R)^2 (1 + 2^-12) with R rounded up, so every slot the lemma does not
// exclude is kept. Slots without a centre join no set and have none; only the
// words of slots below the count are written (and read). The tiles j are split
// over gridDim.z workgroups (each writes its own words), so that a head's few
// 64-slot blocks a still give the chip enough workgroups.
template <int D>
__global__ __launch_bounds__(256) void cand_bits_kernel(CentView cv, const int32_t* __restrict__ mcount,
                                                        const float* __restrict__ rad,
                                                        const float* __restrict__ drift,
                                                        uint32_t* __restrict__ cbits, int cwords, int am) {
    constexpr int KC = D / 32;
    constexpr int LD = D + 8;
    __shared__ __attribute__((aligned(16))) u16 sh_hi[64 * LD];
    __shared__ __attribute__((aligned(16))) u16 sh_lo[64 * LD];
    __shared__ float sh_n2[64];
    const int bh = blockIdx.y;
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, g = l >> 4, c16 = l & 15;
    const int M = mcount ? min(mcount[bh], cv.m) : cv.m;
    const int MA = min(M, am);  // slots that get a set
    const int a0 = blockIdx.x * 64;
    if (a0 >= MA) return;  // no row carries these labels
    const int64_t sbase = (int64_t)bh * cv.cap + cv.base;
    const int a = a0 + w * 16 + c16;
    const int ac = min(a, MA - 1);
    bf16x8 ah[KC], al[KC];
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
        ah[kc] = ld_bf16x8(cv.c_hi + (sbase + ac) * D + kc * 32 + g * 8);
        al[kc] = ld_bf16x8(cv.c_lo + (sbase + ac) * D + kc * 32 + g * 8);
    }
    const int jtiles = ((M + 63) / 64 + gridDim.z - 1) / gridDim.z;
    const int jb0 = blockIdx.z * jtiles * 64, jb1 = min(M, jb0 + jtiles * 64);
    if (jb0 >= jb1) return;
    const float na2 = cv.cn2[sbase + ac];
    float lim = -INFINITY;  // no set for slots without a centre or past the count
    if (a < MA && na2 < INFINITY) {
        const float R = (rad[sbase + a] + (drift ? drift[sbase + a] : 0.0f)) * (1.0f + 0x1.0p-20f);
        lim = 4.0f * R * R * (1.0f + 0x1.0p-12f);
    }
    for (int j0 = jb0; j0 < jb1; j0 += 64) {
        __syncthreads();
        for (int i = tid; i < 64 * (D / 8); i += 256) {
            const int r = i / (D / 8), c = (i % (D / 8)) * 8;
            const int64_t j = sbase + min(j0 + r, M - 1);
            *reinterpret_cast<u32x4*>(&sh_hi[r * LD + c]) = *reinterpret_cast<const u32x4*>(cv.c_hi + j * D + c);
            *reinterpret_cast<u32x4*>(&sh_lo[r * LD + c]) = *reinterpret_cast<const u32x4*>(cv.c_lo + j * D + c);
        }
        if (tid < 64) sh_n2[tid] = j0 + tid < M ? cv.cn2[sbase + j0 + tid] : INFINITY;
        __syncthreads();
        uint32_t bits[2] = {0u, 0u};
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kc = 0; kc < KC; ++kc) {
                const int off = (cb * 16 + c16) * LD + kc * 32 + g * 8;
                const bf16x8 jh = *reinterpret_cast<const bf16x8*>(&sh_hi[off]);
                const bf16x8 jl = *reinterpret_cast<const bf16x8*>(&sh_lo[off]);
                acc = mfma16(jh, ah[kc], acc);
                acc = mfma16(jl, ah[kc], acc);
                acc = mfma16(jh, al[kc], acc);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float nj2 = sh_n2[cb * 16 + g * 4 + i];  // +inf: no centre, never kept
                const float s2 = (na2 + nj2) - 2.0f * acc[i];
                const bool keep = nj2 < INFINITY && s2 - 0x1.0p-13f * (na2 + nj2) <= lim;
                const int jb = cb * 16 + g * 4 + i;  // position in the tile
                bits[jb >> 5] |= (uint32_t)keep << (jb & 31);
            }
        }
        // the four lanes holding column c16 cover disjoint bits: OR them together
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            bits[h] |= __shfl_xor(bits[h], 16);
            bits[h] |= __shfl_xor(bits[h], 32);
        }
        const int wd = (j0 >> 5) + (g & 1);
        if (g < 2 && a < MA && wd < cwords) cbits[(sbase + a) * cwords + wd] = bits[g & 1];
    }
}

hipError_t launch_cand_bits(const Prob& p, CentView cv, const int32_t* mcount, const float* rad,
                            const float* drift, uint32_t* cbits, int cwords, hipStream_t s, int am) {
    if (am < 0 || am > cv.m) am = cv.m;
    if (am == 0) return hipSuccess;
    // split the j tiles so that the grid has about 2048 workgroups (at most 8 splits)
    const int ablocks = (am + 63) / 64;
    const int js = std::max(1, std::min(8, (2048 + ablocks * p.BH - 1) / (ablocks * p.BH)));
    dim3 grid((unsigned)ablocks, (unsigned)p.BH, (unsigned)js);
    if (p.D == 64)
        hipLaunchKernelGGL(cand_bits_kernel<64>, grid, dim3(256), 0, s, cv, mcount, rad, drift, cbits, cwords, am);
    else
        hipLaunchKernelGGL(cand_bits_kernel<128>, grid, dim3(256), 0, s, cv, mcount, rad, drift, cbits, cwords, am);
    return hipGetLastError();
}

// Triangle inequality: the new distance to the row's centre is at most
// ub + drift[label], and to any other centre at least lb - max drift, so
// ub' < lb' keeps the label strictly nearest (the f32 sums and differences are
// rounded outward by 2^-22 of themselves). A workgroup takes 2048 rows (8 per
// thread), finds the largest drift of its head itself and appends its rows to
// redo in row order with one atomic (same-address atomics cost about 0.3 us
// each, so one per wave would dominate).
constexpr int BF_ROWS = 8;
__global__ __launch_bounds__(256) void bound_filter_kernel(int N, RowSet rs, CentView cv,
                                                           const int32_t* __restrict__ labels,
                                                           float* __restrict__ ub, float* __restrict__ lb,
                                                           const float* __restrict__ drift,
                                                           int32_t* __restrict__ rlist,
                                                           int32_t* __restrict__ rcount) {
    __shared__ float sh_m[4];
    __shared__ int sh_c[4 * BF_ROWS];
    __shared__ int sh_base;
    const int bh = blockIdx.y;
    if (rs.active && !rs.active[bh]) return;
    const int n = rs.nrows ? rs.nrows[bh] : N;
    const int r0 = blockIdx.x * 256 * BF_ROWS;
    if (r0 >= n) return;
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
    const float* dr = drift + (int64_t)bh * cv.cap + cv.base;
    float dm = 0.0f;
    for (int j = tid; j < cv.m; j += 256) {
        const float v = dr[j];
        dm = fmaxf(dm, v == v ? v : INFINITY);  // a NaN drift disables the test
    }
    dm = wave_max(dm);
    if (lane == 0) sh_m[w] = dm;
    __syncthreads();
    dm = fmaxf(fmaxf(sh_m[0], sh_m[1]), fmaxf(sh_m[2], sh_m[3]));
    uint64_t masks[BF_ROWS];
#pragma unroll
    for (int i = 0; i < BF_ROWS; ++i) {
        const int r = r0 + i * 256 + tid;
        bool redo = false;
        if (r < n) {
            const int64_t ix = (int64_t)bh * N + r;
            const float u = (ub[ix] + dr[labels[ix]]) * (1.0f + 0x1.0p-22f);
            const float lo = (lb[ix] - dm) * (1.0f - 0x1.0p-22f);
            if (u < lo) {
                ub[ix] = u;
                lb[ix] = lo;
            } else {
                redo = true;
            }
        }
        masks[i] = __ballot(redo);
        if (lane == 0) sh_c[i * 4 + w] = __popcll(masks[i]);
    }
    __syncthreads();
    if (tid == 0) {
        int tot = 0;
        for (int c = 0; c < 4 * BF_ROWS; ++c) {
            const int v = sh_c[c];
            sh_c[c] = tot;
            tot += v;
        }
        sh_base = tot ? atomicAdd(&rcount[bh], tot) : 0;
    }
    __syncthreads();
    const int base = sh_base;
    const uint64_t below = (1ull << lane) - 1ull;
#pragma unroll
    for (int i = 0; i < BF_ROWS; ++i)
        if ((masks[i] >> lane) & 1ull)
            rlist[(int64_t)bh * N + base + sh_c[i * 4 + w] + __popcll(masks[i] & below)] = r0 + i * 256 + tid;
}

hipError_t launch_bound_filter(const Prob& p, RowSet rs, CentView cv, const int32_t* labels,
                               float* ub, float* lb, const float* drift, int32_t* rlist,
                               int32_t* rcount, hipStream_t s) {
    dim3 grid((unsigned)((p.N + 256 * BF_ROWS - 1) / (256 * BF_ROWS)), (unsigned)p.BH);
    hipLaunchKernelGGL(bound_filter_kernel, grid, dim3(256), 0, s, p.N, rs, cv, labels, ub, lb, drift,
                       rlist, rcount);
    return hipGetLastError();
}

// ------------------------------------------------------------------ assignment
// Workgroup = 4 waves x 64 rows. The centres stream through LDS in tiles of 64
// (bf16 hi and lo parts, double-buffered, the next tile loaded while the
// current one is contracted); each wave computes S^T = C . X^T with 16x16x32
// bf16 MFMAs (rows of the MFMA = centres, columns = points), so a lane owns
// one point per 16-point block and 16 centres per tile. For each centre it
// forms
//   d'_j = ||c_j||^2 + B - 2 s (x . c_j)      (s = 1 / ||x|| for queries, else 1)
// with a per-workgroup offset B that makes every d' positive, and keeps the
// smallest and second-smallest sort keys of d' (bits of d' with the centre's
// position in the tile in the 4 low mantissa bits; 4 VALU ops per distance).
// The contraction error of one d' is at most err = ERR_X s||x|| max||c|| +
// ERR_C max||c||^2 + 2^-22 (max||c||^2 + B + 2 s||x|| max||c||) (hi/lo residual,
// f32 accumulation, rounding of ||c||^2 + B and of the final fma, with margin),
// and the key moves a value by less than 2^-19 of itself. A row whose best two
// keys are not separated by 2 err + 2^-17 d2 is flagged, with the band edge
// thr = best - B + 3 err + 2^-17 best (in units of ||c||^2 - 2 s x.c).
//
// CAND mode runs the same contraction over the flagged rows only, without the
// offset, and appends every centre with ||c_j||^2 - 2 s x.c_j <= thr to the
// row's candidate list; the centre tiles are split over gridDim.z workgroups.
// The exact nearest centre is among the candidates, so exact f64 distances of
// the candidates decide the label (cand_exact_kernel); a row with no or more
// than CAND_CAP candidates goes to the full exact scan (launch_refine).
// The row and the centre are read 16 elements at a time with 16-byte loads (a
// few in flight per chunk instead of one dependent load per element); the f64
// arithmetic is the definition's, in index order.
template <typename T, int D>
__device__ double exact_d2(const T* xr, int normalize, const float* c) {
#pragma clang fp contract(off)
    constexpr int CH = 16;
    double nrm = 1.0;
    if (normalize) {
        // ||x|| as seq_norm: squares summed in index order in f64, floored at 1e-12
        double q = 0.0;
#pragma unroll 1
        for (int k = 0; k < D; k += CH) {
            float a[8], b[8];
            load8<T>(xr + k, a);
            load8<T>(xr + k + 8, b);
#pragma unroll
            for (int i = 0; i < 8; ++i) q += (double)a[i] * (double)a[i];
#pragma unroll
            for (int i = 0; i < 8; ++i) q += (double)b[i] * (double)b[i];
        }
        nrm = sqrt(q);
        nrm = nrm < 1e-12 ? 1e-12 : nrm;
    }
    double s = 0.0;
#pragma unroll 1
    for (int k = 0; k < D; k += CH) {
        float xv[CH], cv[CH];
        load8<T>(xr + k, *reinterpret_cast<float(*)[8]>(&xv[0]));
        load8<T>(xr + k + 8, *reinterpret_cast<float(*)[8]>(&xv[8]));
        load8<float>(c + k, *reinterpret_cast<float(*)[8]>(&cv[0]));
        load8<float>(c + k + 8, *reinterpret_cast<float(*)[8]>(&cv[8]));
#pragma unroll
        for (int i = 0; i < CH; ++i) {
            const float xh = normalize ? (float)((double)xv[i] / nrm) : xv[i];
            const double df = (double)xh - (double)cv[i];
            s += df * df;
        }
    }
    return s;
}

// Sort key of one distance for the running minimum: d' >= 0 (see below), so
// its bit pattern orders as an unsigned integer; the 4 low mantissa bits are
// replaced by the position of the centre among the lane's 16 in the tile.
__device__ __forceinline__ uint32_t dist_key(float d, uint32_t pos) {
    return (__float_as_uint(d) & ~15u) | pos;
}
// Second smallest of {a, b, c} given a <= b: the median.
__device__ __forceinline__ uint32_t med3_u32(uint32_t a, uint32_t b, uint32_t c) {
    uint32_t r;
    asm("v_med3_u32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
    return r;
}

// Settles one row from its best and second-best sort keys (merged over lanes,
// or over centre-tile splits): label, flag list entry, distance bounds.
template <bool FOLD, bool F32X>
__device__ __forceinline__ void assign_settle(uint32_t k1, uint32_t k2, int bj, float xn, float c2max,
                                              float bwg, int bh, int N, int rr, const RowSet& rs,
                                              int32_t* __restrict__ labels, const FlagSet& fs) {
    constexpr float ERR_X = F32X ? 0x1.0p-12f : 0x1.0p-13f;
    constexpr float ERR_C = 0x1.0p-21f;
    const float cmax = sqrtf(c2max);
    // keys are d' >= 0, or (FOLD) -d'/2 < 0; +-inf and NaN are not finite
    auto fin = [](uint32_t k) { return FOLD ? (k >= 0x80000000u && k < 0xff800000u) : k < 0x7f800000u; };
    auto dec = [](uint32_t k) { return FOLD ? -2.0f * __uint_as_float(k) : __uint_as_float(k); };
    const bool finite = fin(k1);
    const int64_t li = (int64_t)bh * N +
                       (rs.by_token ? rs.rows[(int64_t)bh * N + rr] : rr);
    // no finite distance (no centre, or a NaN row): slot 0, and the row is flagged
    labels[li] = finite ? bj : 0;
    const float d1 = dec(k1);
    const float d2 = fin(k2) ? dec(k2) : INFINITY;
    // contraction error of one d' (hi/lo residual and f32 accumulation,
    // plus the rounding of ||c||^2 + B and of the final fma); the key
    // truncation moves a value by less than 2^-19 of itself
    // (FOLD: up to 16 f32 roundings of accumulator values as large as
    // (||c||^2 + B) / 2 + s||x|| ||c||, i.e. 2^-19 of the same sum in d' units)
    const float err = ERR_X * xn * cmax + ERR_C * c2max +
                      (FOLD ? 0x1.0p-19f : 0x1.0p-22f) * (c2max + bwg + 2.0f * xn * cmax);
    const bool settled = finite && d2 - d1 > 2.0f * err + 0x1.0p-17f * d2;
    if (fs.ub) {
        // distance bounds: squared distance = d' - B + (s||x||)^2; every d'
        // within err + 2^-19 d' of the contraction's, (s||x||)^2 within
        // (D + 4) 2^-24 of itself, f32 roundings far below the margin mg
        const float mg = err + 0x1.0p-15f * (c2max + bwg + 2.0f * xn * cmax);
        const float x2 = xn * xn;
        float u = INFINITY, lo = 0.0f;
        if (settled) {
            u = sqrtf(fmaxf((d1 + mg - bwg) + x2 * (1.0f + 0x1.0p-15f), 0.0f)) * (1.0f + 0x1.0p-20f);
            lo = sqrtf(fmaxf((d2 - mg - bwg) + x2 * (1.0f - 0x1.0p-15f), 0.0f)) * (1.0f - 0x1.0p-20f);
        }
        fs.ub[li] = u;
        fs.lb[li] = lo;
    }
    if (!settled) {
        const int fpos = atomicAdd(&fs.count[bh], 1);
        fs.list[(int64_t)bh * N + fpos] = rr;
        fs.ccount[(int64_t)bh * N + fpos] = 0;
        // band edge in the units of ||c||^2 - 2 s x.c (the CAND pass has no B)
        fs.thr[(int64_t)bh * N + fpos] =
            finite ? (d1 - bwg) + 3.0f * err + 0x1.0p-17f * d1 : -INFINITY;
    }
}

// FOLD (rows not rescaled, s = 1; assignment pass only): the MFMA accumulators
// start at -(||c_j||^2 + B) / 2, so they end at a_j = x.c_j - (||c_j||^2 + B) / 2
// = -d'_j / 2 < 0, and the bit patterns of these negative values, read as
// unsigned integers, already order the distances ascending: the fma is
// dropped (3 VALU ops per distance). The accumulator then carries the centre
// term through the f32 accumulation, which the error bound allows for.
// bf16 rows, D = 64: 128 registers at most, four workgroups per CU
//
// GATHER (pruned assignment): the rows come sorted by their current label, so
// a workgroup's 256 rows carry a short range of labels [a0, a1]; the centres
// it contracts with are the union of those labels' candidate sets, gathered
// by index into the same LDS tiles (the union of the bit sets is compacted to
// an index list in slot order; a workgroup whose union passes UCAP takes every
// slot). Every row's nearest centre is in its own label's set, so the argmin,
// the certificate and the row's upper bound are those of the full
// contraction; the lower bound covers only the gathered centres and is not
// used after a pruned round.
#ifndef ADC_CAND_BLOCKS
#define ADC_CAND_BLOCKS 8
#endif
#ifndef ADC_CAND_TPS
#define ADC_CAND_TPS 2
#endif
constexpr int CAND_BLOCKS = ADC_CAND_BLOCKS;  // candidate pass: workgroups per head along the rows
constexpr int CAND_TPS = ADC_CAND_TPS;        // and 64-slot centre tiles per workgroup
template <typename T, int D, bool F32X, bool CAND, bool FOLD, bool GATHER>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(D == 64 && !F32X ? 4 : 1, 8)))
void assign_kernel(const T* __restrict__ X, int N, RowSet rs,
                                                     const float* __restrict__ inv_norm,
                                                     int normalize, CentView cv,
                                                     const int32_t* __restrict__ mcount,
                                                     int32_t* __restrict__ labels, FlagSet fs,
                                                     int tiles_per_split, int32_t* __restrict__ split_rec) {
    constexpr int KC = D / 32;
    constexpr int LD = D + 8;
    __shared__ __attribute__((aligned(16))) u16 sh_hi[2][64 * LD];
    __shared__ __attribute__((aligned(16))) u16 sh_lo[2][64 * LD];
    __shared__ float sh_c2[2][64];
    __shared__ float sh_red[2][4];
    constexpr int UCAP = ucap<D>();
    __shared__ uint16_t ulist[GATHER ? UCAP : 1];

    const int bh = blockIdx.y;
    if (rs.active && !rs.active[bh]) return;
    const int n = CAND ? fs.count[bh] : (rs.nrows ? rs.nrows[bh] : N);
    if ((int)blockIdx.x * 256 >= n) return;
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, g = l >> 4, c16 = l & 15;
    const int M = mcount ? min(mcount[bh], cv.m) : cv.m;
    const int64_t cbase = (int64_t)bh * cv.cap + cv.base;
    const int ntiles_all = (M + 63) / 64;
    const bool tsplit = CAND || split_rec != nullptr;
    const int t_begin = tsplit ? blockIdx.z * tiles_per_split : 0;
    const int t_end = tsplit ? min(ntiles_all, t_begin + tiles_per_split) : ntiles_all;
    if (tsplit && t_begin >= t_end) return;
    // one 256-row block (CAND: a small grid walks the flagged rows' blocks x,
    // x + gridDim.x, ... through the jump at the end; every other pass covers
    // its one block and has no such jump)
    int row_base = blockIdx.x * 256;
[[maybe_unused]] next_block:

    bf16x8 xh[4][KC];
    bf16x8 xl[4][F32X ? KC : 1];
    float sc[4], xn[4], thr[4];
    int rr[4];
    bool ok[4];
#pragma unroll
    for (int pb = 0; pb < 4; ++pb) {
        const int e = row_base + w * 64 + pb * 16 + c16;
        ok[pb] = e < n;
        int r = e;
        thr[pb] = 0.0f;
        if constexpr (CAND) {
            r = ok[pb] ? fs.list[(int64_t)bh * N + e] : 0;
            thr[pb] = ok[pb] ? fs.thr[(int64_t)bh * N + e] : -INFINITY;
        }
        rr[pb] = r;
        int64_t tok = 0;
        if (ok[pb]) tok = rs.rows ? rs.rows[(int64_t)bh * N + r] : r;
        const T* xp = row_ptr(X, N, D, bh, tok);
        float ss = 0.0f;
#pragma unroll
        for (int kc = 0; kc < KC; ++kc) {
            if constexpr (F32X) {
                float v[8];
                if (ok[pb]) {
                    load8<T>(xp + kc * 32 + g * 8, v);
                } else {
#pragma unroll
                    for (int i = 0; i < 8; ++i) v[i] = 0.0f;
                }
#pragma unroll
                for (int i = 0; i < 8; ++i) ss += v[i] * v[i];
                xh[pb][kc] = pack_bf16x8(v);
                float lo[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) lo[i] = v[i] - bf2f(xh[pb][kc][i]);
                xl[pb][kc] = pack_bf16x8(lo);
            } else {
                // bf16 rows are MFMA operands as they stand
                uint4 raw = make_uint4(0u, 0u, 0u, 0u);
                if (ok[pb]) raw = *reinterpret_cast<const uint4*>(xp + kc * 32 + g * 8);
                xh[pb][kc] = __builtin_bit_cast(bf16x8, raw);
                const uint32_t wd[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float a = __uint_as_float(wd[i] << 16), b = __uint_as_float(wd[i] & 0xFFFF0000u);
                    ss += a * a;
                    ss += b * b;
                }
            }
        }
        ss += __shfl_xor(ss, 16);
        ss += __shfl_xor(ss, 32);
        sc[pb] = (inv_norm && ok[pb]) ? inv_norm[(int64_t)bh * N + tok] : 1.0f;
        xn[pb] = sc[pb] * sqrtf(ss);
    }

    // GATHER: the centres of this workgroup (see above); U = -1 means every slot
    int U = -1;
    if constexpr (GATHER) {
        uint32_t* bits = reinterpret_cast<uint32_t*>(&sh_hi[1][0]);  // free until the first tile swap
        const int nwords = (M + 31) / 32;
        const int last = min(row_base + 255, n - 1);
        const int32_t* gl = cv.glab ? cv.glab : labels;
        const int a0 = gl[(int64_t)bh * N + rs.rows[(int64_t)bh * N + row_base]];
        const int a1 = gl[(int64_t)bh * N + rs.rows[(int64_t)bh * N + last]];
        const int64_t sbase = (int64_t)bh * cv.cap + cv.base;
        for (int i = tid; i < nwords; i += 256) {
            uint32_t word = 0u;
            for (int a = a0; a <= a1; ++a) word |= cv.cbits[(sbase + a) * cv.cwords + i];
            bits[i] = word;
        }
        __syncthreads();
        // compaction in slot order: thread i takes words i, i + 256, ...; a wave
        // scan and the four wave totals place them
        int total = 0;
        for (int w0 = 0; w0 < nwords; w0 += 256) {
            const int wi = w0 + tid;
            const uint32_t word = wi < nwords ? bits[wi] : 0u;
            const int cnt = __popc(word);
            int incl = cnt;
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                const int v = __shfl_up(incl, o);
                if (l >= o) incl += v;
            }
            if (l == 63) sh_red[0][w] = __int_as_float(incl);
            __syncthreads();
            int before = total + incl - cnt;
            for (int i = 0; i < w; ++i) before += __float_as_int(sh_red[0][i]);
            int tot = 0;
            for (int i = 0; i < 4; ++i) tot += __float_as_int(sh_red[0][i]);
            uint32_t wd = word;
            while (wd) {
                const int b = __ffs(wd) - 1;
                wd &= wd - 1;
                if (before < UCAP) ulist[before] = (uint16_t)(wi * 32 + b);
                ++before;
            }
            total += tot;
            __syncthreads();
        }
        U = (total > UCAP || total == 0) ? -1 : total;
        __syncthreads();
    }
    const int ntiles_g = U >= 0 ? (U + 63) / 64 : ntiles_all;
    const int t_end_g = GATHER ? ntiles_g : t_end;

    // Assignment pass: d'_j = ||c_j||^2 + B - 2 s (x . c_j) with one offset B per
    // workgroup, B = max_rows (s||x||)^2 + 2^-10 (max_rows s||x|| + max||c||)^2.
    // d'_j - B + (s||x||)^2 is the squared distance, so d' > 0 by a margin far
    // above the contraction error and the argmin is unchanged.
    float c2max = 0.0f, bwg = 0.0f;
    if constexpr (!CAND) {
        float cm = 0.0f, xm = 0.0f;
        for (int j = tid; j < M; j += 256) {
            const float c2 = cv.cn2[cbase + j];
            if (c2 < INFINITY) cm = fmaxf(cm, c2);
        }
#pragma unroll
        for (int pb = 0; pb < 4; ++pb) xm = fmaxf(xm, xn[pb]);
        cm = wave_max(cm);
        xm = wave_max(xm);
        if (l == 0) { sh_red[0][w] = cm; sh_red[1][w] = xm; }
        __syncthreads();
        c2max = fmaxf(fmaxf(sh_red[0][0], sh_red[0][1]), fmaxf(sh_red[0][2], sh_red[0][3]));
        xm = fmaxf(fmaxf(sh_red[1][0], sh_red[1][1]), fmaxf(sh_red[1][2], sh_red[1][3]));
        const float t = xm + sqrtf(c2max);
        bwg = xm * xm + 0x1.0p-10f * t * t;
    }
    float kx[4];
#pragma unroll
    for (int pb = 0; pb < 4; ++pb) kx[pb] = -2.0f * sc[pb];
    uint32_t b1[4], b2[4];
    int tb[4];
#pragma unroll
    for (int pb = 0; pb < 4; ++pb) { b1[pb] = 0xffffffffu; b2[pb] = 0xffffffffu; tb[pb] = 0; }

    // Centre tiles: double-buffered in LDS, the next tile in flight in registers
    // while the current one is contracted. The loads are unconditional, from
    // clamped slots; slots past M get ||c||^2 = +inf.
    u32x4 ph[D / 32], pl[D / 32];
    float pc2;
    // slot of tile position q (GATHER: through the index list)
    auto slot_at = [&](int q) __attribute__((always_inline)) -> int {
        if constexpr (GATHER) {
            if (U >= 0) return ulist[min(q, U - 1)];
        }
        return min(q, M - 1);
    };
    const int lim = (GATHER && U >= 0) ? U : M;  // tile positions that hold a slot
#define ADC_LOAD_TILE(TILE)                                                                  \
    do {                                                                                   \
        _Pragma("unroll") for (int i = 0; i < D / 32; ++i) {                               \
            const int c = tid + i * 256;                                                   \
            const int64_t j = cbase + slot_at((TILE) * 64 + c / (D / 8));                  \
            ph[i] = *reinterpret_cast<const u32x4*>(cv.c_hi + j * D + (c % (D / 8)) * 8); \
            pl[i] = *reinterpret_cast<const u32x4*>(cv.c_lo + j * D + (c % (D / 8)) * 8); \
        }                                                                                  \
        pc2 = cv.cn2[cbase + slot_at((TILE) * 64 + (tid & 63))];                           \
    } while (0)
#define ADC_STORE_TILE(TILE, BUF)                                                          \
    do {                                                                                   \
        _Pragma("unroll") for (int i = 0; i < D / 32; ++i) {                               \
            const int c = tid + i * 256;                                                   \
            const int o = (c / (D / 8)) * LD + (c % (D / 8)) * 8;                          \
            *reinterpret_cast<u32x4*>(&sh_hi[BUF][o]) = ph[i];                             \
            *reinterpret_cast<u32x4*>(&sh_lo[BUF][o]) = pl[i];                             \
        }                                                                                  \
        if (tid < 64)                                                                      \
            sh_c2[BUF][tid] = FOLD ? ((TILE) * 64 + tid < lim ? -0.5f * (pc2 + bwg) : -INFINITY) \
                                   : ((TILE) * 64 + tid < lim ? pc2 + bwg : INFINITY);        \
    } while (0)
    if (t_begin < t_end_g) {
        ADC_LOAD_TILE(t_begin);
        ADC_STORE_TILE(t_begin, 0);
    }
    __syncthreads();

    for (int tile = t_begin; tile < t_end_g; ++tile) {
        const int buf = (tile - t_begin) & 1;
        ADC_LOAD_TILE(min(tile + 1, t_end_g - 1));
        uint32_t prev[4];
#pragma unroll
        for (int pb = 0; pb < 4; ++pb) prev[pb] = b1[pb];
        uint64_t hits = 0;  // CAND: candidates of this tile, bit pb*16 + cb*4 + i
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) {
            const f32x4 c2v = *reinterpret_cast<const f32x4*>(&sh_c2[buf][cb * 16 + g * 4]);
            f32x4 acc[4];
#pragma unroll
            for (int pb = 0; pb < 4; ++pb) acc[pb] = FOLD ? c2v : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kc = 0; kc < KC; ++kc) {
                const int off = (cb * 16 + c16) * LD + kc * 32 + g * 8;
                const bf16x8 ah = *reinterpret_cast<const bf16x8*>(&sh_hi[buf][off]);
                const bf16x8 al = *reinterpret_cast<const bf16x8*>(&sh_lo[buf][off]);
#pragma unroll
                for (int pb = 0; pb < 4; ++pb) {
                    acc[pb] = mfma16(ah, xh[pb][kc], acc[pb]);
                    acc[pb] = mfma16(al, xh[pb][kc], acc[pb]);
                    if constexpr (F32X) acc[pb] = mfma16(ah, xl[pb][kc], acc[pb]);
                }
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
#pragma unroll
                for (int pb = 0; pb < 4; ++pb) {
                    const float dv = FOLD ? acc[pb][i] : fmaf(kx[pb], acc[pb][i], c2v[i]);
                    if constexpr (CAND) {
                        const int j = tile * 64 + cb * 16 + g * 4 + i;
                        if (j < M && dv <= thr[pb]) hits |= 1ull << (pb * 16 + cb * 4 + i);
                    } else {
                        const uint32_t key = dist_key(dv, (uint32_t)(cb * 4 + i));
                        b2[pb] = med3_u32(b1[pb], b2[pb], key);
                        b1[pb] = min(b1[pb], key);
                    }
                }
            }
        }
        if constexpr (!CAND) {
#pragma unroll
            for (int pb = 0; pb < 4; ++pb) tb[pb] = b1[pb] != prev[pb] ? tile : tb[pb];
        } else {
            while (hits) {
                const int bit = __ffsll((unsigned long long)hits) - 1;
                hits &= hits - 1;
                const int pb = bit >> 4, cb = (bit >> 2) & 3, i = bit & 3;
                const int64_t fe = (int64_t)bh * N + row_base + w * 64 + pb * 16 + c16;
                const int pos = atomicAdd(&fs.ccount[fe], 1);
                if (pos < CAND_CAP) fs.cand[fe * CAND_CAP + pos] = tile * 64 + cb * 16 + g * 4 + i;
            }
        }
        ADC_STORE_TILE(tile + 1, buf ^ 1);
        __syncthreads();
    }
#undef ADC_LOAD_TILE
#undef ADC_STORE_TILE

    if constexpr (!CAND) {
#pragma unroll
        for (int pb = 0; pb < 4; ++pb) {
            const uint32_t pos = b1[pb] & 15u;
            int bj = tb[pb] * 64 + (int)(pos >> 2) * 16 + g * 4 + (int)(pos & 3u);
            if constexpr (GATHER) bj = slot_at(bj);
#pragma unroll
            for (int o = 16; o <= 32; o <<= 1) {
                const uint32_t ob1 = __shfl_xor(b1[pb], o);
                const uint32_t ob2 = __shfl_xor(b2[pb], o);
                const int obj = __shfl_xor(bj, o);
                const bool take = ob1 < b1[pb] || (ob1 == b1[pb] && obj < bj);
                b2[pb] = min(max(b1[pb], ob1), min(b2[pb], ob2));
                if (take) { b1[pb] = ob1; bj = obj; }
            }
            if (g == 0 && ok[pb]) {
                if (split_rec) {
                    // centre-tile split: this split's best two keys, merged by assign_merge_kernel
                    const int64_t P = (int64_t)gridDim.y * N, e = (int64_t)bh * N + rr[pb];
                    const int z = blockIdx.z, S = gridDim.z;
                    split_rec[(3 * z) * P + e] = (int32_t)b1[pb];
                    split_rec[(3 * z + 1) * P + e] = (int32_t)b2[pb];
                    split_rec[(3 * z + 2) * P + e] = bj;
                    if (z == 0) {
                        split_rec[(3 * S) * P + e] = __float_as_int(xn[pb]);
                        split_rec[(3 * S + 1) * P + e] = __float_as_int(bwg);
                        split_rec[(3 * S + 2) * P + e] = __float_as_int(c2max);
                    }
                } else {
                    assign_settle<FOLD, F32X>(b1[pb], b2[pb], bj, xn[pb], c2max, bwg, bh, N, rr[pb], rs,
                                              labels, fs);
                }
            }
        }
    }
    if constexpr (CAND) {
        __syncthreads();  // the next block reuses the LDS tiles
        row_base += (int)gridDim.x * 256;
        if (row_base < n) goto next_block;
    }
}

template <bool CAND, bool FOLD, bool GATHER = false>
static void launch_assign_t(const Prob& p, dim3 grid, const void* x, RowSet rs,
                            const float* inv_norm, int normalize, CentView cv,
                            const int32_t* mcount, int32_t* labels, FlagSet fs, int tps,
                            hipStream_t s, int32_t* rec = nullptr) {
    if (p.bf16) {
        auto k = p.D == 64 ? assign_kernel<u16, 64, false, CAND, FOLD, GATHER>
                           : assign_kernel<u16, 128, false, CAND, FOLD, GATHER>;
        hipLaunchKernelGGL(k, grid, dim3(256), 0, s, (const u16*)x, p.N, rs, inv_norm, normalize, cv,
                           mcount, labels, fs, tps, rec);
    } else {
        auto k = p.D == 64 ? assign_kernel<float, 64, true, CAND, FOLD, GATHER>
                           : assign_kernel<float, 128, true, CAND, FOLD, GATHER>;
        hipLaunchKernelGGL(k, grid, dim3(256), 0, s, (const float*)x, p.N, rs, inv_norm, normalize,
                           cv, mcount, labels, fs, tps, rec);
    }
}

// Labels of the flagged rows from their candidate lists: lane (row, c) computes
// the exact f64 distance (index order, as the definition) to candidate c, and
// the 16 lanes of a row take the minimum, ties to the lowest slot. Rows with no
// or too many candidates go to the full exact scan.
template <typename T, int D>
__global__ __launch_bounds__(256) void cand_exact_kernel(const T* __restrict__ X, int N,
                                                         int normalize, RowSet rs, CentView cv,
                                                         FlagSet fs, int32_t* __restrict__ labels) {
    const int bh = blockIdx.y;
    if (rs.active && !rs.active[bh]) return;
    const int count = fs.count[bh];
    const int w = threadIdx.x >> 6, l = threadIdx.x & 63, ci = l & 15;
    const int64_t cbase = (int64_t)bh * cv.cap + cv.base;
    for (int base = blockIdx.x * 16; base < count; base += gridDim.x * 16) {
        const int e = base + w * 4 + (l >> 4);
        const bool okr = e < count;
        const int64_t fe = (int64_t)bh * N + (okr ? e : 0);
        const int nc = okr ? fs.ccount[fe] : 0;
        const int r = okr ? fs.list[fe] : 0;
        double d = INFINITY;
        int j = 0x7fffffff;
        const int64_t tok = (okr && rs.rows) ? rs.rows[(int64_t)bh * N + r] : r;
        if (okr && nc <= CAND_CAP && ci < nc) {
            j = fs.cand[fe * CAND_CAP + ci];
            d = exact_d2<T, D>(row_ptr(X, N, D, bh, tok), normalize, cv.cent + (cbase + j) * D);
        }
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) {
            const double od = __shfl_xor(d, o);
            const int oj = __shfl_xor(j, o);
            if (od < d || (od == d && oj < j)) { d = od; j = oj; }
        }
        if (okr && ci == 0) {
            if (nc > CAND_CAP || nc == 0) {
                const int pos = atomicAdd(&fs.over_count[bh], 1);
                fs.over[(int64_t)bh * N + pos] = r;
            } else {
                labels[(int64_t)bh * N + (rs.by_token ? tok : r)] = j;
                // an upper bound on the row's distance to its centre (the exact
                // value, rounded up)
                if (fs.ub) fs.ub[(int64_t)bh * N + (rs.by_token ? tok : r)] = (float)sqrt(d) * (1.0f + 0x1.0p-20f);
            }
        }
    }
}

// ------------------------------------------------------------------ exact recheck
// One wave per row: squared distances to every slot holding a centre, summed
// over dimensions in index order in f64 (as the definition), argmin with ties
// to the lowest slot. Used for rows whose uncertainty band holds too many
// centres (degenerate data such as repeated points).
template <typename T, int D>
__global__ __launch_bounds__(256) void refine_kernel(const T* __restrict__ X, int N, int normalize,
                                                     RowSet rs, CentView cv,
                                                     const int32_t* __restrict__ mcount,
                                                     const int32_t* __restrict__ flag_list,
                                                     const int32_t* __restrict__ flag_count,
                                                     int32_t* __restrict__ labels, float* __restrict__ ub) {
#pragma clang fp contract(off)
    __shared__ float xs[4][D];
    const int bh = blockIdx.y;
    if (rs.active && !rs.active[bh]) return;
    const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
    const int cnt = flag_count[bh];
    const int M = mcount ? min(mcount[bh], cv.m) : cv.m;
    const int64_t cbase = (int64_t)bh * cv.cap + cv.base;
    for (int base = blockIdx.x * 4; base < cnt; base += gridDim.x * 4) {
        const int e = base + w;
        const bool live = e < cnt;
        int r = 0;
        int64_t tok = 0;
        if (live) {
            r = flag_list[(int64_t)bh * N + e];
            tok = rs.rows ? rs.rows[(int64_t)bh * N + r] : r;
            const T* xr = row_ptr(X, N, D, bh, tok);
            double nrm = 1.0;
            if (normalize) {
                double v = (l == 0) ? seq_norm(xr, D) : 0.0;
                nrm = __shfl(v, 0);
            }
            for (int d = l; d < D; d += 64) {
                float xv = elem<T>::load(xr, d);
                xs[w][d] = normalize ? (float)((double)xv / nrm) : xv;
            }
        }
        __syncthreads();
        if (live) {
            double best = INFINITY;
            int bj = 0x7fffffff;
            for (int j = l; j < M; j += 64) {
                if (!(cv.cn2[cbase + j] < INFINITY)) continue;
                const float* cp = cv.cent + (cbase + j) * D;
                double s = 0.0;
                for (int d = 0; d < D; ++d) {
                    double df = (double)xs[w][d] - (double)cp[d];
                    s += df * df;
                }
                if (s < best) { best = s; bj = j; }
            }
#pragma unroll
            for (int o = 32; o > 0; o >>= 1) {
                const double ob = __shfl_xor(best, o);
                const int oj = __shfl_xor(bj, o);
                if (ob < best || (ob == best && oj < bj)) { best = ob; bj = oj; }
            }
            if (l == 0 && bj != 0x7fffffff) {
                labels[(int64_t)bh * N + (rs.by_token ? tok : r)] = bj;
                if (ub) ub[(int64_t)bh * N + (rs.by_token ? tok : r)] = (float)sqrt(best) * (1.0f + 0x1.0p-20f);
            }
        }
        __syncthreads();
    }
}

static hipError_t launch_refine_full(const Prob& p, const void* x, int normalize, RowSet rs,
                                     CentView cv, const int32_t* mcount, const int32_t* list,
                                     const int32_t* count, int32_t* labels, float* ub, hipStream_t s) {
    dim3 grid(8u, (unsigned)p.BH);
    if (p.bf16) {
        auto k = p.D == 64 ? refine_kernel<u16, 64> : refine_kernel<u16, 128>;
        hipLaunchKernelGGL(k, grid, dim3(256), 0, s, (const u16*)x, p.N, normalize, rs, cv, mcount,
                           list, count, labels, ub);
    } else {
        auto k = p.D == 64 ? refine_kernel<float, 64> : refine_kernel<float, 128>;
        hipLaunchKernelGGL(k, grid, dim3(256), 0, s, (const float*)x, p.N, normalize, rs, cv, mcount,
                           list, count, labels, ub);
    }
    return hipGetLastError();
}

// One thread per row: merges the best two keys of the centre-tile splits (ties
// to the lowest slot, as across lanes) and settles the row.
template <bool FOLD, bool F32X>
__global__ __launch_bounds__(256) void assign_merge_kernel(int N, RowSet rs, int M, const int32_t* __restrict__ mcount,
                                                           const int32_t* __restrict__ rec,
                                                           int nsplit, int tps, int32_t* __restrict__ labels,
                                                           FlagSet fs) {
    const int bh = blockIdx.y;
    if (rs.active && !rs.active[bh]) return;
    const int n = rs.nrows ? rs.nrows[bh] : N;
    const int e = blockIdx.x * 256 + threadIdx.x;
    if (e >= n) return;
    // the splits that ran: those holding a tile of the head's first M slots
    const int Mh = mcount ? min(mcount[bh], M) : M;
    const int nz = min(nsplit, ((Mh + 63) / 64 + tps - 1) / tps);
    const int64_t P = (int64_t)gridDim.y * N, ix = (int64_t)bh * N + e;
    uint32_t k1 = 0xffffffffu, k2 = 0xffffffffu;
    int bj = 0;
    for (int z = 0; z < nz; ++z) {
        const uint32_t o1 = (uint32_t)rec[(3 * z) * P + ix], o2 = (uint32_t)rec[(3 * z + 1) * P + ix];
        const int oj = rec[(3 * z + 2) * P + ix];
        const bool take = o1 < k1 || (o1 == k1 && oj < bj);
        k2 = min(max(k1, o1), min(k2, o2));
        if (take) { k1 = o1; bj = oj; }
    }
    assign_settle<FOLD, F32X>(k1, k2, bj, __int_as_float(rec[(3 * nsplit) * P + ix]),
                              __int_as_float(rec[(3 * nsplit + 2) * P + ix]),
                              __int_as_float(rec[(3 * nsplit + 1) * P + ix]), bh, N, e, rs, labels, fs);
}

// ------------------------------------------------------------------ fixed points
// Lloyd rounds over a row subset (the later key stages): lact[bh] says whether
// head bh still iterates. A round whose labels all equal the previous round's
// leaves the head at its fixed point (the update would reproduce the centres,
// every later round the labels), so the head's remaining round kernels can
// return at once.
__global__ void conv_init_kernel(int BH, const uint8_t* __restrict__ active, uint8_t* __restrict__ lact,
                                 int32_t* __restrict__ chg) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < BH) {
        lact[i] = active ? active[i] : 1;
        chg[i] = 0;
    }
}

// prev <- labels over the head's rows; with compare, chg[bh] = 1 if any differed
__global__ __launch_bounds__(256) void label_cmp_kernel(int N, RowSet rs, const int32_t* __restrict__ labels,
                                                        int32_t* __restrict__ prev, int32_t* __restrict__ chg,
                                                        int compare) {
    const int bh = blockIdx.y;
    if (rs.active && !rs.active[bh]) return;
    const int n = rs.nrows ? rs.nrows[bh] : N;
    bool diff = false;
    for (int r = blockIdx.x * 256 + threadIdx.x; r < n; r += gridDim.x * 256) {
        const int64_t ix = (int64_t)bh * N + (rs.by_token ? rs.rows[(int64_t)bh * N + r] : r);
        const int lab = labels[ix];
        diff |= compare && prev[ix] != lab;
        prev[ix] = lab;
    }
    if (__ballot(diff) != 0 && (threadIdx.x & 63) == 0) chg[bh] = 1;
}

// after a compared round: a head whose labels did not change stops
__global__ void conv_step_kernel(int BH, uint8_t* __restrict__ lact, int32_t* __restrict__ chg) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < BH) {
        if (lact[i] && chg[i] == 0) lact[i] = 0;
        chg[i] = 0;
    }
}

hipError_t launch_conv_init(const Prob& p, const uint8_t* active, uint8_t* lact, int32_t* chg, hipStream_t s) {
    hipLaunchKernelGGL(conv_init_kernel, dim3((unsigned)((p.BH + 255) / 256)), dim3(256), 0, s, p.BH, active,
                       lact, chg);
    return hipGetLastError();
}

hipError_t launch_conv_round(const Prob& p, RowSet rs, const int32_t* labels, int32_t* prev, uint8_t* lact,
                             int32_t* chg, bool compare, hipStream_t s) {
    const unsigned gx = (unsigned)std::min(32, (p.N + 255) / 256);
    hipLaunchKernelGGL(label_cmp_kernel, dim3(gx, (unsigned)p.BH), dim3(256), 0, s, p.N, rs, labels, prev, chg,
                       compare ? 1 : 0);
    if (compare)
        hipLaunchKernelGGL(conv_step_kernel, dim3((unsigned)((p.BH + 255) / 256)), dim3(256), 0, s, p.BH, lact,
                           chg);
    return hipGetLastError();
}

hipError_t launch_assign(const Prob& p, const void* x, RowSet rs, const float* inv_norm,
                         int normalize, CentView cv, const int32_t* mcount, int32_t* labels,
                         FlagSet fs, hipStream_t s, int split, bool counts_zeroed) {
    hipError_t e = hipSuccess;
    if (!counts_zeroed) {
        hipLaunchKernelGGL(zero2_i32_kernel, dim3((unsigned)((p.BH + 255) / 256)), dim3(256), 0, s,
                           fs.count, fs.over_count, p.BH);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    dim3 grid((unsigned)((p.N + 255) / 256), (unsigned)p.BH);
    const bool fold = !normalize && !inv_norm;  // rows not rescaled: folded assignment pass
    const int tiles_m = (cv.m + 63) / 64;
    if (split > 1 && tiles_m >= 2) {
        // few rows: the centre tiles are split over gridDim.z (at most 4, so the
        // 3 per split + 3 record planes fit in the candidate scratch), the best
        // two keys of every split go to that scratch and a merge settles the rows
        // (with mcount, splits past a head's first mcount slots do not run and
        // the merge leaves them out)
        const int ns = min(split, 4);
        const int tps = (tiles_m + ns - 1) / ns;
        const int nz = (tiles_m + tps - 1) / tps;
        static_assert(3 * 4 + 3 <= CAND_CAP, "split records exceed the candidate scratch");
        dim3 sgrid(grid.x, grid.y, (unsigned)nz);
        if (fold)
            launch_assign_t<false, true>(p, sgrid, x, rs, inv_norm, normalize, cv, mcount, labels, fs, tps, s, fs.cand);
        else
            launch_assign_t<false, false>(p, sgrid, x, rs, inv_norm, normalize, cv, mcount, labels, fs, tps, s, fs.cand);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        auto mk = fold ? (p.bf16 ? assign_merge_kernel<true, false> : assign_merge_kernel<true, true>)
                       : (p.bf16 ? assign_merge_kernel<false, false> : assign_merge_kernel<false, true>);
        hipLaunchKernelGGL(mk, grid, dim3(256), 0, s, p.N, rs, cv.m, mcount, (const int32_t*)fs.cand, nz, tps,
                           labels, fs);
    } else if (cv.cbits) {
        if (fold)
            launch_assign_t<false, true, true>(p, grid, x, rs, inv_norm, normalize, cv, mcount, labels, fs, 0, s);
        else
            launch_assign_t<false, false, true>(p, grid, x, rs, inv_norm, normalize, cv, mcount, labels, fs, 0, s);
    } else if (fold) {
        launch_assign_t<false, true>(p, grid, x, rs, inv_norm, normalize, cv, mcount, labels, fs, 0, s);
    } else {
        launch_assign_t<false, false>(p, grid, x, rs, inv_norm, normalize, cv, mcount, labels, fs, 0, s);
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;
    // candidate pass over every slot (also after a pruned pass): the flagged rows
    // are a few percent, so a grid of CAND_BLOCKS workgroups per head walks their
    // 256-row blocks, and the centre tiles are split CAND_TPS per workgroup
    const int tiles = (cv.m + 63) / 64;
    const int cbx = std::min(CAND_BLOCKS, (p.N + 255) / 256);
    dim3 cgrid((unsigned)cbx, (unsigned)p.BH, (unsigned)((tiles + CAND_TPS - 1) / CAND_TPS));
    launch_assign_t<true, false>(p, cgrid, x, rs, inv_norm, normalize, cv, mcount, labels, fs, CAND_TPS, s);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    // 16 flagged rows per workgroup step; 128 workgroups per head take the usual
    // 1-3 % of the rows in one step each
    const dim3 egrid(128, (unsigned)p.BH);
    if (p.bf16) {
        auto k = p.D == 64 ? cand_exact_kernel<u16, 64> : cand_exact_kernel<u16, 128>;
        hipLaunchKernelGGL(k, egrid, dim3(256), 0, s, (const u16*)x, p.N, normalize, rs, cv, fs, labels);
    } else {
        auto k = p.D == 64 ? cand_exact_kernel<float, 64> : cand_exact_kernel<float, 128>;
        hipLaunchKernelGGL(k, egrid, dim3(256), 0, s, (const float*)x, p.N, normalize, rs, cv, fs, labels);
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;
    return launch_refine_full(p, x, normalize, rs, cv, mcount, fs.over, fs.over_count, labels, fs.ub, s);
}

// ------------------------------------------------------------------ update
// Wave W takes the sorted rows [64 W, 64 W + 64): it stages them in LDS (RS
// rows at a time) with coalesced 16-byte loads, all in flight at once, then
// walks them with one lane per dimension, summing each run of equal labels in
// row order. A run is a whole cluster unless it touches the start of the range
// with the cluster begun in the wave before (its sum goes to part[W][0]) or
// the end of the range with the cluster going on in the next wave
// (part[W][1]); whole clusters are stored to sums. Every value has one
// writer, so the sums do not depend on scheduling.
// With ub (by token; may be null) the same walk also takes the largest ub of
// each run: rad[slot] for whole clusters, part radii beside the part sums.
// LOOP (row lists whose size is on the device: the keys left in U, a few
// percent of N): a capped grid whose waves walk W, W + 4 gridDim.x, ...
constexpr int UPDATE_LOOP_BLOCKS = 32;
template <typename T, int D, bool LOOP = false>
__global__ __launch_bounds__(256) void update_accum_kernel(const T* __restrict__ X, int N, RowSet rs,
                                                           const float* __restrict__ inv_norm,
                                                           const int32_t* __restrict__ labels,
                                                           CentView cv,
                                                           const int32_t* __restrict__ order,
                                                           const float* __restrict__ ub,
                                                           float* __restrict__ rad,
                                                           float* __restrict__ part_rad) {
    constexpr int E = D / 64;
    constexpr int RS = 32;                         // rows staged at once (two batches per wave)
    constexpr int LDX = D + 16 / (int)sizeof(T);   // padded row stride (elements)
    constexpr int CPR = D / 8;                     // 8-element chunks per row
    constexpr int RPI = 64 / CPR;                  // rows per wave instruction
    constexpr int W8 = (int)sizeof(T) / 2;         // 16-byte words per 8-element chunk
    __shared__ __attribute__((aligned(16))) T xs[4][RS * LDX];
    const int bh = blockIdx.y;
    if (rs.active && !rs.active[bh]) return;
    const int n = rs.nrows ? rs.nrows[bh] : N;
    const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
    auto range = [&](const int wv) __attribute__((always_inline)) {  // wave range W = wv
    const int base = wv * 64;
    const int32_t* ord = order + (int64_t)bh * N;
    const int32_t* lab_h = labels + (int64_t)bh * N;
    const int r0 = base + l;
    const bool okr = r0 < n;
    const int r = okr ? ord[r0] : 0;
    const int lab_l = okr ? lab_h[r] : -1;
    const int tok_l = okr ? (rs.rows ? rs.rows[(int64_t)bh * N + r] : r) : 0;
    const float s_l = (inv_norm && okr) ? inv_norm[(int64_t)bh * N + tok_l] : 1.0f;
    const float u_l = (ub && okr) ? ub[(int64_t)bh * N + tok_l] : 0.0f;
    const int rows_here = min(64, n - base);
    // labels of the sorted rows just before and just after the range
    const int lab_prev = base > 0 ? lab_h[ord[base - 1]] : -1;
    const int lab_next = base + 64 < n ? lab_h[ord[base + 64]] : -1;
    const int64_t cbase = (int64_t)bh * cv.cap + cv.base;
    float* pw = cv.part + ((int64_t)bh * cv.nwav + wv) * 2 * D;
    T* xw = xs[w];
    float acc[E];
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] = 0.0f;
    int cur = -1;
    bool cur_lead = false;
    float umax = 0.0f;  // largest ub of the current run (lane 0's copy is used)
    auto flush = [&](bool trail) __attribute__((always_inline)) {
        float* dst = cur_lead ? pw : (trail ? pw + D : cv.sums + (cbase + cur) * D);
#pragma unroll
        for (int e = 0; e < E; ++e) dst[l + 64 * e] = acc[e];
        if (ub && l == 0) {
            float* rd = cur_lead ? part_rad + ((int64_t)bh * cv.nwav + wv) * 2
                                 : (trail ? part_rad + ((int64_t)bh * cv.nwav + wv) * 2 + 1 : rad + cbase + cur);
            *rd = umax;
        }
    };
    // the rows of the next batch are loaded into registers while the current
    // batch is walked; chunk c of row q goes to lane (q % RPI) * CPR + c, and
    // rows past the end read row 0
    u32x4 pre[RS / RPI][W8];
    auto load_batch = [&](int h0) __attribute__((always_inline)) {
#pragma unroll
        for (int it = 0; it < RS / RPI; ++it) {
            const int q = it * RPI + l / CPR, c = l % CPR;
            const int tok = __shfl(tok_l, h0 + q);
            const T* src = row_ptr(X, N, D, bh, tok) + c * 8;
#pragma unroll
            for (int k = 0; k < W8; ++k) pre[it][k] = *reinterpret_cast<const u32x4*>(src + 4 * k);
        }
    };
    load_batch(0);
    for (int h0 = 0; h0 < rows_here; h0 += RS) {
#pragma unroll
        for (int it = 0; it < RS / RPI; ++it) {
            const int q = it * RPI + l / CPR, c = l % CPR;
#pragma unroll
            for (int k = 0; k < W8; ++k) *reinterpret_cast<u32x4*>(&xw[q * LDX + c * 8 + 4 * k]) = pre[it][k];
        }
        if (h0 + RS < rows_here) load_batch(h0 + RS);
        // lanes read rows other lanes wrote
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        const int qend = min(RS, rows_here - h0);
        for (int q = 0; q < qend; ++q) {
            const int lab = __builtin_amdgcn_readlane(lab_l, h0 + q);
            const float s = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(s_l), h0 + q));
            if (lab != cur) {
                if (cur >= 0) flush(false);
                cur = lab;
                cur_lead = h0 + q == 0 && lab == lab_prev;
                umax = 0.0f;
#pragma unroll
                for (int e = 0; e < E; ++e) acc[e] = 0.0f;
            }
            if (ub) umax = fmaxf(umax, __int_as_float(__builtin_amdgcn_readlane(__float_as_int(u_l), h0 + q)));
#pragma unroll
            for (int e = 0; e < E; ++e) acc[e] += s * elem<T>::load(xw, q * LDX + l + 64 * e);
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
    if (cur >= 0) flush(rows_here == 64 && cur == lab_next);
    };
    if constexpr (LOOP) {
        for (int wv = blockIdx.x * 4 + w; wv * 64 < n; wv += gridDim.x * 4) range(wv);
    } else {
        const int wv = blockIdx.x * 4 + w;
        if (wv * 64 < n) range(wv);
    }
}

hipError_t launch_update_accum(const Prob& p, const void* x, RowSet rs, const float* inv_norm,
                               const int32_t* labels, CentView cv, const int32_t* order,
                               hipStream_t s, const float* ub, float* rad, float* part_rad) {
    dim3 grid((unsigned)((p.N + 255) / 256), (unsigned)p.BH);
    // a row list with its size on the device walks wave ranges from a capped grid
    const bool subset = rs.rows != nullptr && rs.nrows != nullptr;
    if (subset) grid.x = min(grid.x, (unsigned)UPDATE_LOOP_BLOCKS);
#define ADC_UPD(TT, DD)                                                                                   \
    hipLaunchKernelGGL((subset ? update_accum_kernel<TT, DD, true> : update_accum_kernel<TT, DD, false>), grid, \
                       dim3(256), 0, s, (const TT*)x, p.N, rs, inv_norm, labels, cv, order, ub, rad, part_rad)
    if (p.bf16) {
        if (p.D == 64) ADC_UPD(u16, 64);
        else ADC_UPD(u16, 128);
    } else {
        if (p.D == 64) ADC_UPD(float, 64);
        else ADC_UPD(float, 128);
    }
#undef ADC_UPD
    return hipGetLastError();
}

// ------------------------------------------------------------------ stage records
template <int D>
__global__ __launch_bounds__(256) void copy_slots_kernel(CentView cv, const uint8_t* __restrict__ active,
                                                         float* __restrict__ dst) {
    const int bh = blockIdx.y;
    if (active && !active[bh]) return;
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= (int64_t)cv.m * D) return;
    const int64_t o = ((int64_t)bh * cv.cap + cv.base) * D + i;
    dst[o] = cv.cent[o];
}

hipError_t launch_copy_slots(const Prob& p, CentView cv, const uint8_t* active, float* dst,
                             hipStream_t s) {
    dim3 grid((unsigned)(((int64_t)cv.m * p.D + 255) / 256), (unsigned)p.BH);
    if (p.D == 64)
        hipLaunchKernelGGL(copy_slots_kernel<64>, grid, dim3(256), 0, s, cv, active, dst);
    else
        hipLaunchKernelGGL(copy_slots_kernel<128>, grid, dim3(256), 0, s, cv, active, dst);
    return hipGetLastError();
}

__global__ __launch_bounds__(256) void trace_stage_kernel(int N, RowSet rs, const int32_t* __restrict__ labels,
                                                          int base, int t, int32_t* __restrict__ stage_labels,
                                                          int32_t* __restrict__ stage_base) {
    const int bh = blockIdx.y;
    if (rs.active && !rs.active[bh]) return;
    const int n = rs.nrows ? rs.nrows[bh] : N;
    const int r = blockIdx.x * 256 + threadIdx.x;
    if (r == 0 && stage_base) stage_base[bh * TRACE_STAGES + t] = base;
    if (r >= n || !stage_labels) return;
    const int64_t tok = rs.rows ? rs.rows[(int64_t)bh * N + r] : r;
    stage_labels[((int64_t)bh * TRACE_STAGES + t) * N + tok] = base + labels[(int64_t)bh * N + r];
}

hipError_t launch_trace_stage(const Prob& p, RowSet rs, const int32_t* labels, int base, int t,
                              int32_t* stage_labels, int32_t* stage_base, hipStream_t s) {
    if (t >= TRACE_STAGES) return hipSuccess;
    dim3 grid((unsigned)((p.N + 255) / 256), (unsigned)p.BH);
    hipLaunchKernelGGL(trace_stage_kernel, grid, dim3(256), 0, s, p.N, rs, labels, base, t, stage_labels,
                       stage_base);
    return hipGetLastError();
}

// ------------------------------------------------------------------ multi-stage bookkeeping
__global__ void stage_reset_kernel(int BH, int N, StageState st) {
    int bh = blockIdx.x * blockDim.x + threadIdx.x;
    if (bh >= BH) return;
    st.nu[bh] = N;
    st.slots[bh] = 0;
    st.full[bh] = 0;
    st.active[bh] = 1;
    st.n_stages[bh] = 0;
    st.tau[bh] = 0.0;
    if (st.stage_sizes)
        for (int i = 0; i < 8; ++i) st.stage_sizes[bh * 8 + i] = -1;
}

hipError_t launch_stage_reset(const Prob& p, StageState st, hipStream_t s) {
    hipLaunchKernelGGL(stage_reset_kernel, dim3((p.BH + 63) / 64), dim3(64), 0, s, p.BH, p.N, st);
    return hipGetLastError();
}

// Algorithm 1 loop head: a head runs stage t while U is non-empty and fewer
// than Nmax slots are used; U non-empty at Nmax sets F.
__global__ void stage_begin_kernel(int BH, StageState st, int t, int nmax) {
    int bh = blockIdx.x * blockDim.x + threadIdx.x;
    if (bh >= BH) return;
    const int nu = st.nu[bh], slots = st.slots[bh];
    const bool act = nu > 0 && slots < nmax;
    if (nu > 0 && slots >= nmax) st.full[bh] = 1;
    st.active[bh] = act ? 1 : 0;
    if (act) {
        st.n_stages[bh] = t + 1;
        if (st.stage_sizes && t < 8) st.stage_sizes[bh * 8 + t] = nu;
    }
}

hipError_t launch_stage_begin(const Prob& p, StageState st, int t, int nmax, hipStream_t s) {
    hipLaunchKernelGGL(stage_begin_kernel, dim3((p.BH + 63) / 64), dim3(64), 0, s, p.BH, st, t, nmax);
    return hipGetLastError();
}

// Euclidean distance of each clustered row to its stage centre, in f64. Eight
// lanes share a row: each sums the squared differences of its chunks of 8
// dimensions in index order, and the eight partial sums are combined in a
// fixed tree, so the result is deterministic (it differs from an index-order
// sum only by f64 rounding).
template <typename T>
__global__ __launch_bounds__(256) void stage_dist_kernel(const T* __restrict__ x, int N, int D,
                                                         RowSet rs, const int32_t* __restrict__ labels,
                                                         CentView cv, double* __restrict__ dist) {
#pragma clang fp contract(off)
    const int bh = blockIdx.y;
    if (rs.active && !rs.active[bh]) return;
    const int n = rs.nrows ? rs.nrows[bh] : N;
    const int sub = threadIdx.x & 7;
    // a row list (the keys left in U) comes with a capped grid: blocks of 32
    // rows, grid-strided
    for (int r0 = blockIdx.x * 32; r0 < n; r0 += gridDim.x * 32) {
    const int r = r0 + (threadIdx.x >> 3);
    const bool ok = r < n;
    double s = 0.0;
    if (ok) {
        const int64_t tok = rs.rows ? rs.rows[(int64_t)bh * N + r] : r;
        const T* xr = row_ptr(x, N, D, bh, tok);
        const float* c = cv.cent + ((int64_t)bh * cv.cap + cv.base + labels[(int64_t)bh * N + r]) * D;
        for (int d0 = sub * 8; d0 < D; d0 += 64) {
            float xv[8];
            load8<T>(xr + d0, xv);
            const float4 c0 = *reinterpret_cast<const float4*>(c + d0);
            const float4 c1 = *reinterpret_cast<const float4*>(c + d0 + 4);
            const float cc[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const double df = (double)xv[i] - (double)cc[i];
                s += df * df;
            }
        }
    }
    s += __shfl_xor(s, 1);
    s += __shfl_xor(s, 2);
    s += __shfl_xor(s, 4);
    if (ok && sub == 0) dist[(int64_t)bh * N + r] = sqrt(s);
    }
}

hipError_t launch_stage_dist(const Prob& p, const void* k, RowSet rs, const int32_t* labels,
                             CentView cv, double* dist, hipStream_t s) {
    dim3 grid((unsigned)((p.N + 31) / 32), (unsigned)p.BH);
    if (rs.rows && rs.nrows) grid.x = min(grid.x, 256u);
    if (p.bf16)
        hipLaunchKernelGGL(stage_dist_kernel<u16>, grid, dim3(256), 0, s, (const u16*)k, p.N, p.D,
                           rs, labels, cv, dist);
    else
        hipLaunchKernelGGL(stage_dist_kernel<float>, grid, dim3(256), 0, s, (const float*)k, p.N,
                           p.D, rs, labels, cv, dist);
    return hipGetLastError();
}

// tau = tau_mult x mean distance over all N keys (stage 0 clusters every key).
// Fixed reduction order: strided per-thread sums, then a tree.
__global__ __launch_bounds__(1024) void stage_tau_kernel(int N, StageState st, double tau_mult) {
    __shared__ double part[16];
    const int bh = blockIdx.x;
    if (!st.active[bh]) return;
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
    const double* dd = st.dist + (int64_t)bh * N;
    // fixed order: four interleaved sums per thread, a butterfly over the wave,
    // then the 16 waves in order
    double p0 = 0.0, p1 = 0.0, p2 = 0.0, p3 = 0.0;
    int r = tid;
    for (; r + 3 * 1024 < N; r += 4 * 1024) {
        p0 += dd[r];
        p1 += dd[r + 1024];
        p2 += dd[r + 2048];
        p3 += dd[r + 3072];
    }
    for (; r < N; r += 1024) p0 += dd[r];
    const double sw = wave_sum_d((p0 + p1) + (p2 + p3));
    if (l == 0) part[w] = sw;
    __syncthreads();
    if (tid == 0) {
        double t = 0.0;
        for (int i = 0; i < 16; ++i) t += part[i];
        st.tau[bh] = tau_mult * t / (double)N;
    }
}

hipError_t launch_stage_tau(const Prob& p, StageState st, double tau_mult, hipStream_t s) {
    hipLaunchKernelGGL(stage_tau_kernel, dim3(p.BH), dim3(1024), 0, s, p.N, st, tau_mult);
    return hipGetLastError();
}

// U <- {u in U : dist(u) >= tau}, order kept (Algorithm 1 steps 11-16); slots += m_t.
// Each thread takes 8 consecutive entries of a 8192-entry chunk; a wave scan and
// the 16 wave totals give every kept entry its place.
__global__ __launch_bounds__(1024) void stage_compact_kernel(int N, StageState st,
                                                             const int32_t* __restrict__ u_in,
                                                             int32_t* __restrict__ u_out, int m_t) {
    constexpr int PER = 8;
    __shared__ int wsum[16];
    const int bh = blockIdx.x;
    if (!st.active[bh]) return;
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
    const int nu = st.nu[bh];
    const double tau = st.tau[bh];
    const double* dd = st.dist + (int64_t)bh * N;
    int running = 0;
    for (int base = 0; base < nu; base += 1024 * PER) {
        const int r0 = base + tid * PER;
        uint32_t keepm = 0;
        int cnt = 0;
#pragma unroll
        for (int j = 0; j < PER; ++j) {
            const int r = r0 + j;
            const bool keep = r < nu && !(dd[r] < tau);
            keepm |= (uint32_t)keep << j;
            cnt += keep;
        }
        int incl = cnt;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int v = __shfl_up(incl, o);
            if (l >= o) incl += v;
        }
        if (l == 63) wsum[w] = incl;
        __syncthreads();
        int before = 0, tot = 0;
        for (int i = 0; i < 16; ++i) {
            const int v = wsum[i];
            before += i < w ? v : 0;
            tot += v;
        }
        int pos = running + before + incl - cnt;
#pragma unroll
        for (int j = 0; j < PER; ++j) {
            if ((keepm >> j) & 1u) {
                const int r = r0 + j;
                u_out[(int64_t)bh * N + pos++] = u_in ? u_in[(int64_t)bh * N + r] : r;
            }
        }
        running += tot;
        __syncthreads();
    }
    if (tid == 0) {
        st.nu[bh] = running;
        st.slots[bh] += m_t;
    }
}

hipError_t launch_stage_compact(const Prob& p, StageState st, const int32_t* u_in, int32_t* u_out,
                                int m_t, hipStream_t s) {
    hipLaunchKernelGGL(stage_compact_kernel, dim3(p.BH), dim3(1024), 0, s, p.N, st, u_in, u_out, m_t);
    return hipGetLastError();
}

__global__ void stage_end_kernel(int BH, StageState st, int nmax, int32_t* n_clusters,
                                 uint8_t* full_out, float* tau_out) {
    int bh = blockIdx.x * blockDim.x + threadIdx.x;
    if (bh >= BH) return;
    const int nu = st.nu[bh], slots = st.slots[bh];
    if (nu > 0 && slots >= nmax) st.full[bh] = 1;
    n_clusters[bh] = slots;
    full_out[bh] = st.full[bh];
    tau_out[bh] = (float)st.tau[bh];
    const int t = st.n_stages[bh];
    if (st.stage_sizes && t < 8) st.stage_sizes[bh * 8 + t] = nu;
}

hipError_t launch_stage_end(const Prob& p, StageState st, int t_total, int nmax,
                            int32_t* n_clusters, uint8_t* full_out, float* tau_out, hipStream_t s) {
    (void)t_total;
    hipLaunchKernelGGL(stage_end_kernel, dim3((p.BH + 63) / 64), dim3(64), 0, s, p.BH, st, nmax,
                       n_clusters, full_out, tau_out);
    return hipGetLastError();
}

}  // namespace adc
