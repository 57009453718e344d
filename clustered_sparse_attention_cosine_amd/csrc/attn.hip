// Variable-length block-sparse attention for gfx950 (AdaCluster paper,
// Algorithm 3 steps 8-9): every query of q-cluster a attends, with an exact
// online softmax, to the keys of the slots selected for a.
//
// Layout. cluster_k leaves K and V slot-contiguous, so the keys of a selection
// are a list of contiguous key ranges ("runs"; slots with no members never
// break a run). The queries of a q-cluster are read through its permutation.
//
// Kernel. A work item is (head, q-cluster, chunk of 64 query rows); four waves
// own 16 rows each. Key/value tiles of 64 rows are staged in LDS (K row-major,
// V transposed) and shared by the waves. Scores are computed as
// S^T = K Q^T with 16x16x32 bf16 MFMAs so that a lane owns one query column,
// the output as O^T += V^T P^T reusing the score registers as the B operand.
#include <math.h>
#include "common.hpp"
#include "kernels.hpp"

namespace adc {

hipError_t fill_i32(int32_t* p, int64_t n, int32_t v, hipStream_t s);

// ------------------------------------------------------------------ runs
__global__ __launch_bounds__(256) void build_runs_kernel(int64_t rows, int Cq, int Ck,
                                                         const int32_t* __restrict__ k_offsets,
                                                         const uint32_t* __restrict__ mask,
                                                         int run_cap, int32_t* __restrict__ run_start,
                                                         int32_t* __restrict__ run_pos,
                                                         int32_t* __restrict__ n_runs) {
    const int64_t row = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (row >= rows) return;
    const int64_t bh = row / Cq;
    const int words = (Ck + 31) / 32;
    const uint32_t* m = mask + row * words;
    const int32_t* off = k_offsets + bh * (Ck + 1);
    int32_t* rs = run_start + row * run_cap;
    int32_t* rp = run_pos + row * (run_cap + 1);
    int nr = 0, pos = 0, cs = -1, ce = -1;
    for (int wd = 0; wd < words; ++wd) {
        uint32_t bits = m[wd];
        while (bits) {
            const int b = wd * 32 + __ffs(bits) - 1;
            bits &= bits - 1;
            if (b >= Ck) break;
            const int s = off[b], e = off[b + 1];
            if (e <= s) continue;
            if (s == ce) {
                ce = e;
            } else {
                if (cs >= 0 && nr < run_cap) { rs[nr] = cs; rp[nr] = pos; pos += ce - cs; ++nr; }
                cs = s;
                ce = e;
            }
        }
    }
    if (cs >= 0 && nr < run_cap) { rs[nr] = cs; rp[nr] = pos; pos += ce - cs; ++nr; }
    rp[nr] = pos;
    n_runs[row] = nr;
}

hipError_t launch_build_runs(const Prob& p, int Cq, int Ck, const int32_t* k_offsets,
                             const uint32_t* mask, int run_cap, int32_t* run_start,
                             int32_t* run_pos, int32_t* n_runs, hipStream_t s) {
    const int64_t rows = (int64_t)p.BH * Cq;
    hipLaunchKernelGGL(build_runs_kernel, dim3((unsigned)((rows + 255) / 256)), dim3(256), 0, s, rows,
                       Cq, Ck, k_offsets, mask, run_cap, run_start, run_pos, n_runs);
    return hipGetLastError();
}

// ------------------------------------------------------------------ work list
__global__ __launch_bounds__(256) void worklist_kernel(int64_t rows, int Cq,
                                                       const int32_t* __restrict__ q_offsets,
                                                       int32_t* __restrict__ items,
                                                       int32_t* __restrict__ n_items) {
    const int64_t row = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (row >= rows) return;
    const int64_t bh = row / Cq;
    const int a = (int)(row % Cq);
    const int32_t* qo = q_offsets + bh * (Cq + 1);
    const int na = qo[a + 1] - qo[a];
    const int ch = (na + ATTN_ROWS - 1) / ATTN_ROWS;
    if (ch == 0) return;
    const int base = atomicAdd(n_items, ch);
    for (int c = 0; c < ch; ++c) {
        items[2 * (int64_t)(base + c)] = (int32_t)bh;
        items[2 * (int64_t)(base + c) + 1] = a | (c << 16);
    }
}

hipError_t launch_worklist(const Prob& p, int Cq, const int32_t* q_offsets, int32_t* items,
                           int32_t* n_items, hipStream_t s) {
    hipError_t e = fill_i32(n_items, 1, 0, s);
    if (e != hipSuccess) return e;
    const int64_t rows = (int64_t)p.BH * Cq;
    hipLaunchKernelGGL(worklist_kernel, dim3((unsigned)((rows + 255) / 256)), dim3(256), 0, s, rows,
                       Cq, q_offsets, items, n_items);
    return hipGetLastError();
}

// ------------------------------------------------------------------ attention
template <typename T> __device__ __forceinline__ void load_row8_bits(const T* p, bool ok, uint32_t (&w)[4]);
template <> __device__ __forceinline__ void load_row8_bits<u16>(const u16* p, bool ok, uint32_t (&w)[4]) {
    uint4 r = make_uint4(0, 0, 0, 0);
    if (ok) r = *reinterpret_cast<const uint4*>(p);
    w[0] = r.x; w[1] = r.y; w[2] = r.z; w[3] = r.w;
}
template <> __device__ __forceinline__ void load_row8_bits<float>(const float* p, bool ok, uint32_t (&w)[4]) {
    float v[8];
    if (ok) {
        load8<float>(p, v);
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = 0.0f;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
        w[i] = (uint32_t)f2bf_bits(v[2 * i]) | ((uint32_t)f2bf_bits(v[2 * i + 1]) << 16);
}

template <typename T, int D>
__global__ __launch_bounds__(256) void attn_kernel(int N, int Cq, const T* __restrict__ Q,
                                                   const int32_t* __restrict__ q_perm,
                                                   const int32_t* __restrict__ q_off,
                                                   const T* __restrict__ Kp, const T* __restrict__ Vp,
                                                   const int32_t* __restrict__ run_start,
                                                   const int32_t* __restrict__ run_pos,
                                                   const int32_t* __restrict__ n_runs, int run_cap,
                                                   const int32_t* __restrict__ items,
                                                   const int32_t* __restrict__ n_items, float sl2,
                                                   T* __restrict__ O, float* __restrict__ lse) {
    constexpr int KC = D / 32;   // 32-wide chunks of the head dimension
    constexpr int DB = D / 16;   // 16-row blocks of O^T
    constexpr int LDK = D + 8;   // padded LDS strides (elements)
    constexpr int LDV = 64 + 8;
    __shared__ __attribute__((aligned(16))) u16 Ks[64 * LDK];
    __shared__ __attribute__((aligned(16))) u16 Vt[D * LDV];
    __shared__ int win_s[65], win_p[65];
    __shared__ int krow[64];
    __shared__ int sh_r0;

    const int it = blockIdx.x;
    if (it >= *n_items) return;
    const int bh = items[2 * it];
    const int packed = items[2 * it + 1];
    const int a = packed & 0xFFFF, ch = packed >> 16;
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, g = l >> 4, c16 = l & 15;

    const int32_t* qo = q_off + (int64_t)bh * (Cq + 1);
    const int row0 = qo[a] + ch * ATTN_ROWS;
    const int nrows = min(ATTN_ROWS, qo[a + 1] - row0);
    const int rowi = w * 16 + c16;
    const bool qok = rowi < nrows;
    const bool wave_live = w * 16 < nrows;
    const int64_t qtok = qok ? q_perm[(int64_t)bh * N + row0 + rowi] : 0;

    bf16x8 qf[KC];
    {
        const T* qr = Q + ((int64_t)bh * N + qtok) * D;
#pragma unroll
        for (int kc = 0; kc < KC; ++kc) {
            uint32_t wv[4];
            load_row8_bits<T>(qr + kc * 32 + g * 8, qok, wv);
            qf[kc] = __builtin_bit_cast(bf16x8, make_uint4(wv[0], wv[1], wv[2], wv[3]));
        }
    }

    const int64_t rbase = (int64_t)bh * Cq + a;
    const int R = n_runs[rbase];
    const int32_t* rs = run_start + rbase * run_cap;
    const int32_t* rp = run_pos + rbase * (run_cap + 1);
    const int total = rp[R];
    const T* Kh = Kp + (int64_t)bh * N * D;
    const T* Vh = Vp + (int64_t)bh * N * D;

    float m_run = -INFINITY, l_part = 0.0f;
    f32x4 o[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) o[db] = f32x4{0.f, 0.f, 0.f, 0.f};
    int r0 = 0;

    for (int t0 = 0; t0 < total; t0 += 64) {
        // key rows of positions t0 .. t0+63 of the concatenated selection
        if (tid < 65) {
            const int k = r0 + tid;
            win_p[tid] = k <= R ? rp[k] : 0x7fffffff;
            win_s[tid] = k < R ? rs[k] : 0;
        }
        __syncthreads();
        if (tid < 64) {
            const int P = t0 + tid;
            int row = -1;
            if (P < total) {
                int lo = 0, hi = 64;
                while (lo < hi) {
                    const int mid = (lo + hi + 1) >> 1;
                    if (win_p[mid] <= P) lo = mid; else hi = mid - 1;
                }
                row = win_s[lo] + (P - win_p[lo]);
            }
            krow[tid] = row;
            if (tid == 0) {
                const int nxt = t0 + 64;
                int lo = 0, hi = 64;
                while (lo < hi) {
                    const int mid = (lo + hi + 1) >> 1;
                    if (win_p[mid] <= nxt) lo = mid; else hi = mid - 1;
                }
                sh_r0 = r0 + lo;
            }
        }
        __syncthreads();
        // K tile, row-major
#pragma unroll
        for (int i = 0; i < D / 32; ++i) {
            const int c = tid + i * 256;
            const int kr = c / (D / 8), c8 = c % (D / 8);
            const int row = krow[kr];
            uint32_t wv[4];
            load_row8_bits<T>(Kh + (int64_t)(row < 0 ? 0 : row) * D + c8 * 8, row >= 0, wv);
            *reinterpret_cast<uint4*>(&Ks[kr * LDK + c8 * 8]) = make_uint4(wv[0], wv[1], wv[2], wv[3]);
        }
        // V tile, transposed: Vt[d][key]
#pragma unroll
        for (int i = 0; i < D / 64; ++i) {
            const int c = tid + i * 256;
            const int kk = c % 32, c8 = c / 32;
            const int ra = krow[2 * kk], rb = krow[2 * kk + 1];
            uint32_t va[4], vb[4];
            load_row8_bits<T>(Vh + (int64_t)(ra < 0 ? 0 : ra) * D + c8 * 8, ra >= 0, va);
            load_row8_bits<T>(Vh + (int64_t)(rb < 0 ? 0 : rb) * D + c8 * 8, rb >= 0, vb);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint32_t lo_w = (va[j] & 0xFFFFu) | (vb[j] << 16);
                const uint32_t hi_w = (va[j] >> 16) | (vb[j] & 0xFFFF0000u);
                *reinterpret_cast<uint32_t*>(&Vt[(c8 * 8 + 2 * j) * LDV + 2 * kk]) = lo_w;
                *reinterpret_cast<uint32_t*>(&Vt[(c8 * 8 + 2 * j + 1) * LDV + 2 * kk]) = hi_w;
            }
        }
        __syncthreads();
        const int r0_next = sh_r0;

        if (wave_live) {
            f32x4 sc[4];
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
                sc[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kc = 0; kc < KC; ++kc) {
                    const bf16x8 ka = *reinterpret_cast<const bf16x8*>(&Ks[(kb * 16 + c16) * LDK + kc * 32 + g * 8]);
                    sc[kb] = mfma16(ka, qf[kc], sc[kb]);
                }
            }
            float mx = -INFINITY;
#pragma unroll
            for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int pos = t0 + kb * 16 + g * 4 + i;
                    const float v = pos < total ? sc[kb][i] * sl2 : -INFINITY;
                    sc[kb][i] = v;
                    mx = fmaxf(mx, v);
                }
            mx = fmaxf(mx, __shfl_xor(mx, 16));
            mx = fmaxf(mx, __shfl_xor(mx, 32));
            const float m_new = fmaxf(m_run, mx);
            const float base = (m_new == -INFINITY) ? 0.0f : m_new;
            const float alpha = __builtin_amdgcn_exp2f(m_run - base);
            float lsum = 0.0f;
#pragma unroll
            for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float pv = __builtin_amdgcn_exp2f(sc[kb][i] - base);
                    sc[kb][i] = pv;
                    lsum += pv;
                }
            l_part = l_part * alpha + lsum;
#pragma unroll
            for (int db = 0; db < DB; ++db) o[db] *= alpha;
#pragma unroll
            for (int kc2 = 0; kc2 < 2; ++kc2) {
                bf16x8 pb;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    pb[j] = f2bf(sc[2 * kc2][j]);
                    pb[4 + j] = f2bf(sc[2 * kc2 + 1][j]);
                }
#pragma unroll
                for (int db = 0; db < DB; ++db) {
                    const u16* vp = &Vt[(db * 16 + c16) * LDV + kc2 * 32 + g * 4];
                    const uint2 lo = *reinterpret_cast<const uint2*>(vp);
                    const uint2 hi = *reinterpret_cast<const uint2*>(vp + 16);
                    const bf16x8 va = __builtin_bit_cast(bf16x8, make_uint4(lo.x, lo.y, hi.x, hi.y));
                    o[db] = mfma16(va, pb, o[db]);
                }
            }
            m_run = m_new;
        }
        __syncthreads();
        r0 = r0_next;
    }

    float l_tot = l_part + __shfl_xor(l_part, 16);
    l_tot += __shfl_xor(l_tot, 32);
    if (qok) {
        const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
        T* orow = O + ((int64_t)bh * N + qtok) * D;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int i = 0; i < 4; ++i) elem<T>::store(orow, db * 16 + g * 4 + i, o[db][i] * inv);
        if (g == 0 && lse)
            lse[(int64_t)bh * N + qtok] =
                l_tot > 0.0f ? (m_run + __log2f(l_tot)) * 0.69314718055994531f : -INFINITY;
    }
}

hipError_t launch_attention(const Prob& p, int Cq, const void* q, const int32_t* q_perm,
                            const int32_t* q_offsets, const void* k_perm, const void* v_perm,
                            const int32_t* run_start, const int32_t* run_pos, const int32_t* n_runs,
                            int run_cap, const int32_t* items, const int32_t* n_items, int max_items,
                            float scale, void* out, float* lse, hipStream_t s) {
    if (max_items <= 0) return hipSuccess;
    const float sl2 = scale * 1.4426950408889634f;
    dim3 grid((unsigned)max_items);
    if (p.bf16) {
        auto k = p.D == 64 ? attn_kernel<u16, 64> : attn_kernel<u16, 128>;
        hipLaunchKernelGGL(k, grid, dim3(256), 0, s, p.N, Cq, (const u16*)q, q_perm, q_offsets,
                           (const u16*)k_perm, (const u16*)v_perm, run_start, run_pos, n_runs,
                           run_cap, items, n_items, sl2, (u16*)out, lse);
    } else {
        auto k = p.D == 64 ? attn_kernel<float, 64> : attn_kernel<float, 128>;
        hipLaunchKernelGGL(k, grid, dim3(256), 0, s, p.N, Cq, (const float*)q, q_perm, q_offsets,
                           (const float*)k_perm, (const float*)v_perm, run_start, run_pos, n_runs,
                           run_cap, items, n_items, sl2, (float*)out, lse);
    }
    return hipGetLastError();
}

}  // namespace adc
