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
// 8 consecutive elements as packed bf16 words: the value (hi) and, for f32
// inputs, the rounding residual (lo), so f32 data is carried as hi + lo.
template <typename T>
__device__ __forceinline__ void load_row8_split(const T* p, bool ok, uint32_t (&hi)[4],
                                                uint32_t (&lo)[4]);
template <>
__device__ __forceinline__ void load_row8_split<u16>(const u16* p, bool ok, uint32_t (&hi)[4],
                                                     uint32_t (&lo)[4]) {
    uint4 r = make_uint4(0, 0, 0, 0);
    if (ok) r = *reinterpret_cast<const uint4*>(p);
    hi[0] = r.x; hi[1] = r.y; hi[2] = r.z; hi[3] = r.w;
    lo[0] = lo[1] = lo[2] = lo[3] = 0;
}
template <>
__device__ __forceinline__ void load_row8_split<float>(const float* p, bool ok, uint32_t (&hi)[4],
                                                       uint32_t (&lo)[4]) {
    float v[8];
    if (ok) {
        load8<float>(p, v);
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = 0.0f;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const u16 h0 = f2bf_bits(v[2 * i]), h1 = f2bf_bits(v[2 * i + 1]);
        const u16 l0 = f2bf_bits(v[2 * i] - bf_bits2f(h0));
        const u16 l1 = f2bf_bits(v[2 * i + 1] - bf_bits2f(h1));
        hi[i] = (uint32_t)h0 | ((uint32_t)h1 << 16);
        lo[i] = (uint32_t)l0 | ((uint32_t)l1 << 16);
    }
}

// PREC (f32 inputs): operands carried as bf16 hi + lo and every product of
// order <= 1 accumulated (3 MFMAs per product instead of 1), which keeps the
// result near f32 accuracy. TO is the output element type.
template <typename T, int D, typename TO>
__global__ __launch_bounds__(256) void attn_kernel(int N, int Cq, const T* __restrict__ Q,
                                                   const int32_t* __restrict__ q_perm,
                                                   const int32_t* __restrict__ q_off,
                                                   const T* __restrict__ Kp, const T* __restrict__ Vp,
                                                   const int32_t* __restrict__ run_start,
                                                   const int32_t* __restrict__ run_pos,
                                                   const int32_t* __restrict__ n_runs, int run_cap,
                                                   const int32_t* __restrict__ items,
                                                   const int32_t* __restrict__ n_items, float sl2,
                                                   TO* __restrict__ O, float* __restrict__ lse) {
    constexpr bool PREC = sizeof(T) == 4;
    constexpr int NP = PREC ? 2 : 1;  // stored parts per operand
    constexpr int KC = D / 32;        // 32-wide chunks of the head dimension
    constexpr int DB = D / 16;        // 16-row blocks of O^T
    constexpr int LDK = D + 8;        // padded LDS strides (elements)
    constexpr int LDV = 64 + 8;
    __shared__ __attribute__((aligned(16))) u16 Ks[NP][64 * LDK];
    __shared__ __attribute__((aligned(16))) u16 Vt[NP][D * LDV];
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

    bf16x8 qf[NP][KC];
    {
        const T* qr = Q + ((int64_t)bh * N + qtok) * D;
#pragma unroll
        for (int kc = 0; kc < KC; ++kc) {
            uint32_t hv[4], lv[4];
            load_row8_split<T>(qr + kc * 32 + g * 8, qok, hv, lv);
            qf[0][kc] = __builtin_bit_cast(bf16x8, make_uint4(hv[0], hv[1], hv[2], hv[3]));
            if constexpr (PREC)
                qf[NP - 1][kc] = __builtin_bit_cast(bf16x8, make_uint4(lv[0], lv[1], lv[2], lv[3]));
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
            uint32_t hv[4], lv[4];
            load_row8_split<T>(Kh + (int64_t)(row < 0 ? 0 : row) * D + c8 * 8, row >= 0, hv, lv);
            *reinterpret_cast<uint4*>(&Ks[0][kr * LDK + c8 * 8]) = make_uint4(hv[0], hv[1], hv[2], hv[3]);
            if constexpr (PREC)
                *reinterpret_cast<uint4*>(&Ks[NP - 1][kr * LDK + c8 * 8]) = make_uint4(lv[0], lv[1], lv[2], lv[3]);
        }
        // V tile, transposed: Vt[d][key]
#pragma unroll
        for (int i = 0; i < D / 64; ++i) {
            const int c = tid + i * 256;
            const int kk = c % 32, c8 = c / 32;
            const int ra = krow[2 * kk], rb = krow[2 * kk + 1];
            uint32_t va[NP][4], vb[NP][4];
            uint32_t scratch[4];
            load_row8_split<T>(Vh + (int64_t)(ra < 0 ? 0 : ra) * D + c8 * 8, ra >= 0, va[0],
                               PREC ? va[NP - 1] : scratch);
            load_row8_split<T>(Vh + (int64_t)(rb < 0 ? 0 : rb) * D + c8 * 8, rb >= 0, vb[0],
                               PREC ? vb[NP - 1] : scratch);
#pragma unroll
            for (int pp = 0; pp < NP; ++pp)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    uint32_t lo_w, hi_w;
                    if constexpr (PREC) {
                        lo_w = (va[pp][j] & 0xFFFFu) | (vb[pp][j] << 16);
                        hi_w = (va[pp][j] >> 16) | (vb[pp][j] & 0xFFFF0000u);
                    } else {
                        // bf16 -> fp16 is exact for |v| in the fp16 normal range
                        lo_w = pack_h2(__uint_as_float(va[pp][j] << 16), __uint_as_float(vb[pp][j] << 16));
                        hi_w = pack_h2(__uint_as_float(va[pp][j] & 0xFFFF0000u),
                                       __uint_as_float(vb[pp][j] & 0xFFFF0000u));
                    }
                    *reinterpret_cast<uint32_t*>(&Vt[pp][(c8 * 8 + 2 * j) * LDV + 2 * kk]) = lo_w;
                    *reinterpret_cast<uint32_t*>(&Vt[pp][(c8 * 8 + 2 * j + 1) * LDV + 2 * kk]) = hi_w;
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
                    const int off = (kb * 16 + c16) * LDK + kc * 32 + g * 8;
                    const bf16x8 ka = *reinterpret_cast<const bf16x8*>(&Ks[0][off]);
                    if constexpr (PREC) {
                        const bf16x8 kl = *reinterpret_cast<const bf16x8*>(&Ks[NP - 1][off]);
                        sc[kb] = mfma16(kl, qf[0][kc], sc[kb]);
                        sc[kb] = mfma16(ka, qf[NP - 1][kc], sc[kb]);
                    }
                    sc[kb] = mfma16(ka, qf[0][kc], sc[kb]);
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
                if constexpr (PREC) {
                    bf16x8 pb, pl;
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        pb[j] = f2bf(sc[2 * kc2][j]);
                        pb[4 + j] = f2bf(sc[2 * kc2 + 1][j]);
                        pl[j] = f2bf(sc[2 * kc2][j] - bf2f(pb[j]));
                        pl[4 + j] = f2bf(sc[2 * kc2 + 1][j] - bf2f(pb[4 + j]));
                    }
#pragma unroll
                    for (int db = 0; db < DB; ++db) {
                        const int off = (db * 16 + c16) * LDV + kc2 * 32 + g * 4;
                        const uint2 lo0 = *reinterpret_cast<const uint2*>(&Vt[0][off]);
                        const uint2 hi0 = *reinterpret_cast<const uint2*>(&Vt[0][off + 16]);
                        const uint2 lo1 = *reinterpret_cast<const uint2*>(&Vt[NP - 1][off]);
                        const uint2 hi1 = *reinterpret_cast<const uint2*>(&Vt[NP - 1][off + 16]);
                        const bf16x8 va = __builtin_bit_cast(bf16x8, make_uint4(lo0.x, lo0.y, hi0.x, hi0.y));
                        const bf16x8 vl = __builtin_bit_cast(bf16x8, make_uint4(lo1.x, lo1.y, hi1.x, hi1.y));
                        o[db] = mfma16(vl, pb, o[db]);
                        o[db] = mfma16(va, pl, o[db]);
                        o[db] = mfma16(va, pb, o[db]);
                    }
                } else {
                    // P.V in fp16 (11-bit significand): probabilities lose at most 2^-12
                    const uint4 pw = make_uint4(pack_h2(sc[2 * kc2][0], sc[2 * kc2][1]),
                                                pack_h2(sc[2 * kc2][2], sc[2 * kc2][3]),
                                                pack_h2(sc[2 * kc2 + 1][0], sc[2 * kc2 + 1][1]),
                                                pack_h2(sc[2 * kc2 + 1][2], sc[2 * kc2 + 1][3]));
                    const f16x8 ph = __builtin_bit_cast(f16x8, pw);
#pragma unroll
                    for (int db = 0; db < DB; ++db) {
                        const int off = (db * 16 + c16) * LDV + kc2 * 32 + g * 4;
                        const uint2 lo0 = *reinterpret_cast<const uint2*>(&Vt[0][off]);
                        const uint2 hi0 = *reinterpret_cast<const uint2*>(&Vt[0][off + 16]);
                        const f16x8 vh = __builtin_bit_cast(f16x8, make_uint4(lo0.x, lo0.y, hi0.x, hi0.y));
                        o[db] = mfma16h(vh, ph, o[db]);
                    }
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
        TO* orow = O + ((int64_t)bh * N + qtok) * D;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int i = 0; i < 4; ++i) elem<TO>::store(orow, db * 16 + g * 4 + i, o[db][i] * inv);
        if (g == 0 && lse)
            lse[(int64_t)bh * N + qtok] =
                l_tot > 0.0f ? (m_run + __log2f(l_tot)) * 0.69314718055994531f : -INFINITY;
    }
}

template <typename T, typename TO>
static void launch_attn_t(const Prob& p, dim3 grid, int Cq, const void* q, const int32_t* q_perm,
                          const int32_t* q_offsets, const void* k_perm, const void* v_perm,
                          const int32_t* run_start, const int32_t* run_pos, const int32_t* n_runs,
                          int run_cap, const int32_t* items, const int32_t* n_items, float sl2,
                          void* out, float* lse, hipStream_t s) {
    auto k = p.D == 64 ? attn_kernel<T, 64, TO> : attn_kernel<T, 128, TO>;
    hipLaunchKernelGGL(k, grid, dim3(256), 0, s, p.N, Cq, (const T*)q, q_perm, q_offsets,
                       (const T*)k_perm, (const T*)v_perm, run_start, run_pos, n_runs, run_cap,
                       items, n_items, sl2, (TO*)out, lse);
}

hipError_t launch_attention(const Prob& p, int Cq, const void* q, const int32_t* q_perm,
                            const int32_t* q_offsets, const void* k_perm, const void* v_perm,
                            const int32_t* run_start, const int32_t* run_pos, const int32_t* n_runs,
                            int run_cap, const int32_t* items, const int32_t* n_items, int max_items,
                            float scale, void* out, int out_f32, float* lse, hipStream_t s) {
    if (max_items <= 0) return hipSuccess;
    const float sl2 = scale * 1.4426950408889634f;
    dim3 grid((unsigned)max_items);
    if (p.bf16) {
        if (out_f32)
            launch_attn_t<u16, float>(p, grid, Cq, q, q_perm, q_offsets, k_perm, v_perm, run_start,
                                      run_pos, n_runs, run_cap, items, n_items, sl2, out, lse, s);
        else
            launch_attn_t<u16, u16>(p, grid, Cq, q, q_perm, q_offsets, k_perm, v_perm, run_start,
                                    run_pos, n_runs, run_cap, items, n_items, sl2, out, lse, s);
    } else {
        launch_attn_t<float, float>(p, grid, Cq, q, q_perm, q_offsets, k_perm, v_perm, run_start,
                                    run_pos, n_runs, run_cap, items, n_items, sl2, out, lse, s);
    }
    return hipGetLastError();
}

}  // namespace adc
