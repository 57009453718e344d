// Critical-cluster selection for gfx950 (AdaCluster paper, section 3.2.3 and
// Algorithm 3 steps 6-7).
//
// Scores. Eq. (1) bounds q.k over a cluster by sum_d max(q_d max K_d, q_d min K_d).
// With q+ = max(q, 0), q- = min(q, 0) and K+/K- read as the per-cluster,
// per-dimension max / min, that sum equals q+ . K+ + q- . K- (Eq. (2)): one
// contraction of width 2D, done here on bf16 matrix cores. The f32 query side
// is split into three bf16 terms (residual 2^-24); bf16 key statistics are
// exact in one term, f32 ones are split too, and every product of combined
// order <= 2 is accumulated, which keeps the scores at about f32 accuracy.
//
// Top-p. For each q-cluster row: l_b = S_ab * scale + ln n_b over slots with
// members; the cut value T (the l of the last selected slot) is found by
// bisection on the order-preserving integer image of l, using deterministic
// block sums of exp(l - max l); slots with l above T are selected, slots equal
// to T are taken in index order until the mass reaches top_p.
#include <math.h>
#include "common.hpp"
#include "kernels.hpp"

namespace adc {

// ------------------------------------------------------------------ scores
// Grid: (Cq / 64, Ck / 256, BH); 4 waves, each 16 q-clusters x 256 slots.
template <typename TK, int D, int MODE>  // MODE 0: quest (width 2D), 1: centroid (width D)
__global__ __launch_bounds__(256) void scores_kernel(int Cq, int Ck, const float* __restrict__ qrep,
                                                     const TK* __restrict__ kmax,
                                                     const TK* __restrict__ kmin,
                                                     const float* __restrict__ kcent,
                                                     const int32_t* __restrict__ k_sizes,
                                                     const int32_t* __restrict__ n_clusters,
                                                     float* __restrict__ S) {
    constexpr int KD = MODE == 0 ? 2 * D : D;
    constexpr int KC = KD / 32;
    constexpr bool AF32 = (MODE == 1) || sizeof(TK) == 4;  // key side needs a split
    constexpr int KA = AF32 ? 3 : 1;
    constexpr int LD = KD + 8;
    __shared__ __attribute__((aligned(16))) u16 sa[KA][64 * LD];

    const int bh = blockIdx.z;
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, g = l >> 4, c16 = l & 15;
    const int a = blockIdx.x * 64 + w * 16 + c16;
    const bool aok = a < Cq;
    const int ncl = min(n_clusters[bh], Ck);

    // query side: 3-term split of [q+, q-] (or q)
    bf16x8 qb[3][KC];
    const float* qp = qrep + ((int64_t)bh * Cq + (aok ? a : 0)) * D;
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
        float v[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int k = kc * 32 + g * 8 + i;
            float x = 0.0f;
            if (aok) {
                if (MODE == 0) {
                    const float qv = qp[k < D ? k : k - D];
                    x = k < D ? fmaxf(qv, 0.0f) : fminf(qv, 0.0f);
                } else {
                    x = qp[k];
                }
            }
            v[i] = x;
        }
        float r1[8], r2[8];
        qb[0][kc] = pack_bf16x8(v);
#pragma unroll
        for (int i = 0; i < 8; ++i) r1[i] = v[i] - bf2f(qb[0][kc][i]);
        qb[1][kc] = pack_bf16x8(r1);
#pragma unroll
        for (int i = 0; i < 8; ++i) r2[i] = r1[i] - bf2f(qb[1][kc][i]);
        qb[2][kc] = pack_bf16x8(r2);
    }

    for (int tile = 0; tile < 4; ++tile) {
        const int b0 = blockIdx.y * 256 + tile * 64;
        if (b0 >= Ck) break;
        __syncthreads();
        // stage 64 slots x KD of the key side (KA terms)
        for (int c = tid; c < 64 * (KD / 8); c += 256) {
            const int row = c / (KD / 8), col8 = c % (KD / 8);
            const int b = b0 + row;
            float v[8];
            if (b < Ck) {
                const int k0 = col8 * 8;
                const int64_t base = ((int64_t)bh * Ck + b) * D;
                if (MODE == 0) {
                    const TK* src = k0 < D ? kmax + base + k0 : kmin + base + (k0 - D);
                    load8<TK>(src, v);
                } else {
                    load8<float>(kcent + base + k0, v);
                }
            } else {
#pragma unroll
                for (int i = 0; i < 8; ++i) v[i] = 0.0f;
            }
            bf16x8 t0 = pack_bf16x8(v);
            *reinterpret_cast<bf16x8*>(&sa[0][row * LD + col8 * 8]) = t0;
            if constexpr (KA == 3) {
                float r1[8], r2[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) r1[i] = v[i] - bf2f(t0[i]);
                bf16x8 t1 = pack_bf16x8(r1);
#pragma unroll
                for (int i = 0; i < 8; ++i) r2[i] = r1[i] - bf2f(t1[i]);
                *reinterpret_cast<bf16x8*>(&sa[1][row * LD + col8 * 8]) = t1;
                *reinterpret_cast<bf16x8*>(&sa[KA - 1][row * LD + col8 * 8]) = pack_bf16x8(r2);
            }
        }
        __syncthreads();
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kc = 0; kc < KC; ++kc) {
                const int off = (cb * 16 + c16) * LD + kc * 32 + g * 8;
                const bf16x8 a0 = *reinterpret_cast<const bf16x8*>(&sa[0][off]);
                // smallest terms first
                acc = mfma16(a0, qb[2][kc], acc);
                acc = mfma16(a0, qb[1][kc], acc);
                if constexpr (KA == 3) {
                    const bf16x8 a1 = *reinterpret_cast<const bf16x8*>(&sa[1][off]);
                    const bf16x8 a2 = *reinterpret_cast<const bf16x8*>(&sa[KA - 1][off]);
                    acc = mfma16(a2, qb[0][kc], acc);
                    acc = mfma16(a1, qb[1][kc], acc);
                    acc = mfma16(a1, qb[0][kc], acc);
                }
                acc = mfma16(a0, qb[0][kc], acc);
            }
            // lane holds slots b0 + cb*16 + 4g + i for q-cluster a: one 16-byte
            // store (and one 16-byte read of the slot sizes) where the four fit
            if (aok) {
                float* dst = S + ((int64_t)bh * Cq + a) * Ck;
                const int b = b0 + cb * 16 + g * 4;
                const int32_t* ksz = k_sizes + (int64_t)bh * Ck;
                if (b + 3 < Ck && ((reinterpret_cast<uintptr_t>(dst + b) | reinterpret_cast<uintptr_t>(ksz + b)) & 15) == 0) {
                    const int4 ks = *reinterpret_cast<const int4*>(ksz + b);
                    float4 out;
                    out.x = (b < ncl && ks.x > 0) ? acc[0] : -INFINITY;
                    out.y = (b + 1 < ncl && ks.y > 0) ? acc[1] : -INFINITY;
                    out.z = (b + 2 < ncl && ks.z > 0) ? acc[2] : -INFINITY;
                    out.w = (b + 3 < ncl && ks.w > 0) ? acc[3] : -INFINITY;
                    *reinterpret_cast<float4*>(dst + b) = out;
                } else {
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        if (b + i < Ck) dst[b + i] = (b + i < ncl && ksz[b + i] > 0) ? acc[i] : -INFINITY;
                    }
                }
            }
        }
    }
}

hipError_t launch_scores(const Prob& p, int Cq, int Ck, const float* qrep, const void* kmax,
                         const void* kmin, const float* kcent, int score_mode,
                         const int32_t* k_sizes, const int32_t* n_clusters, float* S,
                         hipStream_t s) {
    dim3 grid((unsigned)((Cq + 63) / 64), (unsigned)((Ck + 255) / 256), (unsigned)p.BH);
    if (score_mode == 0) {
        if (p.bf16) {
            auto k = p.D == 64 ? scores_kernel<u16, 64, 0> : scores_kernel<u16, 128, 0>;
            hipLaunchKernelGGL(k, grid, dim3(256), 0, s, Cq, Ck, qrep, (const u16*)kmax,
                               (const u16*)kmin, kcent, k_sizes, n_clusters, S);
        } else {
            auto k = p.D == 64 ? scores_kernel<float, 64, 0> : scores_kernel<float, 128, 0>;
            hipLaunchKernelGGL(k, grid, dim3(256), 0, s, Cq, Ck, qrep, (const float*)kmax,
                               (const float*)kmin, kcent, k_sizes, n_clusters, S);
        }
    } else {
        auto k = p.D == 64 ? scores_kernel<float, 64, 1> : scores_kernel<float, 128, 1>;
        hipLaunchKernelGGL(k, grid, dim3(256), 0, s, Cq, Ck, qrep, (const float*)nullptr,
                           (const float*)nullptr, kcent, k_sizes, n_clusters, S);
    }
    return hipGetLastError();
}

// ------------------------------------------------------------------ block reductions
// Deterministic: per-thread partial, xor-butterfly inside each wave, then the
// four wave results added in wave order.
__device__ __forceinline__ float block_sum4(float v, float* red) {
    v = wave_sum(v);
    const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
    __syncthreads();
    if (l == 0) red[w] = v;
    __syncthreads();
    return ((red[0] + red[1]) + red[2]) + red[3];
}
__device__ __forceinline__ int block_sum4_i(int v, int* red) {
    v = wave_sum_i(v);
    const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
    __syncthreads();
    if (l == 0) red[w] = v;
    __syncthreads();
    return red[0] + red[1] + red[2] + red[3];
}
__device__ __forceinline__ float block_max4(float v, float* red) {
    v = wave_max(v);
    const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
    __syncthreads();
    if (l == 0) red[w] = v;
    __syncthreads();
    return fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

__device__ __forceinline__ uint32_t order_key(float f) {
    const uint32_t u = __float_as_uint(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
// inverse of order_key
__device__ __forceinline__ float key_value(uint32_t k) {
    return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// One workgroup (256 threads) per (head, q-cluster); thread t owns slots
// 32t .. 32t+31, i.e. mask word t.
template <bool TOPK>
__global__ __launch_bounds__(256) void select_kernel(int Cq, int Ck, const float* __restrict__ S,
                                                     const int32_t* __restrict__ k_sizes,
                                                     const int32_t* __restrict__ n_clusters,
                                                     const uint8_t* __restrict__ full, float scale,
                                                     float top_p, int top_k,
                                                     uint32_t* __restrict__ mask,
                                                     int32_t* __restrict__ sel_keys) {
    __shared__ float redf[4];
    __shared__ int redi[4];
    const int a = blockIdx.x, bh = blockIdx.y;
    const int t = threadIdx.x;
    const int words = (Ck + 31) / 32;
    const int ncl = min(n_clusters[bh], Ck);
    const float* row = S + ((int64_t)bh * Cq + a) * Ck;
    const int32_t* ks = k_sizes + (int64_t)bh * Ck;

    float lv[32];
    uint32_t live = 0;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
        const int b = t * 32 + i;
        const bool ok = t < words && b < ncl && ks[b] > 0;
        if (ok) live |= 1u << i;
        float v = -INFINITY;
        if (ok) v = TOPK ? row[b] : fmaf(row[b], scale, logf((float)ks[b]));
        lv[i] = v;
    }
    uint32_t selw = 0;
    const bool take_all = full[bh] || (!TOPK && top_p >= 1.0f);
    if (take_all) {
        selw = live;
    } else {
        // target: mass (top-p) or count (top-k) the selected set must reach
        float e[32];
        float target;
        if (TOPK) {
            const int nlive = block_sum4_i(__popc(live), redi);
            target = (float)min(top_k, nlive);
#pragma unroll
            for (int i = 0; i < 32; ++i) e[i] = ((live >> i) & 1) ? 1.0f : 0.0f;
        } else {
            float lmax = -INFINITY;
#pragma unroll
            for (int i = 0; i < 32; ++i) lmax = fmaxf(lmax, lv[i]);
            const float mx = block_max4(lmax, redf);
            float part = 0.0f;
#pragma unroll
            for (int i = 0; i < 32; ++i) {
                e[i] = ((live >> i) & 1) ? __expf(lv[i] - mx) : 0.0f;
                part += e[i];
            }
            const float Z = block_sum4(part, redf);
            target = top_p * Z;
        }
        uint32_t key[32];
#pragma unroll
        for (int i = 0; i < 32; ++i) key[i] = ((live >> i) & 1) ? order_key(lv[i]) : 0u;
        // largest T with mass(key >= T) >= target
        uint32_t T = 0;
        for (int bit = 31; bit >= 0; --bit) {
            const uint32_t cand = T | (1u << bit);
            float part = 0.0f;
#pragma unroll
            for (int i = 0; i < 32; ++i) part += key[i] >= cand ? e[i] : 0.0f;
            const float mass = block_sum4(part, redf);
            if (mass >= target) T = cand;
        }
        float above = 0.0f;
        int nties = 0;
        float e_tie = 0.0f;
#pragma unroll
        for (int i = 0; i < 32; ++i) {
            if (((live >> i) & 1) && key[i] > T) { selw |= 1u << i; above += e[i]; }
            if (((live >> i) & 1) && key[i] == T) { ++nties; e_tie = e[i]; }
        }
        const float mass_above = block_sum4(above, redf);
        // tied slots share one l, hence one e: take the first k of them in slot order
        __shared__ float sh_etie;
        __shared__ int sh_take;
        __shared__ int wpre[4];
        if (nties > 0) sh_etie = e_tie;
        int incl = nties;
        const int l = t & 63, w = t >> 6;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int v = __shfl_up(incl, o);
            if (l >= o) incl += v;
        }
        if (l == 63) wpre[w] = incl;
        __syncthreads();
        int before = incl - nties;
        for (int i = 0; i < w; ++i) before += wpre[i];
        const int ties = wpre[0] + wpre[1] + wpre[2] + wpre[3];
        if (t == 0) {
            int k = 0;
            float acc = mass_above;
            while (k < ties) {
                acc += sh_etie;
                ++k;
                if (acc >= target) break;
            }
            sh_take = k;
        }
        __syncthreads();
        const int take = sh_take;
        int rank = before;
#pragma unroll
        for (int i = 0; i < 32; ++i) {
            if (((live >> i) & 1) && key[i] == T) {
                if (rank < take) selw |= 1u << i;
                ++rank;
            }
        }
    }
    int keys = 0;
#pragma unroll
    for (int i = 0; i < 32; ++i)
        if ((selw >> i) & 1) keys += ks[t * 32 + i];
    const int total = block_sum4_i(keys, redi);
    if (t < words) mask[((int64_t)bh * Cq + a) * words + t] = selw;
    if (t == 0) sel_keys[(int64_t)bh * Cq + a] = total;
}

// One wave per (head, q-cluster) row for Ck <= 64 * SPL: lane j owns slots
// j + 64 i (i < SPL), so the slots of a mask word pair come out of one ballot.
// The same rule as select_kernel, with wave-level fixed-order sums (no
// workgroup barriers in the bisection); the last 16 of its 32 steps run over
// the few slots that can still move the cut.
// ln n_b of every slot with members (slots past the head's count or with no
// members: -inf), once per head instead of once per row.
__global__ __launch_bounds__(256) void ln_sizes_kernel(int Ck, const int32_t* __restrict__ k_sizes,
                                                       const int32_t* __restrict__ n_clusters,
                                                       float* __restrict__ ln_sizes) {
    const int bh = blockIdx.y;
    const int b = blockIdx.x * 256 + threadIdx.x;
    if (b >= Ck) return;
    const int n = b < min(n_clusters[bh], Ck) ? k_sizes[(int64_t)bh * Ck + b] : 0;
    ln_sizes[(int64_t)bh * Ck + b] = n > 0 ? logf((float)n) : -INFINITY;
}

template <bool TOPK, int SPL>
__global__ __launch_bounds__(256) void select_wave_kernel(int Cq, int Ck, const float* __restrict__ S,
                                                          const float* __restrict__ ln_sizes,
                                                          const int32_t* __restrict__ k_sizes,
                                                          const int32_t* __restrict__ n_clusters,
                                                          const uint8_t* __restrict__ full, float scale,
                                                          float top_p, int top_k,
                                                          uint32_t* __restrict__ mask,
                                                          int32_t* __restrict__ sel_keys) {
    __shared__ uint32_t bin_key[4][64];
    __shared__ float bin_e[4][64];
    const int bh = blockIdx.y;
    const int l = threadIdx.x & 63;
    const int a = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (a >= Cq) return;
    const int words = (Ck + 31) / 32;
    const float* row = S + ((int64_t)bh * Cq + a) * Ck;
    const float* lns = ln_sizes + (int64_t)bh * Ck;
    const int32_t* ks = k_sizes + (int64_t)bh * Ck;

    // keys (order-preserving integer images of l) are kept; l is recovered from
    // them, so a lane holds SPL keys and SPL weights
    uint32_t key[SPL];
    uint64_t live = 0;
    float lmax = -INFINITY;
#pragma unroll
    for (int i = 0; i < SPL; ++i) {
        const int b = l + 64 * i;
        const float ln = b < Ck ? lns[b] : -INFINITY;
        const bool ok = ln > -INFINITY;
        if (ok) live |= 1ull << i;
        float v = -INFINITY;
        if (ok) v = TOPK ? row[b] : fmaf(row[b], scale, ln);
        lmax = fmaxf(lmax, v);
        key[i] = ok ? order_key(v) : 0u;
    }
    uint64_t sel = 0;
    const bool take_all = full[bh] || (!TOPK && top_p >= 1.0f);
    if (take_all) {
        sel = live;
    } else {
        float e[SPL];
        float target;
        if (TOPK) {
            const int nlive = wave_sum_i(__popcll(live));
            target = (float)min(top_k, nlive);
#pragma unroll
            for (int i = 0; i < SPL; ++i) e[i] = ((live >> i) & 1) ? 1.0f : 0.0f;
        } else {
            const float mx = wave_max(lmax);
            float part = 0.0f;
#pragma unroll
            for (int i = 0; i < SPL; ++i) {
                e[i] = ((live >> i) & 1) ? __expf(key_value(key[i]) - mx) : 0.0f;
                part += e[i];
            }
            target = top_p * wave_sum_dpp(part);
        }
        // largest T with mass(key >= T) >= target: the top 16 bits by bisection
        // over every owned slot, then the low 16 bits over the slots whose top
        // bits equal T's (few: keys within 2^-7 relative of the cut), gathered
        // into a per-wave list in LDS
        uint32_t T = 0;
        for (int bit = 31; bit >= 16; --bit) {
            const uint32_t cand = T | (1u << bit);
            float part = 0.0f;
#pragma unroll
            for (int i = 0; i < SPL; ++i) part += key[i] >= cand ? e[i] : 0.0f;
            if (wave_sum_dpp(part) >= target) T = cand;
        }
        {
            const uint32_t hi = T >> 16;
            float part_hi = 0.0f;
            int nb = 0;
            uint32_t* lk = bin_key[threadIdx.x >> 6];
            float* le = bin_e[threadIdx.x >> 6];
            const uint64_t below = l == 0 ? 0ull : (~0ull >> (64 - l));
#pragma unroll
            for (int i = 0; i < SPL; ++i) {
                const bool lv = (live >> i) & 1;
                part_hi += (lv && (key[i] >> 16) > hi) ? e[i] : 0.0f;
                const bool in = lv && (key[i] >> 16) == hi;
                const uint64_t m = __ballot(in);
                const int pos = nb + __popcll(m & below);
                if (in && pos < 64) {
                    lk[pos] = key[i];
                    le[pos] = e[i];
                }
                nb += __popcll(m);
            }
            const float mass_hi = wave_sum_dpp(part_hi);
            if (nb <= 64) {
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
                __builtin_amdgcn_wave_barrier();
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
                const uint32_t mk = l < nb ? lk[l] : 0u;
                const float me = l < nb ? le[l] : 0.0f;
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
                __builtin_amdgcn_wave_barrier();
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
                for (int bit = 15; bit >= 0; --bit) {
                    const uint32_t cand = T | (1u << bit);
                    if (mass_hi + wave_sum_dpp(mk >= cand ? me : 0.0f) >= target) T = cand;
                }
            } else {
                for (int bit = 15; bit >= 0; --bit) {
                    const uint32_t cand = T | (1u << bit);
                    float part = 0.0f;
#pragma unroll
                    for (int i = 0; i < SPL; ++i) part += key[i] >= cand ? e[i] : 0.0f;
                    if (wave_sum_dpp(part) >= target) T = cand;
                }
            }
        }
        float above = 0.0f, e_tie = 0.0f;
        int nties = 0;
#pragma unroll
        for (int i = 0; i < SPL; ++i) {
            if (((live >> i) & 1) && key[i] > T) { sel |= 1ull << i; above += e[i]; }
            if (((live >> i) & 1) && key[i] == T) { ++nties; e_tie = e[i]; }
        }
        const float mass_above = wave_sum_dpp(above);
        const int ties = wave_sum_i(nties);
        // tied slots share one l, hence one e: take the first k of them in slot order
        const uint64_t has = __ballot(nties > 0);
        const float et = has ? __shfl(e_tie, __ffsll((unsigned long long)has) - 1) : 0.0f;
        int take = 0;
        {
            float acc = mass_above;
            while (take < ties) {
                acc += et;
                ++take;
                if (acc >= target) break;
            }
        }
        int before = 0;  // ties in slots before block i
        const uint64_t below = l == 0 ? 0ull : (~0ull >> (64 - l));
#pragma unroll
        for (int i = 0; i < SPL; ++i) {
            const bool tie = ((live >> i) & 1) && key[i] == T;
            const uint64_t tb = __ballot(tie);
            if (tie && before + __popcll(tb & below) < take) sel |= 1ull << i;
            before += __popcll(tb);
        }
    }
    int keys = 0;
#pragma unroll
    for (int i = 0; i < SPL; ++i) {
        const bool si = (sel >> i) & 1;
        if (si) keys += ks[l + 64 * i];
        const uint64_t wb = __ballot(si);
        const int wd = 2 * i + (l & 1);
        if (l < 2 && wd < words)
            mask[((int64_t)bh * Cq + a) * words + wd] = (uint32_t)(l ? (wb >> 32) : wb);
    }
    const int total = wave_sum_i(keys);
    if (l == 0) sel_keys[(int64_t)bh * Cq + a] = total;
}

template <bool TOPK>
static void launch_select_t(const Prob& p, int Cq, int Ck, const float* S, const int32_t* k_sizes,
                            const int32_t* n_clusters, const uint8_t* full, float scale,
                            float top_p, int top_k, uint32_t* mask, int32_t* sel_keys,
                            float* ln_sizes, hipStream_t s) {
    const dim3 wgrid((unsigned)((Cq + 3) / 4), (unsigned)p.BH);
    if (Ck <= 4096)
        hipLaunchKernelGGL(ln_sizes_kernel, dim3((unsigned)((Ck + 255) / 256), (unsigned)p.BH), dim3(256), 0,
                           s, Ck, k_sizes, n_clusters, ln_sizes);
    if (Ck <= 1024)
        hipLaunchKernelGGL((select_wave_kernel<TOPK, 16>), wgrid, dim3(256), 0, s, Cq, Ck, S, ln_sizes,
                           k_sizes, n_clusters, full, scale, top_p, top_k, mask, sel_keys);
    else if (Ck <= 4096)
        hipLaunchKernelGGL((select_wave_kernel<TOPK, 64>), wgrid, dim3(256), 0, s, Cq, Ck, S, ln_sizes,
                           k_sizes, n_clusters, full, scale, top_p, top_k, mask, sel_keys);
    else
        hipLaunchKernelGGL(select_kernel<TOPK>, dim3((unsigned)Cq, (unsigned)p.BH), dim3(256), 0, s,
                           Cq, Ck, S, k_sizes, n_clusters, full, scale, top_p, top_k, mask, sel_keys);
}

hipError_t launch_topp(const Prob& p, int Cq, int Ck, const float* S, const int32_t* k_sizes,
                       const int32_t* n_clusters, const uint8_t* full, float scale, float top_p,
                       uint32_t* mask, int32_t* sel_keys, float* ln_sizes, hipStream_t s) {
    launch_select_t<false>(p, Cq, Ck, S, k_sizes, n_clusters, full, scale, top_p, 0, mask, sel_keys,
                           ln_sizes, s);
    return hipGetLastError();
}

hipError_t launch_topk(const Prob& p, int Cq, int Ck, const float* S, const int32_t* k_sizes,
                       const int32_t* n_clusters, const uint8_t* full, int top_k, uint32_t* mask,
                       int32_t* sel_keys, float* ln_sizes, hipStream_t s) {
    launch_select_t<true>(p, Cq, Ck, S, k_sizes, n_clusters, full, 1.0f, 1.0f, top_k, mask, sel_keys,
                          ln_sizes, s);
    return hipGetLastError();
}

// ------------------------------------------------------------------ pairs
// Query-key pairs the attention will compute per head: sum over q-clusters of
// (members) x (selected keys), in int64, in a fixed order (per-thread strided
// sums, a wave butterfly, then the four waves in order).
__global__ __launch_bounds__(256) void pairs_kernel(int Cq, const int32_t* __restrict__ q_offsets,
                                                    const int32_t* __restrict__ sel_keys,
                                                    int64_t* __restrict__ pairs) {
    __shared__ long long part[4];
    const int bh = blockIdx.x;
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
    const int32_t* qo = q_offsets + (int64_t)bh * (Cq + 1);
    const int32_t* sk = sel_keys + (int64_t)bh * Cq;
    long long acc = 0;
    for (int a = tid; a < Cq; a += 256) acc += (long long)(qo[a + 1] - qo[a]) * (long long)sk[a];
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o);
    if (l == 0) part[w] = acc;
    __syncthreads();
    if (tid == 0) pairs[bh] = (int64_t)(part[0] + part[1] + part[2] + part[3]);
}

hipError_t launch_pairs(const Prob& p, int Cq, const int32_t* q_offsets, const int32_t* sel_keys,
                        int64_t* pairs, hipStream_t s) {
    hipLaunchKernelGGL(pairs_kernel, dim3((unsigned)p.BH), dim3(256), 0, s, Cq, q_offsets, sel_keys, pairs);
    return hipGetLastError();
}

}  // namespace adc
