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
// members; the cut value T (the l of the last selected slot) is the largest l
// whose mass, the sum of exp(l' - max l) over l' >= l, reaches top_p of the
// total; slots with l above T are selected, slots equal to T are taken in
// index order until the mass reaches top_p. Top-k takes the k largest scores
// by the same rule with unit weights.
#include <math.h>
#include <mutex>
#include "common.hpp"
#include "kernels.hpp"

namespace adc {

// Order-preserving 32-bit image of a float (larger float, larger image;
// never 0 for a non-NaN value, so 0 can mark a slot without members):
// negative values have every bit flipped, others only the sign bit.
__device__ __forceinline__ uint32_t order_key(float f) {
    const uint32_t u = __float_as_uint(f);
    return u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);
}
// inverse of order_key
__device__ __forceinline__ float key_value(uint32_t k) {
    return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// ------------------------------------------------------------------ scores
// A workgroup (4 waves, each 16 q-clusters) scores 64 q-clusters against a
// chunk of tpw consecutive 64-slot tiles of one head. The query side is split
// once and held in registers over the chunk; the key side of each tile is
// staged in LDS, the next tile's loads in flight while the current one is
// contracted.
//
// Work order. A column is (head, chunk): its nqb q-blocks all read the same
// key statistics. Block b runs on XCD b % 8 (round-robin dispatch); columns
// are dealt to the XCDs in turn and each XCD takes its columns one after
// another, q-blocks fastest, so the statistics of the few columns in flight
// on an XCD stay in its L2 while every q-block reads them.
//
// Output: the order key of what the selection ranks, per (q-cluster, slot):
// l = S * scale + ln n_b for top-p (LOGN), the score S itself for top-k; 0 for
// slots without members.
template <typename TK, int D, int MODE>
struct ScoreGeom {
    static constexpr int KD = MODE == 0 ? 2 * D : D;             // contraction width
    static constexpr int CPR = KD / 8;                           // 8-wide chunks per slot row
    static constexpr int RPP = 256 / CPR;                        // slot rows per workgroup pass
    static constexpr int NPASS = 64 / RPP;                       // passes per 64-slot tile
    static constexpr bool SPLIT = (MODE == 1) || sizeof(TK) == 4;  // key side needs a split
    static constexpr int RW = SPLIT ? 2 : 1;                     // 16-byte words per chunk
};

template <typename TK, int D, int MODE, bool LOGN>  // MODE 0: quest (width 2D), 1: centroid (width D)
__global__ __launch_bounds__(256) void scores_kernel(int Cq, int Ck, int nkc, int ncols, int nqb, int tpw,
                                                     const float* __restrict__ qrep,
                                                     const TK* __restrict__ kmax,
                                                     const TK* __restrict__ kmin,
                                                     const float* __restrict__ kcent,
                                                     const int32_t* __restrict__ k_sizes,
                                                     const int32_t* __restrict__ n_clusters,
                                                     float scale, uint32_t* __restrict__ keys) {
    using G = ScoreGeom<TK, D, MODE>;
    constexpr int KD = G::KD;
    constexpr int KC = KD / 32;
    constexpr int KA = G::SPLIT ? 3 : 1;
    constexpr int LD = KD + 8;
    __shared__ __attribute__((aligned(16))) u16 sa[KA][64 * LD];
    __shared__ __attribute__((aligned(16))) float lgn[64];      // ln n (top-p) or 0
    __shared__ __attribute__((aligned(16))) uint32_t lmask[64];  // ~0 for a slot with members

    const int xcd = blockIdx.x & 7, jb = blockIdx.x >> 3;
    const int cl = jb / nqb, qb = jb - cl * nqb;
    const int col = cl * 8 + xcd;
    if (col >= ncols) return;
    const int bh = col / nkc, chunk = col - bh * nkc;
    const int t0 = chunk * tpw;
    const int ntl = min(tpw, (Ck + 63) / 64 - t0);  // >= 1: chunk < nkc

    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, g = l >> 4, c16 = l & 15;
    const int a = qb * 64 + w * 16 + c16;
    const bool aok = a < Cq;
    const int ncl = min(n_clusters[bh], Ck);

    // key side: this thread's chunk column and its rows tid / CPR + RPP p
    const int col8 = tid % G::CPR, row0 = tid / G::CPR, k0 = col8 * 8;
    const TK* ksrc;
    if constexpr (MODE == 0) ksrc = (k0 < D ? kmax + k0 : kmin + (k0 - D)) + (int64_t)bh * Ck * D;
    else ksrc = reinterpret_cast<const TK*>(kcent + k0 + (int64_t)bh * Ck * D);
    u32x4 raw[G::NPASS * G::RW];
    // the key-side words of tile t of the chunk into raw (clamped to the last slot)
#define ADC_LOAD_TILE(t)                                                                   \
    do {                                                                                   \
        _Pragma("unroll") for (int ps = 0; ps < G::NPASS; ++ps) {                          \
            const int slot = min((t0 + (t)) * 64 + row0 + G::RPP * ps, Ck - 1);            \
            const u32x4* src = reinterpret_cast<const u32x4*>(ksrc + (int64_t)slot * D);   \
            _Pragma("unroll") for (int r = 0; r < G::RW; ++r) raw[ps * G::RW + r] = src[r]; \
        }                                                                                  \
    } while (0)
    ADC_LOAD_TILE(0);

    // query side: 3-term split of [q+, q-] (or q); each 8-wide chunk lies in
    // one half of the width, read as two 16-byte loads
    bf16x8 qb3[3][KC];
    const float* qp = qrep + ((int64_t)bh * Cq + (aok ? a : 0)) * D;
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
        const int q0 = kc * 32 + g * 8;
        float v[8];
        load8<float>(qp + (q0 < D ? q0 : q0 - D), v);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            float x = aok ? v[i] : 0.0f;
            if (MODE == 0) x = q0 < D ? fmaxf(x, 0.0f) : fminf(x, 0.0f);
            v[i] = x;
        }
        float r1[8], r2[8];
        qb3[0][kc] = pack_bf16x8(v);
#pragma unroll
        for (int i = 0; i < 8; ++i) r1[i] = v[i] - bf2f(qb3[0][kc][i]);
        qb3[1][kc] = pack_bf16x8(r1);
#pragma unroll
        for (int i = 0; i < 8; ++i) r2[i] = r1[i] - bf2f(qb3[1][kc][i]);
        qb3[2][kc] = pack_bf16x8(r2);
    }

    const int32_t* ksz = k_sizes + (int64_t)bh * Ck;
    uint32_t* const dst = keys + ((int64_t)bh * Cq + (aok ? a : 0)) * Ck;
    const bool vec4 = (Ck & 3) == 0;  // rows 16-byte aligned: whole 4-slot groups stored at once
    for (int t = 0; t < ntl; ++t) {
        const int b0 = (t0 + t) * 64;
        __syncthreads();  // the previous tile is no longer read
        if (tid < 64) {
            const int b = b0 + tid;
            const int n = b < Ck ? ksz[b] : 0;
            const bool live = b < ncl && n > 0;
            lgn[tid] = (live && LOGN) ? logf((float)n) : 0.0f;
            lmask[tid] = live ? ~0u : 0u;
        }
#pragma unroll
        for (int ps = 0; ps < G::NPASS; ++ps) {
            u16* d0 = &sa[0][(row0 + G::RPP * ps) * LD + k0];
            if constexpr (!G::SPLIT) {
                // bf16 statistics are copied as they are
                *reinterpret_cast<u32x4*>(d0) = raw[ps];
            } else {
                float v[8];
                if constexpr (G::RW == 2) {
                    const float4 x0 = __builtin_bit_cast(float4, raw[2 * ps]);
                    const float4 x1 = __builtin_bit_cast(float4, raw[2 * ps + 1]);
                    v[0] = x0.x; v[1] = x0.y; v[2] = x0.z; v[3] = x0.w;
                    v[4] = x1.x; v[5] = x1.y; v[6] = x1.z; v[7] = x1.w;
                } else {
                    const uint32_t wd[4] = {raw[ps].x, raw[ps].y, raw[ps].z, raw[ps].w};
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        v[2 * i] = __uint_as_float(wd[i] << 16);
                        v[2 * i + 1] = __uint_as_float(wd[i] & 0xFFFF0000u);
                    }
                }
                const bf16x8 s0 = pack_bf16x8(v);
                float r1[8], r2[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) r1[i] = v[i] - bf2f(s0[i]);
                const bf16x8 s1 = pack_bf16x8(r1);
#pragma unroll
                for (int i = 0; i < 8; ++i) r2[i] = r1[i] - bf2f(s1[i]);
                const int o = (row0 + G::RPP * ps) * LD + k0;
                *reinterpret_cast<bf16x8*>(&sa[0][o]) = s0;
                *reinterpret_cast<bf16x8*>(&sa[1][o]) = s1;
                *reinterpret_cast<bf16x8*>(&sa[KA - 1][o]) = pack_bf16x8(r2);
            }
        }
        __syncthreads();
        if (t + 1 < ntl) ADC_LOAD_TILE(t + 1);  // in flight during the contraction
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kc = 0; kc < KC; ++kc) {
                const int off = (cb * 16 + c16) * LD + kc * 32 + g * 8;
                const bf16x8 a0 = *reinterpret_cast<const bf16x8*>(&sa[0][off]);
                // smallest terms first
                acc = mfma16(a0, qb3[2][kc], acc);
                acc = mfma16(a0, qb3[1][kc], acc);
                if constexpr (KA == 3) {
                    const bf16x8 a1 = *reinterpret_cast<const bf16x8*>(&sa[1][off]);
                    const bf16x8 a2 = *reinterpret_cast<const bf16x8*>(&sa[KA - 1][off]);
                    acc = mfma16(a2, qb3[0][kc], acc);
                    acc = mfma16(a1, qb3[1][kc], acc);
                    acc = mfma16(a1, qb3[0][kc], acc);
                }
                acc = mfma16(a0, qb3[0][kc], acc);
            }
            // lane holds slots b0 + cb*16 + 4g + i for q-cluster a: one 16-byte
            // store where the four fit
            if (aok) {
                const int b = b0 + cb * 16 + g * 4;
                const float4 lg4 = *reinterpret_cast<const float4*>(&lgn[cb * 16 + g * 4]);
                const uint4 m4 = *reinterpret_cast<const uint4*>(&lmask[cb * 16 + g * 4]);
                uint4 out;
                out.x = order_key(LOGN ? fmaf(acc[0], scale, lg4.x) : acc[0]) & m4.x;
                out.y = order_key(LOGN ? fmaf(acc[1], scale, lg4.y) : acc[1]) & m4.y;
                out.z = order_key(LOGN ? fmaf(acc[2], scale, lg4.z) : acc[2]) & m4.z;
                out.w = order_key(LOGN ? fmaf(acc[3], scale, lg4.w) : acc[3]) & m4.w;
                if (vec4) {
                    if (b < Ck) *reinterpret_cast<uint4*>(dst + b) = out;
                } else {
                    const uint32_t o4[4] = {out.x, out.y, out.z, out.w};
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        if (b + i < Ck) dst[b + i] = o4[i];
                }
            }
        }
    }
}

#undef ADC_LOAD_TILE

hipError_t launch_scores(const Prob& p, int Cq, int Ck, const float* qrep, const void* kmax,
                         const void* kmin, const float* kcent, int score_mode, bool logn, float scale,
                         const int32_t* k_sizes, const int32_t* n_clusters, uint32_t* keys,
                         hipStream_t s) {
    // tiles per workgroup: the largest of 16, 8, 4, 2, 1 that still gives 2048
    // workgroups (the query split is amortised over the chunk; below that the
    // grid would not fill the chip)
    const int nqb = (Cq + 63) / 64;
    const int ntiles = (Ck + 63) / 64;
    int tpw = 16;
    while (tpw > 1 && (int64_t)p.BH * nqb * ((ntiles + tpw - 1) / tpw) < 2048) tpw >>= 1;
    const int nkc = (ntiles + tpw - 1) / tpw;
    const int ncols = p.BH * nkc;
    const dim3 grid((unsigned)(8 * ((ncols + 7) / 8) * nqb));
#define ADC_SCORES(TK, MODE, KMAX, KMIN)                                                              \
    do {                                                                                            \
        auto k = p.D == 64 ? (logn ? scores_kernel<TK, 64, MODE, true> : scores_kernel<TK, 64, MODE, false>)   \
                           : (logn ? scores_kernel<TK, 128, MODE, true> : scores_kernel<TK, 128, MODE, false>); \
        hipLaunchKernelGGL(k, grid, dim3(256), 0, s, Cq, Ck, nkc, ncols, nqb, tpw, qrep, (const TK*)(KMAX), \
                           (const TK*)(KMIN), kcent, k_sizes, n_clusters, scale, keys);               \
    } while (0)
    if (score_mode == 0) {
        if (p.bf16)
            ADC_SCORES(u16, 0, kmax, kmin);
        else
            ADC_SCORES(float, 0, kmax, kmin);
    } else {
        ADC_SCORES(float, 1, nullptr, nullptr);
    }
#undef ADC_SCORES
    return hipGetLastError();
}

// ------------------------------------------------------------------ top-p / top-k
// Wave reductions and scans on DPP row shifts and row broadcasts (no lane
// index arithmetic, nothing for the compiler to keep in registers). The scan
// is the inclusive Hillis-Steele sum inside each row of 16 lanes (lanes
// shifted in from outside the row read 0), then the row totals carried
// forward by the two row broadcasts; lane 63 ends with the total.
template <int CTRL, int ROWS>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, ROWS, 0xf, ROWS == 0xf);
}
template <int CTRL, int ROWS>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t v) {
    return ((uint64_t)dpp_u32<CTRL, ROWS>((uint32_t)(v >> 32)) << 32) | dpp_u32<CTRL, ROWS>((uint32_t)v);
}
__device__ __forceinline__ uint64_t wave_scan_u64(uint64_t v) {
    v += dpp_u64<0x111, 0xf>(v);  // row_shr:1
    v += dpp_u64<0x112, 0xf>(v);  // row_shr:2
    v += dpp_u64<0x114, 0xf>(v);  // row_shr:4
    v += dpp_u64<0x118, 0xf>(v);  // row_shr:8
    v += dpp_u64<0x142, 0xa>(v);  // row_bcast:15 into rows 1 and 3
    v += dpp_u64<0x143, 0xc>(v);  // row_bcast:31 into rows 2 and 3
    return v;
}
__device__ __forceinline__ uint64_t lane_u64(uint64_t v, int lane) {
    return ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(v >> 32), lane) << 32) |
           (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, lane);
}
__device__ __forceinline__ uint64_t wave_sum_u64(uint64_t v) { return lane_u64(wave_scan_u64(v), 63); }
__device__ __forceinline__ int wave_sum_i32(int v) {
    v += (int)dpp_u32<0x111, 0xf>((uint32_t)v);
    v += (int)dpp_u32<0x112, 0xf>((uint32_t)v);
    v += (int)dpp_u32<0x114, 0xf>((uint32_t)v);
    v += (int)dpp_u32<0x118, 0xf>((uint32_t)v);
    v += (int)dpp_u32<0x142, 0xa>((uint32_t)v);
    v += (int)dpp_u32<0x143, 0xc>((uint32_t)v);
    return __builtin_amdgcn_readlane(v, 63);
}
// max (unsigned) over the wave: shifted-in zeros are the identity
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
    v = max(v, dpp_u32<0x111, 0xf>(v));
    v = max(v, dpp_u32<0x112, 0xf>(v));
    v = max(v, dpp_u32<0x114, 0xf>(v));
    v = max(v, dpp_u32<0x118, 0xf>(v));
    v = max(v, dpp_u32<0x142, 0xa>(v));
    v = max(v, dpp_u32<0x143, 0xc>(v));
    return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// Selection by a mass histogram. A workgroup of W waves, W = ceil(Ck / 1024),
// takes the rows (q-clusters) a = blockIdx.x + gridDim.x j of head blockIdx.y
// one after another: thread t owns slots t + 64 W i (i < 16), so it holds 16
// keys of a row in registers (and the sizes of its slots, the same for every
// row of the head), each of the workgroup's loads of a row is contiguous, and
// the next row's keys are loaded while the current one is worked on.
//
// Weights are fixed point: e_b = exp(l_b - max l) as an integer multiple of
// 2^-31 (top-k: e_b = 1), so every mass below is an exact integer sum and the
// result does not depend on the order of the additions. The rule is the one
// stated above: T = the largest order key with mass(key >= T) >= target,
// target = top_p * Z (top-k: min(k, live slots)); keys above T are selected,
// keys equal to T in slot order until the mass reaches the target.
//
// 1. The live slots go into SEL_NB buckets by (max l - l) * width (the last
//    bucket takes everything further down), their weights summed per bucket
//    with LDS atomics (exact: integers).
// 2. Each wave scans the histogram for the cut bucket: the first whose
//    cumulative mass reaches the target. Buckets are monotone in l, so every
//    key of an earlier bucket is above every key of the cut bucket.
// 3. The cut bucket's slots (a few dozen, usually) are gathered in LDS; lane j
//    takes the j-th and sums the weights of the gathered keys >= its own,
//    which gives T directly. A cut bucket with more than SEL_LIST slots (many
//    keys within one bucket width) is settled by bisection over the 32-bit
//    images instead, with the same integer masses.
constexpr int SEL_NB = 1024;
constexpr int SEL_LIST = 64;
constexpr int SEL_KPL = 16;         // keys per thread
constexpr float SEL_WIDTH = 64.0f;  // buckets per unit of l

__device__ __forceinline__ uint32_t sel_weight(float v, float mx) {
    // exp(v - mx) in (0, 1] times 2^31, truncated (fits 32 bits)
    return (uint32_t)(__expf(v - mx) * 2147483648.0f);
}
__device__ __forceinline__ int sel_bucket(float v, float mx, float width) {
    const float x = (mx - v) * width;  // >= 0, monotone in v; NaN (no key) -> last
    return x < (float)(SEL_NB - 1) ? (int)x : SEL_NB - 1;
}

// At W = 8 (Ck > 4096) the registers are held to 128, so that two 8-wave
// workgroups fit a CU (measured 2.10 -> 1.90 ms over 49K rows of 8192 slots,
// though a few values spill; at W = 4 the same bound was slower).
template <bool TOPK, int W>
__global__ __launch_bounds__(64 * W) __attribute__((amdgpu_waves_per_eu(W == 8 ? 4 : 1, 8))) void select_hist_kernel(int Cq, int Ck, const uint32_t* __restrict__ K,
                                                             const int32_t* __restrict__ k_sizes,
                                                             const uint8_t* __restrict__ full, float scale,
                                                             float top_p, int top_k,
                                                             uint32_t* __restrict__ mask,
                                                             int32_t* __restrict__ sel_keys) {
    constexpr int NT = 64 * W;
    // histogram plus one spare counter per thread: the last bucket and the
    // slots without members go to the thread's spare, so no lane contends for
    // them; the spares are summed as the last bucket. Bucket k sits at
    // k + k / 16: lane l's 16 buckets in the scan are then 17 words apart, not
    // 16 (which put every lane on the same two banks).
    constexpr int HB = SEL_NB + SEL_NB / 16;  // padded buckets; spares follow
    __shared__ uint64_t H[HB + NT];
    __shared__ uint32_t LK[W][SEL_LIST];  // per wave: the cut bucket's keys,
    __shared__ uint32_t LE[W][SEL_LIST];  // weights
    __shared__ uint32_t LS[W][SEL_LIST];  // and slots, in the wave's slot order
    __shared__ uint64_t red64[2][W];
    __shared__ uint32_t redu[W];
    __shared__ int redi[W];
    __shared__ int redk[W];
    __shared__ int tcnt[W][SEL_KPL];
    __shared__ uint64_t mw[W][SEL_KPL];  // per wave: the mask ballots of a row
    __shared__ int sh_tie;
    const int bh = blockIdx.y;
    const int tid = threadIdx.x, w = tid >> 6;
    const int words = (Ck + 31) / 32;
    // top-k orders by the score itself and buckets by score * scale
    const float width = TOPK ? SEL_WIDTH * scale : SEL_WIDTH;
    const bool take_all = full[bh] || (!TOPK && top_p >= 1.0f);
    // Rows and sizes are read through buffer resources of one row (Ck words):
    // a slot past Ck reads 0 (no key, no members) without any per-slot test,
    // and the per-slot offsets are scalars, so no address registers are held.
    auto row_rsrc = [&](int r) __attribute__((always_inline)) {
        return __builtin_amdgcn_make_buffer_rsrc((void*)(K + ((int64_t)bh * Cq + r) * Ck), (short)0, Ck * 4,
                                                 0x00020000);
    };
    int ksz[SEL_KPL];
    uint32_t nxt[SEL_KPL];
    {
        const auto rs = __builtin_amdgcn_make_buffer_rsrc((void*)(k_sizes + (int64_t)bh * Ck), (short)0, Ck * 4,
                                                          0x00020000);
        const auto rk = row_rsrc(min((int)blockIdx.x, Cq - 1));
#pragma unroll
        for (int i = 0; i < SEL_KPL; ++i) {
            ksz[i] = (int)__builtin_amdgcn_raw_buffer_load_b32(rs, tid * 4, NT * i * 4, 0);
            nxt[i] = __builtin_amdgcn_raw_buffer_load_b32(rk, tid * 4, NT * i * 4, 0);
        }
    }
    for (int a = blockIdx.x; a < Cq; a += gridDim.x) {
    // thread indices hidden from the compiler per row, so that what derives
    // from them (slot numbers, LDS addresses, lane masks) is recomputed per row
    // instead of held in registers across the loop
    int tr = tid;
    asm volatile("" : "+v"(tr));
    const int lr = tr & 63;
    const uint64_t below_r = lr == 0 ? 0ull : (~0ull >> (64 - lr));
    // order keys of lr (0: no members, never selected)
    uint32_t key[SEL_KPL];
    uint32_t kmx = 0u;
    int nlive = 0;
#pragma unroll
    for (int i = 0; i < SEL_KPL; ++i) {
        key[i] = nxt[i];
        kmx = max(kmx, key[i]);
        nlive += key[i] != 0u;
    }
    if (a + (int)gridDim.x < Cq) {
        // the next row's keys, in flight while this row is worked on
        const auto rk = row_rsrc(a + gridDim.x);
#pragma unroll
        for (int i = 0; i < SEL_KPL; ++i) nxt[i] = __builtin_amdgcn_raw_buffer_load_b32(rk, tr * 4, NT * i * 4, 0);
    }
    for (int j = tr; j < HB + NT; j += NT) H[j] = 0ull;
    kmx = wave_max_u32(kmx);
    nlive = wave_sum_i32(nlive);
    if (lr == 0) {
        redu[w] = kmx;
        redi[w] = nlive;
    }
    __syncthreads();
    kmx = redu[0];
    nlive = redi[0];
#pragma unroll
    for (int v = 1; v < W; ++v) {
        kmx = max(kmx, redu[v]);
        nlive += redi[v];
    }
    const float mx = kmx ? key_value(kmx) : -INFINITY;

    // selected: key > T, or key == T in a slot up to last_tie
    uint32_t T = 1u;  // every live key is > 1: all of them
    int last_tie = -1;
    if (!(take_all || kmx == 0u)) {
        uint64_t zp = 0;
#pragma unroll
        for (int i = 0; i < SEL_KPL; ++i) {
            const bool lv = key[i] != 0u;
            const float v = key_value(key[i]);
            const uint32_t e = lv ? (TOPK ? 1u : sel_weight(v, mx)) : 0u;
            const int bk = sel_bucket(v, mx, width);
            zp += e;
            atomicAdd(reinterpret_cast<unsigned long long*>(&H[(lv && bk < SEL_NB - 1) ? bk + (bk >> 4) : HB + tr]),
                      (unsigned long long)e);
        }
        zp = wave_sum_u64(zp);
        if (lr == 0) red64[0][w] = zp;
        __syncthreads();
        uint64_t Z = 0, tail = 0;
#pragma unroll
        for (int v = 0; v < W; ++v) {
            Z += red64[0][v];
            tail += H[HB + 64 * v + lr];
        }
        tail = wave_sum_u64(tail);
        uint64_t tq;
        if (TOPK) {
            tq = (uint64_t)min(top_k, nlive);
        } else {
            tq = (uint64_t)ceil((double)top_p * (double)Z);
            tq = max(tq, (uint64_t)1);
        }
        // cut bucket (every wave alike): lane lr holds buckets 16 lr .. 16 lr + 15
        constexpr int PB = SEL_NB / 64;
        auto hval = [&](int j) __attribute__((always_inline)) -> uint64_t {
            const int bk = lr * PB + j;
            return bk == SEL_NB - 1 ? tail : H[bk + (bk >> 4)];
        };
        uint64_t part = 0;
#pragma unroll
        for (int j = 0; j < PB; ++j) part += hval(j);
        uint64_t c = wave_scan_u64(part) - part;
        int cut = SEL_NB;
        uint64_t before = 0;
#pragma unroll
        for (int j = 0; j < PB; ++j) {
            const uint64_t hj = hval(j);
            if (cut == SEL_NB && c + hj >= tq) {
                cut = lr * PB + j;
                before = c;
            }
            c += hj;
        }
        // the first lane with a cut (the totals reach Z >= tq, so one has)
        const uint64_t has_cut = __ballot(cut < SEL_NB);
        const int cl = (int)__ffsll((unsigned long long)has_cut) - 1;
        cut = __builtin_amdgcn_readlane(cut, cl);
        const uint64_t above = lane_u64(before, cl);

        // gather the cut bucket per wave, in the wave's slot order
        int nw = 0;
#pragma unroll
        for (int i = 0; i < SEL_KPL; ++i) {
            const float v = key_value(key[i]);
            const bool in = key[i] != 0u && sel_bucket(v, mx, width) == cut;
            const uint64_t m = __ballot(in);
            const int pos = nw + __popcll(m & below_r);
            if (in && pos < SEL_LIST) {
                LK[w][pos] = key[i];
                LE[w][pos] = TOPK ? 1u : sel_weight(v, mx);
                LS[w][pos] = (uint32_t)(tr + NT * i);
            }
            nw += __popcll(m);
        }
        if (lr == 0) redi[w] = nw;
        __syncthreads();
        int n = 0;
        int nv[W];
#pragma unroll
        for (int v = 0; v < W; ++v) {
            nv[v] = redi[v];
            n += nv[v];
        }
        uint64_t gt;    // mass of the keys above T
        uint64_t take;  // ties of T to take
        if (n <= SEL_LIST) {
            // lane j takes entry j of the waves' lists one after another
            // (every wave alike)
            uint32_t kj = 0u, ej = 0u, sj = 0u;
            {
                int off = 0;
#pragma unroll
                for (int v = 0; v < W; ++v) {
                    if (lr >= off && lr < off + nv[v]) {
                        kj = LK[v][lr - off];
                        ej = LE[v][lr - off];
                        sj = LS[v][lr - off];
                    }
                    off += nv[v];
                }
            }
            const bool has = lr < n;
            // weight of the gathered keys >= kj: entry i broadcast from lane i
            // (registers, no LDS round trip per entry)
            const int nu = __builtin_amdgcn_readfirstlane(n);
            uint64_t M = 0;
            for (int i = 0; i < nu; ++i) {
                const uint32_t ki = (uint32_t)__builtin_amdgcn_readlane((int)kj, i);
                const uint32_t ei = (uint32_t)__builtin_amdgcn_readlane((int)ej, i);
                M += ki >= kj ? (uint64_t)ei : 0ull;
            }
            T = wave_max_u32((has && above + M >= tq) ? kj : 0u);
            gt = above + wave_sum_u64((has && kj > T) ? (uint64_t)ej : 0ull);
            const uint64_t eT = TOPK ? 1ull : (uint64_t)sel_weight(key_value(T), mx);
            take = eT > 0 ? (tq - gt + eT - 1) / eT : ~0ull;
            // the take-th tie by slot: its rank among the ties is take - 1 (the
            // ties are the lanes holding T; usually one)
            const bool tie = has && kj == T;
            const uint64_t tmask = __ballot(tie);
            int rank = 0;
            for (uint64_t m = tmask; m; m &= m - 1) {
                const int i = (int)__ffsll((unsigned long long)m) - 1;
                rank += (uint32_t)__builtin_amdgcn_readlane((int)sj, i) < sj ? 1 : 0;
            }
            const uint64_t ntie = __popcll(tmask);
            if (take >= ntie) last_tie = Ck;
            else last_tie = (int)wave_max_u32((tie && (uint64_t)rank == take - 1) ? sj + 1 : 0u) - 1;
        } else {
            // bisection: the largest T whose mass (buckets above + the cut
            // bucket's keys >= T) reaches tq; T lies in the cut bucket
            T = 0u;
#pragma unroll 1
            for (int bit = 31; bit >= 0; --bit) {
                const uint32_t cand = T | (1u << bit);
                uint64_t mp = 0;
#pragma unroll
                for (int i = 0; i < SEL_KPL; ++i) {
                    const float v = key_value(key[i]);
                    const bool in = key[i] >= cand && sel_bucket(v, mx, width) == cut;
                    mp += in ? (TOPK ? 1u : sel_weight(v, mx)) : 0u;
                }
                mp = wave_sum_u64(mp);
                const int buf = bit & 1;  // alternate buffers: one barrier per step
                if (lr == 0) red64[buf][w] = mp;
                __syncthreads();
                uint64_t m = 0;
#pragma unroll
                for (int v = 0; v < W; ++v) m += red64[buf][v];
                if (above + m >= tq) T = cand;
            }
            uint64_t gp = 0;
#pragma unroll
            for (int i = 0; i < SEL_KPL; ++i) {
                const float v = key_value(key[i]);
                const bool in = key[i] > T && sel_bucket(v, mx, width) == cut;
                gp += in ? (TOPK ? 1u : sel_weight(v, mx)) : 0u;
            }
            gp = wave_sum_u64(gp);
            // tie counts per (wave, block) for the last tie taken
#pragma unroll
            for (int i = 0; i < SEL_KPL; ++i) {
                const int c2 = __popcll(__ballot(key[i] == T));
                if (lr == 0) tcnt[w][i] = c2;
            }
            __syncthreads();  // every wave has read red64[1] of the last step
            if (lr == 0) red64[1][w] = gp;
            __syncthreads();
            gt = above;
#pragma unroll
            for (int v = 0; v < W; ++v) gt += red64[1][v];
            const uint64_t eT = TOPK ? 1ull : (uint64_t)sel_weight(key_value(T), mx);
            take = eT > 0 ? (tq - gt + eT - 1) / eT : ~0ull;
            // slot order: block i, then wave, then lane
            uint64_t seen = 0;
            int fi = -1, fw = -1;
            uint64_t r = 0;
            for (int i = 0; i < SEL_KPL && fi < 0; ++i)
                for (int v = 0; v < W && fi < 0; ++v) {
                    const uint64_t c2 = (uint64_t)tcnt[v][i];
                    if (seen + c2 >= take) {
                        fi = i;
                        fw = v;
                        r = take - seen;
                    }
                    seen += c2;
                }
            if (fi < 0) {
                last_tie = Ck;  // fewer ties than take: all of them
            } else {
                if (w == fw) {
                    // the r-th tie of this wave's block fi
                    uint64_t mm = 0;
#pragma unroll
                    for (int i = 0; i < SEL_KPL; ++i) {
                        const uint64_t bb = __ballot(key[i] == T);
                        if (i == fi) mm = bb;
                    }
                    for (uint64_t q = r; q > 1; --q) mm &= mm - 1;
                    if (lr == 0) sh_tie = NT * fi + 64 * fw + (int)__ffsll((unsigned long long)mm) - 1;
                }
                __syncthreads();
                last_tie = sh_tie;
            }
        }
    }
    // mark: key > T, or key == T up to the last tie taken. Wave w's ballot over
    // block i is mask word 2 W i + 2 w + h (half h): staged in LDS, then lane
    // 2 i + h stores it.
    int keys = 0;
#pragma unroll
    for (int i = 0; i < SEL_KPL; ++i) {
        const int b = tr + NT * i;
        const bool si = key[i] > T || (key[i] == T && b <= last_tie);
        keys += si ? ksz[i] : 0;
        const uint64_t wb = __ballot(si);
        if (lr == 0) mw[w][i] = wb;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    if (lr < 2 * SEL_KPL) {
        const int wd = 2 * W * (lr >> 1) + 2 * w + (lr & 1);
        if (wd < words) mask[((int64_t)bh * Cq + a) * words + wd] = reinterpret_cast<const uint32_t*>(mw[w])[lr];
    }
    keys = wave_sum_i32(keys);
    if (lr == 0) redk[w] = keys;
    // also the end of every use of this row's shared data
    __syncthreads();
    if (tr == 0) {
        int total = 0;
#pragma unroll
        for (int v = 0; v < W; ++v) total += redk[v];
        sel_keys[(int64_t)bh * Cq + a] = total;
    }
    }
}

// Workgroups of `threads` threads of kernel k resident at once on the current
// device (its compute units times what registers and LDS allow per unit);
// found once per (kernel, device).
static int resident_blocks(const void* k, int threads) {
    struct Entry { const void* k; int dev, n; };
    static Entry cache[64];
    static int used = 0;
    static std::mutex mu;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) dev = 0;
    std::lock_guard<std::mutex> lock(mu);
    for (int i = 0; i < used; ++i)
        if (cache[i].k == k && cache[i].dev == dev) return cache[i].n;
    int cus = 256, per_cu = 1, n = 0, b = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0) cus = n;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&b, k, threads, 0) == hipSuccess && b > 0) per_cu = b;
    if (used < 64) cache[used++] = Entry{k, dev, cus * per_cu};
    return cus * per_cu;
}

template <bool TOPK>
static void launch_select_t(const Prob& p, int Cq, int Ck, const uint32_t* keys, const int32_t* k_sizes,
                            const uint8_t* full, float scale, float top_p, int top_k, uint32_t* mask,
                            int32_t* sel_keys, hipStream_t s) {
    const int W = (Ck + 64 * SEL_KPL - 1) / (64 * SEL_KPL);
    // as many workgroups of W waves as are resident at once over the chip
    // (no second, partly filled round), each over a strided share of one
    // head's rows
#define ADC_SEL(WW)                                                                                      \
    do {                                                                                                 \
        auto k = select_hist_kernel<TOPK, WW>;                                                           \
        const int per_head = max(1, min(Cq, resident_blocks((const void*)k, 64 * WW) / p.BH));          \
        hipLaunchKernelGGL(k, dim3((unsigned)per_head, (unsigned)p.BH), dim3(64 * WW), 0, s, Cq, Ck,    \
                           keys, k_sizes, full, scale, top_p, top_k, mask, sel_keys);                    \
    } while (0)
    if (W <= 1)
        ADC_SEL(1);
    else if (W <= 2)
        ADC_SEL(2);
    else if (W <= 4)
        ADC_SEL(4);
    else
        ADC_SEL(8);
#undef ADC_SEL
}

hipError_t launch_topp(const Prob& p, int Cq, int Ck, const uint32_t* keys, const int32_t* k_sizes,
                       const uint8_t* full, float top_p, uint32_t* mask, int32_t* sel_keys, hipStream_t s) {
    launch_select_t<false>(p, Cq, Ck, keys, k_sizes, full, 1.0f, top_p, 0, mask, sel_keys, s);
    return hipGetLastError();
}

hipError_t launch_topk(const Prob& p, int Cq, int Ck, const uint32_t* keys, const int32_t* k_sizes,
                       const uint8_t* full, float scale, int top_k, uint32_t* mask, int32_t* sel_keys,
                       hipStream_t s) {
    launch_select_t<true>(p, Cq, Ck, keys, k_sizes, full, scale, 1.0f, top_k, mask, sel_keys, s);
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
