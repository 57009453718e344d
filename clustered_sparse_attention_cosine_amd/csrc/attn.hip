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
// Work items (q-cluster a, chunk c of ATTN_ROWS rows) of head bh are written in
// q-cluster order to items[bh * cap ...] (cap = Cq + ceil(N / ATTN_ROWS) bounds
// their number), one workgroup per head. Launching the attention grid over
// heads in order keeps the workgroups in flight on one or two heads at a time,
// so their K'/V' stay in the last-level cache.
__global__ __launch_bounds__(256) void worklist_kernel(int Cq, int cap,
                                                       const int32_t* __restrict__ q_offsets,
                                                       int32_t* __restrict__ items,
                                                       int32_t* __restrict__ n_items) {
    __shared__ int wsum[4];
    const int bh = blockIdx.x;
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
    const int32_t* qo = q_offsets + (int64_t)bh * (Cq + 1);
    int32_t* out = items + (int64_t)bh * cap;
    int running = 0;
    for (int base = 0; base < Cq; base += 256) {
        const int a = base + tid;
        const int ch = a < Cq ? (qo[a + 1] - qo[a] + ATTN_ROWS - 1) / ATTN_ROWS : 0;
        int incl = ch;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int v = __shfl_up(incl, o);
            if (l >= o) incl += v;
        }
        if (l == 63) wsum[w] = incl;
        __syncthreads();
        int before = running + incl - ch;
        for (int i = 0; i < w; ++i) before += wsum[i];
        for (int c = 0; c < ch; ++c) out[before + c] = a | (c << 16);
        running += wsum[0] + wsum[1] + wsum[2] + wsum[3];
        __syncthreads();
    }
    if (tid == 0) n_items[bh] = running;
}

hipError_t launch_worklist(const Prob& p, int Cq, int cap, const int32_t* q_offsets,
                           int32_t* items, int32_t* n_items, hipStream_t s) {
    hipLaunchKernelGGL(worklist_kernel, dim3((unsigned)p.BH), dim3(256), 0, s, Cq, cap, q_offsets,
                       items, n_items);
    return hipGetLastError();
}

// ------------------------------------------------------------------ attention
// 8 consecutive elements as packed bf16 words: the value (hi) and, for f32
// inputs, the rounding residual (lo), so f32 data is carried as hi + lo.
template <typename T>
__device__ __forceinline__ void load_row8_split(const T* p, bool ok, uint32_t (&hi)[4],
                                                uint32_t (&lo)[4]);
// The load is unconditional (p must be a valid address; callers clamp it) and
// `ok` only selects zeros, so no branch hides the load from the counters.
template <>
__device__ __forceinline__ void load_row8_split<u16>(const u16* p, bool ok, uint32_t (&hi)[4],
                                                     uint32_t (&lo)[4]) {
    const uint4 r = *reinterpret_cast<const uint4*>(p);
    hi[0] = ok ? r.x : 0u;
    hi[1] = ok ? r.y : 0u;
    hi[2] = ok ? r.z : 0u;
    hi[3] = ok ? r.w : 0u;
    lo[0] = lo[1] = lo[2] = lo[3] = 0;
}
template <>
__device__ __forceinline__ void load_row8_split<float>(const float* p, bool ok, uint32_t (&hi)[4],
                                                       uint32_t (&lo)[4]) {
    float v[8];
    load8<float>(p, v);
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = ok ? v[i] : 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const u16 h0 = f2bf_bits(v[2 * i]), h1 = f2bf_bits(v[2 * i + 1]);
        const u16 l0 = f2bf_bits(v[2 * i] - bf_bits2f(h0));
        const u16 l1 = f2bf_bits(v[2 * i + 1] - bf_bits2f(h1));
        hi[i] = (uint32_t)h0 | ((uint32_t)h1 << 16);
        lo[i] = (uint32_t)l0 | ((uint32_t)l1 << 16);
    }
}

// Window of 64 runs starting at run r0, loaded by one wave: lane k fetches the
// first position and first key row of run r0 + k, and every lane the first
// position of run r0 + 64. Loads are clamped and unconditional; validity is
// applied where the values are used (tile_rows), so nothing waits here.
struct RunWindow {
    int r0, vp, vs, v64;
};

__device__ __forceinline__ void load_window(int lane, int r0, int R, const int32_t* rs,
                                            const int32_t* rp, RunWindow& wd) {
    const int k = r0 + lane;
    wd.r0 = r0;
    wd.vp = rp[min(k, R)];
    wd.vs = rs[max(min(k, R - 1), 0)];
    wd.v64 = rp[min(r0 + 64, R)];
}

// Key rows of one 64-position tile of the concatenated selection, computed by
// one wave without LDS. Lane k holds run r0 + k: its first position wp
// (INT_MAX past the last run) and first key row ws; run r0 holds position t0.
// The run holding position t0 + lane is (number of run starts <= t0 + lane) - 1,
// counted from a 64-bit mask of the starts inside the tile. Writes krow[lane]
// (-1 past the selection) and returns the run holding position t0 + 64.
__device__ __forceinline__ int tile_rows(int lane, int t0, int total, int R, const RunWindow& wd,
                                         int* krow, bool write) {
    const int r0 = wd.r0;
    const int wp = r0 + lane <= R ? wd.vp : 0x7fffffff;
    const int ws = r0 + lane < R ? wd.vs : 0;
    const int wp64 = r0 + 64 <= R ? wd.v64 : 0x7fffffff;
    const int s = wp - t0;
    uint32_t lo = 0, hi = 0;
    if (lane == 0) lo = 1u;
    if (s >= 0 && s < 32) lo |= 1u << s;
    else if (s >= 32 && s < 64) hi |= 1u << (s - 32);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        lo |= __shfl_xor(lo, o);
        hi |= __shfl_xor(hi, o);
    }
    const uint64_t starts = ((uint64_t)hi << 32) | lo;
    const uint64_t upto = lane == 63 ? ~0ull : ((2ull << lane) - 1ull);
    const int k = __popcll(starts & upto) - 1;
    const int rs_k = __shfl(ws, k), rp_k = __shfl(wp, k);
    const int P = t0 + lane;
    if (write) krow[lane] = P < total ? rs_k + (P - rp_k) : -1;
    const int c = __popcll(__ballot(wp <= t0 + 64));
    return (c == 64 && wp64 <= t0 + 64) ? r0 + 64 : r0 + c - 1;
}

// Raw 16-byte chunk: 8 bf16 words (4 registers) or 8 floats (8 registers).
template <typename T> struct Raw8 { uint32_t w[4]; };
template <> struct Raw8<float> { uint32_t w[8]; };

template <typename T>
__device__ __forceinline__ void load_raw8(const T* p, Raw8<T>& r) {
    const uint4 a = *reinterpret_cast<const uint4*>(p);
    r.w[0] = a.x; r.w[1] = a.y; r.w[2] = a.z; r.w[3] = a.w;
    if constexpr (sizeof(T) == 4) {
        const uint4 b = *reinterpret_cast<const uint4*>(p + 4);
        r.w[4] = b.x; r.w[5] = b.y; r.w[6] = b.z; r.w[7] = b.w;
    }
}

// Raw chunk -> packed bf16 words (hi) and, for f32, the rounding residual (lo).
template <typename T>
__device__ __forceinline__ void split_raw8(const Raw8<T>& r, bool ok, uint32_t (&hi)[4],
                                           uint32_t (&lo)[4]) {
    if constexpr (sizeof(T) == 2) {
#pragma unroll
        for (int i = 0; i < 4; ++i) { hi[i] = ok ? r.w[i] : 0u; lo[i] = 0u; }
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float v0 = ok ? __uint_as_float(r.w[2 * i]) : 0.0f;
            const float v1 = ok ? __uint_as_float(r.w[2 * i + 1]) : 0.0f;
            const u16 h0 = f2bf_bits(v0), h1 = f2bf_bits(v1);
            const u16 l0 = f2bf_bits(v0 - bf_bits2f(h0)), l1 = f2bf_bits(v1 - bf_bits2f(h1));
            hi[i] = (uint32_t)h0 | ((uint32_t)h1 << 16);
            lo[i] = (uint32_t)l0 | ((uint32_t)l1 << 16);
        }
    }
}

// Global -> register staging of one K/V tile (64 key rows), NT threads. Loads
// are issued unconditionally from clamped rows and held raw; masking and
// conversion happen in tile_store, so the loads stay in flight until then.
template <typename T, int D, int NT>
struct TileRegs {
    static constexpr int KTASK = 64 * (D / 8);      // 16-byte chunks of the K tile
    static constexpr int VTASK = 32 * (D / 8);      // (key pair, 8 dims) tasks of the V tile
    static constexpr int KT = (KTASK + NT - 1) / NT;
    static constexpr int VT = (VTASK + NT - 1) / NT;
    Raw8<T> k[KT];
    Raw8<T> va[VT], vb[VT];
    bool aok[VT], bok[VT];
};

template <typename T, int D, int NT>
__device__ __forceinline__ void tile_load(TileRegs<T, D, NT>& r, int tid, const int* krow,
                                          const T* Kh, const T* Vh) {
    // krow entries are -1 (past the selection) or key rows of this head
    using TR = TileRegs<T, D, NT>;
#pragma unroll
    for (int i = 0; i < TR::KT; ++i) {
        const int c = tid + i * NT;
        if (TR::KTASK % NT != 0 && c >= TR::KTASK) break;
        const int kr = c / (D / 8), c8 = c % (D / 8);
        const int row = krow[kr];
        load_raw8<T>(Kh + (int64_t)(row < 0 ? 0 : row) * D + c8 * 8, r.k[i]);
    }
#pragma unroll
    for (int i = 0; i < TR::VT; ++i) {
        const int c = tid + i * NT;
        if (TR::VTASK % NT != 0 && c >= TR::VTASK) break;
        const int kk = c % 32, c8 = c / 32;
        const int ra = krow[2 * kk], rb = krow[2 * kk + 1];
        r.aok[i] = ra >= 0;
        r.bok[i] = rb >= 0;
        load_raw8<T>(Vh + (int64_t)(ra < 0 ? 0 : ra) * D + c8 * 8, r.va[i]);
        load_raw8<T>(Vh + (int64_t)(rb < 0 ? 0 : rb) * D + c8 * 8, r.vb[i]);
    }
}

// Register -> LDS: K row-major, V transposed (fp16 for bf16 inputs, bf16 hi/lo for f32).
template <typename T, int D, int NP, int NT, int LDK, int LDV>
__device__ __forceinline__ void tile_store(const TileRegs<T, D, NT>& r, int tid,
                                           u16 (*Ks)[64 * LDK], u16 (*Vt)[D * LDV]) {
    using TR = TileRegs<T, D, NT>;
    constexpr bool PREC = NP == 2;
#pragma unroll
    for (int i = 0; i < TR::KT; ++i) {
        const int c = tid + i * NT;
        if (TR::KTASK % NT != 0 && c >= TR::KTASK) break;
        const int kr = c / (D / 8), c8 = c % (D / 8);
        uint32_t hv[4], lv[4];
        split_raw8<T>(r.k[i], true, hv, lv);
        *reinterpret_cast<uint4*>(&Ks[0][kr * LDK + c8 * 8]) = make_uint4(hv[0], hv[1], hv[2], hv[3]);
        if constexpr (PREC)
            *reinterpret_cast<uint4*>(&Ks[NP - 1][kr * LDK + c8 * 8]) = make_uint4(lv[0], lv[1], lv[2], lv[3]);
    }
#pragma unroll
    for (int i = 0; i < TR::VT; ++i) {
        const int c = tid + i * NT;
        if (TR::VTASK % NT != 0 && c >= TR::VTASK) break;
        const int kk = c % 32, c8 = c / 32;
        uint32_t va[2][4], vb[2][4];
        split_raw8<T>(r.va[i], r.aok[i], va[0], va[1]);
        split_raw8<T>(r.vb[i], r.bok[i], vb[0], vb[1]);
#pragma unroll
        for (int pp = 0; pp < NP; ++pp)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint32_t a = va[pp][j], b = vb[pp][j];
                uint32_t lo_w, hi_w;
                if constexpr (PREC) {
                    lo_w = (a & 0xFFFFu) | (b << 16);
                    hi_w = (a >> 16) | (b & 0xFFFF0000u);
                } else {
                    // bf16 -> fp16 is exact for |v| inside the fp16 normal range
                    lo_w = pack_h2(__uint_as_float(a << 16), __uint_as_float(b << 16));
                    hi_w = pack_h2(__uint_as_float(a & 0xFFFF0000u), __uint_as_float(b & 0xFFFF0000u));
                }
                *reinterpret_cast<uint32_t*>(&Vt[pp][(c8 * 8 + 2 * j) * LDV + 2 * kk]) = lo_w;
                *reinterpret_cast<uint32_t*>(&Vt[pp][(c8 * 8 + 2 * j + 1) * LDV + 2 * kk]) = hi_w;
            }
    }
}

// Online-softmax update of one 16-query block over one 64-key tile (the lane
// holds query c16 and keys kb*16 + 4g + i). Scores come in raw; sl2 = scale *
// log2(e) is applied inside the exponent.
template <int DB>
__device__ __forceinline__ void softmax_block(f32x4 (&sc)[4], float sl2, bool mask_tail, int t0,
                                              int g, int total, float& m_run, float& l_part,
                                              f32x4 (&o)[DB]) {
    if (mask_tail) {
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (t0 + kb * 16 + g * 4 + i >= total) sc[kb][i] = -INFINITY;
    }
    float mx = fmaxf(fmaxf(sc[0][0], sc[0][1]), fmaxf(sc[0][2], sc[0][3]));
#pragma unroll
    for (int kb = 1; kb < 4; ++kb)
        mx = fmaxf(mx, fmaxf(fmaxf(sc[kb][0], sc[kb][1]), fmaxf(sc[kb][2], sc[kb][3])));
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx * sl2);
    const float base = (m_new == -INFINITY) ? 0.0f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m_run - base);
    float lsum = 0.0f;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float pv = __builtin_amdgcn_exp2f(fmaf(sc[kb][i], sl2, -base));
            sc[kb][i] = pv;
            lsum += pv;
        }
    l_part = fmaf(l_part, alpha, lsum);
    if (alpha != 1.0f) {
#pragma unroll
        for (int db = 0; db < DB; ++db) o[db] *= alpha;
    }
    m_run = m_new;
}

// A work item is (head, q-cluster, chunk of ATTN_ROWS query rows); the NT/64
// waves each own RB blocks of 16 rows (a block with no rows is skipped). K/V
// tiles of 64 keys are double-buffered in LDS: the global loads of tile t+1
// are in flight while tile t is computed, and the key rows of tile t+2 are
// looked up by wave 0 at the same time, so one barrier per tile suffices.
// PREC (f32 inputs): operands carried as bf16 hi + lo and every product of
// order <= 1 accumulated (3 MFMAs per product instead of 1), near f32 accuracy.
template <typename T, int D, typename TO, int NT, int RB>
__global__ __launch_bounds__(NT) void attn_kernel(int N, int Cq, const T* __restrict__ Q,
                                                  const int32_t* __restrict__ q_perm,
                                                  const int32_t* __restrict__ q_off,
                                                  const T* __restrict__ Kp, const T* __restrict__ Vp,
                                                  const int32_t* __restrict__ run_start,
                                                  const int32_t* __restrict__ run_pos,
                                                  const int32_t* __restrict__ n_runs, int run_cap,
                                                  const int32_t* __restrict__ items,
                                                  const int32_t* __restrict__ n_items, int cap,
                                                  float sl2, TO* __restrict__ O,
                                                  float* __restrict__ lse) {
    static_assert((NT / 64) * RB * 16 == ATTN_ROWS, "waves x blocks must cover a work item");
    constexpr bool PREC = sizeof(T) == 4;
    constexpr int NP = PREC ? 2 : 1;  // stored parts per operand
    constexpr int KC = D / 32;        // 32-wide chunks of the head dimension
    constexpr int DB = D / 16;        // 16-row blocks of O^T
    constexpr int LDK = D + 8;        // padded LDS strides (elements)
    constexpr int LDV = 64 + 8;
    __shared__ __attribute__((aligned(16))) u16 Ks[2][NP][64 * LDK];
    __shared__ __attribute__((aligned(16))) u16 Vt[2][NP][D * LDV];
    __shared__ int krow[4][64];

    const int bh = blockIdx.x / cap;
    if ((int)(blockIdx.x % cap) >= n_items[bh]) return;
    const int packed = items[blockIdx.x];
    const int a = packed & 0xFFFF, ch = packed >> 16;
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, g = l >> 4, c16 = l & 15;

    const int32_t* qo = q_off + (int64_t)bh * (Cq + 1);
    const int row0 = qo[a] + ch * ATTN_ROWS;
    const int nrows = min(ATTN_ROWS, qo[a + 1] - row0);
    bool live[RB];
    bf16x8 qf[RB][NP][KC];
    int64_t qtok[RB];
    bool qok[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        live[rb] = (w * RB + rb) * 16 < nrows;
        const int rowi = (w * RB + rb) * 16 + c16;
        qok[rb] = rowi < nrows;
        qtok[rb] = qok[rb] ? q_perm[(int64_t)bh * N + row0 + rowi] : 0;
        const T* qr = Q + ((int64_t)bh * N + qtok[rb]) * D;
#pragma unroll
        for (int kc = 0; kc < KC; ++kc) {
            uint32_t hv[4], lv[4];
            load_row8_split<T>(qr + kc * 32 + g * 8, qok[rb], hv, lv);
            qf[rb][0][kc] = __builtin_bit_cast(bf16x8, make_uint4(hv[0], hv[1], hv[2], hv[3]));
            if constexpr (PREC)
                qf[rb][NP - 1][kc] = __builtin_bit_cast(bf16x8, make_uint4(lv[0], lv[1], lv[2], lv[3]));
        }
    }

    const int64_t rbase = (int64_t)bh * Cq + a;
    const int R = n_runs[rbase];
    const int32_t* rs = run_start + rbase * run_cap;
    const int32_t* rp = run_pos + rbase * (run_cap + 1);
    const int total = rp[R];
    const int ntiles = (total + 63) / 64;
    const T* Kh = Kp + (int64_t)bh * N * D;
    const T* Vh = Vp + (int64_t)bh * N * D;

    float m_run[RB], l_part[RB];
    f32x4 o[RB][DB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        m_run[rb] = -INFINITY;
        l_part[rb] = 0.0f;
#pragma unroll
        for (int db = 0; db < DB; ++db) o[rb][db] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    // Key rows are looked up three tiles ahead; tiles t+1 and t+2 are in flight
    // in two register sets while tile t is computed from LDS. Every wave issues
    // the same loads every step (tiles past the end read clamped, valid rows and
    // are never used) so the load counters stay exact and no wait reaches back
    // past the tile being consumed. Every wave computes the row lookup; wave 0
    // writes it.
    RunWindow wd;
    load_window(l, 0, R, rs, rp, wd);
    int r_next = tile_rows(l, 0, total, R, wd, krow[0], w == 0);
#pragma unroll
    for (int j = 1; j < 3; ++j) {
        load_window(l, r_next, R, rs, rp, wd);
        r_next = tile_rows(l, j * 64, total, R, wd, krow[j], w == 0);
    }
    load_window(l, r_next, R, rs, rp, wd);
    __syncthreads();
    TileRegs<T, D, NT> tr0, tr1;
    tile_load<T, D, NT>(tr0, tid, krow[0], Kh, Vh);
    tile_load<T, D, NT>(tr1, tid, krow[1], Kh, Vh);
    tile_store<T, D, NP, NT, LDK, LDV>(tr0, tid, Ks[0], Vt[0]);
    __syncthreads();

    // one tile: look up t+3, prefetch t+2 into the register set tile t used,
    // compute t, store t+1 into the other LDS buffer
    auto step = [&](int t, auto& tr_mine, auto& tr_next) {
        const int b = t & 1;
        const int t0 = t * 64;
        const int rn = tile_rows(l, t0 + 192, total, R, wd, krow[(t + 3) & 3], w == 0);
        load_window(l, rn, R, rs, rp, wd);
        tile_load<T, D, NT>(tr_mine, tid, krow[(t + 2) & 3], Kh, Vh);
        if (t < ntiles && live[0]) {
                const bool mask_tail = t0 + 64 > total;
                f32x4 sc[RB][4];
    #pragma unroll
                for (int kb = 0; kb < 4; ++kb) {
    #pragma unroll
                    for (int rb = 0; rb < RB; ++rb) sc[rb][kb] = f32x4{0.f, 0.f, 0.f, 0.f};
    #pragma unroll
                    for (int kc = 0; kc < KC; ++kc) {
                        const int off = (kb * 16 + c16) * LDK + kc * 32 + g * 8;
                        const bf16x8 ka = *reinterpret_cast<const bf16x8*>(&Ks[b][0][off]);
                        bf16x8 kl;
                        if constexpr (PREC) kl = *reinterpret_cast<const bf16x8*>(&Ks[b][NP - 1][off]);
    #pragma unroll
                        for (int rb = 0; rb < RB; ++rb) {
                            if (rb > 0 && !live[rb]) continue;
                            if constexpr (PREC) {
                                sc[rb][kb] = mfma16(kl, qf[rb][0][kc], sc[rb][kb]);
                                sc[rb][kb] = mfma16(ka, qf[rb][NP - 1][kc], sc[rb][kb]);
                            }
                            sc[rb][kb] = mfma16(ka, qf[rb][0][kc], sc[rb][kb]);
                        }
                    }
                }
    #pragma unroll
                for (int rb = 0; rb < RB; ++rb) {
                    if (rb > 0 && !live[rb]) continue;
                    softmax_block<DB>(sc[rb], sl2, mask_tail, t0, g, total, m_run[rb], l_part[rb], o[rb]);
                }
    #pragma unroll
                for (int kc2 = 0; kc2 < 2; ++kc2) {
                    if constexpr (PREC) {
                        bf16x8 pb[RB], pl[RB];
    #pragma unroll
                        for (int rb = 0; rb < RB; ++rb)
    #pragma unroll
                            for (int j = 0; j < 4; ++j) {
                                pb[rb][j] = f2bf(sc[rb][2 * kc2][j]);
                                pb[rb][4 + j] = f2bf(sc[rb][2 * kc2 + 1][j]);
                                pl[rb][j] = f2bf(sc[rb][2 * kc2][j] - bf2f(pb[rb][j]));
                                pl[rb][4 + j] = f2bf(sc[rb][2 * kc2 + 1][j] - bf2f(pb[rb][4 + j]));
                            }
    #pragma unroll
                        for (int db = 0; db < DB; ++db) {
                            const int off = (db * 16 + c16) * LDV + kc2 * 32 + g * 4;
                            const uint2 lo0 = *reinterpret_cast<const uint2*>(&Vt[b][0][off]);
                            const uint2 hi0 = *reinterpret_cast<const uint2*>(&Vt[b][0][off + 16]);
                            const uint2 lo1 = *reinterpret_cast<const uint2*>(&Vt[b][NP - 1][off]);
                            const uint2 hi1 = *reinterpret_cast<const uint2*>(&Vt[b][NP - 1][off + 16]);
                            const bf16x8 va = __builtin_bit_cast(bf16x8, make_uint4(lo0.x, lo0.y, hi0.x, hi0.y));
                            const bf16x8 vl = __builtin_bit_cast(bf16x8, make_uint4(lo1.x, lo1.y, hi1.x, hi1.y));
    #pragma unroll
                            for (int rb = 0; rb < RB; ++rb) {
                                if (rb > 0 && !live[rb]) continue;
                                o[rb][db] = mfma16(vl, pb[rb], o[rb][db]);
                                o[rb][db] = mfma16(va, pl[rb], o[rb][db]);
                                o[rb][db] = mfma16(va, pb[rb], o[rb][db]);
                            }
                        }
                    } else {
                        // P.V in fp16 (11-bit significand): probabilities lose at most 2^-12
                        f16x8 ph[RB];
    #pragma unroll
                        for (int rb = 0; rb < RB; ++rb)
                            ph[rb] = __builtin_bit_cast(
                                f16x8, make_uint4(pack_h2(sc[rb][2 * kc2][0], sc[rb][2 * kc2][1]),
                                                  pack_h2(sc[rb][2 * kc2][2], sc[rb][2 * kc2][3]),
                                                  pack_h2(sc[rb][2 * kc2 + 1][0], sc[rb][2 * kc2 + 1][1]),
                                                  pack_h2(sc[rb][2 * kc2 + 1][2], sc[rb][2 * kc2 + 1][3])));
    #pragma unroll
                        for (int db = 0; db < DB; ++db) {
                            const int off = (db * 16 + c16) * LDV + kc2 * 32 + g * 4;
                            const uint2 lo0 = *reinterpret_cast<const uint2*>(&Vt[b][0][off]);
                            const uint2 hi0 = *reinterpret_cast<const uint2*>(&Vt[b][0][off + 16]);
                            const f16x8 vh = __builtin_bit_cast(f16x8, make_uint4(lo0.x, lo0.y, hi0.x, hi0.y));
    #pragma unroll
                            for (int rb = 0; rb < RB; ++rb) {
                                if (rb > 0 && !live[rb]) continue;
                                o[rb][db] = mfma16h(vh, ph[rb], o[rb][db]);
                            }
                        }
                    }
                }
            }
            tile_store<T, D, NP, NT, LDK, LDV>(tr_next, tid, Ks[b ^ 1], Vt[b ^ 1]);
        __syncthreads();
    };
    for (int t = 0; t < ntiles; t += 2) {
        step(t, tr0, tr1);
        step(t + 1, tr1, tr0);
    }

#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        float l_tot = l_part[rb] + __shfl_xor(l_part[rb], 16);
        l_tot += __shfl_xor(l_tot, 32);
        if (qok[rb]) {
            const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
            TO* orow = O + ((int64_t)bh * N + qtok[rb]) * D;
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    elem<TO>::store(orow, db * 16 + g * 4 + i, o[rb][db][i] * inv);
            if (g == 0 && lse)
                lse[(int64_t)bh * N + qtok[rb]] =
                    l_tot > 0.0f ? (m_run[rb] + __log2f(l_tot)) * 0.69314718055994531f : -INFINITY;
        }
    }
}

// Threads per workgroup and 16-row blocks per wave of the attention kernel.
#ifndef ADC_ATTN_NT
#define ADC_ATTN_NT 512
#endif
constexpr int ATTN_NT = ADC_ATTN_NT;
constexpr int ATTN_RB = ATTN_ROWS / 16 / (ATTN_NT / 64);

template <typename T, typename TO>
static void launch_attn_t(const Prob& p, dim3 grid, int Cq, const void* q, const int32_t* q_perm,
                          const int32_t* q_offsets, const void* k_perm, const void* v_perm,
                          const int32_t* run_start, const int32_t* run_pos, const int32_t* n_runs,
                          int run_cap, const int32_t* items, const int32_t* n_items, int cap,
                          float sl2, void* out, float* lse, hipStream_t s) {
    auto k = p.D == 64 ? attn_kernel<T, 64, TO, ATTN_NT, ATTN_RB> : attn_kernel<T, 128, TO, ATTN_NT, ATTN_RB>;
    hipLaunchKernelGGL(k, grid, dim3(ATTN_NT), 0, s, p.N, Cq, (const T*)q, q_perm, q_offsets,
                       (const T*)k_perm, (const T*)v_perm, run_start, run_pos, n_runs, run_cap,
                       items, n_items, cap, sl2, (TO*)out, lse);
}

hipError_t launch_attention(const Prob& p, int Cq, const void* q, const int32_t* q_perm,
                            const int32_t* q_offsets, const void* k_perm, const void* v_perm,
                            const int32_t* run_start, const int32_t* run_pos, const int32_t* n_runs,
                            int run_cap, const int32_t* items, const int32_t* n_items, int cap,
                            float scale, void* out, int out_f32, float* lse, hipStream_t s) {
    if (cap <= 0) return hipSuccess;
    const float sl2 = scale * 1.4426950408889634f;
    dim3 grid((unsigned)((int64_t)p.BH * cap));
    if (p.bf16) {
        if (out_f32)
            launch_attn_t<u16, float>(p, grid, Cq, q, q_perm, q_offsets, k_perm, v_perm, run_start,
                                      run_pos, n_runs, run_cap, items, n_items, cap, sl2, out, lse, s);
        else
            launch_attn_t<u16, u16>(p, grid, Cq, q, q_perm, q_offsets, k_perm, v_perm, run_start,
                                    run_pos, n_runs, run_cap, items, n_items, cap, sl2, out, lse, s);
    } else {
        launch_attn_t<float, float>(p, grid, Cq, q, q_perm, q_offsets, k_perm, v_perm, run_start,
                                    run_pos, n_runs, run_cap, items, n_items, cap, sl2, out, lse, s);
    }
    return hipGetLastError();
}

}  // namespace adc
