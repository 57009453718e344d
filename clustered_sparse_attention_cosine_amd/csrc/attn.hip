// Variable-length block-sparse attention for gfx950 (AdaCluster paper,
// Algorithm 3 steps 8-9): every query of q-cluster a attends, with an exact
// online softmax, to the keys of the slots selected for a.
//
// Layout. cluster_k leaves K and V slot-contiguous, so the keys of a selection
// are a list of contiguous key ranges ("runs"; slots with no members never
// break a run). The queries of a q-cluster are read through its permutation.
//
// Kernel. A work item is (head, q-cluster, chunk of 128 query rows); eight
// waves own 16 rows each. Key/value tiles of 64 rows are copied into LDS
// (both row-major, 16-byte chunks swizzled) and shared by the waves. Scores
// are computed as S^T = K Q^T with 16x16x32 MFMAs so that a lane owns one
// query column, the output as O^T += V^T P^T with the probabilities of the
// score registers as the B operand and V^T read by transposing LDS loads.
#include <math.h>
#include <algorithm>
#include <mutex>
#include <type_traits>
#include "../../include/adacluster.h"
#include "common.hpp"
#include "kernels.hpp"

namespace adc {

hipError_t fill_i32(int32_t* p, int64_t n, int32_t v, hipStream_t s);

// ------------------------------------------------------------------ runs
// The selected slots of one (head, q-cluster) row as contiguous key runs: a run
// continues while the next selected non-empty slot starts where the previous
// one ended. One wave per row; lane L owns slots 64 L .. 64 L + 63 of each
// 4096-slot chunk (mask words 2 L and 2 L + 1). Pass 1: every lane counts its
// runs and keys; wave scans give the run index and key position of each lane's
// first new run (a lane's first run continues the last one of the lanes before
// it when they touch). Pass 2 writes the runs. The result is that of a
// sequential walk over the slots. run_cap (Ck / 2 + 2) exceeds the largest
// possible number of runs, ceil(Ck / 2).
__global__ __launch_bounds__(256) void build_runs_kernel(int64_t rows, int Cq, int Ck,
                                                         const int32_t* __restrict__ k_offsets,
                                                         const uint32_t* __restrict__ mask,
                                                         int run_cap, int32_t* __restrict__ run_start,
                                                         int32_t* __restrict__ run_pos,
                                                         int32_t* __restrict__ n_runs) {
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= rows) return;
    const int l = threadIdx.x & 63;
    const int64_t bh = row / Cq;
    const int words = (Ck + 31) / 32;
    const uint32_t* m = mask + row * words;
    const int32_t* off = k_offsets + bh * (Ck + 1);
    int32_t* rs = run_start + row * run_cap;
    int32_t* rp = run_pos + row * (run_cap + 1);
    int nr = 0, pos = 0, ce = -1;  // runs and keys so far, end of the last run (wave-uniform)
    for (int c0 = 0; c0 < Ck; c0 += 4096) {
        const int b0 = c0 + 64 * l;
        uint64_t bits = 0;
        if (b0 < Ck) {
            const int w0 = b0 / 32;
            const uint32_t lo = m[w0];
            const uint32_t hi = w0 + 1 < words ? m[w0 + 1] : 0u;
            bits = (uint64_t)lo | ((uint64_t)hi << 32);
            if (Ck - b0 < 64) bits &= (1ull << (Ck - b0)) - 1ull;
        }
        int cnt = 0, keys = 0, fs = -1, le = -1;
        for (uint64_t t = bits; t; t &= t - 1) {
            const int b = b0 + __ffsll((unsigned long long)t) - 1;
            const int s = off[b], e = off[b + 1];
            if (e <= s) continue;
            if (fs < 0) fs = s;
            if (s != le) ++cnt;
            le = e;
            keys += e - s;
        }
        // end of the last run of the lanes before this one (key ends grow with the slot)
        int pmax = le;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int v = __shfl_up(pmax, o);
            if (l >= o) pmax = max(pmax, v);
        }
        int prev_le = __shfl_up(pmax, 1);
        prev_le = max(l == 0 ? -1 : prev_le, ce);
        const int newr = cnt - ((cnt > 0 && fs == prev_le) ? 1 : 0);
        int ir = newr, ik = keys;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int vr = __shfl_up(ir, o), vk = __shfl_up(ik, o);
            if (l >= o) {
                ir += vr;
                ik += vk;
            }
        }
        int idx = nr + ir - newr, p = pos + ik - keys, le2 = prev_le;
        for (uint64_t t = bits; t; t &= t - 1) {
            const int b = b0 + __ffsll((unsigned long long)t) - 1;
            const int s = off[b], e = off[b + 1];
            if (e <= s) continue;
            if (s != le2) {
                if (idx < run_cap) {
                    rs[idx] = s;
                    rp[idx] = p;
                }
                ++idx;
            }
            p += e - s;
            le2 = e;
        }
        nr += __shfl(ir, 63);
        pos += __shfl(ik, 63);
        ce = max(ce, __shfl(pmax, 63));
    }
    if (l == 0) {
        const int n = min(nr, run_cap);
        rp[n] = pos;
        n_runs[row] = n;
    }
}

hipError_t launch_build_runs(const Prob& p, int Cq, int Ck, const int32_t* k_offsets,
                             const uint32_t* mask, int run_cap, int32_t* run_start,
                             int32_t* run_pos, int32_t* n_runs, hipStream_t s) {
    const int64_t rows = (int64_t)p.BH * Cq;
    hipLaunchKernelGGL(build_runs_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, s, rows,
                       Cq, Ck, k_offsets, mask, run_cap, run_start, run_pos, n_runs);
    return hipGetLastError();
}

// ------------------------------------------------------------------ work list
// Work items (q-cluster a, chunk c of ATTN_ROWS rows) of head bh, one
// workgroup per head, with the inclusive prefix of their estimated cost. The
// list has two parts: first the items of the head's large q-clusters (those
// whose first item costs more than twice the mean item cost over all heads:
// heads differ, and on some workloads one head's q-clusters select most of
// its keys), written
// to part bh = items[bh * cap ...], then the others, part BH + bh (cap = Cq +
// ceil(N / ATTN_ROWS) bounds each part). Within a part the q-clusters go in
// the order of the middle key of their selection (the key row at half of the
// selected keys, K being slot-ordered): items that run at the same time on one
// XCD then read nearby key tiles, which its L2 can share; ties keep q-cluster
// order. Running the large items first leaves the small ones for the end of
// the kernel, where the last item of each workgroup sets when it finishes.
// An item's cost is its number of 64-key tiles times (4 + its live waves): the
// time per tile of a work item grows by about a quarter of its 4-wave value
// per 16-row wave of query rows (measured on uniform synthetic layouts).
__device__ __forceinline__ uint32_t item_cost(int tiles, int rows) {
    return (uint32_t)tiles * (uint32_t)(4 + (min(rows, ATTN_ROWS) + 15) / 16);
}

constexpr int WL_SORT = 8192;  // q-clusters a head can have (the slot capacity)

// Items and summed item cost of head bh (one workgroup per head), for the mean
// item cost over every head that the work list compares against.
__global__ __launch_bounds__(256) void item_load_kernel(int Cq, const int32_t* __restrict__ q_offsets,
                                                        const int32_t* __restrict__ run_pos,
                                                        const int32_t* __restrict__ n_runs, int run_cap,
                                                        uint64_t* __restrict__ load) {
    __shared__ uint64_t wl[4];
    __shared__ int wn[4];
    const int bh = blockIdx.x;
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
    const int32_t* qo = q_offsets + (int64_t)bh * (Cq + 1);
    uint64_t cost = 0;
    int n = 0;
    for (int a = tid; a < Cq; a += 256) {
        const int rows = qo[a + 1] - qo[a];
        const int ch = (rows + ATTN_ROWS - 1) / ATTN_ROWS;
        if (ch == 0) continue;
        const int64_t row = (int64_t)bh * Cq + a;
        const int tiles = (run_pos[row * (run_cap + 1) + n_runs[row]] + 63) / 64;
        for (int c = 0; c < ch; ++c) cost += item_cost(tiles, rows - c * ATTN_ROWS);
        n += ch;
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        cost += __shfl_xor(cost, o);
        n += __shfl_xor(n, o);
    }
    if (l == 0) {
        wl[w] = cost;
        wn[w] = n;
    }
    __syncthreads();
    if (tid == 0) {
        load[2 * bh] = wl[0] + wl[1] + wl[2] + wl[3];
        load[2 * bh + 1] = (uint64_t)(wn[0] + wn[1] + wn[2] + wn[3]);
    }
}

__global__ __launch_bounds__(256) void worklist_kernel(int Cq, int cap, int BH,
                                                       const uint64_t* __restrict__ load,
                                                       const int32_t* __restrict__ q_offsets,
                                                       const int32_t* __restrict__ run_start,
                                                       const int32_t* __restrict__ run_pos,
                                                       const int32_t* __restrict__ n_runs,
                                                       int run_cap, int32_t* __restrict__ items,
                                                       int32_t* __restrict__ n_items,
                                                       uint32_t* __restrict__ cost_pre,
                                                       uint32_t* __restrict__ n_cost) {
    __shared__ int wsum[4];
    __shared__ uint32_t wcost[4];
    __shared__ uint64_t wtot[4], wtot2[4];
    __shared__ uint64_t order[WL_SORT];
    const int bh = blockIdx.x;
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
    const int32_t* qo = q_offsets + (int64_t)bh * (Cq + 1);
    auto tiles_of = [&](int a) __attribute__((always_inline)) -> int {
        const int64_t row = (int64_t)bh * Cq + a;
        return (run_pos[row * (run_cap + 1) + n_runs[row]] + 63) / 64;
    };
    // item count and summed cost over every head, for the mean item cost
    uint64_t tot_cost = 0, tot_items = 0;
    for (int i = tid; i < BH; i += 256) {
        tot_cost += load[2 * i];
        tot_items += load[2 * i + 1];
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        tot_cost += __shfl_xor(tot_cost, o);
        tot_items += __shfl_xor(tot_items, o);
    }
    if (l == 0) {
        wtot[w] = tot_cost;
        wtot2[w] = tot_items;
    }
    __syncthreads();
    const uint64_t all_cost = wtot[0] + wtot[1] + wtot[2] + wtot[3];
    const uint64_t all_items = wtot2[0] + wtot2[1] + wtot2[2] + wtot2[3];
    // large: first item cost > 2 * mean item cost, i.e. cost * items > 2 * sum
    auto large = [&](int tiles, int rows) __attribute__((always_inline)) -> bool {
        return (uint64_t)item_cost(tiles, rows) * all_items > 2ull * all_cost;
    };
    __syncthreads();
    // sort keys: (small?, middle key row of the selection, q-cluster); the
    // q-clusters with no selection make no items
    int np2 = 1;
    while (np2 < Cq) np2 <<= 1;
    for (int a = tid; a < np2; a += 256) {
        uint64_t key = ~0ull;  // padding sorts last
        if (a < Cq) {
            const int64_t row = (int64_t)bh * Cq + a;
            const int R = n_runs[row];
            const int32_t* rp = run_pos + row * (run_cap + 1);
            const int total = rp[R];
            uint32_t mid = 0;
            if (total > 0) {
                // the run holding position total / 2: largest r with rp[r] <= total / 2
                const int half = total / 2;
                int lo = 0, hi = R - 1;
                while (lo < hi) {
                    const int m = (lo + hi + 1) >> 1;
                    if (rp[m] <= half) lo = m; else hi = m - 1;
                }
                mid = (uint32_t)(run_start[row * run_cap + lo] + (half - rp[lo]));
            }
            const bool big = large((total + 63) / 64, qo[a + 1] - qo[a]);
            key = ((uint64_t)(big ? 0u : 1u) << 63) | ((uint64_t)mid << 32) | (uint32_t)a;
        }
        order[a] = key;
    }
    __syncthreads();
    // bitonic sort of np2 keys in LDS
    for (int k = 2; k <= np2; k <<= 1) {
        for (int j = k >> 1; j > 0; j >>= 1) {
            for (int i = tid; i < np2; i += 256) {
                const int ixj = i ^ j;
                if (ixj > i) {
                    const uint64_t x = order[i], y = order[ixj];
                    const bool up = (i & k) == 0;
                    if ((x > y) == up) {
                        order[i] = y;
                        order[ixj] = x;
                    }
                }
            }
            __syncthreads();
        }
    }
    // one pass per part over the sorted q-clusters, each taking those of its part
    for (int part = 0; part < 2; ++part) {
        const int vh = part * BH + bh;
        int32_t* out = items + (int64_t)vh * cap;
        uint32_t* cout = cost_pre + (int64_t)vh * cap;
        int running = 0;
        uint32_t running_cost = 0;
        for (int base = 0; base < Cq; base += 256) {
            const uint64_t key = base + tid < Cq ? order[base + tid] : ~0ull;
            const int a = base + tid < Cq ? (int)(uint32_t)key : Cq;
            const bool mine = a < Cq && (int)(key >> 63) == part;
            const int rows = mine ? qo[a + 1] - qo[a] : 0;
            const int ch = (rows + ATTN_ROWS - 1) / ATTN_ROWS;
            const int tiles = ch > 0 ? tiles_of(a) : 0;
            uint32_t cq = 0;
            for (int c = 0; c < ch; ++c) cq += item_cost(tiles, rows - c * ATTN_ROWS);
            int incl = ch;
            uint32_t cincl = cq;
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                const int v = __shfl_up(incl, o);
                const uint32_t vc = __shfl_up(cincl, o);
                if (l >= o) {
                    incl += v;
                    cincl += vc;
                }
            }
            if (l == 63) {
                wsum[w] = incl;
                wcost[w] = cincl;
            }
            __syncthreads();
            int before = running + incl - ch;
            uint32_t cbefore = running_cost + cincl - cq;
            for (int i = 0; i < w; ++i) {
                before += wsum[i];
                cbefore += wcost[i];
            }
            for (int c = 0; c < ch; ++c) {
                cbefore += item_cost(tiles, rows - c * ATTN_ROWS);
                out[before + c] = a | (c << 16);
                cout[before + c] = cbefore;
            }
            running += wsum[0] + wsum[1] + wsum[2] + wsum[3];
            running_cost += wcost[0] + wcost[1] + wcost[2] + wcost[3];
            __syncthreads();
        }
        if (tid == 0) {
            n_items[vh] = running;
            n_cost[vh] = running_cost;
        }
    }
}

// head_pos[v] = number of work items of the list parts before part v,
// head_cost[v] = their summed cost; entry NP holds the totals (NP parts).
__global__ __launch_bounds__(1024) void head_scan_kernel(int BH, const int32_t* __restrict__ n_items,
                                                         const uint32_t* __restrict__ n_cost,
                                                         int32_t* __restrict__ head_pos,
                                                         uint64_t* __restrict__ head_cost) {
    __shared__ int wsum[16];
    __shared__ uint64_t wcost[16];
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
    int running = 0;
    uint64_t running_cost = 0;
    if (tid == 0) {
        head_pos[0] = 0;
        head_cost[0] = 0;
    }
    for (int base = 0; base < BH; base += 1024) {
        const int i = base + tid;
        const int v = i < BH ? n_items[i] : 0;
        const uint64_t vc = i < BH ? n_cost[i] : 0;
        int incl = v;
        uint64_t cincl = vc;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int u = __shfl_up(incl, o);
            const uint64_t uc = __shfl_up(cincl, o);
            if (l >= o) {
                incl += u;
                cincl += uc;
            }
        }
        if (l == 63) {
            wsum[w] = incl;
            wcost[w] = cincl;
        }
        __syncthreads();
        int before = running;
        uint64_t cbefore = running_cost;
        for (int k = 0; k < w; ++k) {
            before += wsum[k];
            cbefore += wcost[k];
        }
        if (i < BH) {
            head_pos[i + 1] = before + incl;
            head_cost[i + 1] = cbefore + cincl;
        }
        for (int k = 0; k < 16; ++k) {
            running += wsum[k];
            running_cost += wcost[k];
        }
        __syncthreads();
    }
}

// Each half of the list (the large items of every head, then the others) is
// cut into eight stretches of equal estimated cost, one per XCD: stretch
// 8 h + x holds the items of half h whose cost prefix lies in the x-th eighth
// of that half's cost, so every XCD has its share of both. Also clears the
// sixteen stretch counters.
__device__ __forceinline__ uint64_t cost_before(int i, int NV, int cap, const int32_t* head_pos,
                                                const uint64_t* head_cost, const uint32_t* cost_pre) {
    int lo = 0, hi = NV;  // head_pos[lo] <= i < head_pos[hi]
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (head_pos[mid] <= i) lo = mid; else hi = mid;
    }
    const int j = i - head_pos[lo];
    return head_cost[lo] + (j > 0 ? cost_pre[(int64_t)lo * cap + j - 1] : 0u);
}

__global__ __launch_bounds__(64) void xcd_split_kernel(int BH, int cap, const int32_t* __restrict__ head_pos,
                                                       const uint64_t* __restrict__ head_cost,
                                                       const uint32_t* __restrict__ cost_pre,
                                                       int32_t* __restrict__ xcd_start,
                                                       int32_t* __restrict__ xcd_ctr) {
    const int x = threadIdx.x;
    if (x > 16) return;
    const int NV = 2 * BH;
    const int n_total = head_pos[NV];
    if (x < 16) xcd_ctr[x] = 0;
    if (x == 16) {
        xcd_start[16] = n_total;
        return;
    }
    const int h = x >> 3, j = x & 7;
    const int i_lo = h == 0 ? 0 : head_pos[BH], i_hi = h == 0 ? head_pos[BH] : n_total;
    const uint64_t c_lo = h == 0 ? 0 : head_cost[BH], c_hi = h == 0 ? head_cost[BH] : head_cost[NV];
    const uint64_t target = c_lo + (c_hi - c_lo) * (uint64_t)j / 8u;
    int lo = i_lo, hi = i_hi;  // smallest i in [i_lo, i_hi] with cost_before(i) >= target
    while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (cost_before(mid, NV, cap, head_pos, head_cost, cost_pre) >= target) hi = mid; else lo = mid + 1;
    }
    xcd_start[x] = lo;
}

hipError_t launch_worklist(const Prob& p, int Cq, int cap, const int32_t* q_offsets,
                           const int32_t* run_start, const int32_t* run_pos, const int32_t* n_runs,
                           int run_cap, const AttnSched& sc, hipStream_t s) {
    if (Cq > WL_SORT) return hipErrorInvalidValue;
    hipLaunchKernelGGL(item_load_kernel, dim3((unsigned)p.BH), dim3(256), 0, s, Cq, q_offsets, run_pos, n_runs,
                       run_cap, sc.load);
    hipLaunchKernelGGL(worklist_kernel, dim3((unsigned)p.BH), dim3(256), 0, s, Cq, cap, p.BH,
                       (const uint64_t*)sc.load, q_offsets,
                       run_start, run_pos, n_runs, run_cap, sc.items, sc.n_items, sc.cost_pre, sc.n_cost);
    hipLaunchKernelGGL(head_scan_kernel, dim3(1), dim3(1024), 0, s, 2 * p.BH, sc.n_items, sc.n_cost,
                       sc.head_pos, sc.head_cost);
    hipLaunchKernelGGL(xcd_split_kernel, dim3(1), dim3(64), 0, s, p.BH, cap, sc.head_pos, sc.head_cost,
                       sc.cost_pre, sc.xcd_start, sc.xcd_ctr);
    return hipGetLastError();
}

// ------------------------------------------------------------------ operand planes
// The attention kernel reads 16-bit operand planes. bf16 inputs: K' is used as
// it is and V' is converted once to fp16 here (the P.V product runs in fp16),
// scaled per head by a power of two 2^e chosen from the head's largest |v|
// so that it lands in [2^14, 2^15): no finite bf16 value overflows fp16, and
// every value within 2^-28 of the largest keeps all its bits (smaller ones are
// rounded to the fp16 subnormal grid, an absolute error below 2^-25 of the
// largest |v|). The output is multiplied back by 2^-e, which is exact. f32
// inputs: K' and V' are split into bf16 hi + lo planes (x = hi + lo to 2^-16
// relative), which keep the f32 range.

// Exponent e of the head's fp16 scale from its largest |v| (bf16 magnitude
// bits; 0 for an all-zero head), kept where 2^e and 2^-e are normal floats.
__device__ __forceinline__ int v_scale_exp(uint32_t vmax_bits) {
    if (vmax_bits == 0) return 0;
    const int E = vmax_bits >= 0x80u ? (int)(vmax_bits >> 7) - 127 : -127;  // floor(log2 |v|max)
    return min(126, max(-126, 14 - E));
}
__device__ __forceinline__ float pow2f(int e) { return __uint_as_float((uint32_t)(127 + e) << 23); }

// Largest bf16 magnitude (as its bit pattern, which orders finite values) per
// head: VMAX_WG workgroups per head, each thread with VMAX_PER independent
// 16-byte loads in flight per step, and one atomic per workgroup (atomics on
// one address serialise, so their number is kept small).
constexpr int VMAX_PER = 8;
constexpr int VMAX_WG = 32;
__global__ __launch_bounds__(256) void vmax_kernel(const u16* __restrict__ x, int64_t per_head8,
                                                   uint32_t* __restrict__ vmax) {
    const int bh = blockIdx.y;
    const uint4* xh = reinterpret_cast<const uint4*>(x + (int64_t)bh * per_head8 * 8);
    const int64_t stride = (int64_t)gridDim.x * 256;
    uint32_t m = 0;
    for (int64_t i0 = (int64_t)blockIdx.x * 256 + threadIdx.x; i0 < per_head8; i0 += VMAX_PER * stride) {
        uint4 r[VMAX_PER];
#pragma unroll
        for (int u = 0; u < VMAX_PER; ++u) {
            const int64_t i = i0 + u * stride;
            r[u] = i < per_head8 ? xh[i] : make_uint4(0u, 0u, 0u, 0u);
        }
#pragma unroll
        for (int u = 0; u < VMAX_PER; ++u) {
            const uint32_t w[4] = {r[u].x, r[u].y, r[u].z, r[u].w};
#pragma unroll
            for (int k = 0; k < 4; ++k) m = max(m, max(w[k] & 0x7FFFu, (w[k] >> 16) & 0x7FFFu));
        }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, o));
    __shared__ uint32_t wm[4];
    if ((threadIdx.x & 63) == 0) wm[threadIdx.x >> 6] = m;
    __syncthreads();
    if (threadIdx.x == 0) atomicMax(&vmax[bh], max(max(wm[0], wm[1]), max(wm[2], wm[3])));
}

__global__ __launch_bounds__(256) void planes_f16_kernel(const u16* __restrict__ x, int64_t per_head8,
                                                         const uint32_t* __restrict__ vmax,
                                                         u16* __restrict__ out) {
    const int bh = blockIdx.y;
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= per_head8) return;
    const float sc = pow2f(v_scale_exp(vmax[bh]));
    const int64_t o = ((int64_t)bh * per_head8 + i) * 8;
    const uint4 r = *reinterpret_cast<const uint4*>(x + o);
    const uint32_t w[4] = {r.x, r.y, r.z, r.w};
    uint32_t h[4];
#pragma unroll
    for (int k = 0; k < 4; ++k)
        h[k] = pack_h2(__uint_as_float(w[k] << 16) * sc, __uint_as_float(w[k] & 0xFFFF0000u) * sc);
    *reinterpret_cast<uint4*>(out + o) = make_uint4(h[0], h[1], h[2], h[3]);
}

__global__ __launch_bounds__(256) void planes_split_kernel(const float* __restrict__ x, int64_t n8,
                                                           u16* __restrict__ hi, u16* __restrict__ lo) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n8) return;
    float v[8];
    load8<float>(x + i * 8, v);
    uint32_t h[4], l[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const u16 h0 = f2bf_bits(v[2 * k]), h1 = f2bf_bits(v[2 * k + 1]);
        const u16 l0 = f2bf_bits(v[2 * k] - bf_bits2f(h0)), l1 = f2bf_bits(v[2 * k + 1] - bf_bits2f(h1));
        h[k] = (uint32_t)h0 | ((uint32_t)h1 << 16);
        l[k] = (uint32_t)l0 | ((uint32_t)l1 << 16);
    }
    *reinterpret_cast<uint4*>(hi + i * 8) = make_uint4(h[0], h[1], h[2], h[3]);
    *reinterpret_cast<uint4*>(lo + i * 8) = make_uint4(l[0], l[1], l[2], l[3]);
}

hipError_t launch_planes(const Prob& p, const void* k, const void* v, u16* k_hi, u16* k_lo,
                         u16* v_hi, u16* v_lo, uint32_t* vmax, hipStream_t s) {
    const int64_t n8 = (int64_t)p.BH * p.N * p.D / 8;
    if (n8 <= 0) return hipSuccess;
    if (p.bf16) {
        const int64_t ph8 = (int64_t)p.N * p.D / 8;
        hipError_t e = fill_i32((int32_t*)vmax, p.BH, 0, s);
        if (e != hipSuccess) return e;
        const unsigned gx = (unsigned)std::min<int64_t>(VMAX_WG, (ph8 + 256 * VMAX_PER - 1) / (256 * VMAX_PER));
        hipLaunchKernelGGL(vmax_kernel, dim3(gx, p.BH), dim3(256), 0, s, (const u16*)v, ph8, vmax);
        hipLaunchKernelGGL(planes_f16_kernel, dim3((unsigned)((ph8 + 255) / 256), p.BH), dim3(256), 0, s,
                           (const u16*)v, ph8, (const uint32_t*)vmax, v_hi);
    } else {
        const dim3 grid((unsigned)((n8 + 255) / 256));
        hipLaunchKernelGGL(planes_split_kernel, grid, dim3(256), 0, s, (const float*)k, n8, k_hi, k_lo);
        hipLaunchKernelGGL(planes_split_kernel, grid, dim3(256), 0, s, (const float*)v, n8, v_hi, v_lo);
    }
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

// Key rows of one 64-position tile of the concatenated selection, computed by
// one wave. rn is the run holding position t0 (uniform). Lane k looks at the
// start of run rn + 1 + k; the offsets of the starts inside (t0, t0 + 64) are
// gathered into a 64-bit mask (an OR over the wave), and lane p counts the
// starts at offsets <= p: run rn + count holds position t0 + p. Writes
// krow[p] (-1 past the selection) and returns the run holding position
// t0 + 64. rs/rp may point to LDS or to global memory.
__device__ __forceinline__ int tile_rows(int lane, int t0, int total, int R, int rn,
                                         const int32_t* rs, const int32_t* rp, int* krow) {
    const int rk = rn + 1 + lane;
    const int off = rp[min(rk, R)] - t0;  // rp[R] = total; off >= 1
    const bool inside = rk < R && off < 64;
    const uint32_t lo = wave_or(inside && off < 32 ? 1u << off : 0u);
    const uint32_t hi = wave_or(inside && off >= 32 ? 1u << (off - 32) : 0u);
    const uint64_t starts = ((uint64_t)hi << 32) | lo;
    const uint64_t upto = lane == 63 ? ~0ull : ((2ull << lane) - 1ull);
    const int r = min(rn + (int)__popcll(starts & upto), R - 1);
    const int P = t0 + lane;
    const int row = rs[max(r, 0)] + (P - rp[max(r, 0)]);
    krow[lane] = P < total ? row : -1;
    return rn + (int)__popcll(__ballot(rk < R && off <= 64));
}

// K/V tiles in LDS. A tile is 64 key rows of NP 16-bit planes of K, then NP of
// V, each plane row-major with unpadded rows of RB = 2 D bytes; the 16-byte
// chunks of row r are stored XOR-swizzled (logical chunk c at physical chunk
// c ^ tile_swz<D>(r)) so that the column reads of the fragments below spread
// over the banks. With 128-byte rows (D = 64) the row parity already splits
// the banks and the XOR is r & 7; with 256-byte rows every row starts on the
// same bank, and the transposing V reads (four rows, two 16-byte chunks and
// both 8-byte halves per 16 lanes) need the 8 chunk pairs they touch to be
// distinct, which 2 (r & 7) gives and r & 7 does not (it maps two rows onto
// one pair: measured as LDS bank conflicts on every V read of the D = 128
// kernel). Tiles are copied from global memory straight into LDS by the
// 16-byte global->LDS loads: one wave instruction fills 1 KB of a plane, lane
// j the j-th 16 bytes, so the swizzle is applied by choosing which global
// chunk each lane fetches. NB tiles are in flight (the copy of tile t + NB - 1
// is issued while tile t is computed).
template <int D>
__device__ __forceinline__ int tile_swz(int r) {
    return D == 64 ? (r & 7) : 2 * (r & 7);
}

template <int D, int NP, int NT>
struct TileGeom {
    static constexpr int RB = 2 * D;                    // bytes per row of a plane
    static constexpr int PLANE = 64 * RB;               // bytes per plane of a tile
    static constexpr int TILE = 2 * NP * PLANE;         // K planes, then V planes
    // tiles resident: three for 16 KB tiles (bf16, D = 64), so that three
    // workgroups fit a CU's LDS; two beyond (two workgroups per CU for 32 KB
    // tiles: bf16 D = 128, f32 D = 64)
    static constexpr int NB = TILE <= 16384 ? 3 : 2;
    static constexpr int NW = NT / 64;
    static constexpr int IPW = PLANE / 1024 / NW;       // 1 KB blocks per plane per wave
    static constexpr int L = 2 * NP * IPW;              // copies per wave per tile
    static_assert(IPW >= 1 && (PLANE / 1024) % NW == 0, "plane blocks must divide among the waves");
};

typedef __attribute__((address_space(3))) void lds_void;

// Issue the copy of one tile into the LDS buffer `buf`: wave w fills blocks
// w * IPW .. w * IPW + IPW - 1 of every plane. Rows past the selection
// (krow = -1) read row 0: their scores are masked to -inf, so their
// probabilities are exactly 0 and the finite values they carry never reach
// the output.
template <int D, int NP, int NT>
__device__ __forceinline__ void tile_copy(unsigned char* buf, int w, int lane, const int* krow,
                                          const u16* K0, const u16* K1, const u16* V0,
                                          const u16* V1) {
    using G = TileGeom<D, NP, NT>;
#pragma unroll
    for (int i = 0; i < G::IPW; ++i) {
        const int blk = w * G::IPW + i;
        const int off = blk * 1024 + 16 * lane;
        const int r = off / G::RB;
        const int lc = ((off % G::RB) / 16) ^ tile_swz<D>(r);
        const int64_t goff = (int64_t)max(krow[r], 0) * D + lc * 8;
        unsigned char* dst = buf + blk * 1024;
        __builtin_amdgcn_global_load_lds(K0 + goff, (lds_void*)dst, 16, 0, 0);
        __builtin_amdgcn_global_load_lds(V0 + goff, (lds_void*)(dst + NP * G::PLANE), 16, 0, 0);
        if constexpr (NP == 2) {
            __builtin_amdgcn_global_load_lds(K1 + goff, (lds_void*)(dst + G::PLANE), 16, 0, 0);
            __builtin_amdgcn_global_load_lds(V1 + goff, (lds_void*)(dst + 3 * G::PLANE), 16, 0, 0);
        }
    }
}

// Wait until at most N of this wave's tile copies are outstanding (copies
// complete in issue order) and its LDS accesses are done, then meet the other
// waves. The barrier is an opaque statement to the compiler (no memory access
// moves across it), so it waits for exactly what is asked here instead of for
// every copy in flight.
template <int N>
__device__ __forceinline__ void tiles_ready_barrier() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (0 << 8) | ((N >> 4) << 14));
    asm volatile("s_barrier" ::: "memory");
}

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

// Transposed 16x32 fragment of a row-major V plane for the A operand of
// O^T += V^T P^T. Lane L (group G = L/16) receives V[key][d] for d = L%16 of a
// 16-column block and the 8 keys 32c + 4G + {0..3}, 32c + 16 + 4G + {0..3}: the
// key order of the lane's probabilities. In each 16-lane group of a
// ds_read_tr16_b64, source lane a + 4j points at columns 4a..4a+3 of key row j
// and destination lane 4a + b collects column b of source lanes a, a + 4,
// a + 8, a + 12. `p` is the lane's address for the first four keys; the
// second four are 16 rows further (same swizzle, as 16 is a multiple of 8).
template <int RB>
__device__ __forceinline__ uint4 v_frag(const unsigned char* p) {
    const v4i16 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)p);
    const v4i16 y = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(p + 16 * RB));
    const uint2 xu = __builtin_bit_cast(uint2, x), yu = __builtin_bit_cast(uint2, y);
    return make_uint4(xu.x, xu.y, yu.x, yu.y);
}

// Online softmax of one 16-query block over NKB 16-key blocks of a tile (the
// lane holds query c16 and keys kb*16 + 4g + i of the blocks). Scores come in raw; sl2 = scale *
// log2(e) is applied inside the exponent. LAST: positions >= total get
// probability 0. FIRST: the first tile of the item sets the running maximum m.
//
// m (log2 units) is raised only when some score of the wave exceeds m + 8, a
// test each lane makes on its own maximum against thr = (m + 8) / sl2 (the
// maximum across the four lanes of a query is formed only then); otherwise
// the stale m is kept, so every probability is at most 2^8 (exact as an f32
// summand, finite in fp16) and O is not rescaled. The result is the same
// softmax: numerator and denominator share the factor 2^-m whatever m is.
// The row sums are accumulated by the matrix cores (a block of ones in the
// P.V product), so they are part of o and rescaled with it.
template <int DB, int NKB>
__device__ __forceinline__ void softmax_tile(f32x4 (&sc)[NKB], float sl2, int lim, bool last,
                                             bool first, float& m_run, float& thr,
                                             f32x4 (&o)[DB + 1]) {
    if (last) {
        // lim = total - (block start + 4g): keys kb*16 + i >= lim are past the selection
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (kb * 16 + i >= lim) sc[kb][i] = -INFINITY;
    }
    float mx = fmaxf(fmaxf(sc[0][0], sc[0][1]), sc[0][2]);
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            if (kb > 0 || i > 2) mx = fmaxf(mx, sc[kb][i]);
    if (first || __ballot(mx > thr) != 0) {
        // the first tile holds position 0 of the selection, so its maximum is finite
        const float mq = col_max4(mx) * sl2;
        const float m_new = first ? (mq > -INFINITY ? mq : 0.0f) : fmaxf(m_run, mq);
        const float alpha = first ? 0.0f : __builtin_amdgcn_exp2f(m_run - m_new);
#pragma unroll
        for (int db = 0; db <= DB; ++db) o[db] *= alpha;
        m_run = m_new;
        thr = (m_new + 8.0f) / sl2;
    }
    const float nb = -m_run;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) sc[kb][i] = __builtin_amdgcn_exp2f(fmaf(sc[kb][i], sl2, nb));
}

// A work item is (head, q-cluster, chunk of ATTN_ROWS = 128 query rows); wave
// w of the eight owns rows 16w..16w+15 (a wave past the item's rows only
// helps with the tile staging and the run lookups).
//
// K/V tiles of 64 keys are copied straight into NB LDS buffers: while tile t
// is computed the copies of tiles t+1 .. t+NB-1 are in flight and the last
// wave looks up the key rows of tile t+NB, so one barrier per tile suffices
// and no register staging is needed. Operands are 16-bit planes (NP = 1: K
// bf16, V fp16; NP = 2: bf16 hi and lo of f32 data, every product of order
// <= 1 accumulated, three MFMAs per product, near f32 accuracy).
template <typename T, int D, typename TO, int WPE>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(WPE, 8)))
void attn_kernel(int N, int Cq, const T* __restrict__ Q, const int32_t* __restrict__ q_perm,
                 const int32_t* __restrict__ q_off, const u16* __restrict__ K0,
                 const u16* __restrict__ K1, const u16* __restrict__ V0,
                 const u16* __restrict__ V1, const int32_t* __restrict__ run_start,
                 const int32_t* __restrict__ run_pos, const int32_t* __restrict__ n_runs,
                 int run_cap, const int32_t* __restrict__ items,
                 const int32_t* __restrict__ head_pos, const int32_t* __restrict__ xcd_start,
                 int32_t* __restrict__ xcd_ctr, int BH, int cap, float sl2,
                 const uint32_t* __restrict__ vmax, TO* __restrict__ O, float* __restrict__ lse) {
    constexpr int NT = 512;
    static_assert((NT / 64) * 16 == ATTN_ROWS, "eight waves of 16 rows cover a work item");
    constexpr bool PREC = sizeof(T) == 4;
    constexpr int NP = PREC ? 2 : 1;  // operand planes
    constexpr int KC = D / 32;        // 32-wide chunks of the head dimension
    constexpr int DB = D / 16;        // 16-row blocks of O^T
    using TG = TileGeom<D, NP, NT>;
    constexpr int RB = TG::RB;
    constexpr int NB = TG::NB;
    constexpr bool LATE_COPY = D == 128;
    // one array per buffer, always indexed by a compile-time buffer number, so
    // the compiler's wait analysis sees that a copy into one buffer does not
    // touch the buffer being read
    __shared__ __attribute__((aligned(1024))) unsigned char tb0[TG::TILE], tb1[TG::TILE];
    __shared__ __attribute__((aligned(1024))) unsigned char tb2[NB > 2 ? TG::TILE : 16];
    __shared__ __attribute__((aligned(1024))) unsigned char tb3[NB > 3 ? TG::TILE : 16];
    auto buf = [&](auto j_c) __attribute__((always_inline)) -> unsigned char* {
        constexpr int J = decltype(j_c)::value % NB;
        if constexpr (J == 0) return tb0;
        else if constexpr (J == 1) return tb1;
        else if constexpr (J == 2) return tb2;
        else return tb3;
    };
    __shared__ int krow[4][64];
    // the work item's runs (first key row, first position) when they fit
    constexpr int RL = 256;
    __shared__ int run_s[RL], run_p[RL + 1];

    __shared__ int sh_item;

    // Work order: workgroup b runs on XCD x = b % 8 (round-robin dispatch) and
    // takes the items of stretch x (its share of the large items) in list
    // order from that stretch's counter, then those of stretch 8 + x (its
    // share of the others). The stretches are contiguous (a few heads,
    // q-clusters in order), so the workgroups in flight on one XCD read
    // overlapping key ranges through its own L2, and they carry about equal
    // estimated cost. A workgroup whose stretch is used up takes items from
    // the other XCDs' stretches of the same half in turn (x + 1, x + 2, ...
    // mod 8): the cost estimate is off by a few percent per XCD (the XCDs
    // finished 4-14 % of the kernel apart without this). Every counter value
    // names at most one item, so each item is taken once; a workgroup exits
    // after it has found all sixteen stretches used up.
    const int xq = blockIdx.x & 7;
    int kk = 0;  // position in this workgroup's order of stretches (thread 0's copy is used)
    for (;;) {
    if (threadIdx.x == 0) {
        int xs = (kk & 8) | ((xq + kk) & 7);
        int it = xcd_start[xs] + atomicAdd(&xcd_ctr[xs], 1);
        while (it >= xcd_start[xs + 1] && ++kk < 16) {
            xs = (kk & 8) | ((xq + kk) & 7);
            it = xcd_start[xs] + atomicAdd(&xcd_ctr[xs], 1);
        }
        sh_item = kk < 16 ? it : -1;
    }
    __syncthreads();
    const int item = __builtin_amdgcn_readfirstlane(sh_item);
    if (item < 0) break;
    int hlo = 0, hhi = 2 * BH;  // list part: head_pos[hlo] <= item < head_pos[hhi]
    while (hhi - hlo > 1) {
        const int mid = (hlo + hhi) >> 1;
        if (__builtin_amdgcn_readfirstlane(head_pos[mid]) <= item) hlo = mid; else hhi = mid;
    }
    const int bh = hlo < BH ? hlo : hlo - BH;
    const int packed = __builtin_amdgcn_readfirstlane(
        items[(int64_t)hlo * cap + item - __builtin_amdgcn_readfirstlane(head_pos[hlo])]);
    const int a = packed & 0xFFFF, ch = packed >> 16;
    const int tid = threadIdx.x, l = tid & 63, g = l >> 4, c16 = l & 15;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);

    const int32_t* qo = q_off + (int64_t)bh * (Cq + 1);
    const int row0 = __builtin_amdgcn_readfirstlane(qo[a]) + ch * ATTN_ROWS;
    const int nrows = min(ATTN_ROWS, __builtin_amdgcn_readfirstlane(qo[a + 1]) - row0);
    const bool live = w * 16 < nrows;
    const int rowi = w * 16 + c16;
    const bool qok = rowi < nrows;
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
    const int R = __builtin_amdgcn_readfirstlane(n_runs[rbase]);
    const int32_t* rs = run_start + rbase * run_cap;
    const int32_t* rp = run_pos + rbase * (run_cap + 1);
    const int total = __builtin_amdgcn_readfirstlane(rp[R]);
    const int ntiles = (total + 63) / 64;
    const int64_t hoff = (int64_t)bh * N * D;
    const u16* const Kh0 = K0 + hoff;
    const u16* const Vh0 = V0 + hoff;
    const u16* const Kh1 = PREC ? K1 + hoff : Kh0;
    const u16* const Vh1 = PREC ? V1 + hoff : Vh0;

    float m_run = 0.0f;  // running maximum (log2 units), set by the first tile
    float thr = 0.0f;    // (m_run + 8) / sl2: a raw score above it raises m_run
    f32x4 o[DB + 1];  // O^T blocks and the row-sum block
#pragma unroll
    for (int db = 0; db <= DB; ++db) o[db] = f32x4{0.f, 0.f, 0.f, 0.f};
    // per-lane byte offsets (swizzled) of the K fragment reads (key row c16,
    // chunk 4 kc + g) and of the transposed V reads (key row 4g + j, columns
    // 16 db + 4a .. + 3)
    int koff[KC], voff[DB];
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) koff[kc] = c16 * RB + 16 * ((4 * kc + g) ^ tile_swz<D>(c16));
    {
        const int rv = 4 * g + ((l & 15) >> 2);
#pragma unroll
        for (int db = 0; db < DB; ++db)
            voff[db] = rv * RB + 16 * ((2 * db + ((l & 3) >> 1)) ^ tile_swz<D>(rv)) + (l & 1) * 8;
    }

    // Run lookups read the run list from LDS (copied once here; a list longer
    // than RL is read from global memory instead). They are made by the last
    // wave, which has no query rows in most work items.
    const bool runs_lds = R <= RL;
    constexpr int LW = NT / 64 - 1;
    for (int i = tid; i < R && runs_lds; i += NT) run_s[i] = rs[i];
    for (int i = tid; i <= R && runs_lds; i += NT) run_p[i] = rp[i];
    __syncthreads();
    int rn = 0;
    auto lookup = [&](int t) __attribute__((always_inline)) {
        if (runs_lds) rn = tile_rows(l, t * 64, total, R, rn, run_s, run_p, krow[t & 3]);
        else rn = tile_rows(l, t * 64, total, R, rn, rs, rp, krow[t & 3]);
    };
    if (w == LW) {
#pragma unroll
        for (int t = 0; t < NB; ++t) lookup(t);
    }
    __syncthreads();
    // tiles 0 .. NB - 2 here; step t issues tile t + NB - 1
    tile_copy<D, NP, NT>(buf(std::integral_constant<int, 0>{}), w, l, krow[0], Kh0, Kh1, Vh0, Vh1);
    if constexpr (NB > 2)
        tile_copy<D, NP, NT>(buf(std::integral_constant<int, 1>{}), w, l, krow[1], Kh0, Kh1, Vh0, Vh1);
    if constexpr (NB > 3)
        tile_copy<D, NP, NT>(buf(std::integral_constant<int, 2>{}), w, l, krow[2], Kh0, Kh1, Vh0, Vh1);

    // Scores of the tile in buffer tb, then its softmax and P.V (first position p0).
    constexpr int NKB = 4;
    auto scores = [&](const unsigned char* tb, f32x4 (&sc)[NKB]) __attribute__((always_inline)) {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
            sc[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kc = 0; kc < KC; ++kc) {
                const unsigned char* kp = tb + kb * 16 * RB + koff[kc];
                const bf16x8 ka = *reinterpret_cast<const bf16x8*>(kp);
                if constexpr (PREC) {
                    const bf16x8 kl = *reinterpret_cast<const bf16x8*>(kp + TG::PLANE);
                    sc[kb] = mfma16(kl, qf[0][kc], sc[kb]);
                    sc[kb] = mfma16(ka, qf[NP - 1][kc], sc[kb]);
                }
                sc[kb] = mfma16(ka, qf[0][kc], sc[kb]);
            }
        }
    };
    auto finish = [&](const unsigned char* tb, f32x4 (&sc)[NKB], int p0, bool first) __attribute__((always_inline)) {
        softmax_tile<DB, NKB>(sc, sl2, total - p0 - 4 * g, p0 + 64 > total, first, m_run, thr, o);
#pragma unroll
        for (int h = 0; h < NKB / 2; ++h) {
            const unsigned char* vb0 = tb + NP * TG::PLANE + h * 32 * RB;
            if constexpr (PREC) {
                const unsigned char* vb1 = vb0 + TG::PLANE;
                const bf16x8 ones = __builtin_bit_cast(bf16x8, make_uint4(0x3F803F80u, 0x3F803F80u,
                                                                          0x3F803F80u, 0x3F803F80u));
                bf16x8 pb, pl;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    pb[j] = f2bf(sc[2 * h][j]);
                    pb[4 + j] = f2bf(sc[2 * h + 1][j]);
                    pl[j] = f2bf(sc[2 * h][j] - bf2f(pb[j]));
                    pl[4 + j] = f2bf(sc[2 * h + 1][j] - bf2f(pb[4 + j]));
                }
#pragma unroll
                for (int db = 0; db < DB; ++db) {
                    const bf16x8 va = __builtin_bit_cast(bf16x8, v_frag<RB>(vb0 + voff[db]));
                    const bf16x8 vl = __builtin_bit_cast(bf16x8, v_frag<RB>(vb1 + voff[db]));
                    o[db] = mfma16(vl, pb, o[db]);
                    o[db] = mfma16(va, pl, o[db]);
                    o[db] = mfma16(va, pb, o[db]);
                }
                o[DB] = mfma16(ones, pl, o[DB]);
                o[DB] = mfma16(ones, pb, o[DB]);
            } else {
                // P.V in fp16 (11-bit significand): probabilities lose at most 2^-12
                const f16x8 ones = __builtin_bit_cast(f16x8, make_uint4(0x3C003C00u, 0x3C003C00u,
                                                                        0x3C003C00u, 0x3C003C00u));
                const f16x8 ph = __builtin_bit_cast(
                    f16x8, make_uint4(pack_h2(sc[2 * h][0], sc[2 * h][1]), pack_h2(sc[2 * h][2], sc[2 * h][3]),
                                      pack_h2(sc[2 * h + 1][0], sc[2 * h + 1][1]),
                                      pack_h2(sc[2 * h + 1][2], sc[2 * h + 1][3])));
                // the V fragments in groups of VG blocks, every read of a group in
                // flight before its first product (measured: 2 at D = 64, 4 at D = 128)
                constexpr int VG = D == 64 ? 2 : 4;
#pragma unroll
                for (int d0 = 0; d0 < DB; d0 += VG) {
                    uint4 vf[VG];
#pragma unroll
                    for (int i = 0; i < VG; ++i) vf[i] = v_frag<RB>(vb0 + voff[d0 + i]);
#pragma unroll
                    for (int i = 0; i < VG; ++i)
                        o[d0 + i] = mfma16h(__builtin_bit_cast(f16x8, vf[i]), ph, o[d0 + i]);
                }
                o[DB] = mfma16h(ones, ph, o[DB]);
            }
        }
    };

    // One tile (t % NB == J): wait for this wave's copy of tile t (the copies of
    // the NB - 2 later tiles already issued may stay in flight) and meet the
    // other waves, so tile t is in LDS and buffer (t - 1) % NB is no longer
    // read; then the last wave looks up tile t + NB, every wave issues its part
    // of the copy of tile t + NB - 1 into buffer (t - 1) % NB, and tile t is
    // computed. Steps run in whole rounds of NB, and every step copies a tile
    // (past the selection: row 0 repeated, one cache line, never used), so every
    // wait counts the same copies on every path.
    auto step = [&](int t, auto j_c) __attribute__((always_inline)) {
        constexpr int J = decltype(j_c)::value;
        tiles_ready_barrier<TG::L * (NB - 2)>();
        if (w == LW) lookup(t + NB);
        const bool act = t < ntiles && live;
        f32x4 sc[NKB];
        // D = 128: the score fragments are read before the key rows of the
        // copy, so the two LDS latencies overlap (measured 4 % faster on
        // 32.8K tokens; at D = 64 the later copy issue cost 2 %)
        if (LATE_COPY && act) scores(buf(j_c), sc);
        tile_copy<D, NP, NT>(buf(std::integral_constant<int, J + NB - 1>{}), w, l,
                             krow[(t + NB - 1) & 3], Kh0, Kh1, Vh0, Vh1);
        if (act) {
            if (!LATE_COPY) scores(buf(j_c), sc);
            finish(buf(j_c), sc, t * 64, t == 0);
        }
    };
    for (int t = 0; t < ntiles; t += NB) {
        step(t, std::integral_constant<int, 0>{});
        step(t + 1, std::integral_constant<int, 1>{});
        if constexpr (NB > 2) step(t + 2, std::integral_constant<int, 2>{});
        if constexpr (NB > 3) step(t + 3, std::integral_constant<int, 3>{});
    }

    if (qok) {
        const float l_tot = o[DB][0];  // every row of the ones block holds the sum
        // the fp16 V plane of a bf16 head carries the factor 2^e: undo it here
        const float vinv = PREC ? 1.0f : pow2f(-v_scale_exp(vmax[bh]));
        const float inv = l_tot > 0.0f ? vinv / l_tot : 0.0f;
        TO* orow = O + ((int64_t)bh * N + qtok) * D;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int i = 0; i < 4; ++i) elem<TO>::store(orow, db * 16 + g * 4 + i, o[db][i] * inv);
        if (g == 0 && lse)
            lse[(int64_t)bh * N + qtok] =
                l_tot > 0.0f ? (m_run + __log2f(l_tot)) * 0.69314718055994531f : -INFINITY;
    }
    __syncthreads();  // LDS (runs, tiles, sh_item) is reused by the next item
    }
}

#ifndef ADC_ATTN_WPE64
#define ADC_ATTN_WPE64 6
#endif
constexpr int ATTN_WPE64 = ADC_ATTN_WPE64;  // waves per SIMD asked of the bf16 D=64 kernel

// Compute units of the current device (read once per device).
static int cu_count() {
    static int cached[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
    if (cached[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
            n = 256;
        cached[dev] = n;
    }
    return cached[dev];
}

template <typename T, typename TO>
static void launch_attn_t(const Prob& p, int Cq, const void* q, const int32_t* q_perm,
                          const int32_t* q_offsets, const u16* k0, const u16* k1, const u16* v0,
                          const u16* v1, const int32_t* run_start, const int32_t* run_pos,
                          const int32_t* n_runs, int run_cap, const AttnSched& sc, int cap,
                          float sl2, const uint32_t* vmax, void* out, float* lse, hipStream_t s) {
    // waves per SIMD: three workgroups per CU for bf16 D = 64 (80 registers,
    // three 16 KB tile buffers), two for bf16 D = 128 and f32 D = 64 (at most
    // 128 registers, two 32 KB buffers), one for f32 D = 128 (64 KB tiles)
    constexpr int W64 = sizeof(T) == 2 ? ATTN_WPE64 : 4;
    constexpr int W128 = sizeof(T) == 2 ? 4 : 2;
    const int wpe = p.D == 64 ? W64 : W128;
    auto k = p.D == 64 ? attn_kernel<T, 64, TO, W64> : attn_kernel<T, 128, TO, W128>;
    // as many workgroups as fit at once (wpe * 4 SIMDs / 8 waves per CU), but
    // no more than the work items can be (cap per head), in whole rounds of the
    // eight XCDs: a workgroup without an item still visits every stretch
    const int per_cu = std::max(1, wpe / 2);
    const int64_t wgs = std::min<int64_t>((int64_t)cu_count() * per_cu, (int64_t)p.BH * cap);
    const dim3 grid((unsigned)((wgs + 7) / 8 * 8));
    hipLaunchKernelGGL(k, grid, dim3(512), 0, s, p.N, Cq, (const T*)q, q_perm, q_offsets, k0, k1,
                       v0, v1, run_start, run_pos, n_runs, run_cap, sc.items, sc.head_pos,
                       sc.xcd_start, sc.xcd_ctr, p.BH, cap, sl2, vmax, (TO*)out, lse);
}

// ------------------------------------------------------------------ allocation-free scratch
// Workspace of adacluster_sparse_attn_noalloc: one static array per device
// (the code object's copy on each GPU), held until the process ends. Host code
// never passes the array's name to a kernel: it takes the device address
// hipGetSymbolAddress returns for the current device, once per device, and
// hands that address on as the workspace.
static __device__ __align__(256) unsigned char scratch[ADC_NOALLOC_SCRATCH_BYTES];

hipError_t noalloc_scratch(void** out) {
    constexpr int MAX_DEVICES = 64;
    static std::mutex mu;
    static void* ptrs[MAX_DEVICES] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= MAX_DEVICES) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!ptrs[dev]) {
        void* ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!ptr) return hipErrorInvalidSymbol;
        ptrs[dev] = ptr;
    }
    *out = ptrs[dev];
    return hipSuccess;
}

hipError_t launch_attention(const Prob& p, int Cq, const void* q, const int32_t* q_perm,
                            const int32_t* q_offsets, const u16* k0, const u16* k1,
                            const u16* v0, const u16* v1, const int32_t* run_start,
                            const int32_t* run_pos, const int32_t* n_runs, int run_cap,
                            const AttnSched& sc, int cap, float scale, const uint32_t* vmax,
                            void* out, int out_f32, float* lse, hipStream_t s) {
    if (cap <= 0) return hipSuccess;
    const float sl2 = scale * 1.4426950408889634f;
    if (p.bf16) {
        if (out_f32)
            launch_attn_t<u16, float>(p, Cq, q, q_perm, q_offsets, k0, k1, v0, v1, run_start,
                                      run_pos, n_runs, run_cap, sc, cap, sl2, vmax, out, lse, s);
        else
            launch_attn_t<u16, u16>(p, Cq, q, q_perm, q_offsets, k0, k1, v0, v1, run_start,
                                    run_pos, n_runs, run_cap, sc, cap, sl2, vmax, out, lse, s);
    } else {
        launch_attn_t<float, float>(p, Cq, q, q_perm, q_offsets, k0, k1, v0, v1, run_start,
                                    run_pos, n_runs, run_cap, sc, cap, sl2, vmax, out, lse, s);
    }
    return hipGetLastError();
}

}  // namespace adc
