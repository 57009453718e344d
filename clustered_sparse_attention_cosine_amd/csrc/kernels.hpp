// Internal launchers of the gfx950 kernels (host side). Every launcher enqueues
// on `stream` and returns the hipError_t of its launch.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace adc {

// Draw-stream tags of the two clustered tensors.
constexpr uint32_t TENSOR_Q = 1, TENSOR_K = 2;

// Workload-independent problem descriptor for one batched launch.
struct Prob {
    int BH;     // B * H independent heads
    int H;      // heads per batch entry (stream keys use b = bh / H, h = bh % H)
    int N;      // rows per head
    int D;      // 64 or 128
    int bf16;   // 1: inputs are bf16 words, 0: f32
};

// ---------------------------------------------------------------- fills (kmeans.hip)
hipError_t fill_i32(int32_t* p, int64_t n, int32_t v, hipStream_t s);
hipError_t fill_u8(uint8_t* p, int64_t n, uint8_t v, hipStream_t s);
hipError_t launch_fixed_info(int BH, int N, int m, int32_t* n_clusters, uint8_t* full, float* tau,
                             int32_t* stage_sizes, hipStream_t s);
// Warm start: clamp the caller's per-head counts to [1, cap] in place and write
// the fixed-path stage record.
hipError_t launch_warm_info(int BH, int N, int cap, int32_t* n_clusters, int32_t* stage_sizes,
                            hipStream_t s);

// ---------------------------------------------------------------- k-means (kmeans.hip)
// 1 / max(||x_i||, 1e-12) per row (norm in f64).
hipError_t launch_inv_norm(const Prob& p, const void* x, float* inv_norm, hipStream_t s);
// xhat_i = x_i / max(||x_i||, 1e-12) in f32 (norm summed in index order, f64).
hipError_t launch_normalize(const Prob& p, const void* x, float* xhat, hipStream_t s);

// Centroid-array view: cent/valid/c_hi/c_lo/cn2 hold `cap` slots per head;
// kernels see slots [base, base + m). sums ([BH][cap][D]) and part
// ([BH][ceil(N/64)][2][D]) hold the member sums of an update (see
// launch_update_accum).
struct CentView {
    float* cent;
    uint8_t* valid;
    uint16_t* c_hi;
    uint16_t* c_lo;
    float* cn2;
    float* sums;
    float* part;
    int nwav;   // waves of 64 sorted rows per head in part (ceil(N / 64))
    int cap;
    int base;
    int m;
    // Pruned assignment (may be null): per slot a, a bit set over the view's
    // slots (cbits [BH][cap][cwords]) of the slots that can be the nearest
    // centre of a row now labelled a.
    const uint32_t* cbits = nullptr;
    int cwords = 0;
    // labels the pruned assignment gathers by (may be null: the labels it
    // writes, read before they are overwritten)
    const int32_t* glab = nullptr;
};
// candidate slots a pruned workgroup gathers (an index list of 16-bit slots in LDS)
template <int D>
constexpr int ucap() { return D == 64 ? 1024 : 4096; }

// Rows a k-means call clusters: rows[bh*N + r] for r < nrows[bh] (NULL: all N
// rows, identity), only for heads with active[bh] != 0 (NULL: all heads).
// With by_token, labels (and the bounds below) are indexed by the row's token
// rows[bh*N + r] rather than by its position r.
struct RowSet {
    const int32_t* rows;
    const int32_t* nrows;
    const uint8_t* active;
    int by_token;
};

// Seeded systematic sample of min(m, n) rows; slots beyond hold no centre.
hipError_t launch_init_sample(const Prob& p, const void* x, int normalize, RowSet rs,
                              CentView cv, uint64_t seed, uint32_t tensor, uint32_t stage,
                              hipStream_t s);
// Seeded k-means++ (one workgroup per head). xf: f32 rows to cluster (the
// normalised queries, or NULL to read `x` directly); d2/chosen are scratch.
hipError_t launch_init_kmeanspp(const Prob& p, const void* x, const float* xf, RowSet rs,
                                CentView cv, uint64_t seed, uint32_t tensor, uint32_t stage,
                                double* d2, uint8_t* chosen, hipStream_t s);
// Centroid prep: split into bf16 hi/lo, squared norms (+inf where no centre).
// With soff != NULL (the offsets [BH][m + 1] of the rows sorted by label that
// launch_update_accum walked) it first moves every slot with members to the
// mean of its members' sums; then with drift != NULL also drift[slot] >=
// ||new - old|| (0 where no centre). zero_a/b/c (may be null): per-head
// counters [BH] cleared on the way.
// With rad (and part_rad, the update's part radii) it also completes each
// slot's radius: the largest ub of its rows (0 for a slot without rows).
hipError_t launch_finalize(const Prob& p, CentView cv, const uint8_t* active, const int32_t* soff,
                           hipStream_t s, float* drift = nullptr, int32_t* zero_a = nullptr,
                           int32_t* zero_b = nullptr, int32_t* zero_c = nullptr,
                           float* rad = nullptr, const float* part_rad = nullptr);
// Fixed points of Lloyd rounds over row subsets (see kmeans.hip): lact = active
// (1 for all without), chg = 0; after each round's assignment prev <- labels,
// and from the second round a head whose labels all stayed gets lact = 0.
hipError_t launch_conv_init(const Prob& p, const uint8_t* active, uint8_t* lact, int32_t* chg, hipStream_t s);
hipError_t launch_conv_round(const Prob& p, RowSet rs, const int32_t* labels, int32_t* prev, uint8_t* lact,
                             int32_t* chg, bool compare, hipStream_t s);
// Flag lists of the certified assignment (see kmeans.hip).
struct FlagSet {
    int32_t* list;
    int32_t* count;
    float* thr;
    int32_t* over;
    int32_t* over_count;
    int32_t* cand;    // [BH, N, CAND_CAP] candidate slots of each flagged row
    int32_t* ccount;  // [BH, N] number of candidates found (may exceed CAND_CAP)
    // optional [BH, N]: upper bound on the distance of each row to the centre it
    // is given and lower bound on its distance to every other centre (+inf / 0
    // for a row the certified pass could not settle)
    float* ub = nullptr;
    float* lb = nullptr;
};
constexpr int CAND_CAP = 16;
// Caller centres [BH][cv.m][D] into slots [cv.base, cv.base + cv.m), marked valid.
hipError_t launch_caller_init(const Prob& p, const float* init, CentView cv, hipStream_t s);
// Warm start: slots [0, count[bh]) of cv (base 0) copy their centres from
// init ([BH][cap][D]) and are marked as holding a centre, the rest are not.
hipError_t launch_warm_init(const Prob& p, const float* init, const int32_t* count, CentView cv,
                            hipStream_t s);
// m_eff[bh] = min(mcount[bh], last slot holding a centre + 1).
hipError_t launch_last_valid(const Prob& p, CentView cv, const int32_t* mcount, int32_t* m_eff,
                             hipStream_t s);
// Nearest centre by a bf16 hi/lo matrix-core contraction with a certified
// error bound; uncertain rows are settled by exact f64 distances of the
// centres inside their uncertainty band (labels are final on return).
// split > 1: for calls over few rows, the centre tiles are also split over up to
// `split` workgroups per row block (same labels; shorter serial chain per row).
// With cv.clist set (pruned assignment): rs.rows lists the rows sorted by
// their current label (by token), and each workgroup contracts its rows only
// with the union of their labels' candidate lists (labels is read for the
// current labels and then overwritten with the new ones).
hipError_t launch_assign(const Prob& p, const void* x, RowSet rs, const float* inv_norm,
                         int normalize, CentView cv, const int32_t* mcount, int32_t* labels,
                         FlagSet fs, hipStream_t s, int split = 0, bool counts_zeroed = false);
// Candidate sets for the pruned assignment (Elkan's first lemma): for slot a
// with radius R = rad[a] + drift[a] (drift may be null), every slot j holding
// a centre with ||c_j - c_a|| <= 2 R (up to a rounding margin taken in the
// safe direction), as bits of cbits [BH][cv.cap][cwords]. A row of a is
// strictly closer to c_a than to any slot left out, so its nearest centre,
// ties included, is in the set. Sets are formed for the slots a < am (am < 0:
// every slot of the view), over every slot of the view.
hipError_t launch_cand_bits(const Prob& p, CentView cv, const int32_t* mcount, const float* rad,
                            const float* drift, uint32_t* cbits, int cwords, hipStream_t s, int am = -1);
// Bound test between Lloyd rounds (every row, rs.rows NULL): a row whose bound on
// its own centre, grown by that centre's drift, stays below its bound on every
// other centre, shrunk by the largest drift, keeps its label and the moved
// bounds; the others are appended to rlist (tokens, rcount[bh] cleared beforehand).
hipError_t launch_bound_filter(const Prob& p, RowSet rs, CentView cv, const int32_t* labels,
                               float* ub, float* lb, const float* drift, int32_t* rlist,
                               int32_t* rcount, hipStream_t s);
// Member sums for the current labels, taken over the rows in `order` (the
// stable sort of the rows by label, [BH][N]) with n rows per head (rs.nrows,
// or N). Wave W sums the runs of equal labels among sorted rows
// [64 W, 64 W + 64) in row order: a cluster whose rows all lie there is stored
// to sums; the part of a longer cluster at the start of the range goes to
// part[W][0], the part at the end to part[W][1], and finalize adds a long
// cluster's parts in wave order. No atomics: the sums do not depend on
// scheduling, so identical inputs give identical centres.
// With ub (an upper bound on each row's distance to its centre, by token) it
// also takes each slot's radius, the largest ub of its rows: rad [BH][cap]
// for clusters inside one wave, part_rad [BH][nwav][2] for the parts that
// finalize combines.
hipError_t launch_update_accum(const Prob& p, const void* x, RowSet rs, const float* inv_norm,
                               const int32_t* labels, CentView cv, const int32_t* order,
                               hipStream_t s, const float* ub = nullptr, float* rad = nullptr,
                               float* part_rad = nullptr);

// Copy of the centres of view cv (slots [base, base + m) of every head with
// active[bh] != 0, active may be null) into dst, same [BH][cap][D] layout.
hipError_t launch_copy_slots(const Prob& p, CentView cv, const uint8_t* active, float* dst,
                             hipStream_t s);
// Record of one stage of Algorithm 1: stage_labels[bh][t][token] = base + the
// stage label of each row of rs (labels by position), stage_base[bh][t] = base,
// for heads running the stage.
constexpr int TRACE_STAGES = 8;
hipError_t launch_trace_stage(const Prob& p, RowSet rs, const int32_t* labels, int base, int t,
                              int32_t* stage_labels, int32_t* stage_base, hipStream_t s);

// ---------------------------------------------------------------- multi-stage state
struct StageState {
    int32_t* nu;         // [BH] |U|
    int32_t* slots;      // [BH] slots used so far
    uint8_t* full;       // [BH] F
    uint8_t* active;     // [BH] stage runs for this head
    int32_t* n_stages;   // [BH]
    double* tau;         // [BH]
    int32_t* u_a;        // [BH][N] U lists (ping-pong)
    int32_t* u_b;
    double* dist;        // [BH][N] stage distances
    int32_t* stage_sizes;  // [BH][8] or NULL
};
hipError_t launch_stage_reset(const Prob& p, StageState st, hipStream_t s);
hipError_t launch_stage_begin(const Prob& p, StageState st, int t, int nmax, hipStream_t s);
hipError_t launch_stage_dist(const Prob& p, const void* k, RowSet rs, const int32_t* labels,
                             CentView cv, double* dist, hipStream_t s);
hipError_t launch_stage_tau(const Prob& p, StageState st, double tau_mult, hipStream_t s);
hipError_t launch_stage_compact(const Prob& p, StageState st, const int32_t* u_in,
                                int32_t* u_out, int m_t, hipStream_t s);
hipError_t launch_stage_end(const Prob& p, StageState st, int t_total, int nmax,
                            int32_t* n_clusters, uint8_t* full_out, float* tau_out,
                            hipStream_t s);

// ---------------------------------------------------------------- diagnostics (diag.hip)
// Per head: MSE, mean distance to the centre and Davies-Bouldin index of a
// clustering given as cluster-contiguous rows x_perm with offsets ([BH][M+1])
// and centres cent ([BH][M][D]); comp[b] = 1 / mean over heads of MSE (may be
// null). Scratch: csq, cdist [BH][M] f64; smean, dbmax [BH][M] f32.
hipError_t launch_compactness(const Prob& p, int M, const void* x_perm, const int32_t* offsets,
                              const float* cent, double* csq, double* cdist, float* smean,
                              float* dbmax, double* mse, double* mean_dist, double* db,
                              double* comp, hipStream_t s);

// ---------------------------------------------------------------- layout (permute.hip)
hipError_t launch_scan_offsets(const Prob& p, const int32_t* cnt, int M, int32_t* sizes_out,
                               int32_t* offsets, hipStream_t s, const uint8_t* active = nullptr);
// Stable counting sort by label (M <= 8192) over segments of SORT_SEG rows:
// sizes [BH][M], offsets [BH][M+1], perm [BH][N] out; seg_cnt
// [BH][sort_segments(N)][M] and total [BH][M] are scratch. With nrows (may be
// null) only the first nrows[bh] rows of a head are sorted; heads with
// active[bh] == 0 (active may be null) are skipped.
constexpr int SORT_SEG = 4096;
static_assert(SORT_SEG % 1024 == 0, "the ranking pass takes 1024 rows per step");
int sort_segments(int N);
hipError_t launch_counting_sort(const Prob& p, const int32_t* labels, int M, int32_t* seg_cnt,
                                int32_t* total, int32_t* sizes, int32_t* offsets, int32_t* perm,
                                hipStream_t s, const int32_t* nrows = nullptr,
                                const uint8_t* active = nullptr);
// Per cluster: member means (of normalised rows when normalize), raw means,
// per-dimension max/min and the permuted copies of x and v.
hipError_t launch_gather_stats(const Prob& p, int M, const int32_t* offsets, const int32_t* perm,
                               const void* x, const void* v, int normalize, float* means,
                               float* raw_means, void* xmax, void* xmin, void* x_perm,
                               void* v_perm, hipStream_t s);

// ---------------------------------------------------------------- selection (select.hip)
hipError_t launch_scores(const Prob& p, int Cq, int Ck, const float* qrep, const void* kmax,
                         const void* kmin, const float* kcent, int score_mode, bool logn, float scale,
                         const int32_t* k_sizes, const int32_t* n_clusters, uint32_t* keys,
                         hipStream_t s);
hipError_t launch_topp(const Prob& p, int Cq, int Ck, const uint32_t* keys, const int32_t* k_sizes,
                       const uint8_t* full, float top_p, uint32_t* mask, int32_t* sel_keys, hipStream_t s);
hipError_t launch_topk(const Prob& p, int Cq, int Ck, const uint32_t* keys, const int32_t* k_sizes,
                       const uint8_t* full, float scale, int top_k, uint32_t* mask, int32_t* sel_keys,
                       hipStream_t s);

// pairs[bh] = sum over q-clusters a of (q_offsets[a + 1] - q_offsets[a]) x sel_keys[a].
hipError_t launch_pairs(const Prob& p, int Cq, const int32_t* q_offsets, const int32_t* sel_keys,
                        int64_t* pairs, hipStream_t s);

// ---------------------------------------------------------------- attention (attn.hip)
hipError_t launch_build_runs(const Prob& p, int Cq, int Ck, const int32_t* k_offsets,
                             const uint32_t* mask, int run_cap, int32_t* run_start,
                             int32_t* run_pos, int32_t* n_runs, hipStream_t s);
// Attention schedule: the work items of each head (q-cluster, 128-row chunk)
// in two halves (large q-clusters first), their cost prefix, per-part totals
// and the sixteen cost-balanced stretches (one per XCD and half) with their
// queue counters.
struct AttnSched {
    // the list holds 2 BH parts: the items of the large q-clusters of every
    // head (part bh), then those of the others (part BH + bh)
    int32_t* items;      // [2 BH][cap] a | chunk << 16
    int32_t* n_items;    // [2 BH]
    uint32_t* cost_pre;  // [2 BH][cap] inclusive cost prefix inside the part
    uint32_t* n_cost;    // [2 BH]
    int32_t* head_pos;   // [2 BH + 1] items before each part
    uint64_t* head_cost; // [2 BH + 1] cost before each part
    int32_t* xcd_start;  // [17] first item of each of the 16 stretches, then the total
    int32_t* xcd_ctr;    // [16] items taken from each stretch
    uint64_t* load;      // [BH][2] summed item cost and item count per head
};
hipError_t launch_worklist(const Prob& p, int Cq, int cap, const int32_t* q_offsets,
                           const int32_t* run_start, const int32_t* run_pos, const int32_t* n_runs,
                           int run_cap, const AttnSched& sc, hipStream_t s);
// Operand planes of the attention kernel. bf16: V' to fp16 scaled per head by
// a power of two (vmax [BH] receives each head's largest |v| as bf16 bits);
// f32: K' and V' split into bf16 hi/lo planes (vmax unused).
hipError_t launch_planes(const Prob& p, const void* k, const void* v, uint16_t* k_hi, uint16_t* k_lo,
                         uint16_t* v_hi, uint16_t* v_lo, uint32_t* vmax, hipStream_t s);
hipError_t launch_attention(const Prob& p, int Cq, const void* q, const int32_t* q_perm,
                            const int32_t* q_offsets, const uint16_t* k0, const uint16_t* k1,
                            const uint16_t* v0, const uint16_t* v1, const int32_t* run_start,
                            const int32_t* run_pos, const int32_t* n_runs, int run_cap,
                            const AttnSched& sc, int cap, float scale, const uint32_t* vmax,
                            void* out, int out_f32, float* lse, hipStream_t s);

constexpr int ATTN_ROWS = 128;  // query rows per attention work item

// Device address of this device's static scratch array (ADC_NOALLOC_SCRATCH_BYTES
// bytes), looked up once per device.
hipError_t noalloc_scratch(void** ptr);

}  // namespace adc
