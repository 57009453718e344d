// C ABI of the clustered sparse attention library: argument checks (all before
// the first launch), workspace carving and the order of kernel launches for
// each stage. The method follows "AdaCluster: Adaptive Query-Key Clustering for
// Sparse Attention in Video Generation" (arXiv 2604.18348v1); the per-stage
// citations are in include/adacluster.h and next to each kernel.
#include <hip/hip_runtime.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>
#include <algorithm>

#include "../../include/adacluster.h"
#include "kernels.hpp"

using namespace adc;

namespace {

thread_local char g_err[512] = "";

int32_t fail(int32_t code, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return code;
}

#define HIPCHK(expr)                                                                      \
    do {                                                                                  \
        hipError_t e_ = (expr);                                                           \
        if (e_ != hipSuccess) return fail(ADC_EHIP, "%s: %s", #expr, hipGetErrorString(e_)); \
    } while (0)

constexpr int MAX_CLUSTERS = 8192;

// Lloyd rounds after the first contract each row only with its label's
// candidate slots (the full contraction gives the same labels).
#ifndef ADC_PRUNE
#define ADC_PRUNE 1
#endif
constexpr bool g_prune = ADC_PRUNE != 0;
constexpr int MAX_N = 1 << 21;

// Bump allocator over the caller's workspace: pieces at 256-byte aligned
// device addresses. The base is first rounded up to a multiple of 256, which
// the 256 bytes of slack every *_workspace() size adds to the measured total
// cover. With base == nullptr it only measures.
struct Carver {
    char* base;
    size_t used = 0;
    explicit Carver(void* b)
        : base(b ? (char*)(((uintptr_t)b + 255) & ~(uintptr_t)255) : nullptr) {}
    template <typename T>
    T* take(size_t count) {
        size_t off = (used + 255) & ~size_t(255);
        used = off + count * sizeof(T);
        return base ? reinterpret_cast<T*>(base + off) : nullptr;
    }
};

int32_t check_shape(const adc_shape* s) {
    if (!s) return fail(ADC_EINVAL, "shape is NULL");
    if (s->B < 1 || s->H < 1 || s->N < 1)
        return fail(ADC_ESHAPE, "B, H, N must be >= 1 (got %d, %d, %d)", s->B, s->H, s->N);
    if (s->N > MAX_N) return fail(ADC_ESHAPE, "N = %d exceeds %d", s->N, MAX_N);
    if (s->D != 64 && s->D != 128) return fail(ADC_ESHAPE, "D must be 64 or 128 (got %d)", s->D);
    if (s->dtype != ADC_F32 && s->dtype != ADC_BF16)
        return fail(ADC_EDTYPE, "dtype must be ADC_F32 or ADC_BF16 (got %d)", s->dtype);
    if ((int64_t)s->B * s->H > 65535) return fail(ADC_ESHAPE, "B*H = %lld exceeds 65535",
                                                   (long long)s->B * s->H);
    return ADC_OK;
}

int32_t check_clusters(const char* what, int32_t c) {
    if (c < 1 || c > MAX_CLUSTERS) return fail(ADC_ESHAPE, "%s = %d outside [1, %d]", what, c, MAX_CLUSTERS);
    return ADC_OK;
}

Prob make_prob(const adc_shape* s) {
    Prob p;
    p.BH = s->B * s->H;
    p.H = s->H;
    p.N = s->N;
    p.D = s->D;
    p.bf16 = s->dtype == ADC_BF16;
    return p;
}

#define REQ(ptr) \
    if (!(ptr)) return fail(ADC_EINVAL, "%s is NULL", #ptr)

// ------------------------------------------------------------------ workspace plans
struct KmeansWs {
    float* inv_norm = nullptr;
    int32_t* flag_list = nullptr;
    int32_t* flag_count = nullptr;
    float* flag_thr = nullptr;
    int32_t* over_list = nullptr;
    int32_t* over_count = nullptr;
    int32_t* cand = nullptr;
    int32_t* ccount = nullptr;
    uint8_t* valid = nullptr;
    uint16_t* c_hi = nullptr;
    uint16_t* c_lo = nullptr;
    float* cn2 = nullptr;
    float* sums = nullptr;
    float* part = nullptr;
    int nwav = 0;
    float* xhat = nullptr;
    double* d2 = nullptr;
    uint8_t* chosen = nullptr;
    int32_t* hist = nullptr;
    int32_t* seg_cnt = nullptr;
    int32_t* m_eff = nullptr;
    // distance bounds of the Lloyd rounds over every row
    float* ub = nullptr;
    float* lb = nullptr;
    int32_t* rlist = nullptr;
    int32_t* rcount = nullptr;
    float* drift = nullptr;
    // pruned assignment: slot radii and candidate lists
    float* rad = nullptr;
    float* part_rad = nullptr;
    uint32_t* cbits = nullptr;
    int cwords = 0;
    // row-subset rounds (later key stages): each row's previous label, and per
    // head whether it is still iterating and whether a label changed
    int32_t* prev_lab = nullptr;
    uint8_t* lact = nullptr;
    int32_t* chg = nullptr;
};

void plan_kmeans(Carver& c, const Prob& p, int cap, bool want_inv, bool kpp, bool want_xhat,
                 KmeansWs& w) {
    const size_t bhn = (size_t)p.BH * p.N;
    const size_t bhc = (size_t)p.BH * cap;
    if (want_inv) w.inv_norm = c.take<float>(bhn);
    w.flag_list = c.take<int32_t>(bhn);
    w.flag_count = c.take<int32_t>(p.BH);
    w.flag_thr = c.take<float>(bhn);
    w.over_list = c.take<int32_t>(bhn);
    w.over_count = c.take<int32_t>(p.BH);
    w.cand = c.take<int32_t>(bhn * CAND_CAP);
    w.ccount = c.take<int32_t>(bhn);
    w.valid = c.take<uint8_t>(bhc);
    w.c_hi = c.take<uint16_t>(bhc * p.D);
    w.c_lo = c.take<uint16_t>(bhc * p.D);
    w.cn2 = c.take<float>(bhc);
    w.sums = c.take<float>(bhc * p.D);
    w.nwav = (p.N + 63) / 64;
    w.part = c.take<float>((size_t)p.BH * w.nwav * 2 * p.D);
    w.hist = c.take<int32_t>(bhc);
    w.seg_cnt = c.take<int32_t>(bhc * sort_segments(p.N));
    w.m_eff = c.take<int32_t>(p.BH);
    w.ub = c.take<float>(bhn);
    w.lb = c.take<float>(bhn);
    w.rlist = c.take<int32_t>(bhn);
    w.rcount = c.take<int32_t>(p.BH);
    w.drift = c.take<float>(bhc);
    w.rad = c.take<float>(bhc);
    w.part_rad = c.take<float>((size_t)p.BH * w.nwav * 2);
    w.cwords = (cap + 31) / 32;
    w.cbits = c.take<uint32_t>(bhc * w.cwords);
    if (kpp) {
        if (want_xhat) w.xhat = c.take<float>(bhn * p.D);
        w.d2 = c.take<double>(bhn);
        w.chosen = c.take<uint8_t>(bhn);
    }
}

struct StageWs {
    StageState st{};
    int32_t* labels_u = nullptr;
    // stage 0: the labels of every key and the keys sorted by them, kept for the
    // pruned final assignment
    int32_t* lab0 = nullptr;
    int32_t* perm0 = nullptr;
};

void plan_stages(Carver& c, const Prob& p, StageWs& w) {
    const size_t bhn = (size_t)p.BH * p.N;
    w.st.nu = c.take<int32_t>(p.BH);
    w.st.slots = c.take<int32_t>(p.BH);
    w.st.full = c.take<uint8_t>(p.BH);
    w.st.active = c.take<uint8_t>(p.BH);
    w.st.n_stages = c.take<int32_t>(p.BH);
    w.st.tau = c.take<double>(p.BH);
    w.st.u_a = c.take<int32_t>(bhn);
    w.st.u_b = c.take<int32_t>(bhn);
    w.st.dist = c.take<double>(bhn);
    w.labels_u = c.take<int32_t>(bhn);
    w.lab0 = c.take<int32_t>(bhn);
    w.perm0 = c.take<int32_t>(bhn);
}

FlagSet flags_of(const KmeansWs& w) {
    return FlagSet{w.flag_list, w.flag_count, w.flag_thr, w.over_list, w.over_count, w.cand,
                   w.ccount};
}

CentView make_view(float* cent, const KmeansWs& w, int cap, int base, int m) {
    CentView v;
    v.cent = cent;
    v.valid = w.valid;
    v.c_hi = w.c_hi;
    v.c_lo = w.c_lo;
    v.cn2 = w.cn2;
    v.sums = w.sums;
    v.part = w.part;
    v.nwav = w.nwav;
    v.cap = cap;
    v.base = base;
    v.m = m;
    return v;
}

// Scratch for the row order of the centroid updates: the caller's layout
// outputs (sizes [BH][>= m], offsets [BH][>= m + 1], perm [BH][N]), which the
// layout pass overwrites afterwards.
struct SortScratch {
    int32_t* sizes;
    int32_t* offsets;
    int32_t* perm;
};

// Lloyd rounds on one centroid view. With final_update the last round also
// moves the centres (multi-stage stages need the stage centres); otherwise the
// last centres are left to the exact member means of the layout pass. Each
// update takes the rows sorted by the round's labels (stable counting sort,
// about 47 us at 75.6K rows x 30 heads), so every cluster is one run of rows
// and its sum is formed without atomics, in a fixed order.
// On every row (rs.rows null) the rounds also keep distance bounds (Hamerly's
// test): from the second round on, only rows whose bounds no longer prove
// their label are assigned again; the others keep it, which the exact
// assignment would too. snap (may be null, [BH][cap][D]) receives the centres
// of view cv as they are just before the last assignment. With final_radii
// (every row, final_update) the last update also leaves each cluster's radius
// and drift for candidate sets of a later pruned assignment, and ss.perm holds
// the rows sorted by the last labels.
hipError_t lloyd(const Prob& p, const void* x, int normalize, RowSet rs, const float* inv_norm,
                 CentView cv, int iters, bool final_update, int32_t* labels, const KmeansWs& w,
                 hipStream_t s, const int32_t* mcount, const SortScratch& ss, float* snap = nullptr,
                 bool final_radii = false) {
    hipError_t e;
    const bool bounds = !rs.rows;
    FlagSet fs = flags_of(w);
    if (bounds) {
        fs.ub = w.ub;
        fs.lb = w.lb;
    }
    // Row subsets (the later key stages): a head whose round leaves every label
    // as the previous round left it has reached its fixed point: the update
    // would give the centres it already holds and every later round the same
    // labels again. It is marked done on the device (rl.active), and the
    // remaining kernels of its rounds return at once; results are those of
    // running every round.
    const bool conv = rs.rows && w.lact;
    RowSet rl = rs;
    if (conv) {
        if ((e = launch_conv_init(p, rs.active, w.lact, w.chg, s))) return e;
        rl.active = w.lact;
    }
    for (int it = 0; it < iters; ++it) {
        RowSet ra = rl;
        CentView ca = cv;
        if (bounds && it > 0) {
            if (g_prune) {
                // pruned round: the rows in the order of the previous round's sort,
                // each contracted only with the slots its label's radius allows
                if ((e = launch_cand_bits(p, cv, mcount, w.rad, w.drift, w.cbits, w.cwords, s))) return e;
                ra = RowSet{ss.perm, nullptr, rs.active, 1};
                ca.cbits = w.cbits;
                ca.cwords = w.cwords;
            } else {
                if ((e = launch_bound_filter(p, rs, cv, labels, w.ub, w.lb, w.drift, w.rlist, w.rcount, s)))
                    return e;
                ra = RowSet{w.rlist, w.rcount, rs.active, 1};
            }
        }
        if (snap && it + 1 == iters && (e = launch_copy_slots(p, cv, rs.active, snap, s))) return e;
        // a row subset (later stages: the few keys left in U) also splits the centre tiles
        // from the second round on, the previous round's finalize cleared the flag counts
        if ((e = launch_assign(p, x, ra, inv_norm, normalize, ca, mcount, labels, fs, s, rs.rows ? 4 : 0,
                               it > 0)))
            return e;
        if (it + 1 < iters || final_update) {
            if (conv && (e = launch_conv_round(p, rl, labels, w.prev_lab, w.lact, w.chg, it > 0, s))) return e;
            // the next round's candidate sets need each cluster's radius (the
            // largest upper bound of its rows), taken by the same sorted walk
            const bool keep = it + 1 < iters || final_radii;  // bounds move on
            const bool radii = bounds && g_prune && keep;
            if ((e = launch_counting_sort(p, labels, cv.m, w.seg_cnt, w.hist, ss.sizes, ss.offsets, ss.perm,
                                          s, rl.nrows, rl.active)))
                return e;
            if ((e = launch_update_accum(p, x, rl, inv_norm, labels, cv, ss.perm, s, radii ? w.ub : nullptr,
                                         w.rad, w.part_rad)))
                return e;
            if (bounds && keep) {
                if ((e = launch_finalize(p, cv, rl.active, ss.offsets, s, w.drift, w.flag_count, w.over_count,
                                         w.rcount, radii ? w.rad : nullptr, w.part_rad)))
                    return e;
            } else if ((e = launch_finalize(p, cv, rl.active, ss.offsets, s, nullptr, w.flag_count,
                                            w.over_count))) {
                return e;
            }
        }
    }
    return hipSuccess;
}

hipError_t init_centres(const Prob& p, const void* x, int normalize, RowSet rs, CentView cv, int init,
                        const float* init_cent, uint64_t seed, uint32_t tensor, uint32_t stage,
                        const KmeansWs& w, hipStream_t s) {
    hipError_t e = hipSuccess;
    if (init == ADC_INIT_SAMPLE) {
        e = launch_init_sample(p, x, normalize, rs, cv, seed, tensor, stage, s);
    } else if (init == ADC_INIT_KMEANSPP) {
        const float* xf = nullptr;
        if (normalize) {
            if ((e = launch_normalize(p, x, w.xhat, s))) return e;
            xf = w.xhat;
        }
        e = launch_init_kmeanspp(p, x, xf, rs, cv, seed, tensor, stage, w.d2, w.chosen, s);
    } else {
        // caller centres: [BH][m][D] copied into slots [base, base + m)
        e = launch_caller_init(p, init_cent, cv, s);
    }
    return e;
}

}  // namespace

extern "C" {

int32_t adacluster_abi_version(void) { return ADACLUSTER_ABI_VERSION; }

const char* adacluster_last_error(void) { return g_err; }

// ====================================================================== cluster_q
static int32_t check_q(const adc_shape* shape, const adc_q_params* prm) {
    int32_t st = check_shape(shape);
    if (st) return st;
    if (!prm) return fail(ADC_EINVAL, "params is NULL");
    if ((st = check_clusters("n_clusters", prm->n_clusters))) return st;
    if (prm->iters < 1 || prm->iters > 1000) return fail(ADC_EINVAL, "iters = %d outside [1, 1000]", prm->iters);
    if (prm->init < 0 || prm->init > 2) return fail(ADC_EINVAL, "init = %d unknown", prm->init);
    return ADC_OK;
}

static void plan_q(Carver& c, const adc_shape* shape, const adc_q_params* prm, KmeansWs& w) {
    Prob p = make_prob(shape);
    plan_kmeans(c, p, prm->n_clusters, true, prm->init == ADC_INIT_KMEANSPP, true, w);
}

size_t adacluster_cluster_q_workspace(const adc_shape* shape, const adc_q_params* prm) {
    if (check_q(shape, prm)) return 0;
    Carver c(nullptr);
    KmeansWs w;
    plan_q(c, shape, prm, w);
    return c.used + 256;
}

int32_t adacluster_cluster_q(const adc_shape* shape, const adc_q_params* prm, const void* q,
                             const float* init_centroids, int32_t* assign, float* centroids,
                             int32_t* sizes, float* qrep, int32_t* perm, int32_t* offsets,
                             void* workspace, size_t workspace_bytes, void* stream) {
    int32_t st = check_q(shape, prm);
    if (st) return st;
    REQ(q); REQ(assign); REQ(centroids); REQ(sizes); REQ(qrep); REQ(perm); REQ(offsets); REQ(workspace);
    if (prm->init == ADC_INIT_CALLER && !init_centroids)
        return fail(ADC_EINVAL, "init == ADC_INIT_CALLER needs init_centroids");
    if (workspace_bytes < adacluster_cluster_q_workspace(shape, prm))
        return fail(ADC_EWORKSPACE, "workspace of %zu bytes is below the %zu required", workspace_bytes,
                    adacluster_cluster_q_workspace(shape, prm));
    hipStream_t s = (hipStream_t)stream;
    Prob p = make_prob(shape);
    const int Cq = prm->n_clusters;
    Carver c(workspace);
    KmeansWs w;
    plan_q(c, shape, prm, w);

    HIPCHK(launch_inv_norm(p, q, w.inv_norm, s));
    CentView cv = make_view(centroids, w, Cq, 0, Cq);
    RowSet all{nullptr, nullptr, nullptr};
    HIPCHK(init_centres(p, q, 1, all, cv, prm->init, init_centroids, prm->seed, TENSOR_Q, 0, w, s));
    HIPCHK(launch_finalize(p, cv, nullptr, nullptr, s));
    const SortScratch ss{sizes, offsets, perm};
    HIPCHK(lloyd(p, q, 1, all, w.inv_norm, cv, prm->iters, false, assign, w, s, nullptr, ss));
    HIPCHK(launch_counting_sort(p, assign, Cq, w.seg_cnt, w.hist, sizes, offsets, perm, s));
    HIPCHK(launch_gather_stats(p, Cq, offsets, perm, q, nullptr, 1, centroids, qrep, nullptr,
                               nullptr, nullptr, nullptr, s));
    return ADC_OK;
}

// ====================================================================== cluster_k
static int32_t check_k(const adc_shape* shape, const adc_k_params* prm) {
    int32_t st = check_shape(shape);
    if (st) return st;
    if (!prm) return fail(ADC_EINVAL, "params is NULL");
    if ((st = check_clusters("base_clusters", prm->base_clusters))) return st;
    if ((st = check_clusters("max_clusters", prm->max_clusters))) return st;
    if (prm->max_clusters < prm->base_clusters)
        return fail(ADC_ESHAPE, "max_clusters (%d) < base_clusters (%d)", prm->max_clusters,
                    prm->base_clusters);
    if (prm->iters < 1 || prm->iters > 1000) return fail(ADC_EINVAL, "iters = %d outside [1, 1000]", prm->iters);
    if (prm->init < 0 || prm->init > 2) return fail(ADC_EINVAL, "init = %d unknown", prm->init);
    if (!(prm->tau_mult >= 0.0f) || prm->tau_mult > 1e6f)
        return fail(ADC_EINVAL, "tau_mult must be a finite value >= 0");
    if (prm->adaptive < ADC_K_FIXED || prm->adaptive > ADC_K_WARM)
        return fail(ADC_EINVAL, "adaptive = %d unknown", prm->adaptive);
    if (prm->adaptive == ADC_K_STAGED && prm->init == ADC_INIT_CALLER)
        return fail(ADC_EUNSUPPORTED, "caller centres need FIXED or WARM (warm steps keep counts fixed)");
    if (prm->adaptive == ADC_K_WARM && prm->init != ADC_INIT_CALLER)
        return fail(ADC_EINVAL, "WARM starts from the previous centres: init must be ADC_INIT_CALLER");
    return ADC_OK;
}

static void plan_k(Carver& c, const adc_shape* shape, const adc_k_params* prm, KmeansWs& w,
                   StageWs& sw) {
    Prob p = make_prob(shape);
    plan_kmeans(c, p, prm->max_clusters, false, prm->init == ADC_INIT_KMEANSPP, false, w);
    if (prm->adaptive == ADC_K_STAGED) {
        plan_stages(c, p, sw);
        w.prev_lab = c.take<int32_t>((size_t)p.BH * p.N);
        w.lact = c.take<uint8_t>(p.BH);
        w.chg = c.take<int32_t>(p.BH);
    }
}

size_t adacluster_cluster_k_workspace(const adc_shape* shape, const adc_k_params* prm) {
    if (check_k(shape, prm)) return 0;
    Carver c(nullptr);
    KmeansWs w;
    StageWs sw;
    plan_k(c, shape, prm, w, sw);
    return c.used + 256;
}

static int32_t cluster_k_impl(const adc_shape* shape, const adc_k_params* prm, const void* k,
                              const void* v, const float* init_centroids, int32_t* n_clusters,
                              uint8_t* full_attn, float* tau, int32_t* assign, float* centroids,
                              int32_t* sizes, void* kmax, void* kmin, int32_t* perm,
                              int32_t* offsets, void* k_perm, void* v_perm, int32_t* stage_sizes,
                              const adc_k_trace* tr, void* workspace, size_t workspace_bytes,
                              void* stream) {
    int32_t st = check_k(shape, prm);
    if (st) return st;
    REQ(k); REQ(v); REQ(n_clusters); REQ(full_attn); REQ(tau); REQ(assign); REQ(centroids);
    REQ(sizes); REQ(kmax); REQ(kmin); REQ(perm); REQ(offsets); REQ(k_perm); REQ(v_perm);
    REQ(workspace);
    if (prm->init == ADC_INIT_CALLER && !init_centroids)
        return fail(ADC_EINVAL, "init == ADC_INIT_CALLER needs init_centroids");
    if (tr && prm->adaptive != ADC_K_STAGED)
        return fail(ADC_EUNSUPPORTED, "a stage record needs the STAGED mode");
    const size_t need = adacluster_cluster_k_workspace(shape, prm);
    if (workspace_bytes < need)
        return fail(ADC_EWORKSPACE, "workspace of %zu bytes is below the %zu required", workspace_bytes, need);
    hipStream_t s = (hipStream_t)stream;
    Prob p = make_prob(shape);
    const int nmax = prm->max_clusters, m0 = prm->base_clusters;
    Carver c(workspace);
    KmeansWs w;
    StageWs sw;
    plan_k(c, shape, prm, w, sw);

    HIPCHK(fill_i32((int32_t*)centroids, (int64_t)p.BH * nmax * p.D, 0, s));
    HIPCHK(fill_u8(w.valid, (int64_t)p.BH * nmax, 0, s));
    RowSet all{nullptr, nullptr, nullptr};
    const SortScratch ss{sizes, offsets, perm};

    if (prm->adaptive == ADC_K_WARM) {
        // steady state (section 3.2.2): per-head counts kept, previous centres as init
        HIPCHK(launch_warm_info(p.BH, p.N, nmax, n_clusters, stage_sizes, s));
        CentView cv = make_view(centroids, w, nmax, 0, nmax);
        HIPCHK(launch_warm_init(p, init_centroids, n_clusters, cv, s));
        HIPCHK(launch_finalize(p, cv, nullptr, nullptr, s));
        HIPCHK(lloyd(p, k, 0, all, nullptr, cv, prm->iters, false, assign, w, s, n_clusters, ss));
    } else if (prm->adaptive == ADC_K_FIXED) {
        CentView cv = make_view(centroids, w, nmax, 0, m0);
        HIPCHK(init_centres(p, k, 0, all, cv, prm->init, init_centroids, prm->seed, TENSOR_K, 0, w, s));
        HIPCHK(launch_finalize(p, cv, nullptr, nullptr, s));
        HIPCHK(lloyd(p, k, 0, all, nullptr, cv, prm->iters, false, assign, w, s, nullptr, ss));
        HIPCHK(launch_fixed_info(p.BH, p.N, m0, n_clusters, full_attn, tau, stage_sizes, s));
    } else {
        if (tr) {
            if (tr->stage_labels)
                HIPCHK(fill_i32(tr->stage_labels, (int64_t)p.BH * TRACE_STAGES * p.N, -1, s));
            if (tr->stage_base) HIPCHK(fill_i32(tr->stage_base, (int64_t)p.BH * TRACE_STAGES, -1, s));
            if (tr->last_centroids)
                HIPCHK(fill_i32((int32_t*)tr->last_centroids, (int64_t)p.BH * nmax * p.D, 0, s));
        }
        StageState S = sw.st;
        S.stage_sizes = stage_sizes;
        HIPCHK(launch_stage_reset(p, S, s));
        int base = 0, t = 0;
        int32_t* u_cur = S.u_a;
        int32_t* u_next = S.u_b;
        while (base < nmax) {
            int mt = (t == 0) ? m0 : (m0 << std::min(t - 1, 20));
            mt = std::min(mt, nmax - base);
            HIPCHK(launch_stage_begin(p, S, t, nmax, s));
            RowSet rs{t == 0 ? nullptr : u_cur, S.nu, S.active};
            CentView cv = make_view(centroids, w, nmax, base, mt);
            HIPCHK(init_centres(p, k, 0, rs, cv, prm->init, nullptr, prm->seed, TENSOR_K, (uint32_t)t, w, s));
            HIPCHK(launch_finalize(p, cv, S.active, nullptr, s));
            // stage 0 (every key) keeps its labels, its row order and its radii for
            // the pruned final assignment
            int32_t* lab = t == 0 ? sw.lab0 : sw.labels_u;
            const SortScratch ss_t{sizes, offsets, t == 0 ? sw.perm0 : perm};
            // from stage 1 on, slots at or past the stage's row count hold no
            // centre (the init fills min(m_t, |U_t|)), so the contractions stop there
            HIPCHK(lloyd(p, k, 0, rs, nullptr, cv, prm->iters, true, lab, w, s, t == 0 ? nullptr : S.nu, ss_t,
                         tr ? tr->last_centroids : nullptr, t == 0 && g_prune));
            if (tr) HIPCHK(launch_trace_stage(p, rs, lab, base, t, tr->stage_labels, tr->stage_base, s));
            HIPCHK(launch_stage_dist(p, k, rs, lab, cv, S.dist, s));
            if (t == 0) HIPCHK(launch_stage_tau(p, S, (double)prm->tau_mult, s));
            HIPCHK(launch_stage_compact(p, S, t == 0 ? nullptr : u_cur, u_next, mt, s));
            std::swap(u_cur, u_next);
            base += mt;
            ++t;
        }
        HIPCHK(launch_stage_end(p, S, t, nmax, n_clusters, full_attn, tau, s));
        // final assignment over every slot that holds a centre (Algorithm 1 step 20)
        CentView cvf = make_view(centroids, w, nmax, 0, nmax);
        if (tr) {
            if (tr->stage_centroids) HIPCHK(launch_copy_slots(p, cvf, nullptr, tr->stage_centroids, s));
            if (tr->slot_valid)
                HIPCHK(hipMemcpyAsync(tr->slot_valid, w.valid, (size_t)p.BH * nmax, hipMemcpyDeviceToDevice, s));
        }
        HIPCHK(launch_finalize(p, cvf, nullptr, nullptr, s));
        // slots after the last one holding a centre (the unfilled end of the last
        // stage) are left out of the contraction
        HIPCHK(launch_last_valid(p, cvf, n_clusters, w.m_eff, s));
        if (g_prune) {
            // pruned: every key is within its stage-0 cluster's radius of that
            // centre, so only the slots within twice the radius can be nearer
            // (Elkan's lemma); the keys go in the order of their stage-0 labels
            HIPCHK(launch_cand_bits(p, cvf, w.m_eff, w.rad, w.drift, w.cbits, w.cwords, s, m0));
            CentView cg = cvf;
            cg.cbits = w.cbits;
            cg.cwords = w.cwords;
            cg.glab = sw.lab0;
            HIPCHK(launch_assign(p, k, RowSet{sw.perm0, nullptr, nullptr, 1}, nullptr, 0, cg, w.m_eff, assign,
                                 flags_of(w), s));
        } else {
            HIPCHK(launch_assign(p, k, all, nullptr, 0, cvf, w.m_eff, assign, flags_of(w), s));
        }
    }
    HIPCHK(launch_counting_sort(p, assign, nmax, w.seg_cnt, w.hist, sizes, offsets, perm, s));
    HIPCHK(launch_gather_stats(p, nmax, offsets, perm, k, v, 0, centroids, nullptr, kmax, kmin,
                               k_perm, v_perm, s));
    return ADC_OK;
}

int32_t adacluster_cluster_k(const adc_shape* shape, const adc_k_params* prm, const void* k,
                             const void* v, const float* init_centroids, int32_t* n_clusters,
                             uint8_t* full_attn, float* tau, int32_t* assign, float* centroids,
                             int32_t* sizes, void* kmax, void* kmin, int32_t* perm,
                             int32_t* offsets, void* k_perm, void* v_perm, int32_t* stage_sizes,
                             void* workspace, size_t workspace_bytes, void* stream) {
    return cluster_k_impl(shape, prm, k, v, init_centroids, n_clusters, full_attn, tau, assign,
                          centroids, sizes, kmax, kmin, perm, offsets, k_perm, v_perm, stage_sizes,
                          nullptr, workspace, workspace_bytes, stream);
}

int32_t adacluster_cluster_k_trace(const adc_shape* shape, const adc_k_params* prm, const void* k,
                                   const void* v, int32_t* n_clusters, uint8_t* full_attn,
                                   float* tau, int32_t* assign, float* centroids, int32_t* sizes,
                                   void* kmax, void* kmin, int32_t* perm, int32_t* offsets,
                                   void* k_perm, void* v_perm, int32_t* stage_sizes,
                                   const adc_k_trace* trace, void* workspace,
                                   size_t workspace_bytes, void* stream) {
    if (!trace) return fail(ADC_EINVAL, "trace is NULL");
    return cluster_k_impl(shape, prm, k, v, nullptr, n_clusters, full_attn, tau, assign, centroids,
                          sizes, kmax, kmin, perm, offsets, k_perm, v_perm, stage_sizes, trace,
                          workspace, workspace_bytes, stream);
}

// ====================================================================== select
static int32_t check_sel_dims(const adc_shape* shape, int32_t Cq, int32_t Ck) {
    int32_t st = check_shape(shape);
    if (st) return st;
    if ((st = check_clusters("Cq", Cq))) return st;
    if ((st = check_clusters("Ck", Ck))) return st;
    return ADC_OK;
}

size_t adacluster_select_workspace(const adc_shape* shape, int32_t Cq, int32_t Ck) {
    if (check_sel_dims(shape, Cq, Ck)) return 0;
    Carver c(nullptr);
    c.take<uint32_t>((size_t)shape->B * shape->H * Cq * Ck);
    return c.used + 256;
}

int32_t adacluster_select(const adc_shape* shape, int32_t Cq, int32_t Ck, const float* qrep,
                          const int32_t* q_offsets, const void* kmax, const void* kmin,
                          const float* centroids, const int32_t* k_sizes,
                          const int32_t* n_clusters, const uint8_t* full_attn, int32_t score,
                          int32_t rule, float top_p, int32_t top_k, float scale,
                          uint32_t* sel_mask, int32_t* sel_keys, int64_t* sel_pairs,
                          void* workspace, size_t workspace_bytes, void* stream) {
    int32_t st = check_sel_dims(shape, Cq, Ck);
    if (st) return st;
    REQ(qrep); REQ(k_sizes); REQ(n_clusters); REQ(full_attn); REQ(sel_mask); REQ(sel_keys); REQ(workspace);
    if (sel_pairs && !q_offsets) return fail(ADC_EINVAL, "sel_pairs needs q_offsets");
    if (score == ADC_SCORE_QUEST) {
        REQ(kmax); REQ(kmin);
    } else if (score == ADC_SCORE_CENTROID) {
        REQ(centroids);
    } else {
        return fail(ADC_EINVAL, "score = %d unknown", score);
    }
    if (rule == ADC_SELECT_TOPP) {
        if (!(top_p > 0.0f && top_p <= 1.0f)) return fail(ADC_EINVAL, "top_p must be in (0, 1]");
    } else if (rule == ADC_SELECT_TOPK) {
        if (top_k < 1) return fail(ADC_EINVAL, "top_k must be >= 1");
    } else {
        return fail(ADC_EINVAL, "rule = %d unknown", rule);
    }
    if (!(scale > 0.0f) || scale > 1e30f) return fail(ADC_EINVAL, "scale must be a finite value > 0");
    const size_t need = adacluster_select_workspace(shape, Cq, Ck);
    if (workspace_bytes < need)
        return fail(ADC_EWORKSPACE, "workspace of %zu bytes is below the %zu required", workspace_bytes, need);
    hipStream_t s = (hipStream_t)stream;
    Prob p = make_prob(shape);
    Carver c(workspace);
    // the ranking keys of every (q-cluster, slot) pair; the selection reads them once
    uint32_t* keys = c.take<uint32_t>((size_t)p.BH * Cq * Ck);
    const bool topp = rule == ADC_SELECT_TOPP;
    HIPCHK(launch_scores(p, Cq, Ck, qrep, kmax, kmin, centroids, score, topp, scale, k_sizes, n_clusters, keys,
                         s));
    if (topp)
        HIPCHK(launch_topp(p, Cq, Ck, keys, k_sizes, full_attn, top_p, sel_mask, sel_keys, s));
    else
        HIPCHK(launch_topk(p, Cq, Ck, keys, k_sizes, full_attn, scale, top_k, sel_mask, sel_keys, s));
    if (sel_pairs) HIPCHK(launch_pairs(p, Cq, q_offsets, sel_keys, sel_pairs, s));
    return ADC_OK;
}

// ====================================================================== sparse attention
struct AttnWs {
    int run_cap;
    int cap;   // work items per head (upper bound)
    int32_t* run_start;
    int32_t* run_pos;
    int32_t* n_runs;
    AttnSched sched;
    uint16_t* planes[4];     // 16-bit operand planes: V fp16 (bf16 inputs); K hi, K lo, V hi, V lo (f32)
    uint32_t* vmax;          // [BH] largest |v| per head (bf16 bits): the fp16 plane's scale
};

static void plan_attn(Carver& c, const adc_shape* shape, int32_t Cq, int32_t Ck, AttnWs& w) {
    const size_t rows = (size_t)shape->B * shape->H * Cq;
    w.run_cap = Ck / 2 + 2;
    w.cap = Cq + (shape->N + ATTN_ROWS - 1) / ATTN_ROWS;
    w.run_start = c.take<int32_t>(rows * w.run_cap);
    w.run_pos = c.take<int32_t>(rows * (w.run_cap + 1));
    w.n_runs = c.take<int32_t>(rows);
    const size_t BH = (size_t)shape->B * shape->H;
    w.sched.items = c.take<int32_t>(2 * BH * w.cap);
    w.sched.n_items = c.take<int32_t>(2 * BH);
    w.sched.cost_pre = c.take<uint32_t>(2 * BH * w.cap);
    w.sched.n_cost = c.take<uint32_t>(2 * BH);
    w.sched.head_pos = c.take<int32_t>(2 * BH + 1);
    w.sched.head_cost = c.take<uint64_t>(2 * BH + 1);
    w.sched.xcd_start = c.take<int32_t>(17);
    w.sched.xcd_ctr = c.take<int32_t>(16);
    w.sched.load = c.take<uint64_t>(2 * BH);
    const size_t elems = (size_t)shape->B * shape->H * shape->N * shape->D;
    for (int i = 0; i < 4; ++i) w.planes[i] = nullptr;
    w.vmax = c.take<uint32_t>(BH);
    if (shape->dtype == ADC_BF16) {
        w.planes[2] = c.take<uint16_t>(elems);
    } else {
        for (int i = 0; i < 4; ++i) w.planes[i] = c.take<uint16_t>(elems);
    }
}

size_t adacluster_sparse_attn_workspace(const adc_shape* shape, int32_t Cq, int32_t Ck) {
    if (check_sel_dims(shape, Cq, Ck)) return 0;
    Carver c(nullptr);
    AttnWs w;
    plan_attn(c, shape, Cq, Ck, w);
    return c.used + 256;
}

static int32_t sparse_attn_impl(const adc_shape* shape, int32_t Cq, int32_t Ck, const void* q,
                                const int32_t* q_perm, const int32_t* q_offsets, const void* k_perm,
                                const void* v_perm, const int32_t* k_offsets,
                                const uint32_t* sel_mask, float scale, void* out, int32_t out_dtype,
                                float* lse, void* workspace, size_t workspace_bytes, void* stream,
                                bool noalloc) {
    int32_t st = check_sel_dims(shape, Cq, Ck);
    if (st) return st;
    REQ(q); REQ(q_perm); REQ(q_offsets); REQ(k_perm); REQ(v_perm); REQ(k_offsets); REQ(sel_mask);
    REQ(out);
    if (!noalloc) REQ(workspace);
    if (!(scale > 0.0f) || scale > 1e30f) return fail(ADC_EINVAL, "scale must be a finite value > 0");
    if (out_dtype != ADC_F32 && !(out_dtype == ADC_BF16 && shape->dtype == ADC_BF16))
        return fail(ADC_EDTYPE, "out_dtype must be ADC_F32, or ADC_BF16 with bf16 inputs");
    const size_t need = adacluster_sparse_attn_workspace(shape, Cq, Ck);
    if (noalloc) {
        if (need > (size_t)ADC_NOALLOC_SCRATCH_BYTES)
            return fail(ADC_EWORKSPACE,
                        "this shape needs %zu bytes of scratch, above the %zu bytes the allocation-free "
                        "entry point holds per device; call adacluster_sparse_attn with a workspace",
                        need, (size_t)ADC_NOALLOC_SCRATCH_BYTES);
        hipError_t e = noalloc_scratch(&workspace);
        if (e != hipSuccess) return fail(ADC_EHIP, "scratch lookup: %s", hipGetErrorString(e));
        workspace_bytes = ADC_NOALLOC_SCRATCH_BYTES;
    } else if (workspace_bytes < need) {
        return fail(ADC_EWORKSPACE, "workspace of %zu bytes is below the %zu required", workspace_bytes, need);
    }
    hipStream_t s = (hipStream_t)stream;
    Prob p = make_prob(shape);
    Carver c(workspace);
    AttnWs w;
    plan_attn(c, shape, Cq, Ck, w);
    HIPCHK(launch_build_runs(p, Cq, Ck, k_offsets, sel_mask, w.run_cap, w.run_start, w.run_pos, w.n_runs, s));
    HIPCHK(launch_worklist(p, Cq, w.cap, q_offsets, w.run_start, w.run_pos, w.n_runs, w.run_cap, w.sched, s));
    HIPCHK(launch_planes(p, k_perm, v_perm, w.planes[0], w.planes[1], w.planes[2], w.planes[3], w.vmax, s));
    const uint16_t* k0 = p.bf16 ? (const uint16_t*)k_perm : w.planes[0];
    HIPCHK(launch_attention(p, Cq, q, q_perm, q_offsets, k0, w.planes[1], w.planes[2], w.planes[3],
                            w.run_start, w.run_pos, w.n_runs, w.run_cap, w.sched, w.cap, scale,
                            w.vmax, out, out_dtype == ADC_F32, lse, s));
    return ADC_OK;
}

int32_t adacluster_sparse_attn(const adc_shape* shape, int32_t Cq, int32_t Ck, const void* q,
                               const int32_t* q_perm, const int32_t* q_offsets, const void* k_perm,
                               const void* v_perm, const int32_t* k_offsets,
                               const uint32_t* sel_mask, float scale, void* out,
                               int32_t out_dtype, float* lse, void* workspace,
                               size_t workspace_bytes, void* stream) {
    return sparse_attn_impl(shape, Cq, Ck, q, q_perm, q_offsets, k_perm, v_perm, k_offsets, sel_mask,
                            scale, out, out_dtype, lse, workspace, workspace_bytes, stream, false);
}

int32_t adacluster_sparse_attn_noalloc(const adc_shape* shape, int32_t Cq, int32_t Ck, const void* q,
                                       const int32_t* q_perm, const int32_t* q_offsets,
                                       const void* k_perm, const void* v_perm,
                                       const int32_t* k_offsets, const uint32_t* sel_mask,
                                       float scale, void* out, int32_t out_dtype, float* lse,
                                       void* stream) {
    return sparse_attn_impl(shape, Cq, Ck, q, q_perm, q_offsets, k_perm, v_perm, k_offsets, sel_mask,
                            scale, out, out_dtype, lse, nullptr, 0, stream, true);
}

// ====================================================================== helpers
size_t adacluster_assign_workspace(const adc_shape* shape, int32_t M) {
    if (check_shape(shape) || check_clusters("M", M)) return 0;
    Carver c(nullptr);
    KmeansWs w;
    plan_kmeans(c, make_prob(shape), M, true, false, false, w);
    return c.used + 256;
}

int32_t adacluster_assign(const adc_shape* shape, int32_t M, int32_t normalize, const void* x,
                          const float* centroids, const uint8_t* valid, int32_t* assign,
                          void* workspace, size_t workspace_bytes, void* stream) {
    int32_t st = check_shape(shape);
    if (st) return st;
    if ((st = check_clusters("M", M))) return st;
    REQ(x); REQ(centroids); REQ(assign); REQ(workspace);
    const size_t need = adacluster_assign_workspace(shape, M);
    if (workspace_bytes < need)
        return fail(ADC_EWORKSPACE, "workspace of %zu bytes is below the %zu required", workspace_bytes, need);
    hipStream_t s = (hipStream_t)stream;
    Prob p = make_prob(shape);
    Carver c(workspace);
    KmeansWs w;
    plan_kmeans(c, p, M, true, false, false, w);
    if (valid)
        HIPCHK(hipMemcpyAsync(w.valid, valid, (size_t)p.BH * M, hipMemcpyDeviceToDevice, s));
    else
        HIPCHK(fill_u8(w.valid, (int64_t)p.BH * M, 1, s));
    // centres are only read (finalize without sums does not write them)
    CentView cv = make_view(const_cast<float*>(centroids), w, M, 0, M);
    RowSet all{nullptr, nullptr, nullptr};
    if (normalize) HIPCHK(launch_inv_norm(p, x, w.inv_norm, s));
    HIPCHK(launch_finalize(p, cv, nullptr, nullptr, s));
    HIPCHK(launch_assign(p, x, all, normalize ? w.inv_norm : nullptr, normalize, cv, nullptr,
                         assign, flags_of(w), s));
    return ADC_OK;
}

size_t adacluster_permute_workspace(const adc_shape* shape, int32_t M) {
    if (check_shape(shape) || check_clusters("M", M)) return 0;
    Carver c(nullptr);
    c.take<int32_t>((size_t)shape->B * shape->H * M);
    c.take<int32_t>((size_t)shape->B * shape->H * M * sort_segments(shape->N));
    return c.used + 256;
}

int32_t adacluster_permute(const adc_shape* shape, int32_t M, const int32_t* assign, const void* x,
                           const void* v, int32_t* sizes, int32_t* offsets, int32_t* perm,
                           float* means, void* xmax, void* xmin, void* x_perm, void* v_perm,
                           void* workspace, size_t workspace_bytes, void* stream) {
    int32_t st = check_shape(shape);
    if (st) return st;
    if ((st = check_clusters("M", M))) return st;
    REQ(assign); REQ(x); REQ(sizes); REQ(offsets); REQ(perm); REQ(workspace);
    if (v_perm && !v) return fail(ADC_EINVAL, "v_perm needs v");
    const size_t need = adacluster_permute_workspace(shape, M);
    if (workspace_bytes < need)
        return fail(ADC_EWORKSPACE, "workspace of %zu bytes is below the %zu required", workspace_bytes, need);
    hipStream_t s = (hipStream_t)stream;
    Prob p = make_prob(shape);
    Carver c(workspace);
    int32_t* hist = c.take<int32_t>((size_t)p.BH * M);
    int32_t* seg_cnt = c.take<int32_t>((size_t)p.BH * M * sort_segments(p.N));
    HIPCHK(launch_counting_sort(p, assign, M, seg_cnt, hist, sizes, offsets, perm, s));
    HIPCHK(launch_gather_stats(p, M, offsets, perm, x, v, 0, means, nullptr, xmax, xmin, x_perm,
                               v_perm, s));
    return ADC_OK;
}

// ====================================================================== diagnostics
size_t adacluster_compactness_workspace(const adc_shape* shape, int32_t M) {
    if (check_shape(shape) || check_clusters("M", M)) return 0;
    Carver c(nullptr);
    const size_t n = (size_t)shape->B * shape->H * M;
    c.take<double>(n);
    c.take<double>(n);
    c.take<float>(n);
    c.take<float>(n);
    return c.used + 256;
}

int32_t adacluster_compactness(const adc_shape* shape, int32_t M, const void* x_perm,
                               const int32_t* offsets, const float* centroids, double* mse,
                               double* mean_dist, double* db, double* comp, void* workspace,
                               size_t workspace_bytes, void* stream) {
    int32_t st = check_shape(shape);
    if (st) return st;
    if ((st = check_clusters("M", M))) return st;
    REQ(x_perm); REQ(offsets); REQ(centroids); REQ(mse); REQ(mean_dist); REQ(db); REQ(workspace);
    const size_t need = adacluster_compactness_workspace(shape, M);
    if (workspace_bytes < need)
        return fail(ADC_EWORKSPACE, "workspace of %zu bytes is below the %zu required", workspace_bytes, need);
    hipStream_t s = (hipStream_t)stream;
    Prob p = make_prob(shape);
    Carver c(workspace);
    const size_t n = (size_t)p.BH * M;
    double* csq = c.take<double>(n);
    double* cdist = c.take<double>(n);
    float* smean = c.take<float>(n);
    float* dbmax = c.take<float>(n);
    HIPCHK(launch_compactness(p, M, x_perm, offsets, centroids, csq, cdist, smean, dbmax, mse,
                              mean_dist, db, comp, s));
    return ADC_OK;
}

}  // extern "C"
