/*
 * AdaCluster clustered sparse attention: plain CPU oracle.
 *
 * TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the benchmark's
 * CPU-baseline leg may load this file's library. It shares no code, header,
 * table or helper with the HIP library, and the HIP library never calls it.
 *
 * What it follows: "AdaCluster: Adaptive Query-Key Clustering for Sparse
 * Attention in Video Generation" (Tan, Wang et al., arXiv 2604.18348v1):
 *   section 3.1 and Algorithm 3 step 1   query normalisation + k-means
 *   section 3.2.2, Algorithm 1           multi-stage key clustering
 *   section 4.1 "Platform and configurations"  tau = 1.5 x mean distance
 *   section 3.2.3, Eq. (1)               Quest upper-bound score
 *   Algorithm 3 steps 3-9                 selection and attention over K*, V*
 *   section 3.2.1 and Fig. 10             compactness diagnostics
 * Readings where the paper is silent or garbled are listed beside each step.
 *
 * Arithmetic: tensors are float32; every distance, sum, softmax denominator and
 * cumulative mass is accumulated in double, in index order, with no fast-math
 * and no FMA contraction (build with -ffp-contract=off). Loops marked
 * "omp parallel for" compute independent outputs, so results do not depend on
 * the thread count.
 *
 * Parity status: every function below is pinned by the CPU test suite against
 * brute force, closed forms, invariants or hand-built cases; none is pinned to
 * numbers printed by the paper, which prints no worked example.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORC_INIT_KMEANSPP = 0, ORC_INIT_SAMPLE = 1, ORC_INIT_CALLER = 2 };
enum { ORC_TENSOR_Q = 1, ORC_TENSOR_K = 2 };

void orc_set_threads(int n) {
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

int orc_get_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ---------------------------------------------------------------- random draws
 * The paper describes no cold initialisation (only the warm start of section
 * 3.2.2 "Efficient initialization"). Draws come from SplitMix64 (Steele, Lea and
 * Flood, OOPSLA 2014): the i-th output (i = 0, 1, ...) of a generator whose
 * state starts at s is mix(s + (i + 1) * 0x9E3779B97F4A7C15).
 */
static uint64_t sm64_mix(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

uint64_t orc_splitmix64(uint64_t state, uint64_t i) {
    return sm64_mix(state + (i + 1) * 0x9E3779B97F4A7C15ULL);
}

/* One independent stream per (tensor, stage, batch, head). */
uint64_t orc_stream(uint64_t seed, uint32_t tensor, uint32_t stage, uint32_t b, uint32_t h) {
    uint64_t key = ((uint64_t)(tensor & 0xF) << 60) | ((uint64_t)(stage & 0xFF) << 52) |
                   ((uint64_t)(b & 0x3FFFFFF) << 26) | (uint64_t)(h & 0x3FFFFFF);
    return orc_splitmix64(seed ^ key, 0);
}

/* ---------------------------------------------------------------- distances */
static double sq_dist(const float* a, const float* b, int d) {
    double s = 0.0;
    for (int i = 0; i < d; ++i) {
        double t = (double)a[i] - (double)b[i];
        s += t * t;
    }
    return s;
}

/* Query normalisation, section 3.1 / Algorithm 3 step 1: each query is put on the
 * unit sphere, q / max(||q||, 1e-12); the norm is taken in double, the result is
 * rounded to float32 once. */
void orc_normalize(const float* x, int64_t n, int d, float* out) {
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) {
        const float* r = x + i * d;
        double s = 0.0;
        for (int j = 0; j < d; ++j) s += (double)r[j] * (double)r[j];
        double nrm = sqrt(s);
        if (nrm < 1e-12) nrm = 1e-12;
        for (int j = 0; j < d; ++j) out[i * d + j] = (float)((double)r[j] / nrm);
    }
}

/* ---------------------------------------------------------------- k-means init
 * SAMPLE (reading for the large workloads): a seeded systematic sample over the
 * row order. With r = draw(0) mod n, slot j < m takes row floor((j n + r) / m);
 * these rows are distinct and in range whenever n >= m. When n < m, slot j < n
 * takes row j and slots n..m-1 hold no centre.
 * Returns the number of slots that hold a centre, min(m, n). */
int orc_init_sample(const float* x, int64_t n, int d, int m, uint64_t stream,
                    float* cent, int64_t* picked) {
    memset(cent, 0, sizeof(float) * (size_t)m * d);
    if (n <= 0) return 0;
    int cm = (int64_t)m < n ? m : (int)n;
    uint64_t r = orc_splitmix64(stream, 0) % (uint64_t)n;
    for (int j = 0; j < cm; ++j) {
        int64_t idx = (n >= m) ? (int64_t)(((uint64_t)j * (uint64_t)n + r) / (uint64_t)m) : j;
        if (picked) picked[j] = idx;
        memcpy(cent + (size_t)j * d, x + idx * d, sizeof(float) * d);
    }
    return cm;
}

/* KMEANSPP (Arthur and Vassilvitskii, SODA 2007; the small workload's stated init).
 * First centre: row draw(0) mod n. Centre t >= 1: with D2_i the squared distance
 * of row i to its nearest chosen centre and S = sum_i D2_i (both double, index
 * order), u = (draw(t) >> 11) * 2^-53 * S and the first row whose running sum of
 * D2 exceeds u is chosen. If S == 0 the smallest not-yet-chosen row is chosen.
 * Returns min(m, n). */
int orc_init_kmeanspp(const float* x, int64_t n, int d, int m, uint64_t stream,
                      float* cent, int64_t* picked) {
    memset(cent, 0, sizeof(float) * (size_t)m * d);
    if (n <= 0) return 0;
    int cm = (int64_t)m < n ? m : (int)n;
    double* d2 = (double*)malloc(sizeof(double) * (size_t)n);
    uint8_t* chosen = (uint8_t*)calloc((size_t)n, 1);
    int64_t idx = (int64_t)(orc_splitmix64(stream, 0) % (uint64_t)n);
    for (int t = 0; t < cm; ++t) {
        if (t > 0) {
            double S = 0.0;
            for (int64_t i = 0; i < n; ++i) S += d2[i];
            if (S == 0.0) {
                idx = -1;
                for (int64_t i = 0; i < n; ++i)
                    if (!chosen[i]) { idx = i; break; }
            } else {
                double u = (double)(orc_splitmix64(stream, (uint64_t)t) >> 11) * 0x1.0p-53 * S;
                double run = 0.0;
                idx = n - 1;
                for (int64_t i = 0; i < n; ++i) {
                    run += d2[i];
                    if (run > u) { idx = i; break; }
                }
            }
        }
        chosen[idx] = 1;
        if (picked) picked[t] = idx;
        memcpy(cent + (size_t)t * d, x + idx * d, sizeof(float) * d);
        const float* c = cent + (size_t)t * d;
        #pragma omp parallel for schedule(static)
        for (int64_t i = 0; i < n; ++i) {
            double v = sq_dist(x + i * d, c, d);
            if (t == 0 || v < d2[i]) d2[i] = v;
        }
    }
    free(d2);
    free(chosen);
    return cm;
}

/* ---------------------------------------------------------------- Lloyd steps
 * Assignment: a_i = argmin over slots j with valid[j] (all when valid == NULL)
 * of ||x_i - c_j||^2, ties to the lowest j. best/second (optional) receive the
 * two smallest squared distances, used by the tests' near-tie rule. */
void orc_assign(const float* x, int64_t n, int d, const float* cent, int m,
                const uint8_t* valid, int32_t* lab, double* best, double* second) {
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) {
        double b1 = INFINITY, b2 = INFINITY;
        int32_t arg = -1;
        for (int j = 0; j < m; ++j) {
            if (valid && !valid[j]) continue;
            double v = sq_dist(x + i * d, cent + (size_t)j * d, d);
            if (v < b1) { b2 = b1; b1 = v; arg = j; }
            else if (v < b2) { b2 = v; }
        }
        lab[i] = arg;
        if (best) best[i] = b1;
        if (second) second[i] = b2;
    }
}

/* Update: c_j = mean of the rows assigned to j (double sums in row order, rounded
 * to float32 once); a slot with no rows keeps its centre. sizes[j] = member count. */
void orc_update(const float* x, int64_t n, int d, const int32_t* lab, int m,
                float* cent, int32_t* sizes) {
    double* sum = (double*)calloc((size_t)m * d, sizeof(double));
    memset(sizes, 0, sizeof(int32_t) * (size_t)m);
    for (int64_t i = 0; i < n; ++i) {
        int32_t a = lab[i];
        sizes[a] += 1;
        for (int j = 0; j < d; ++j) sum[(size_t)a * d + j] += (double)x[i * d + j];
    }
    for (int a = 0; a < m; ++a)
        if (sizes[a] > 0)
            for (int j = 0; j < d; ++j)
                cent[(size_t)a * d + j] = (float)(sum[(size_t)a * d + j] / (double)sizes[a]);
    free(sum);
}

/* k-means: init, then `iters` rounds of (assign, update). Labels come from the
 * last assignment and centres from the last update. Slots that hold no centre
 * (j >= the count returned by the init) never attract rows.
 * Returns the number of slots that hold a centre. */
int orc_kmeans(const float* x, int64_t n, int d, int m, int iters, int init,
               uint64_t stream, const float* init_cent, float* cent, int32_t* lab,
               int32_t* sizes) {
    int cm;
    if (init == ORC_INIT_CALLER) {
        memcpy(cent, init_cent, sizeof(float) * (size_t)m * d);
        cm = m;
    } else if (init == ORC_INIT_KMEANSPP) {
        cm = orc_init_kmeanspp(x, n, d, m, stream, cent, NULL);
    } else {
        cm = orc_init_sample(x, n, d, m, stream, cent, NULL);
    }
    uint8_t* valid = (uint8_t*)malloc((size_t)m);
    for (int j = 0; j < m; ++j) valid[j] = (uint8_t)(j < cm);
    if (n == 0) memset(sizes, 0, sizeof(int32_t) * (size_t)m);
    for (int t = 0; t < iters && n > 0; ++t) {
        orc_assign(x, n, d, cent, m, valid, lab, NULL, NULL);
        orc_update(x, n, d, lab, m, cent, sizes);
    }
    free(valid);
    return cm;
}

/* ---------------------------------------------------------------- permutation
 * Cluster-contiguous order (the gather K[Index], V[Index] of Algorithm 3 step 8):
 * off = exclusive scan of the cluster sizes (m + 1 entries); inside a cluster the
 * rows keep ascending index order. */
void orc_permute(const int32_t* lab, int64_t n, int m, int32_t* perm, int32_t* off) {
    int32_t* cur = (int32_t*)calloc((size_t)m + 1, sizeof(int32_t));
    for (int64_t i = 0; i < n; ++i) cur[lab[i] + 1] += 1;
    for (int a = 0; a < m; ++a) cur[a + 1] += cur[a];
    memcpy(off, cur, sizeof(int32_t) * ((size_t)m + 1));
    for (int64_t i = 0; i < n; ++i) perm[cur[lab[i]]++] = (int32_t)i;
    free(cur);
}

/* ---------------------------------------------------------------- query side
 * Algorithm 3 step 1: A_q, C_q <- KMeans(Normalize(Q)). Reading: plain Euclidean
 * Lloyd on the normalised queries, centres are member means and are not
 * renormalised. qrep_a (the cluster's representative for scoring) is the double
 * mean of the raw (unnormalised) member queries; empty clusters get zeros. */
void orc_cluster_q(const float* q, int64_t n, int d, int cq, int iters, int init,
                   uint64_t seed, int b, int h, const float* init_cent,
                   int32_t* lab, float* cent, int32_t* sizes, float* qrep,
                   int32_t* perm, int32_t* off) {
    float* qh = (float*)malloc(sizeof(float) * (size_t)n * d);
    orc_normalize(q, n, d, qh);
    uint64_t stream = orc_stream(seed, ORC_TENSOR_Q, 0, (uint32_t)b, (uint32_t)h);
    orc_kmeans(qh, n, d, cq, iters, init, stream, init_cent, cent, lab, sizes);
    double* acc = (double*)calloc((size_t)cq * d, sizeof(double));
    for (int64_t i = 0; i < n; ++i)
        for (int j = 0; j < d; ++j) acc[(size_t)lab[i] * d + j] += (double)q[i * d + j];
    for (int a = 0; a < cq; ++a)
        for (int j = 0; j < d; ++j)
            qrep[(size_t)a * d + j] = sizes[a] > 0 ? (float)(acc[(size_t)a * d + j] / sizes[a]) : 0.0f;
    orc_permute(lab, n, cq, perm, off);
    free(acc);
    free(qh);
}

/* ---------------------------------------------------------------- key side
 * Per-cluster, per-dimension max and min of the member keys (the max(K_d),
 * min(K_d) of Eq. (1)); empty clusters get zeros. */
void orc_cluster_minmax(const float* k, int64_t n, int d, const int32_t* lab, int m,
                        float* kmax, float* kmin) {
    uint8_t* seen = (uint8_t*)calloc((size_t)m, 1);
    memset(kmax, 0, sizeof(float) * (size_t)m * d);
    memset(kmin, 0, sizeof(float) * (size_t)m * d);
    for (int64_t i = 0; i < n; ++i) {
        int32_t a = lab[i];
        float* mx = kmax + (size_t)a * d;
        float* mn = kmin + (size_t)a * d;
        const float* r = k + i * d;
        if (!seen[a]) {
            memcpy(mx, r, sizeof(float) * d);
            memcpy(mn, r, sizeof(float) * d);
            seen[a] = 1;
        } else {
            for (int j = 0; j < d; ++j) {
                if (r[j] > mx[j]) mx[j] = r[j];
                if (r[j] < mn[j]) mn[j] = r[j];
            }
        }
    }
    free(seen);
}

/* Algorithm 1 (MultiStageClustering), section 3.2.2, with these readings:
 *  - "U <- D" (a garbled symbol) is read as U <- all keys of the head.
 *  - step 11 iterates over the keys still in U, measured against their centre
 *    from the current stage; keys already removed stay removed.
 *  - stage sizes: m_0 = m0, m_t = m0 * 2^(t-1) for t >= 1 (clamped so the slot
 *    count never passes nmax); |C| counts slots, m_t per stage, so with
 *    nmax = 4 m0 the count ends in {m0, 2 m0, 4 m0}.
 *  - tau (section 4.1): tau_mult times the mean, over all n keys, of the
 *    Euclidean (not squared) distance to their stage-0 centre.
 *  - a key leaves U when its distance is strictly below tau (step 13).
 *  - step 20: every key goes to its nearest slot that holds a centre; then each
 *    slot's centre is refreshed to its member mean (no members: unchanged),
 *    and sizes, per-dimension max/min and the cluster-contiguous order follow.
 * adaptive == 0 is the fixed-count path: one k-means with m0 clusters, F = 0,
 * tau = 0. stage_u[t] receives |U| at the start of stage t (up to 8 stages).
 */
void orc_cluster_k(const float* k, int64_t n, int d, int m0, int nmax, int iters,
                   double tau_mult, int adaptive, int init, uint64_t seed, int b, int h,
                   const float* init_cent,
                   int32_t* n_slots, uint8_t* full, double* tau, int32_t* n_stages,
                   int64_t* stage_u, int32_t* lab, float* cent, uint8_t* valid,
                   int32_t* sizes, float* kmax, float* kmin, int32_t* perm, int32_t* off) {
    memset(cent, 0, sizeof(float) * (size_t)nmax * d);
    memset(valid, 0, (size_t)nmax);
    *full = 0;
    *tau = 0.0;
    if (!adaptive) {
        uint64_t stream = orc_stream(seed, ORC_TENSOR_K, 0, (uint32_t)b, (uint32_t)h);
        int cm = orc_kmeans(k, n, d, m0, iters, init, stream, init_cent, cent, lab, sizes);
        for (int j = 0; j < m0; ++j) valid[j] = (uint8_t)(j < cm);
        *n_slots = m0;
        *n_stages = 1;
        if (stage_u) stage_u[0] = n;
        orc_cluster_minmax(k, n, d, lab, m0, kmax, kmin);
        orc_permute(lab, n, m0, perm, off);
        return;
    }
    int64_t* U = (int64_t*)malloc(sizeof(int64_t) * (size_t)(n > 0 ? n : 1));
    int64_t nu = n;
    for (int64_t i = 0; i < n; ++i) U[i] = i;
    float* xu = (float*)malloc(sizeof(float) * (size_t)(n > 0 ? n : 1) * d);
    int32_t* lu = (int32_t*)malloc(sizeof(int32_t) * (size_t)(n > 0 ? n : 1));
    double* du = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
    float* ct = (float*)malloc(sizeof(float) * (size_t)nmax * d);
    int32_t* st = (int32_t*)malloc(sizeof(int32_t) * (size_t)nmax);
    int slots = 0, t = 0;
    for (;;) {
        if (nu == 0) break;
        if (slots >= nmax) { *full = 1; break; }
        int mt = (t == 0) ? m0 : (m0 << (t - 1));
        if (mt > nmax - slots) mt = nmax - slots;
        if (stage_u && t < 8) stage_u[t] = nu;
        for (int64_t r = 0; r < nu; ++r) memcpy(xu + r * d, k + U[r] * d, sizeof(float) * d);
        uint64_t stream = orc_stream(seed, ORC_TENSOR_K, (uint32_t)t, (uint32_t)b, (uint32_t)h);
        int cm = orc_kmeans(xu, nu, d, mt, iters, init, stream, NULL, ct, lu, st);
        memcpy(cent + (size_t)slots * d, ct, sizeof(float) * (size_t)mt * d);
        for (int j = 0; j < mt; ++j) valid[slots + j] = (uint8_t)(j < cm);
        for (int64_t r = 0; r < nu; ++r)
            du[r] = sqrt(sq_dist(xu + r * d, ct + (size_t)lu[r] * d, d));
        if (t == 0) {
            double s = 0.0;
            for (int64_t r = 0; r < nu; ++r) s += du[r];
            *tau = tau_mult * s / (double)n;
        }
        int64_t keep = 0;
        for (int64_t r = 0; r < nu; ++r)
            if (!(du[r] < *tau)) U[keep++] = U[r];
        nu = keep;
        slots += mt;
        t += 1;
    }
    *n_slots = slots;
    *n_stages = t;
    if (stage_u && t < 8) stage_u[t] = nu;
    orc_assign(k, n, d, cent, slots, valid, lab, NULL, NULL);
    orc_update(k, n, d, lab, slots, cent, sizes);
    for (int j = slots; j < nmax; ++j) sizes[j] = 0;
    orc_cluster_minmax(k, n, d, lab, slots, kmax, kmin);
    orc_permute(lab, n, slots, perm, off);
    free(U); free(xu); free(lu); free(du); free(ct); free(st);
}

/* ---------------------------------------------------------------- scoring
 * Eq. (1), section 3.2.3, evaluated literally at cluster level (Algorithm 3
 * step 6 read on cluster representatives):
 *   S_ab = sum_d max(qrep_ad * kmax_bd, qrep_ad * kmin_bd).
 * Slots with no members get -inf. */
void orc_quest_scores(const float* qrep, int cq, const float* kmax, const float* kmin,
                      const int32_t* ksizes, int ck, int d, double* S) {
    #pragma omp parallel for schedule(static)
    for (int a = 0; a < cq; ++a) {
        const float* qa = qrep + (size_t)a * d;
        for (int bb = 0; bb < ck; ++bb) {
            if (ksizes[bb] <= 0) { S[(size_t)a * ck + bb] = -INFINITY; continue; }
            double s = 0.0;
            for (int j = 0; j < d; ++j) {
                double hi = (double)qa[j] * (double)kmax[(size_t)bb * d + j];
                double lo = (double)qa[j] * (double)kmin[(size_t)bb * d + j];
                s += hi > lo ? hi : lo;
            }
            S[(size_t)a * ck + bb] = s;
        }
    }
}

/* Centroid score (the prior clustering approach's significance estimate):
 * S_ab = qrep_a . c_b; slots with no members get -inf. */
void orc_centroid_scores(const float* qrep, int cq, const float* cent,
                         const int32_t* ksizes, int ck, int d, double* S) {
    #pragma omp parallel for schedule(static)
    for (int a = 0; a < cq; ++a)
        for (int bb = 0; bb < ck; ++bb) {
            if (ksizes[bb] <= 0) { S[(size_t)a * ck + bb] = -INFINITY; continue; }
            double s = 0.0;
            for (int j = 0; j < d; ++j)
                s += (double)qrep[(size_t)a * d + j] * (double)cent[(size_t)bb * d + j];
            S[(size_t)a * ck + bb] = s;
        }
}

/* ---------------------------------------------------------------- selection */
typedef struct { double key; int32_t idx; } orc_kv;

static int orc_kv_desc(const void* pa, const void* pb) {
    const orc_kv* a = (const orc_kv*)pa;
    const orc_kv* b = (const orc_kv*)pb;
    if (a->key > b->key) return -1;
    if (a->key < b->key) return 1;
    return (a->idx > b->idx) - (a->idx < b->idx);
}

static void set_bit(uint32_t* row, int bb) { row[bb >> 5] |= 1u << (bb & 31); }

/* Top-p critical-cluster selection (the paper's Algorithm 3 step 7 uses
 * argtopk; top-p is the workloads' rule). Per q-cluster a, over slots b with
 * members: l_b = S_ab * scale + ln n_b (the size term turns a per-cluster score
 * into an estimate of the cluster's attention mass, cf. the centre-approximation
 * bound of section 3.2.1). Order by l descending, ties to the lower b; with
 * P_b = exp(l_b - max l) / sum exp(l - max l) (double), select the shortest
 * prefix whose cumulative P reaches p; at least one cluster. full != 0 or
 * p >= 1 selects every slot with members.
 * Diagnostics per row (optional, for the tests' boundary rule): ncut = selected
 * count, cum_before / cum_at = cumulative P before / including the last selected,
 * l_cut = l of the last selected, l_next = l of the first unselected (-inf if none).
 */
void orc_select_topp(const double* S, int cq, int ck, const int32_t* ksizes,
                     double scale, double p, int full, uint32_t* mask,
                     int32_t* sel_keys, int32_t* ncut, double* cum_before,
                     double* cum_at, double* l_cut, double* l_next) {
    int words = (ck + 31) / 32;
    memset(mask, 0, sizeof(uint32_t) * (size_t)cq * words);
    #pragma omp parallel for schedule(dynamic, 4)
    for (int a = 0; a < cq; ++a) {
        uint32_t* row = mask + (size_t)a * words;
        orc_kv* kv = (orc_kv*)malloc(sizeof(orc_kv) * (size_t)(ck > 0 ? ck : 1));
        int ne = 0;
        for (int bb = 0; bb < ck; ++bb)
            if (ksizes[bb] > 0) {
                kv[ne].key = S[(size_t)a * ck + bb] * scale + log((double)ksizes[bb]);
                kv[ne].idx = bb;
                ne++;
            }
        int take = ne;
        double cb = 0.0, ca = 1.0;
        if (!(full || p >= 1.0) && ne > 0) {
            qsort(kv, (size_t)ne, sizeof(orc_kv), orc_kv_desc);
            double mx = kv[0].key, z = 0.0;
            for (int i = 0; i < ne; ++i) z += exp(kv[i].key - mx);
            double cum = 0.0;
            take = ne;
            for (int i = 0; i < ne; ++i) {
                double before = cum;
                cum += exp(kv[i].key - mx) / z;
                if (cum >= p) { take = i + 1; cb = before; ca = cum; break; }
            }
        } else if (ne > 0) {
            qsort(kv, (size_t)ne, sizeof(orc_kv), orc_kv_desc);
        }
        int32_t keys = 0;
        for (int i = 0; i < take; ++i) {
            set_bit(row, kv[i].idx);
            keys += ksizes[kv[i].idx];
        }
        sel_keys[a] = keys;
        if (ncut) ncut[a] = take;
        if (cum_before) cum_before[a] = cb;
        if (cum_at) cum_at[a] = ca;
        if (l_cut) l_cut[a] = take > 0 ? kv[take - 1].key : -INFINITY;
        if (l_next) l_next[a] = take < ne ? kv[take].key : -INFINITY;
        free(kv);
    }
}

/* Top-k selection, Algorithm 3 step 7 (argtopk): the k slots with members and
 * the largest S_ab, ties to the lower b; k' = min(k, slots with members).
 * full != 0 selects every slot with members. */
void orc_select_topk(const double* S, int cq, int ck, const int32_t* ksizes, int topk,
                     int full, uint32_t* mask, int32_t* sel_keys) {
    int words = (ck + 31) / 32;
    memset(mask, 0, sizeof(uint32_t) * (size_t)cq * words);
    #pragma omp parallel for schedule(dynamic, 4)
    for (int a = 0; a < cq; ++a) {
        uint32_t* row = mask + (size_t)a * words;
        orc_kv* kv = (orc_kv*)malloc(sizeof(orc_kv) * (size_t)(ck > 0 ? ck : 1));
        int ne = 0;
        for (int bb = 0; bb < ck; ++bb)
            if (ksizes[bb] > 0) { kv[ne].key = S[(size_t)a * ck + bb]; kv[ne].idx = bb; ne++; }
        qsort(kv, (size_t)ne, sizeof(orc_kv), orc_kv_desc);
        int take = full ? ne : (topk < ne ? topk : ne);
        int32_t keys = 0;
        for (int i = 0; i < take; ++i) { set_bit(row, kv[i].idx); keys += ksizes[kv[i].idx]; }
        sel_keys[a] = keys;
        free(kv);
    }
}

/* ---------------------------------------------------------------- attention
 * Algorithm 3 steps 8-9: for query i in q-cluster a, J_a = every key whose
 * cluster is selected in row a of the mask. z_ij = scale * q_i . k_j (double),
 * m_i = max z, l_i = sum exp(z - m_i), o_i = sum exp(z - m_i) v_j / l_i,
 * lse_i = m_i + ln l_i. Raw (unnormalised) queries are used. Rows whose J_a is
 * empty get o = 0 and lse = -inf. Output in the original token order. */
/* Queries and keys as separate sets: nq query rows with their q-cluster
 * labels qlab, nk key rows with their key-cluster labels klab (the same
 * definition; orc_sparse_attn is the case nq = nk = n). */
void orc_sparse_attn_q(const float* q, int64_t nq, const int32_t* qlab, const float* k,
                       const float* v, int64_t n, int d, const int32_t* klab, int cq, int ck,
                       const uint32_t* mask, double scale, float* out, float* lse) {
    int words = (ck + 31) / 32;
    int64_t* jcount = (int64_t*)calloc((size_t)cq, sizeof(int64_t));
    int64_t** jlist = (int64_t**)calloc((size_t)cq, sizeof(int64_t*));
    uint8_t* used = (uint8_t*)calloc((size_t)cq, 1);
    for (int64_t i = 0; i < nq; ++i) used[qlab[i]] = 1;
    #pragma omp parallel for schedule(dynamic, 1)
    for (int a = 0; a < cq; ++a) {
        if (!used[a]) continue;
        const uint32_t* row = mask + (size_t)a * words;
        int64_t c = 0;
        for (int64_t j = 0; j < n; ++j) {
            int32_t bb = klab[j];
            if ((row[bb >> 5] >> (bb & 31)) & 1u) c++;
        }
        jlist[a] = (int64_t*)malloc(sizeof(int64_t) * (size_t)(c > 0 ? c : 1));
        c = 0;
        for (int64_t j = 0; j < n; ++j) {
            int32_t bb = klab[j];
            if ((row[bb >> 5] >> (bb & 31)) & 1u) jlist[a][c++] = j;
        }
        jcount[a] = c;
    }
    #pragma omp parallel
    {
        double* z = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
        double* acc = (double*)malloc(sizeof(double) * (size_t)d);
        #pragma omp for schedule(dynamic, 16)
        for (int64_t i = 0; i < nq; ++i) {
            int a = qlab[i];
            int64_t c = jcount[a];
            const int64_t* J = jlist[a];
            const float* qi = q + i * d;
            if (c == 0) {
                for (int t = 0; t < d; ++t) out[i * d + t] = 0.0f;
                if (lse) lse[i] = -INFINITY;
                continue;
            }
            double m = -INFINITY;
            for (int64_t r = 0; r < c; ++r) {
                const float* kj = k + J[r] * d;
                double s = 0.0;
                for (int t = 0; t < d; ++t) s += (double)qi[t] * (double)kj[t];
                z[r] = s * scale;
                if (z[r] > m) m = z[r];
            }
            double l = 0.0;
            for (int t = 0; t < d; ++t) acc[t] = 0.0;
            for (int64_t r = 0; r < c; ++r) {
                double w = exp(z[r] - m);
                l += w;
                const float* vj = v + J[r] * d;
                for (int t = 0; t < d; ++t) acc[t] += w * (double)vj[t];
            }
            for (int t = 0; t < d; ++t) out[i * d + t] = (float)(acc[t] / l);
            if (lse) lse[i] = (float)(m + log(l));
        }
        free(z);
        free(acc);
    }
    for (int a = 0; a < cq; ++a) free(jlist[a]);
    free(jlist); free(jcount); free(used);
}

void orc_sparse_attn(const float* q, const float* k, const float* v, int64_t n, int d,
                     const int32_t* qlab, const int32_t* klab, int cq, int ck,
                     const uint32_t* mask, double scale, float* out, float* lse) {
    orc_sparse_attn_q(q, n, qlab, k, v, n, d, klab, cq, ck, mask, scale, out, lse);
}

/* ---------------------------------------------------------------- compactness
 * Section 3.2.1 measures how tight the key clusters of a head are by the mean
 * squared reconstruction error MSE = (1/N) sum_i ||k_i - c(k_i)||^2; a layer's
 * compactness is Comp = 1 / (mean of its heads' MSE). Fig. 10 adds the average
 * intra-cluster distance and the Davies-Bouldin index; the pages give neither
 * formula, so the readings are:
 *   mean_dist = (1/N) sum_i ||k_i - c(k_i)||  (the distance tau is built from),
 *   DB (Davies & Bouldin 1979) over the clusters with members:
 *     s_a = mean distance of a's members to c_a,
 *     DB  = (1/K) sum_a max_{b != a} (s_a + s_b) / ||c_a - c_b||,
 *   where a pair whose centres coincide is left out of the max (a cluster with
 *   no such partner scores 0), and DB = 0 when fewer than two clusters have
 *   members. c is the centre array handed in (slot lab[i] of cent).
 * Outputs: mse, mean_dist, db (double). */
void orc_compactness(const float* x, int64_t n, int d, const int32_t* lab, const float* cent,
                     int m, double* mse, double* mean_dist, double* db) {
    double* s = (double*)calloc((size_t)m, sizeof(double));
    int64_t* cnt = (int64_t*)calloc((size_t)m, sizeof(int64_t));
    double sq = 0.0, dist = 0.0;
    for (int64_t i = 0; i < n; ++i) {
        double v = sq_dist(x + i * d, cent + (size_t)lab[i] * d, d);
        sq += v;
        dist += sqrt(v);
        s[lab[i]] += sqrt(v);
        cnt[lab[i]] += 1;
    }
    *mse = n > 0 ? sq / (double)n : 0.0;
    *mean_dist = n > 0 ? dist / (double)n : 0.0;
    int k = 0;
    for (int a = 0; a < m; ++a)
        if (cnt[a] > 0) {
            s[a] /= (double)cnt[a];
            ++k;
        }
    double* best = (double*)calloc((size_t)m, sizeof(double));
    #pragma omp parallel for schedule(dynamic, 16)
    for (int a = 0; a < m; ++a) {
        if (cnt[a] == 0) continue;
        double mx = 0.0;
        for (int b = 0; b < m; ++b) {
            if (b == a || cnt[b] == 0) continue;
            double dab = sqrt(sq_dist(cent + (size_t)a * d, cent + (size_t)b * d, d));
            if (dab == 0.0) continue;
            double r = (s[a] + s[b]) / dab;
            if (r > mx) mx = r;
        }
        best[a] = mx;
    }
    double acc = 0.0;
    for (int a = 0; a < m; ++a) acc += best[a];
    *db = k >= 2 ? acc / (double)k : 0.0;
    free(best); free(s); free(cnt);
}
