/*
 * adacluster.h - C ABI of the MI355X (gfx950) clustered sparse attention library.
 *
 * The library implements, for one attention layer of a video diffusion
 * transformer, the four stages of AdaCluster ("AdaCluster: Adaptive Query-Key
 * Clustering for Sparse Attention in Video Generation", arXiv 2604.18348v1):
 *   adacluster_cluster_q    section 3.1 and Algorithm 3 step 1
 *   adacluster_cluster_k    section 3.2.2, Algorithm 1, and section 4.1 (tau)
 *   adacluster_select       section 3.2.3 Eq. (1)/(2) and Algorithm 3 step 7
 *   adacluster_sparse_attn  Algorithm 3 steps 3-9
 * plus helpers that expose single steps (adacluster_assign, adacluster_permute)
 * and the compactness diagnostics of section 3.2.1 / Fig. 10
 * (adacluster_compactness).
 *
 * Conventions shared by every entry point
 *   - Tensor pointers are DEVICE pointers to contiguous row-major arrays; the
 *     leading dimensions are [B, H] (one independent problem per (b, h)).
 *     Scalar shape/parameter structs are HOST pointers.
 *   - Ownership: the caller allocates every buffer, including the workspace,
 *     whose size the matching *_workspace() call returns. The library
 *     allocates no device memory and keeps no state between calls.
 *   - Streams: `stream` is a hipStream_t passed as void* (NULL = the null
 *     stream). All work is enqueued on it; no call synchronises the host or
 *     copies device data to the host. Outputs are valid when the stream
 *     reaches the end of the call.
 *   - Alignment: rows and centres are read and written with 16-byte
 *     accesses, so tensor pointers are expected to be 16-byte aligned (as
 *     every hipMalloc and PyTorch allocation is); a less aligned pointer is
 *     still read correctly but slowly.
 *   - Workspace: any device address; the library aligns its pieces itself
 *     (the *_workspace() sizes include the slack for that).
 *   - Determinism: identical inputs, parameters and shapes give bitwise
 *     identical outputs, on any stream and at any concurrency: every sum is
 *     formed in a fixed order (no floating-point atomics), and work queues
 *     only decide which workgroup computes a result, never how.
 *   - Errors: arguments are validated before the first launch; on ADC_EINVAL,
 *     ADC_ESHAPE, ADC_EDTYPE, ADC_EWORKSPACE or ADC_EUNSUPPORTED nothing is
 *     launched and no output is written. ADC_EHIP reports a failed launch; the
 *     outputs are then undefined. adacluster_last_error() returns a
 *     thread-local, library-owned message describing the last failure.
 *   - Supported: D in {64, 128}; dtype ADC_F32 or ADC_BF16 (Q, K, V, the
 *     per-cluster max/min, the permuted K/V and the output share it);
 *     1 <= clusters <= 8192; N >= 1.
 */
#ifndef ADACLUSTER_H
#define ADACLUSTER_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ADACLUSTER_ABI_VERSION 3

typedef enum {
    ADC_OK = 0,
    ADC_EINVAL = -1,       /* null pointer or out-of-range parameter */
    ADC_ESHAPE = -2,       /* unsupported B/H/N/D or cluster count */
    ADC_EDTYPE = -3,       /* unsupported dtype */
    ADC_EWORKSPACE = -4,   /* workspace smaller than *_workspace() */
    ADC_EHIP = -5,         /* a HIP launch failed */
    ADC_EUNSUPPORTED = -6  /* parameter combination not implemented */
} adc_status;

typedef enum { ADC_F32 = 0, ADC_BF16 = 1 } adc_dtype;

/* Cold k-means initialisation (the paper describes only the warm start of
 * section 3.2.2 "Efficient initialization"; see the DESIGN notes):
 *   KMEANSPP  seeded D^2 sampling (Arthur and Vassilvitskii 2007)
 *   SAMPLE    seeded systematic sample: slot j takes row floor((j n + r) / m)
 *   CALLER    centres supplied by the caller (the warm start of section 3.2.2:
 *             later denoising steps begin from the previous step's centres) */
typedef enum { ADC_INIT_KMEANSPP = 0, ADC_INIT_SAMPLE = 1, ADC_INIT_CALLER = 2 } adc_init;

/* Cluster significance: QUEST = Eq. (1) of section 3.2.3 evaluated as the
 * two-matmul form of Eq. (2) with K+ / K- the per-cluster max / min;
 * CENTROID = qrep . key-centre (the prior clustering method's estimate). */
typedef enum { ADC_SCORE_QUEST = 0, ADC_SCORE_CENTROID = 1 } adc_score;

/* Selection rule: TOPP = shortest prefix (by l_b = score*scale + ln n_b)
 * whose softmax mass reaches top_p; TOPK = argtopk of Algorithm 3 step 7. */
typedef enum { ADC_SELECT_TOPP = 0, ADC_SELECT_TOPK = 1 } adc_select;

/* Key clustering mode (adc_k_params.adaptive).
 *   FIXED  one k-means with m0 centres per head
 *   STAGED Algorithm 1: counts chosen per head by the multi-stage loop
 *   WARM   the steady state of section 3.2.2: each head keeps the count (and
 *          the full-attention flag) found by an earlier STAGED call and runs
 *          one k-means from that call's centres */
typedef enum { ADC_K_FIXED = 0, ADC_K_STAGED = 1, ADC_K_WARM = 2 } adc_k_mode;

typedef struct {
    int32_t B, H, N, D;
    int32_t dtype;          /* adc_dtype */
} adc_shape;

typedef struct {
    int32_t n_clusters;     /* Cq */
    int32_t iters;          /* Lloyd iterations, >= 1 */
    int32_t init;           /* adc_init */
    int32_t pad_;
    uint64_t seed;
} adc_q_params;

typedef struct {
    int32_t base_clusters;  /* m0: first-stage count (the fixed count when adaptive == 0;
                               unused when adaptive == 2) */
    int32_t max_clusters;   /* Nmax: slot capacity; adaptive stages are m0, m0, 2 m0, ... */
    int32_t iters;          /* Lloyd iterations per k-means call, >= 1 */
    float tau_mult;         /* tau = tau_mult x mean stage-0 distance (1.5 in section 4.1) */
    int32_t adaptive;       /* adc_k_mode */
    int32_t init;           /* adc_init (adaptive == 1 takes KMEANSPP or SAMPLE,
                               adaptive == 2 takes CALLER only) */
    uint64_t seed;
} adc_k_params;

int32_t adacluster_abi_version(void);
const char* adacluster_last_error(void);

/* ------------------------------------------------------------------------
 * Query clustering: A_q, C_q <- KMeans(Normalize(Q)) (section 3.1, Algorithm 3
 * step 1). Queries are scaled to unit length; Lloyd's algorithm runs
 * `iters` rounds of (assign to the nearest centre, move centres to member
 * means) in the normalised space. Centres are NOT renormalised.
 *   q              [B,H,N,D] dtype            raw queries
 *   init_centroids [B,H,Cq,D] f32 iff init == CALLER, else NULL
 *   assign         [B,H,N] int32   out: cluster of each query (last assignment)
 *   centroids      [B,H,Cq,D] f32  out: member means of the normalised queries
 *                                  (clusters with no members keep their centre)
 *   sizes          [B,H,Cq] int32  out: member counts
 *   qrep           [B,H,Cq,D] f32  out: member means of the RAW queries (the
 *                                  cluster representative used for scoring; 0 if empty)
 *   perm           [B,H,N] int32   out: query ids in cluster-contiguous order,
 *                                  ascending id inside a cluster
 *   offsets        [B,H,Cq+1] int32 out: start of each cluster in perm
 */
size_t adacluster_cluster_q_workspace(const adc_shape* shape, const adc_q_params* params);
int32_t adacluster_cluster_q(const adc_shape* shape, const adc_q_params* params,
                             const void* q, const float* init_centroids,
                             int32_t* assign, float* centroids, int32_t* sizes,
                             float* qrep, int32_t* perm, int32_t* offsets,
                             void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Key clustering, Algorithm 1 (MultiStageClustering) with tau from section 4.1.
 * Stage t clusters the keys still unassigned (U) into m_t = m0 (t = 0),
 * m0 * 2^(t-1) (t >= 1) new slots; tau = tau_mult x the mean Euclidean
 * distance of all keys to their stage-0 centre; a key leaves U when strictly
 * closer than tau to its stage centre. The loop ends when U is empty, or when
 * the slot count reaches Nmax with U non-empty (then full_attn = 1: the head
 * is hard to compress and gets dense attention). Finally every key goes to
 * its nearest slot holding a centre, centres are refreshed to member means,
 * and per-slot max/min and the cluster-contiguous K/V copies are built.
 *   k, v           [B,H,N,D] dtype
 *   init_centroids f32 iff init == CALLER, else NULL: [B,H,m0,D] for FIXED,
 *                  [B,H,Nmax,D] for WARM (normally the `centroids` output of
 *                  the previous call; rows past the head's count are ignored)
 *   n_clusters     [B,H] int32   FIXED/STAGED out: slots used (m0, 2 m0, 4 m0,
 *                  ... <= Nmax). WARM in/out: the per-head count, clamped to
 *                  [1, Nmax] and written back; slots [0, count) start from
 *                  init_centroids and all of them hold a centre
 *   full_attn      [B,H] uint8   FIXED/STAGED out: F of Algorithm 1 (0 for
 *                  FIXED). WARM: read by nobody here and left unchanged (the
 *                  flag found by the STAGED call stays the caller's state)
 *   tau            [B,H] f32     out: threshold (0 for FIXED; left unchanged
 *                  by WARM)
 *   assign         [B,H,N] int32 out: slot of each key
 *   centroids      [B,H,Nmax,D] f32 out: slot centres (unused slots: 0)
 *   sizes          [B,H,Nmax] int32 out: members per slot (0 for empty/unused)
 *   kmax, kmin     [B,H,Nmax,D] dtype out: per-slot, per-dimension max / min
 *                  of the member keys (0 for empty slots)
 *   perm           [B,H,N] int32 out: key ids in slot-contiguous order
 *   offsets        [B,H,Nmax+1] int32 out: slot starts in perm (entries past
 *                  n_clusters repeat N)
 *   k_perm, v_perm [B,H,N,D] dtype out: K and V rows in perm order
 *   stage_sizes    [B,H,8] int32 out (may be NULL): |U| at the start of each
 *                  stage and after the last one, -1 past the end (FIXED and
 *                  WARM: N, then -1)
 * WARM needs init == CALLER; the other modes reject CALLER with STAGED.
 */
size_t adacluster_cluster_k_workspace(const adc_shape* shape, const adc_k_params* params);
int32_t adacluster_cluster_k(const adc_shape* shape, const adc_k_params* params,
                             const void* k, const void* v, const float* init_centroids,
                             int32_t* n_clusters, uint8_t* full_attn, float* tau,
                             int32_t* assign, float* centroids, int32_t* sizes,
                             void* kmax, void* kmin, int32_t* perm, int32_t* offsets,
                             void* k_perm, void* v_perm, int32_t* stage_sizes,
                             void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Key clustering with a record of Algorithm 1's decisions (STAGED mode only),
 * so that each one can be recomputed from the values it was taken on: the
 * labels of every stage's last Lloyd assignment from the centres that
 * assignment measured against, the threshold test of each key (step 13,
 * d(k_i, c(k_i)) < tau) from the stage centres, and the final assignment
 * (step 20) from the slot centres before their refresh to member means.
 * Arguments and results are those of adacluster_cluster_k (init may not be
 * CALLER); every pointer of the record is a device pointer and may be NULL
 * (that part is then not kept). Stages past ADC_TRACE_STAGES are not
 * recorded. Returns ADC_EUNSUPPORTED unless adaptive == ADC_K_STAGED.
 *   stage_centroids [B,H,Nmax,D] f32  each slot's centre as its stage left it
 *                                     (the last update of the stage's k-means;
 *                                     0 where no stage filled the slot)
 *   last_centroids  [B,H,Nmax,D] f32  the centres each stage's last
 *                                     assignment measured against (0 likewise)
 *   slot_valid      [B,H,Nmax] uint8  1 where the slot holds a centre
 *   stage_labels    [B,H,ADC_TRACE_STAGES,N] int32: the slot stage t gave each
 *                                     key it clustered (the keys of U at stage
 *                                     t), -1 for the other keys
 *   stage_base      [B,H,ADC_TRACE_STAGES] int32: first slot of stage t, -1
 *                                     for stages the head did not run
 */
#define ADC_TRACE_STAGES 8
typedef struct {
    float* stage_centroids;
    float* last_centroids;
    uint8_t* slot_valid;
    int32_t* stage_labels;
    int32_t* stage_base;
} adc_k_trace;

int32_t adacluster_cluster_k_trace(const adc_shape* shape, const adc_k_params* params,
                                   const void* k, const void* v, int32_t* n_clusters,
                                   uint8_t* full_attn, float* tau, int32_t* assign,
                                   float* centroids, int32_t* sizes, void* kmax, void* kmin,
                                   int32_t* perm, int32_t* offsets, void* k_perm, void* v_perm,
                                   int32_t* stage_sizes, const adc_k_trace* trace,
                                   void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Critical-cluster selection (section 3.2.3 and Algorithm 3 steps 6-7).
 * For q-cluster a and slot b with members (b < n_clusters[b,h]):
 *   QUEST     S_ab = qrep_a+ . kmax_b + qrep_a- . kmin_b   (Eq. (2) == Eq. (1))
 *   CENTROID  S_ab = qrep_a . centroid_b
 * TOPP: l_b = S_ab * scale + ln sizes_b; the shortest prefix in descending l
 * (ties to the lower b) whose softmax mass reaches top_p, at least one slot.
 * TOPK: the top_k largest S_ab (ties to the lower b).
 * Heads with full_attn = 1, and top_p >= 1, select every slot with members.
 * Precision: the softmax weights exp(l_b - max l) are taken in f32 and
 * truncated to multiples of 2^-31; masses are their exact integer sums, so a
 * cut whose mass is within about 1e-6 of top_p may differ from an exact
 * real-number evaluation by one slot.
 *   qrep       [B,H,Cq,D] f32          kmax, kmin [B,H,Ck,D] dtype (QUEST)
 *   q_offsets  [B,H,Cq+1] int32 (the query clustering's offsets; needed only
 *              for sel_pairs, else may be NULL)
 *   centroids  [B,H,Ck,D] f32 (CENTROID; may be NULL for QUEST)
 *   k_sizes    [B,H,Ck] int32          n_clusters [B,H] int32   full_attn [B,H] uint8
 *   sel_mask   [B,H,Cq,ceil(Ck/32)] uint32 out: bit b of row a set = selected
 *   sel_keys   [B,H,Cq] int32 out: keys covered by the selected slots
 *   sel_pairs  [B,H] int64 out (may be NULL): query-key pairs the attention
 *              computes, sum over a of (members of a) x sel_keys[a]
 * Ck is the slot capacity (Nmax); scale is normally 1/sqrt(D).
 */
size_t adacluster_select_workspace(const adc_shape* shape, int32_t Cq, int32_t Ck);
int32_t adacluster_select(const adc_shape* shape, int32_t Cq, int32_t Ck,
                          const float* qrep, const int32_t* q_offsets, const void* kmax,
                          const void* kmin, const float* centroids, const int32_t* k_sizes,
                          const int32_t* n_clusters, const uint8_t* full_attn,
                          int32_t score, int32_t rule, float top_p, int32_t top_k,
                          float scale, uint32_t* sel_mask, int32_t* sel_keys,
                          int64_t* sel_pairs, void* workspace, size_t workspace_bytes,
                          void* stream);

/* ------------------------------------------------------------------------
 * Sparse attention over the selected key clusters (Algorithm 3 steps 8-9):
 * every query i of q-cluster a attends, with an exact softmax at scale
 * `scale`, to all keys of the slots selected in row a of sel_mask:
 *   o_i = sum_j softmax_j(scale q_i.k_j) v_j,   lse_i = log sum_j exp(scale q_i.k_j)
 * Queries are read through q_perm/q_offsets (cluster-contiguous order) and
 * outputs are written in the original token order. A row with no selected
 * key gets o = 0 and lse = -inf.
 *   q          [B,H,N,D] dtype         q_perm [B,H,N], q_offsets [B,H,Cq+1] int32
 *   k_perm, v_perm [B,H,N,D] dtype     (slot-contiguous copies from cluster_k)
 *   k_offsets  [B,H,Ck+1] int32        sel_mask [B,H,Cq,ceil(Ck/32)] uint32
 *   out        [B,H,N,D] out, element type out_dtype (ADC_F32, or ADC_BF16 only
 *              when the inputs are bf16)
 *   lse        [B,H,N] f32 out (may be NULL)
 * Computation: matrix-core products with f32 accumulation and an online
 * softmax in f32. bf16 inputs: Q.K^T takes the bf16 values as they are (exact
 * operands); for P.V the probabilities (each at most 2^8 after the running
 * maximum) are rounded to fp16 (11-bit significand) and V to fp16 after a
 * per-head power-of-two scaling that puts the head's largest |v| in
 * [2^14, 2^15) (undone exactly on the output), so every finite bf16 V is in
 * range and values down to 2^-28 of the largest keep all their bits; the
 * result is accurate to about 2^-11 of the largest |v| of the head. f32
 * inputs are carried as bf16 hi + lo pairs with three products per
 * contraction, close to f32 accuracy. Inputs must be finite.
 */
size_t adacluster_sparse_attn_workspace(const adc_shape* shape, int32_t Cq, int32_t Ck);
int32_t adacluster_sparse_attn(const adc_shape* shape, int32_t Cq, int32_t Ck,
                               const void* q, const int32_t* q_perm, const int32_t* q_offsets,
                               const void* k_perm, const void* v_perm,
                               const int32_t* k_offsets, const uint32_t* sel_mask,
                               float scale, void* out, int32_t out_dtype, float* lse,
                               void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * adacluster_sparse_attn for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): the same arguments and results without the workspace, which is
 * instead a static array of ADC_NOALLOC_SCRATCH_BYTES per device, held by
 * every GPU the library runs on until the process ends. The call allocates
 * nothing. A shape whose adacluster_sparse_attn_workspace() exceeds the array
 * is rejected with ADC_EWORKSPACE before any launch (256 MiB holds, e.g.,
 * H = 30, N = 17,776, D = 64, Cq = 256, Ck = 1024 and H = 12, N = 32,760,
 * D = 128, Cq = 512, Ck = 2048). All calls on one device share its array:
 * calls that overlap in time on one device (on different streams, or from
 * different threads without ordering) race and give undefined results;
 * calls ordered on one stream are safe, each starts from its own clears.
 */
#define ADC_NOALLOC_SCRATCH_BYTES (256u << 20)
int32_t adacluster_sparse_attn_noalloc(const adc_shape* shape, int32_t Cq, int32_t Ck,
                                       const void* q, const int32_t* q_perm,
                                       const int32_t* q_offsets, const void* k_perm,
                                       const void* v_perm, const int32_t* k_offsets,
                                       const uint32_t* sel_mask, float scale, void* out,
                                       int32_t out_dtype, float* lse, void* stream);

/* ------------------------------------------------------------------------
 * Helper: one assignment step (argmin_j ||x_i - c_j||^2, ties to the lowest j)
 * of the k-means used by both cluster calls. normalize != 0 scales each row of
 * x to unit length first (the query side).
 *   x          [B,H,N,D] dtype     centroids [B,H,M,D] f32
 *   valid      [B,H,M] uint8 (NULL = all slots hold a centre)
 *   assign     [B,H,N] int32 out
 */
size_t adacluster_assign_workspace(const adc_shape* shape, int32_t M);
int32_t adacluster_assign(const adc_shape* shape, int32_t M, int32_t normalize,
                          const void* x, const float* centroids, const uint8_t* valid,
                          int32_t* assign, void* workspace, size_t workspace_bytes,
                          void* stream);

/* ------------------------------------------------------------------------
 * Helper: cluster-contiguous layout from given labels (the gather of
 * Algorithm 3 step 8): sizes, offsets (exclusive scan), a stable permutation
 * (ascending id inside a cluster), member means, per-dimension max/min and
 * the permuted copies of x and v. Optional outputs may be NULL.
 *   assign   [B,H,N] int32 (values in [0, M))
 *   x        [B,H,N,D] dtype; v [B,H,N,D] dtype or NULL
 *   sizes [B,H,M] int32, offsets [B,H,M+1] int32, perm [B,H,N] int32 out
 *   means [B,H,M,D] f32 out or NULL (empty clusters: left unchanged)
 *   xmax, xmin [B,H,M,D] dtype out or NULL; x_perm, v_perm [B,H,N,D] dtype out or NULL
 */
size_t adacluster_permute_workspace(const adc_shape* shape, int32_t M);
int32_t adacluster_permute(const adc_shape* shape, int32_t M, const int32_t* assign,
                           const void* x, const void* v, int32_t* sizes, int32_t* offsets,
                           int32_t* perm, float* means, void* xmax, void* xmin,
                           void* x_perm, void* v_perm, void* workspace,
                           size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Diagnostics: how compact a clustering is (section 3.2.1, where the mean
 * squared reconstruction error of each head and the layer score Comp = 1 / the
 * heads' mean MSE drive the case for per-layer cluster counts; Fig. 10, which
 * compares the average intra-cluster distance and the Davies-Bouldin index).
 * Per head, with c(i) the centre of row i's cluster and only clusters that
 * have members taking part:
 *   mse       = (1/N) sum_i ||x_i - c(i)||^2
 *   mean_dist = (1/N) sum_i ||x_i - c(i)||
 *   db        = (1/K) sum_a max_{b != a, c_b != c_a} (s_a + s_b) / ||c_a - c_b||
 *               with s_a the mean member distance to c_a and K the number of
 *               clusters with members; a cluster with no partner scores 0, and
 *               db = 0 when K < 2 (Davies & Bouldin's index)
 *   comp[b]   = 1 / (mean over the H heads of mse)
 * Inputs are the cluster-contiguous rows and offsets the clusterings write:
 *   x_perm    [B,H,N,D] dtype    rows in cluster order (k_perm of cluster_k)
 *   offsets   [B,H,M+1] int32    cluster starts; must be non-decreasing, 0..N
 *   centroids [B,H,M,D] f32      the centres c
 *   mse, mean_dist, db [B,H] f64 out;  comp [B] f64 out or NULL
 * Row distances are formed in f32 and summed in f64 in a fixed order (the
 * result does not depend on scheduling); centre distances are f32.
 */
size_t adacluster_compactness_workspace(const adc_shape* shape, int32_t M);
int32_t adacluster_compactness(const adc_shape* shape, int32_t M, const void* x_perm,
                               const int32_t* offsets, const float* centroids, double* mse,
                               double* mean_dist, double* db, double* comp, void* workspace,
                               size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* ADACLUSTER_H */
