"""CPU oracle for AdaCluster clustered sparse attention.

TEST INFRASTRUCTURE ONLY: the tests, ``__graft_entry__.smoke()`` and the
benchmark's ``cpu_baseline`` leg are the only callers. The HIP library never
imports, links or runs anything here, and this package imports nothing from it.

The arithmetic lives in ``adacluster_oracle.c`` (plain loops, double
accumulation, no FMA contraction); this module builds it with gcc and wraps it
with numpy. Citations of the paper's steps are in the C source beside each
function.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "adacluster_oracle.c")
# ORACLE_LIB selects another build of the same source (the sanitizer build of
# oracle/sanitize.py); by default the library next to the source is used.
_LIB_PATH = os.environ.get("ORACLE_LIB") or os.path.join(_HERE, "liboracle_adacluster.so")

INIT_KMEANSPP, INIT_SAMPLE, INIT_CALLER = 0, 1, 2
INIT_BY_NAME = {"kmeanspp": INIT_KMEANSPP, "sample": INIT_SAMPLE, "caller": INIT_CALLER}
TENSOR_Q, TENSOR_K = 1, 2

_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle into a shared library next to its source."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
               "-ffp-contract=off", "-fno-fast-math", "-Wall", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _P(t):
    return ctypes.POINTER(t)


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
            build()
        L = ctypes.CDLL(_LIB_PATH)
        f32p, f64p, i32p, i64p, u8p, u32p = (_P(ctypes.c_float), _P(ctypes.c_double),
                                             _P(ctypes.c_int32), _P(ctypes.c_int64),
                                             _P(ctypes.c_uint8), _P(ctypes.c_uint32))
        i64, i32, u64, u32, f64 = (ctypes.c_int64, ctypes.c_int, ctypes.c_uint64,
                                   ctypes.c_uint32, ctypes.c_double)
        sig = {
            "orc_set_threads": (None, [i32]),
            "orc_get_threads": (i32, []),
            "orc_splitmix64": (u64, [u64, u64]),
            "orc_stream": (u64, [u64, u32, u32, u32, u32]),
            "orc_normalize": (None, [f32p, i64, i32, f32p]),
            "orc_init_sample": (i32, [f32p, i64, i32, i32, u64, f32p, i64p]),
            "orc_init_kmeanspp": (i32, [f32p, i64, i32, i32, u64, f32p, i64p]),
            "orc_assign": (None, [f32p, i64, i32, f32p, i32, u8p, i32p, f64p, f64p]),
            "orc_update": (None, [f32p, i64, i32, i32p, i32, f32p, i32p]),
            "orc_kmeans": (i32, [f32p, i64, i32, i32, i32, i32, u64, f32p, f32p, i32p, i32p]),
            "orc_permute": (None, [i32p, i64, i32, i32p, i32p]),
            "orc_cluster_q": (None, [f32p, i64, i32, i32, i32, i32, u64, i32, i32, f32p,
                                     i32p, f32p, i32p, f32p, i32p, i32p]),
            "orc_cluster_minmax": (None, [f32p, i64, i32, i32p, i32, f32p, f32p]),
            "orc_cluster_k": (None, [f32p, i64, i32, i32, i32, i32, f64, i32, i32, u64, i32, i32,
                                     f32p, i32p, u8p, f64p, i32p, i64p, i32p, f32p, u8p, i32p,
                                     f32p, f32p, i32p, i32p]),
            "orc_quest_scores": (None, [f32p, i32, f32p, f32p, i32p, i32, i32, f64p]),
            "orc_centroid_scores": (None, [f32p, i32, f32p, i32p, i32, i32, f64p]),
            "orc_select_topp": (None, [f64p, i32, i32, i32p, f64, f64, i32, u32p, i32p, i32p,
                                       f64p, f64p, f64p, f64p]),
            "orc_select_topk": (None, [f64p, i32, i32, i32p, i32, i32, u32p, i32p]),
            "orc_sparse_attn": (None, [f32p, f32p, f32p, i64, i32, i32p, i32p, i32, i32, u32p,
                                       f64, f32p, f32p]),
            "orc_sparse_attn_q": (None, [f32p, i64, i32p, f32p, f32p, i64, i32, i32p, i32, i32,
                                         u32p, f64, f32p, f32p]),
            "orc_compactness": (None, [f32p, i64, i32, i32p, f32p, i32, f64p, f64p, f64p]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _ptr(a, ctype):
    if a is None:
        return None
    return a.ctypes.data_as(_P(ctype))


def _f32(a):
    return np.ascontiguousarray(a, dtype=np.float32)


def set_threads(n: int) -> None:
    lib().orc_set_threads(int(n))


def get_threads() -> int:
    return int(lib().orc_get_threads())


# ----------------------------------------------------------------- primitives
def splitmix64(state: int, i: int) -> int:
    return int(lib().orc_splitmix64(state & (2**64 - 1), i))


def stream(seed: int, tensor: int, stage: int, b: int, h: int) -> int:
    return int(lib().orc_stream(seed & (2**64 - 1), tensor, stage, b, h))


def normalize(x):
    x = _f32(x)
    n, d = x.shape
    out = np.empty_like(x)
    lib().orc_normalize(_ptr(x, ctypes.c_float), n, d, _ptr(out, ctypes.c_float))
    return out


def init_sample(x, m, strm):
    x = _f32(x)
    n, d = x.shape
    cent = np.empty((m, d), np.float32)
    picked = np.full(m, -1, np.int64)
    cm = lib().orc_init_sample(_ptr(x, ctypes.c_float), n, d, m, strm,
                               _ptr(cent, ctypes.c_float), _ptr(picked, ctypes.c_int64))
    return cent, picked[:cm]


def init_kmeanspp(x, m, strm):
    x = _f32(x)
    n, d = x.shape
    cent = np.empty((m, d), np.float32)
    picked = np.full(m, -1, np.int64)
    cm = lib().orc_init_kmeanspp(_ptr(x, ctypes.c_float), n, d, m, strm,
                                 _ptr(cent, ctypes.c_float), _ptr(picked, ctypes.c_int64))
    return cent, picked[:cm]


def assign(x, cent, valid=None):
    """Returns (labels, best squared distance, second-best squared distance)."""
    x, cent = _f32(x), _f32(cent)
    n, d = x.shape
    m = cent.shape[0]
    lab = np.empty(n, np.int32)
    b1 = np.empty(n, np.float64)
    b2 = np.empty(n, np.float64)
    v = None if valid is None else np.ascontiguousarray(valid, dtype=np.uint8)
    lib().orc_assign(_ptr(x, ctypes.c_float), n, d, _ptr(cent, ctypes.c_float), m,
                     _ptr(v, ctypes.c_uint8), _ptr(lab, ctypes.c_int32),
                     _ptr(b1, ctypes.c_double), _ptr(b2, ctypes.c_double))
    return lab, b1, b2


def update(x, lab, cent):
    """Returns (new centres, sizes); `cent` supplies the centres kept by empty slots."""
    x = _f32(x)
    n, d = x.shape
    cent = _f32(cent).copy()
    m = cent.shape[0]
    lab = np.ascontiguousarray(lab, dtype=np.int32)
    sizes = np.empty(m, np.int32)
    lib().orc_update(_ptr(x, ctypes.c_float), n, d, _ptr(lab, ctypes.c_int32), m,
                     _ptr(cent, ctypes.c_float), _ptr(sizes, ctypes.c_int32))
    return cent, sizes


def kmeans(x, m, iters, init="sample", strm=0, init_cent=None):
    x = _f32(x)
    n, d = x.shape
    cent = np.empty((m, d), np.float32)
    lab = np.empty(n, np.int32)
    sizes = np.empty(m, np.int32)
    ic = None if init_cent is None else _f32(init_cent)
    cm = lib().orc_kmeans(_ptr(x, ctypes.c_float), n, d, m, iters, INIT_BY_NAME[init], strm,
                          _ptr(ic, ctypes.c_float), _ptr(cent, ctypes.c_float),
                          _ptr(lab, ctypes.c_int32), _ptr(sizes, ctypes.c_int32))
    return cent, lab, sizes, int(cm)


def permute(lab, m):
    lab = np.ascontiguousarray(lab, dtype=np.int32)
    n = lab.shape[0]
    perm = np.empty(n, np.int32)
    off = np.empty(m + 1, np.int32)
    lib().orc_permute(_ptr(lab, ctypes.c_int32), n, m, _ptr(perm, ctypes.c_int32),
                      _ptr(off, ctypes.c_int32))
    return perm, off


# ----------------------------------------------------------------- stages (one head)
def cluster_q(q, cq, iters, init="sample", seed=0, b=0, h=0, init_cent=None):
    q = _f32(q)
    n, d = q.shape
    lab = np.empty(n, np.int32)
    cent = np.empty((cq, d), np.float32)
    sizes = np.empty(cq, np.int32)
    qrep = np.empty((cq, d), np.float32)
    perm = np.empty(n, np.int32)
    off = np.empty(cq + 1, np.int32)
    ic = None if init_cent is None else _f32(init_cent)
    lib().orc_cluster_q(_ptr(q, ctypes.c_float), n, d, cq, iters, INIT_BY_NAME[init],
                        seed & (2**64 - 1), b, h, _ptr(ic, ctypes.c_float),
                        _ptr(lab, ctypes.c_int32), _ptr(cent, ctypes.c_float),
                        _ptr(sizes, ctypes.c_int32), _ptr(qrep, ctypes.c_float),
                        _ptr(perm, ctypes.c_int32), _ptr(off, ctypes.c_int32))
    return dict(lab=lab, cent=cent, sizes=sizes, qrep=qrep, perm=perm, off=off)


def cluster_k(k, m0, nmax, iters, tau_mult=1.5, adaptive=True, init="sample", seed=0,
              b=0, h=0, init_cent=None):
    k = _f32(k)
    n, d = k.shape
    n_slots = np.zeros(1, np.int32)
    full = np.zeros(1, np.uint8)
    tau = np.zeros(1, np.float64)
    n_stages = np.zeros(1, np.int32)
    stage_u = np.full(8, -1, np.int64)
    lab = np.empty(n, np.int32)
    cent = np.empty((nmax, d), np.float32)
    valid = np.empty(nmax, np.uint8)
    sizes = np.zeros(nmax, np.int32)
    kmax = np.empty((nmax, d), np.float32)
    kmin = np.empty((nmax, d), np.float32)
    perm = np.empty(n, np.int32)
    off = np.zeros(nmax + 1, np.int32)
    ic = None if init_cent is None else _f32(init_cent)
    lib().orc_cluster_k(_ptr(k, ctypes.c_float), n, d, m0, nmax, iters, float(tau_mult),
                        int(adaptive), INIT_BY_NAME[init], seed & (2**64 - 1), b, h,
                        _ptr(ic, ctypes.c_float), _ptr(n_slots, ctypes.c_int32),
                        _ptr(full, ctypes.c_uint8), _ptr(tau, ctypes.c_double),
                        _ptr(n_stages, ctypes.c_int32), _ptr(stage_u, ctypes.c_int64),
                        _ptr(lab, ctypes.c_int32), _ptr(cent, ctypes.c_float),
                        _ptr(valid, ctypes.c_uint8), _ptr(sizes, ctypes.c_int32),
                        _ptr(kmax, ctypes.c_float), _ptr(kmin, ctypes.c_float),
                        _ptr(perm, ctypes.c_int32), _ptr(off, ctypes.c_int32))
    ns = int(n_slots[0])
    off[ns + 1:] = off[ns]
    return dict(n_slots=ns, full=int(full[0]), tau=float(tau[0]), n_stages=int(n_stages[0]),
                stage_u=stage_u[stage_u >= 0], lab=lab, cent=cent, valid=valid, sizes=sizes,
                kmax=kmax, kmin=kmin, perm=perm, off=off)


def cluster_k_warm(k, prev, iters):
    """A later denoising step (AdaCluster section 3.2.2, "Efficient
    initialization"): the head keeps the slot count and full-attention flag its
    multi-stage clustering found, and runs k-means over the new keys starting
    from the previous step's centres. `prev` is an earlier cluster_k result of
    this head (its n_slots, full and cent). Every one of the count's slots holds
    a centre."""
    m = prev["n_slots"]
    nmax = prev["cent"].shape[0]
    r = cluster_k(k, m, nmax, iters, adaptive=False, init="caller", init_cent=prev["cent"][:m])
    r["full"] = prev["full"]
    r["tau"] = prev["tau"]
    return r


def compactness(x, lab, cent):
    """MSE, average intra-cluster distance and Davies-Bouldin index of one
    head's clustering (section 3.2.1, Fig. 10; readings in the C source)."""
    x, cent = _f32(x), _f32(cent)
    n, d = x.shape
    lab = np.ascontiguousarray(lab, dtype=np.int32)
    out = np.zeros(3, np.float64)
    lib().orc_compactness(_ptr(x, ctypes.c_float), n, d, _ptr(lab, ctypes.c_int32),
                          _ptr(cent, ctypes.c_float), cent.shape[0], _ptr(out[0:], ctypes.c_double),
                          _ptr(out[1:], ctypes.c_double), _ptr(out[2:], ctypes.c_double))
    return dict(mse=float(out[0]), mean_dist=float(out[1]), db=float(out[2]))


def layer_compactness(mses):
    """Comp_l = 1 / (mean of the heads' MSE) (section 3.2.1)."""
    return 1.0 / float(np.mean(mses))


def layer_required_count(k_heads, m0, probe_max, iters=5, tau_mult=1.5, init="sample", seed=0,
                         b=0):
    """Section 3.2.2: Algorithm 1 on each head of a layer with the cap probe_max;
    the layer needs the largest slot count of its heads, and more than the cap
    (probe_max + 1) when some head still had keys left at the cap (F = 1)."""
    worst = 0
    for h, k in enumerate(k_heads):
        r = cluster_k(k, m0, probe_max, iters, tau_mult=tau_mult, adaptive=True, init=init,
                      seed=seed, b=b, h=h)
        worst = max(worst, probe_max + 1 if r["full"] else r["n_slots"])
    return worst


def kmax_for_top_fraction(required, m0, probe_max, top_frac=0.15):
    """Section 4.1: the cap is set so that the top top_frac of layers (the ones
    needing the most clusters) use full attention. Counts come in stage
    boundaries m0 * 2^j, so the cap is the smallest boundary (at most
    probe_max) exceeded by no more than top_frac of the layers."""
    n = len(required)
    j = 0
    while (m0 << j) <= probe_max:
        cap = m0 << j
        over = sum(1 for r in required if r > cap)
        if over <= top_frac * n + 1e-9:
            return cap
        j += 1
    return probe_max


def quest_scores(qrep, kmax, kmin, ksizes):
    qrep, kmax, kmin = _f32(qrep), _f32(kmax), _f32(kmin)
    cq, d = qrep.shape
    ck = kmax.shape[0]
    ks = np.ascontiguousarray(ksizes, dtype=np.int32)
    S = np.empty((cq, ck), np.float64)
    lib().orc_quest_scores(_ptr(qrep, ctypes.c_float), cq, _ptr(kmax, ctypes.c_float),
                           _ptr(kmin, ctypes.c_float), _ptr(ks, ctypes.c_int32), ck, d,
                           _ptr(S, ctypes.c_double))
    return S


def centroid_scores(qrep, cent, ksizes):
    qrep, cent = _f32(qrep), _f32(cent)
    cq, d = qrep.shape
    ck = cent.shape[0]
    ks = np.ascontiguousarray(ksizes, dtype=np.int32)
    S = np.empty((cq, ck), np.float64)
    lib().orc_centroid_scores(_ptr(qrep, ctypes.c_float), cq, _ptr(cent, ctypes.c_float),
                              _ptr(ks, ctypes.c_int32), ck, d, _ptr(S, ctypes.c_double))
    return S


def select_topp(S, ksizes, scale, p, full=False):
    S = np.ascontiguousarray(S, dtype=np.float64)
    cq, ck = S.shape
    words = (ck + 31) // 32
    ks = np.ascontiguousarray(ksizes, dtype=np.int32)
    mask = np.zeros((cq, words), np.uint32)
    sel_keys = np.empty(cq, np.int32)
    ncut = np.empty(cq, np.int32)
    cb, ca, lc, ln = (np.empty(cq, np.float64) for _ in range(4))
    lib().orc_select_topp(_ptr(S, ctypes.c_double), cq, ck, _ptr(ks, ctypes.c_int32),
                          float(scale), float(p), int(bool(full)), _ptr(mask, ctypes.c_uint32),
                          _ptr(sel_keys, ctypes.c_int32), _ptr(ncut, ctypes.c_int32),
                          _ptr(cb, ctypes.c_double), _ptr(ca, ctypes.c_double),
                          _ptr(lc, ctypes.c_double), _ptr(ln, ctypes.c_double))
    return dict(mask=mask, sel_keys=sel_keys, ncut=ncut, cum_before=cb, cum_at=ca,
                l_cut=lc, l_next=ln)


def select_topk(S, ksizes, topk, full=False):
    S = np.ascontiguousarray(S, dtype=np.float64)
    cq, ck = S.shape
    words = (ck + 31) // 32
    ks = np.ascontiguousarray(ksizes, dtype=np.int32)
    mask = np.zeros((cq, words), np.uint32)
    sel_keys = np.empty(cq, np.int32)
    lib().orc_select_topk(_ptr(S, ctypes.c_double), cq, ck, _ptr(ks, ctypes.c_int32),
                          int(topk), int(bool(full)), _ptr(mask, ctypes.c_uint32),
                          _ptr(sel_keys, ctypes.c_int32))
    return dict(mask=mask, sel_keys=sel_keys)


def sparse_attn(q, k, v, qlab, klab, cq, ck, mask, scale):
    q, k, v = _f32(q), _f32(k), _f32(v)
    n, d = q.shape
    qlab = np.ascontiguousarray(qlab, dtype=np.int32)
    klab = np.ascontiguousarray(klab, dtype=np.int32)
    mask = np.ascontiguousarray(mask, dtype=np.uint32)
    out = np.empty((n, d), np.float32)
    lse = np.empty(n, np.float32)
    lib().orc_sparse_attn(_ptr(q, ctypes.c_float), _ptr(k, ctypes.c_float),
                          _ptr(v, ctypes.c_float), n, d, _ptr(qlab, ctypes.c_int32),
                          _ptr(klab, ctypes.c_int32), cq, ck, _ptr(mask, ctypes.c_uint32),
                          float(scale), _ptr(out, ctypes.c_float), _ptr(lse, ctypes.c_float))
    return out, lse


def sparse_attn_rows(q_rows, qlab_rows, k, v, klab, cq, ck, mask, scale):
    """Attention of selected query rows only (the same definition as sparse_attn,
    queries given as their own set with their q-cluster labels)."""
    q, k, v = _f32(q_rows), _f32(k), _f32(v)
    nq, d = q.shape
    n = k.shape[0]
    qlab = np.ascontiguousarray(qlab_rows, dtype=np.int32)
    klab = np.ascontiguousarray(klab, dtype=np.int32)
    mask = np.ascontiguousarray(mask, dtype=np.uint32)
    out = np.empty((nq, d), np.float32)
    lse = np.empty(nq, np.float32)
    lib().orc_sparse_attn_q(_ptr(q, ctypes.c_float), nq, _ptr(qlab, ctypes.c_int32),
                            _ptr(k, ctypes.c_float), _ptr(v, ctypes.c_float), n, d,
                            _ptr(klab, ctypes.c_int32), cq, ck, _ptr(mask, ctypes.c_uint32),
                            float(scale), _ptr(out, ctypes.c_float), _ptr(lse, ctypes.c_float))
    return out, lse


def mask_bits(mask, ck):
    """Boolean [rows, ck] view of a packed selection bitmask."""
    mask = np.asarray(mask, dtype=np.uint32)
    bits = ((mask[..., :, None] >> np.arange(32, dtype=np.uint32)) & 1).astype(bool)
    return bits.reshape(*mask.shape[:-1], -1)[..., :ck]


# ----------------------------------------------------------------- one layer, one head
def layer_head(q, k, v, *, cq, m0, nmax, iters, top_p, init="sample", adaptive=True,
               tau_mult=1.5, seed=0, b=0, h=0, score="quest", rule="topp", top_k=None,
               prev=None, warm_iters=None):
    """The whole clustered-attention layer for one head (Algorithm 3). With
    `prev` (this function's result at the previous denoising step) both
    clusterings start from the previous centres (section 3.2.2) and run
    `warm_iters` Lloyd rounds."""
    d = q.shape[1]
    scale = 1.0 / np.sqrt(d)
    if prev is None:
        Q = cluster_q(q, cq, iters, init=init, seed=seed, b=b, h=h)
        K = cluster_k(k, m0, nmax, iters, tau_mult=tau_mult, adaptive=adaptive, init=init,
                      seed=seed, b=b, h=h)
    else:
        wi = iters if warm_iters is None else warm_iters
        Q = cluster_q(q, cq, wi, init="caller", init_cent=prev["Q"]["cent"])
        K = cluster_k_warm(k, prev["K"], wi)
    ck = K["n_slots"]
    if score == "quest":
        S = quest_scores(Q["qrep"], K["kmax"][:ck], K["kmin"][:ck], K["sizes"][:ck])
    else:
        S = centroid_scores(Q["qrep"], K["cent"][:ck], K["sizes"][:ck])
    if rule == "topp":
        sel = select_topp(S, K["sizes"][:ck], scale, top_p, full=bool(K["full"]))
    else:
        sel = select_topk(S, K["sizes"][:ck], top_k, full=bool(K["full"]))
    out, lse = sparse_attn(q, k, v, Q["lab"], K["lab"], cq, ck, sel["mask"], scale)
    return dict(Q=Q, K=K, S=S, sel=sel, out=out, lse=lse, scale=scale)
