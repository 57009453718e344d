"""MI355X (gfx950) clustered sparse attention: Python binding of libadacluster.so.

Thin ctypes marshalling over the C ABI in include/adacluster.h: every stage runs
in the library's HIP kernels; PyTorch only allocates device memory and supplies
the current stream. There is no CPU fallback: if the library is missing, or a
tensor is not on a ROCm device, the calls raise.

Stages (AdaCluster paper, arXiv 2604.18348v1):
    cluster_q     section 3.1, Algorithm 3 step 1
    cluster_k     section 3.2.2 Algorithm 1, section 4.1 (tau)
    select        section 3.2.3 Eq. (1)/(2), Algorithm 3 steps 6-7
    sparse_attn   Algorithm 3 steps 8-9
    layer         the four in order
"""
from __future__ import annotations

import ctypes
import dataclasses
import math
import os
import re

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libadacluster.so")
HEADER_PATH = os.path.join(os.path.dirname(_HERE), "include", "adacluster.h")

ADC_F32, ADC_BF16 = 0, 1
INIT = {"kmeanspp": 0, "sample": 1, "caller": 2}
SCORE = {"quest": 0, "centroid": 1}
RULE = {"topp": 0, "topk": 1}
K_FIXED, K_STAGED, K_WARM = 0, 1, 2
STATUS = {0: "ADC_OK", -1: "ADC_EINVAL", -2: "ADC_ESHAPE", -3: "ADC_EDTYPE",
          -4: "ADC_EWORKSPACE", -5: "ADC_EHIP", -6: "ADC_EUNSUPPORTED"}


class Shape(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("H", ctypes.c_int32), ("N", ctypes.c_int32),
                ("D", ctypes.c_int32), ("dtype", ctypes.c_int32)]


class QParams(ctypes.Structure):
    _fields_ = [("n_clusters", ctypes.c_int32), ("iters", ctypes.c_int32),
                ("init", ctypes.c_int32), ("pad_", ctypes.c_int32), ("seed", ctypes.c_uint64)]


TRACE_STAGES = 8


class KTrace(ctypes.Structure):
    _fields_ = [("stage_centroids", ctypes.c_void_p), ("last_centroids", ctypes.c_void_p),
                ("slot_valid", ctypes.c_void_p), ("stage_labels", ctypes.c_void_p),
                ("stage_base", ctypes.c_void_p)]


class KParams(ctypes.Structure):
    _fields_ = [("base_clusters", ctypes.c_int32), ("max_clusters", ctypes.c_int32),
                ("iters", ctypes.c_int32), ("tau_mult", ctypes.c_float),
                ("adaptive", ctypes.c_int32), ("init", ctypes.c_int32), ("seed", ctypes.c_uint64)]


_lib = None
_VP = ctypes.c_void_p
_SZ = ctypes.c_size_t
_I32 = ctypes.c_int32
_F32 = ctypes.c_float
_SIGS = {
    "adacluster_abi_version": (_I32, []),
    "adacluster_last_error": (ctypes.c_char_p, []),
    "adacluster_cluster_q_workspace": (_SZ, [_VP, _VP]),
    "adacluster_cluster_q": (_I32, [_VP, _VP] + [_VP] * 8 + [_VP, _SZ, _VP]),
    "adacluster_cluster_k_workspace": (_SZ, [_VP, _VP]),
    "adacluster_cluster_k": (_I32, [_VP, _VP] + [_VP] * 16 + [_VP, _SZ, _VP]),
    "adacluster_select_workspace": (_SZ, [_VP, _I32, _I32]),
    "adacluster_cluster_k_trace": (_I32, [_VP, _VP] + [_VP] * 16 + [_VP, _SZ, _VP]),
    "adacluster_select": (_I32, [_VP, _I32, _I32] + [_VP] * 8 + [_I32, _I32, _F32, _I32, _F32]
                          + [_VP, _VP, _VP, _VP, _SZ, _VP]),
    "adacluster_sparse_attn_workspace": (_SZ, [_VP, _I32, _I32]),
    "adacluster_sparse_attn": (_I32, [_VP, _I32, _I32] + [_VP] * 7
                               + [_F32, _VP, _I32, _VP, _VP, _SZ, _VP]),
    "adacluster_sparse_attn_noalloc": (_I32, [_VP, _I32, _I32] + [_VP] * 7
                                       + [_F32, _VP, _I32, _VP, _VP]),
    "adacluster_assign_workspace": (_SZ, [_VP, _I32]),
    "adacluster_assign": (_I32, [_VP, _I32, _I32, _VP, _VP, _VP, _VP, _VP, _SZ, _VP]),
    "adacluster_permute_workspace": (_SZ, [_VP, _I32]),
    "adacluster_permute": (_I32, [_VP, _I32] + [_VP] * 11 + [_VP, _SZ, _VP]),
    "adacluster_compactness_workspace": (_SZ, [_VP, _I32]),
    "adacluster_compactness": (_I32, [_VP, _I32] + [_VP] * 7 + [_VP, _SZ, _VP]),
}


def lib():
    """Load the HIP library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m clustered_sparse_attention_cosine_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def header_symbols():
    """Names of the entry points declared in include/adacluster.h."""
    with open(HEADER_PATH) as f:
        text = f.read()
    return sorted(set(re.findall(r"\b(adacluster_\w+)\s*\(", text)))


class AdaClusterError(RuntimeError):
    pass


def _check(status):
    if status != 0:
        msg = lib().adacluster_last_error().decode(errors="replace")
        raise AdaClusterError(f"{STATUS.get(status, status)}: {msg}")


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _shape(x: torch.Tensor) -> Shape:
    if x.dim() != 4:
        raise ValueError("expected a [B, H, N, D] tensor")
    if not x.is_cuda:
        raise ValueError("tensors must live on a ROCm device (no CPU path exists)")
    if not x.is_contiguous():
        raise ValueError("tensors must be contiguous")
    if x.dtype == torch.bfloat16:
        dt = ADC_BF16
    elif x.dtype == torch.float32:
        dt = ADC_F32
    else:
        raise ValueError(f"unsupported dtype {x.dtype}")
    B, H, N, D = x.shape
    return Shape(B, H, N, D, dt)


def _workspace(nbytes, device):
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


# ----------------------------------------------------------------- stages
def cluster_q(q, n_clusters, iters=5, init="sample", seed=0, init_centroids=None):
    sh = _shape(q)
    B, H, N, D = q.shape
    dev = q.device
    if init == "caller" and (init_centroids is None
                             or tuple(init_centroids.shape) != (B, H, n_clusters, D)):
        raise ValueError(f"init_centroids must have shape {(B, H, n_clusters, D)}")
    prm = QParams(n_clusters, iters, INIT[init], 0, seed & (2**64 - 1))
    ws_n = lib().adacluster_cluster_q_workspace(ctypes.byref(sh), ctypes.byref(prm))
    if ws_n == 0:
        raise AdaClusterError("invalid cluster_q arguments: " + lib().adacluster_last_error().decode())
    out = dict(
        assign=torch.empty(B, H, N, dtype=torch.int32, device=dev),
        centroids=torch.empty(B, H, n_clusters, D, dtype=torch.float32, device=dev),
        sizes=torch.empty(B, H, n_clusters, dtype=torch.int32, device=dev),
        qrep=torch.empty(B, H, n_clusters, D, dtype=torch.float32, device=dev),
        perm=torch.empty(B, H, N, dtype=torch.int32, device=dev),
        offsets=torch.empty(B, H, n_clusters + 1, dtype=torch.int32, device=dev),
    )
    ws = _workspace(ws_n, dev)
    ic = None if init_centroids is None else init_centroids.contiguous().float()
    _check(lib().adacluster_cluster_q(ctypes.byref(sh), ctypes.byref(prm), _p(q), _p(ic),
                                      _p(out["assign"]), _p(out["centroids"]), _p(out["sizes"]),
                                      _p(out["qrep"]), _p(out["perm"]), _p(out["offsets"]),
                                      _p(ws), ws.numel(), _stream(dev)))
    return out


def cluster_k(k, v, base_clusters, max_clusters=None, iters=5, tau_mult=1.5, adaptive=True,
              init="sample", seed=0, init_centroids=None, n_clusters=None, full=None, tau=None,
              trace=False):
    """adaptive: True (Algorithm 1), False (one k-means with base_clusters) or
    "warm" (keep the per-head counts `n_clusters` and flags `full` of an earlier
    adaptive call and start from its centres `init_centroids`; init is then
    "caller"). The state tensors passed in are copied, not modified.
    trace=True (adaptive only) also returns the record of Algorithm 1's
    decisions under "trace" (adacluster_cluster_k_trace)."""
    sh = _shape(k)
    if v.shape != k.shape or v.dtype != k.dtype:
        raise ValueError("k and v must share shape and dtype")
    _shape(v)
    B, H, N, D = k.shape
    dev = k.device
    warm = adaptive == "warm"
    if warm:
        if init_centroids is None or n_clusters is None or full is None:
            raise ValueError("the warm mode needs init_centroids, n_clusters and full")
        init = "caller"
        mode = K_WARM
        nmax = max_clusters if max_clusters is not None else init_centroids.shape[2]
    else:
        mode = K_STAGED if adaptive else K_FIXED
        nmax = max_clusters if max_clusters is not None else (4 * base_clusters if adaptive else base_clusters)
    if init == "caller":
        rows = nmax if warm else base_clusters
        if init_centroids is None or tuple(init_centroids.shape) != (B, H, rows, D):
            raise ValueError(f"init_centroids must have shape {(B, H, rows, D)}")
    prm = KParams(base_clusters, nmax, iters, tau_mult, mode, INIT[init], seed & (2**64 - 1))
    ws_n = lib().adacluster_cluster_k_workspace(ctypes.byref(sh), ctypes.byref(prm))
    if ws_n == 0:
        raise AdaClusterError("invalid cluster_k arguments: " + lib().adacluster_last_error().decode())

    def state(t, dtype):
        return (torch.empty(B, H, dtype=dtype, device=dev) if t is None
                else t.to(device=dev, dtype=dtype).reshape(B, H).clone())

    out = dict(
        n_clusters=state(n_clusters if warm else None, torch.int32),
        full=state(full if warm else None, torch.uint8),
        tau=(state(tau, torch.float32) if warm and tau is not None
             else torch.zeros(B, H, dtype=torch.float32, device=dev)),
        assign=torch.empty(B, H, N, dtype=torch.int32, device=dev),
        centroids=torch.empty(B, H, nmax, D, dtype=torch.float32, device=dev),
        sizes=torch.empty(B, H, nmax, dtype=torch.int32, device=dev),
        kmax=torch.empty(B, H, nmax, D, dtype=k.dtype, device=dev),
        kmin=torch.empty(B, H, nmax, D, dtype=k.dtype, device=dev),
        perm=torch.empty(B, H, N, dtype=torch.int32, device=dev),
        offsets=torch.empty(B, H, nmax + 1, dtype=torch.int32, device=dev),
        k_perm=torch.empty_like(k),
        v_perm=torch.empty_like(v),
        stage_sizes=torch.empty(B, H, 8, dtype=torch.int32, device=dev),
    )
    ws = _workspace(ws_n, dev)
    ic = None if init_centroids is None else init_centroids.contiguous().float()
    common = [_p(out["n_clusters"]), _p(out["full"]), _p(out["tau"]), _p(out["assign"]),
              _p(out["centroids"]), _p(out["sizes"]), _p(out["kmax"]), _p(out["kmin"]),
              _p(out["perm"]), _p(out["offsets"]), _p(out["k_perm"]), _p(out["v_perm"]),
              _p(out["stage_sizes"])]
    if trace:
        tr = dict(stage_centroids=torch.empty(B, H, nmax, D, dtype=torch.float32, device=dev),
                  last_centroids=torch.empty(B, H, nmax, D, dtype=torch.float32, device=dev),
                  slot_valid=torch.empty(B, H, nmax, dtype=torch.uint8, device=dev),
                  stage_labels=torch.empty(B, H, TRACE_STAGES, N, dtype=torch.int32, device=dev),
                  stage_base=torch.empty(B, H, TRACE_STAGES, dtype=torch.int32, device=dev))
        rec = KTrace(*(t.data_ptr() for t in tr.values()))
        _check(lib().adacluster_cluster_k_trace(
            ctypes.byref(sh), ctypes.byref(prm), _p(k), _p(v), *common, ctypes.byref(rec), _p(ws),
            ws.numel(), _stream(dev)))
        out["trace"] = tr
    else:
        _check(lib().adacluster_cluster_k(
            ctypes.byref(sh), ctypes.byref(prm), _p(k), _p(v), _p(ic), *common, _p(ws), ws.numel(),
            _stream(dev)))
    out["max_clusters"] = nmax
    return out


def select(qrep, K, top_p=0.9, score="quest", rule="topp", top_k=64, scale=None, q_offsets=None):
    """K: the dict returned by cluster_k (or the same keys). With q_offsets (the
    query clustering's offsets) the result also holds "pairs" [B, H] int64, the
    query-key pairs the attention will compute."""
    B, H, Cq, D = qrep.shape
    kmax = K["kmax"]
    Ck = kmax.shape[2]
    sh = Shape(B, H, 1, D, ADC_BF16 if kmax.dtype == torch.bfloat16 else ADC_F32)
    dev = qrep.device
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    words = (Ck + 31) // 32
    out = dict(mask=torch.empty(B, H, Cq, words, dtype=torch.int32, device=dev),
               sel_keys=torch.empty(B, H, Cq, dtype=torch.int32, device=dev),
               pairs=None if q_offsets is None else torch.empty(B, H, dtype=torch.int64, device=dev))
    ws = _workspace(lib().adacluster_select_workspace(ctypes.byref(sh), Cq, Ck), dev)
    _check(lib().adacluster_select(
        ctypes.byref(sh), Cq, Ck, _p(qrep.contiguous()), _p(q_offsets), _p(kmax), _p(K["kmin"]),
        _p(K.get("centroids")), _p(K["sizes"]), _p(K["n_clusters"]), _p(K["full"]), SCORE[score],
        RULE[rule], float(top_p), int(top_k), float(scale), _p(out["mask"]), _p(out["sel_keys"]),
        _p(out["pairs"]), _p(ws), ws.numel(), _stream(dev)))
    return out


def sparse_attn(q, q_perm, q_offsets, k_perm, v_perm, k_offsets, sel_mask, scale=None,
                out=None, lse=None, want_lse=True, out_dtype=torch.float32):
    """Attention of each q-cluster over its selected key slots. The output is f32
    by default (bf16 allowed for bf16 inputs: out_dtype=torch.bfloat16)."""
    sh = _shape(q)
    B, H, N, D = q.shape
    Cq = q_offsets.shape[-1] - 1
    Ck = k_offsets.shape[-1] - 1
    dev = q.device
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype, device=dev)
    odt = ADC_F32 if out.dtype == torch.float32 else ADC_BF16
    if want_lse and lse is None:
        lse = torch.empty(B, H, N, dtype=torch.float32, device=dev)
    ws = _workspace(lib().adacluster_sparse_attn_workspace(ctypes.byref(sh), Cq, Ck), dev)
    _check(lib().adacluster_sparse_attn(
        ctypes.byref(sh), Cq, Ck, _p(q), _p(q_perm), _p(q_offsets), _p(k_perm), _p(v_perm),
        _p(k_offsets), _p(sel_mask), float(scale), _p(out), odt, _p(lse), _p(ws), ws.numel(),
        _stream(dev)))
    return out, lse


def assign(x, centroids, valid=None, normalize=False):
    sh = _shape(x)
    B, H, N, D = x.shape
    M = centroids.shape[2]
    dev = x.device
    lab = torch.empty(B, H, N, dtype=torch.int32, device=dev)
    ws = _workspace(lib().adacluster_assign_workspace(ctypes.byref(sh), M), dev)
    _check(lib().adacluster_assign(ctypes.byref(sh), M, int(bool(normalize)), _p(x),
                                   _p(centroids.contiguous().float()), _p(valid), _p(lab), _p(ws),
                                   ws.numel(), _stream(dev)))
    return lab


def permute(labels, M, x, v=None):
    sh = _shape(x)
    B, H, N, D = x.shape
    dev = x.device
    out = dict(sizes=torch.empty(B, H, M, dtype=torch.int32, device=dev),
               offsets=torch.empty(B, H, M + 1, dtype=torch.int32, device=dev),
               perm=torch.empty(B, H, N, dtype=torch.int32, device=dev),
               means=torch.zeros(B, H, M, D, dtype=torch.float32, device=dev),
               xmax=torch.empty(B, H, M, D, dtype=x.dtype, device=dev),
               xmin=torch.empty(B, H, M, D, dtype=x.dtype, device=dev),
               x_perm=torch.empty_like(x),
               v_perm=None if v is None else torch.empty_like(v))
    ws = _workspace(lib().adacluster_permute_workspace(ctypes.byref(sh), M), dev)
    _check(lib().adacluster_permute(ctypes.byref(sh), M, _p(labels.contiguous()), _p(x), _p(v),
                                    _p(out["sizes"]), _p(out["offsets"]), _p(out["perm"]),
                                    _p(out["means"]), _p(out["xmax"]), _p(out["xmin"]),
                                    _p(out["x_perm"]), _p(out["v_perm"]), _p(ws), ws.numel(),
                                    _stream(dev)))
    return out


def compactness(x_perm, offsets, centroids, want_comp=True):
    """Compactness of a clustering given in cluster order (e.g. the `k_perm`,
    `offsets` and `centroids` of cluster_k): per-head MSE, mean distance to the
    centre and Davies-Bouldin index ([B,H] f64), and Comp ([B] f64)."""
    sh = _shape(x_perm)
    B, H, N, D = x_perm.shape
    M = centroids.shape[2]
    dev = x_perm.device
    if tuple(offsets.shape) != (B, H, M + 1) or tuple(centroids.shape) != (B, H, M, D):
        raise ValueError("offsets must be [B,H,M+1] and centroids [B,H,M,D]")
    out = {n: torch.empty(B, H, dtype=torch.float64, device=dev) for n in ("mse", "mean_dist", "db")}
    out["comp"] = torch.empty(B, dtype=torch.float64, device=dev) if want_comp else None
    ws = _workspace(lib().adacluster_compactness_workspace(ctypes.byref(sh), M), dev)
    _check(lib().adacluster_compactness(ctypes.byref(sh), M, _p(x_perm),
                                        _p(offsets.contiguous()), _p(centroids.contiguous().float()),
                                        _p(out["mse"]), _p(out["mean_dist"]), _p(out["db"]),
                                        _p(out["comp"]), _p(ws), ws.numel(), _stream(dev)))
    return out


@dataclasses.dataclass
class LayerConfig:
    q_clusters: int
    k_base: int
    k_max: int
    top_p: float = 0.9
    iters: int = 5
    init: str = "sample"
    adaptive: bool = True
    tau_mult: float = 1.5
    seed: int = 0
    score: str = "quest"
    rule: str = "topp"
    top_k: int = 64
    warm_iters: int = 5     # Lloyd iterations of the warm steps


_SIDE_STREAMS = {}


def _side_stream(device):
    """A second stream per device (default priority) for the query clustering."""
    idx = torch.device(device).index
    if idx is None:
        idx = torch.cuda.current_device()
    st = _SIDE_STREAMS.get(idx)
    if st is None:
        st = _SIDE_STREAMS[idx] = torch.cuda.Stream(device=idx)
    return st


def cluster_layer(q, k, v, cfg: LayerConfig, prev=None, events=None):
    """Both clusterings of one layer (Algorithm 3 steps 1-2): returns (Q, K).

    The query and key clusterings share no data, so the queries run on a side
    stream while the keys run on the current one; the current stream waits for
    both before this returns, and the query outputs are marked as used on it.
    The key clustering's many small kernels (stages over few keys, sorts,
    updates) leave most of the GPU idle, which the query clustering fills.
    With `prev` both start from the previous step's state (section 3.2.2).
    `events`, if given: five timing events recorded at the query start and end
    (side stream), the key start and end, and the join (current stream)."""
    main = torch.cuda.current_stream(q.device)
    side = _side_stream(q.device)
    side.wait_stream(main)
    # the key clustering (the longer one) is enqueued first so that it starts at
    # once; the query launches follow while it runs
    if events is not None:
        events[2].record(main)
    if prev is None:
        K = cluster_k(k, v, cfg.k_base, cfg.k_max, cfg.iters, cfg.tau_mult, cfg.adaptive,
                      cfg.init, cfg.seed)
    else:
        pk = prev["K"]
        K = cluster_k(k, v, cfg.k_base, pk["max_clusters"], cfg.warm_iters, adaptive="warm",
                      init_centroids=pk["centroids"], n_clusters=pk["n_clusters"],
                      full=pk["full"], tau=pk["tau"])
    if events is not None:
        events[3].record(main)
    with torch.cuda.stream(side):
        if events is not None:
            events[0].record(side)
        if prev is None:
            Q = cluster_q(q, cfg.q_clusters, cfg.iters, cfg.init, cfg.seed)
        else:
            Q = cluster_q(q, cfg.q_clusters, cfg.warm_iters, "caller",
                          init_centroids=prev["Q"]["centroids"])
        if events is not None:
            events[1].record(side)
    main.wait_stream(side)
    for t in Q.values():
        if isinstance(t, torch.Tensor) and t.is_cuda:
            t.record_stream(main)
    if events is not None:
        events[4].record(main)
    return Q, K


def layer(q, k, v, cfg: LayerConfig, prev=None):
    """One clustered-sparse-attention layer (Algorithm 3): returns (out, lse, state).

    With `prev` (the state of this layer at the previous denoising step) the
    layer runs its steady-state form (section 3.2.2): both clusterings start
    from the previous centres, and the keys keep their per-head counts and
    full-attention flags."""
    Q, K = cluster_layer(q, k, v, cfg, prev)
    S = select(Q["qrep"], K, cfg.top_p, cfg.score, cfg.rule, cfg.top_k, q_offsets=Q["offsets"])
    out, lse = sparse_attn(q, Q["perm"], Q["offsets"], K["k_perm"], K["v_perm"], K["offsets"],
                           S["mask"])
    return out, lse, dict(Q=Q, K=K, S=S)


class LayerGraph:
    """One layer (Algorithm 3, cold form) captured once in a HIP graph and
    replayed. The capture records every kernel of both clusterings (the query
    clustering on the side stream, joined back), the selection and the
    attention, about 270 launches at 75.6K tokens, so a replay is one graph
    launch; no kernel of the path issues a memory-set node (buffers are cleared
    by fill kernels) and none synchronizes with the host.

    q, k and v are the graph's input buffers: write the next step's inputs into
    them in place (same shapes, dtypes and device) before replay(). Each replay
    writes the same output tensors (out, lse and the state dict), so copy what
    must outlive the next replay. The workspace of every call is held by the
    graph's memory pool for the graph's lifetime."""

    def __init__(self, q, k, v, cfg: LayerConfig, warmup: int = 2):
        self.q, self.k, self.v, self.cfg = q, k, v, cfg
        main = torch.cuda.current_stream(q.device)
        # warm-up calls outside the capture: library load, side stream, allocator
        s = torch.cuda.Stream(device=q.device)
        s.wait_stream(main)
        with torch.cuda.stream(s):
            for _ in range(max(1, warmup)):
                layer(q, k, v, cfg)
        main.wait_stream(s)
        torch.cuda.synchronize(q.device)
        self.graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.graph):
            self.out, self.lse, self.state = layer(q, k, v, cfg)

    def replay(self):
        """Run the captured layer on the current contents of q, k and v; returns
        (out, lse, state), the tensors the capture produced."""
        self.graph.replay()
        return self.out, self.lse, self.state
