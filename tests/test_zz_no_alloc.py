"""adacluster_sparse_attn_noalloc (the allocation-free variant of the sparse
attention, its workspace a static per-device array) against
adacluster_sparse_attn with a caller workspace, both through the C ABI: two
calls in a row, the second on a smaller input, must give identical bits, and a
shape beyond the array is refused before any launch. Needs an MI355X."""
import ctypes

import numpy as np
import pytest
import torch

import clustered_sparse_attention_cosine_amd as adc
import oracle
import synth
from gpu_util import dev, small_workload

pytestmark = pytest.mark.gpu


def _inputs(H, grid, q_clusters, k_base, seed):
    w = small_workload("cog17k", H=H, grid=grid, text_tokens=0, q_clusters=q_clusters, k_base=k_base)
    g = synth.generate(w, seed=seed)
    nmax = 4 * w.k_base
    qp = np.zeros((1, H, w.N), np.int32)
    qo = np.zeros((1, H, w.q_clusters + 1), np.int32)
    kp = np.zeros((1, H, w.N), np.int32)
    ko = np.zeros((1, H, nmax + 1), np.int32)
    mask = np.zeros((1, H, w.q_clusters, (nmax + 31) // 32), np.uint32)
    for h in range(H):
        q, k, v = (synth.as_f32(g[t][0, h]) for t in "qkv")
        r = oracle.layer_head(q, k, v, cq=w.q_clusters, m0=w.k_base, nmax=nmax, iters=w.iters,
                              top_p=w.top_p, init=w.init, h=h)
        qp[0, h], qo[0, h] = oracle.permute(r["Q"]["lab"], w.q_clusters)
        kp[0, h], ko[0, h] = r["K"]["perm"], r["K"]["off"]
        ns = r["K"]["n_slots"]
        mask[0, h, :, :(ns + 31) // 32] = r["sel"]["mask"]
    kperm = np.take_along_axis(g["k"], kp[..., None].astype(np.int64), axis=2)
    vperm = np.take_along_axis(g["v"], kp[..., None].astype(np.int64), axis=2)
    t = dict(q=dev(g["q"]), qp=dev(qp), qo=dev(qo), kp=dev(kperm), vp=dev(vperm), ko=dev(ko),
             mask=dev(mask.view(np.int32)))
    return w, nmax, t


def _call(w, nmax, t, noalloc):
    L = adc.lib()
    sh = adc.Shape(1, w.H, w.N, w.D, adc.ADC_BF16)
    out = torch.full((1, w.H, w.N, w.D), float("nan"), dtype=torch.float32, device="cuda")
    lse = torch.full((1, w.H, w.N), float("nan"), dtype=torch.float32, device="cuda")
    P = adc._p
    args = [ctypes.byref(sh), w.q_clusters, nmax, P(t["q"]), P(t["qp"]), P(t["qo"]), P(t["kp"]),
            P(t["vp"]), P(t["ko"]), P(t["mask"]), 1.0 / np.sqrt(w.D), P(out), adc.ADC_F32, P(lse)]
    stream = adc._stream(t["q"].device)
    if noalloc:
        st = L.adacluster_sparse_attn_noalloc(*args, stream)
    else:
        n = L.adacluster_sparse_attn_workspace(ctypes.byref(sh), w.q_clusters, nmax)
        ws = torch.empty(n, dtype=torch.uint8, device="cuda")
        st = L.adacluster_sparse_attn(*args, P(ws), n, stream)
    assert st == 0, L.adacluster_last_error()
    torch.cuda.synchronize()
    return out, lse


def test_noalloc_matches_workspace_entry_point():
    # a larger input, then a smaller one (fewer heads, fewer tokens and
    # clusters): the static array keeps the first call's contents, and the
    # second must not see them
    for H, grid, cq, kb, seed in [(3, (3, 24, 40), 40, 24, 0), (2, (2, 12, 20), 12, 6, 1)]:
        w, nmax, t = _inputs(H, grid, cq, kb, seed)
        ref = _call(w, nmax, t, noalloc=False)
        got = _call(w, nmax, t, noalloc=True)
        print(f"H={H} N={w.N}: equal {torch.equal(got[0], ref[0])}")
        assert torch.isfinite(ref[0]).all()
        assert torch.equal(got[0], ref[0]) and torch.equal(got[1], ref[1])


def test_noalloc_refuses_shapes_beyond_its_array():
    # the 75.6K-token layer needs ~760 MB of scratch: refused before any launch
    L = adc.lib()
    sh = adc.Shape(1, 30, 75600, 64, adc.ADC_BF16)
    P = ctypes.c_void_p(16)
    st = L.adacluster_sparse_attn_noalloc(ctypes.byref(sh), 1024, 4096, P, P, P, P, P, P, P, 0.125, P,
                                          adc.ADC_F32, P, None)
    assert st == -4
    assert b"adacluster_sparse_attn with a workspace" in L.adacluster_last_error()
