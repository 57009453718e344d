"""Algorithm 1 (AdaCluster section 3.2.2, tau from section 4.1) checked decision
by decision through the stage record of adacluster_cluster_k_trace, plus the
boundary guarantees of the C ABI: bitwise reproducible outputs, V values over
the whole bf16 range, the pair count of adacluster_select, the selection
kernel for more than 4096 slots, and a workspace at an unaligned address.
Needs an MI355X."""
import math

import numpy as np
import pytest
import torch

import clustered_sparse_attention_cosine_amd as adc
import oracle
import synth
from gpu_util import (check_alg1_head, dev, host, rel_l2, selection_ok, small_workload,
                      topk_ok)

pytestmark = pytest.mark.gpu

CASES = {
    "bf16_d64": ("cog17k", dict(H=2, grid=(3, 20, 50), text_tokens=37, q_clusters=40, k_base=24)),
    "bf16_d128": ("wan33k", dict(H=2, grid=(2, 31, 37), q_clusters=24, k_base=18)),
    # heavy-tailed keys scattered enough that every head runs three stages;
    # the oracle's own run ends head 0 at the slot cap with keys left (F = 1)
    # and empties U on head 1 (F = 0)
    "heavy_tail": ("hun119k", dict(H=2, grid=(2, 16, 20), q_clusters=20, k_base=2, noise_std=2.0)),
    # both heads end at the cap with keys left
    "full_cap": ("hun119k", dict(H=2, grid=(2, 24, 30), q_clusters=20, k_base=4, noise_std=1.5)),
}


def _hostd(d):
    return {n: host(t) for n, t in d.items() if torch.is_tensor(t)}


@pytest.mark.parametrize("case", list(CASES))
def test_alg1_every_decision(case):
    name, kw = CASES[case]
    w = small_workload(name, **kw)
    g = synth.generate(w, seed=0)
    nmax = 4 * w.k_base
    K = adc.cluster_k(dev(g["k"]), dev(g["v"]), w.k_base, nmax, iters=w.iters, adaptive=True,
                      init=w.init, trace=True)
    Kh = _hostd(K)
    tr = _hostd(K["trace"])
    for h in range(w.H):
        kf = synth.as_f32(g["k"][0, h])
        s = check_alg1_head(kf, Kh, tr, h, w.k_base, nmax, tag=case)
        print(f"{case} head {h}: {s} slots {Kh['n_clusters'][0, h]} F {Kh['full'][0, h]}")


def test_alg1_trace_leaves_outputs_unchanged():
    # the record is taken on the side: every output equals the plain call's
    name, kw = CASES["bf16_d64"]
    w = small_workload(name, **kw)
    g = synth.generate(w, seed=0)
    k, v = dev(g["k"]), dev(g["v"])
    a = adc.cluster_k(k, v, w.k_base, 4 * w.k_base, iters=w.iters, adaptive=True, init=w.init)
    b = adc.cluster_k(k, v, w.k_base, 4 * w.k_base, iters=w.iters, adaptive=True, init=w.init,
                      trace=True)
    for n, t in a.items():
        if torch.is_tensor(t):
            assert torch.equal(t, b[n]), n


# ----------------------------------------------------------------- determinism
def test_layer_bitwise_reproducible_with_large_clusters():
    # clusters of several hundred rows span several waves of the centroid
    # update, whose parts are added in a fixed order: two runs (and a run on a
    # second stream beside unrelated work) give identical bits everywhere
    w = small_workload("cog17k", H=3, grid=(4, 30, 45), text_tokens=0, q_clusters=12, k_base=8)
    g = synth.generate(w, seed=1)
    q, k, v = (dev(g[t]) for t in "qkv")
    cfg = adc.LayerConfig(q_clusters=w.q_clusters, k_base=w.k_base, k_max=4 * w.k_base,
                          top_p=w.top_p, iters=w.iters, init=w.init)
    ref = adc.layer(q, k, v, cfg)
    torch.cuda.synchronize()
    sizes = host(ref[2]["Q"]["sizes"])
    assert sizes.max() > 3 * 64  # several update waves per cluster
    side = torch.cuda.Stream()
    for run in range(2):
        busy = torch.randn(2048, 2048, device="cuda")
        if run == 1:
            with torch.cuda.stream(side):
                out = adc.layer(q, k, v, cfg)
                _ = busy @ busy
            torch.cuda.current_stream().wait_stream(side)
        else:
            out = adc.layer(q, k, v, cfg)
        torch.cuda.synchronize()
        assert torch.equal(out[0], ref[0]) and torch.equal(out[1], ref[1])
        for part in ("Q", "K", "S"):
            for n, t in ref[2][part].items():
                if torch.is_tensor(t):
                    assert torch.equal(out[2][part][n], t), (part, n)


# ----------------------------------------------------------------- V over the bf16 range
@pytest.mark.parametrize("vscale", [3.0e5, 1.0e-7, 1.0])
def test_attention_v_range(vscale):
    # bf16 V far beyond the fp16 range (or far below its normal range): the
    # per-head power-of-two scaling of the fp16 plane keeps the result
    # accurate relative to the head's largest |v|; head 1 stays at unit scale
    w = small_workload("cog17k", H=2, grid=(2, 20, 30), text_tokens=0, q_clusters=16, k_base=12)
    g = synth.generate(w, seed=2)
    vf = synth.as_f32(g["v"]).copy()
    vf[0, 0] *= vscale
    vb = synth.f32_to_bf16_bits(vf)
    nmax = 4 * w.k_base
    qp = np.zeros((1, w.H, w.N), np.int32)
    qo = np.zeros((1, w.H, w.q_clusters + 1), np.int32)
    kp = np.zeros((1, w.H, w.N), np.int32)
    ko = np.zeros((1, w.H, nmax + 1), np.int32)
    mask = np.zeros((1, w.H, w.q_clusters, (nmax + 31) // 32), np.uint32)
    refs = []
    for h in range(w.H):
        q, k, v = synth.as_f32(g["q"][0, h]), synth.as_f32(g["k"][0, h]), synth.as_f32(vb[0, h])
        r = oracle.layer_head(q, k, v, cq=w.q_clusters, m0=w.k_base, nmax=nmax, iters=w.iters,
                              top_p=w.top_p, init=w.init, h=h)
        qp[0, h], qo[0, h] = oracle.permute(r["Q"]["lab"], w.q_clusters)
        kp[0, h], ko[0, h] = r["K"]["perm"], r["K"]["off"]
        ns = r["K"]["n_slots"]
        mask[0, h, :, :(ns + 31) // 32] = r["sel"]["mask"]
        refs.append((r, np.abs(v).max()))
    kperm = np.take_along_axis(g["k"], kp[..., None].astype(np.int64), axis=2)
    vperm = np.take_along_axis(vb, kp[..., None].astype(np.int64), axis=2)
    out, lse = adc.sparse_attn(dev(g["q"]), dev(qp), dev(qo), dev(kperm), dev(vperm), dev(ko),
                               dev(mask.view(np.int32)))
    out, lse = host(out), host(lse)
    assert np.all(np.isfinite(out))
    for h in range(w.H):
        r, vmax = refs[h]
        e = rel_l2(out[0, h], r["out"])
        mx = float(np.abs(out[0, h] - r["out"]).max()) / vmax
        print(f"v scale {vscale:g} head {h}: rel-L2 {e:.2e} max-abs / max|v| {mx:.2e}")
        assert e <= 1e-2 and mx <= 2e-3
        assert np.abs(lse[0, h] - r["lse"]).max() <= 1e-2


# ----------------------------------------------------------------- pairs
def test_select_pairs_count():
    name, kw = CASES["bf16_d64"]
    w = small_workload(name, **kw)
    g = synth.generate(w, seed=0)
    cfg = adc.LayerConfig(q_clusters=w.q_clusters, k_base=w.k_base, k_max=4 * w.k_base,
                          top_p=w.top_p, iters=w.iters, init=w.init)
    _, _, st = adc.layer(dev(g["q"]), dev(g["k"]), dev(g["v"]), cfg)
    sizes = host(st["Q"]["sizes"]).astype(np.int64)
    keys = host(st["S"]["sel_keys"]).astype(np.int64)
    assert np.array_equal(host(st["S"]["pairs"]), (sizes * keys).sum(-1))


# ----------------------------------------------------------------- more than 4096 slots
@pytest.mark.parametrize("rule", ["topp", "topk"])
@pytest.mark.parametrize("score", ["quest", "centroid"])
def test_select_wide_capacity(rule, score):
    # slot capacity 8192 (the HunyuanVideo-shaped workload's Nmax) runs the
    # block-per-row selection kernel; inputs are per-slot statistics of a
    # random labelling of bf16 keys, 6000 slots in use, some of them empty
    rng = np.random.default_rng(11)
    H, N, D, Cq, Ck, ns = 2, 24000, 128, 24, 8192, 6000
    kb = synth.f32_to_bf16_bits(rng.standard_normal((H, N, D)).astype(np.float32))
    kf = synth.as_f32(kb)
    qrep = (rng.standard_normal((1, H, Cq, D)) * 0.3).astype(np.float32)
    kmax = np.zeros((1, H, Ck, D), np.uint16)
    kmin = np.zeros((1, H, Ck, D), np.uint16)
    cent = np.zeros((1, H, Ck, D), np.float32)
    sizes = np.zeros((1, H, Ck), np.int32)
    for h in range(H):
        lab = rng.integers(0, ns, N)
        lab[lab % 97 == 5] = 3  # a few slots left empty
        order = np.argsort(lab, kind="stable")
        cnt = np.bincount(lab, minlength=Ck)
        starts = np.concatenate([[0], np.cumsum(cnt)])
        for b in np.flatnonzero(cnt):
            mem = order[starts[b]:starts[b + 1]]
            kmax[0, h, b] = kb[h, mem][np.argmax(kf[h, mem], axis=0), np.arange(D)]
            kmin[0, h, b] = kb[h, mem][np.argmin(kf[h, mem], axis=0), np.arange(D)]
            cent[0, h, b] = kf[h, mem].astype(np.float64).mean(0)
        sizes[0, h] = cnt
    Kd = dict(kmax=dev(kmax), kmin=dev(kmin), sizes=dev(sizes), centroids=dev(cent),
              n_clusters=dev(np.full((1, H), ns, np.int32)), full=dev(np.zeros((1, H), np.uint8)))
    top_k = 300
    res = adc.select(dev(qrep), Kd, top_p=0.9, score=score, rule=rule, top_k=top_k)
    mask = host(res["mask"]).view(np.uint32)
    sel_keys = host(res["sel_keys"])
    scale = 1 / math.sqrt(D)
    for h in range(H):
        sz = sizes[0, h, :ns]
        if score == "quest":
            S = oracle.quest_scores(qrep[0, h], synth.as_f32(kmax[0, h, :ns]),
                                    synth.as_f32(kmin[0, h, :ns]), sz)
        else:
            S = oracle.centroid_scores(qrep[0, h], cent[0, h, :ns], sz)
        gb = oracle.mask_bits(mask[0, h], Ck)
        assert not gb[:, ns:].any()
        gb = gb[:, :ns]
        assert np.array_equal(sel_keys[0, h], (gb * sz[None]).sum(1))
        if rule == "topp":
            sel = oracle.select_topp(S, sz, scale, 0.9)
            bad, differ = selection_ok(gb, sel, S, sz, scale, 0.9)
        else:
            sel = oracle.select_topk(S, sz, top_k)
            bad, differ = topk_ok(gb, oracle.mask_bits(sel["mask"], ns), S)
        print(f"{score} {rule} head {h}: rows differing {differ}, violating {bad}")
        assert bad == 0


# ----------------------------------------------------------------- unaligned workspace
def test_workspace_at_unaligned_address():
    # the library rounds the workspace base up to 256 bytes itself; the size it
    # asks for covers the shift, so a buffer starting 4 bytes into an
    # allocation gives the same results
    name, kw = CASES["bf16_d64"]
    w = small_workload(name, **kw)
    g = synth.generate(w, seed=0)
    q = dev(g["q"])
    ref = adc.cluster_q(q, w.q_clusters, iters=w.iters, init=w.init)
    sh = adc._shape(q)
    prm = adc.QParams(w.q_clusters, w.iters, adc.INIT[w.init], 0, 0)
    need = adc.lib().adacluster_cluster_q_workspace(ctypes_byref(sh), ctypes_byref(prm))
    big = torch.empty(need + 64, dtype=torch.uint8, device="cuda")
    out = {n: torch.empty_like(t) for n, t in ref.items()}
    P = adc._p
    adc._check(adc.lib().adacluster_cluster_q(
        ctypes_byref(sh), ctypes_byref(prm), P(q), None, P(out["assign"]), P(out["centroids"]),
        P(out["sizes"]), P(out["qrep"]), P(out["perm"]), P(out["offsets"]),
        adc.ctypes.c_void_p(big.data_ptr() + 4), need, adc._stream(q.device)))
    torch.cuda.synchronize()
    for n, t in ref.items():
        assert torch.equal(out[n], t), n


def ctypes_byref(x):
    return adc.ctypes.byref(x)
