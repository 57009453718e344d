"""Warm-start steady state (AdaCluster section 3.2.2, "Efficient initialization";
the denoising steps after the first reuse the previous step's centres and keep
each head's key-cluster count): the HIP path's WARM key clustering and the
warm layer, checked against the oracle through the C ABI. Needs an MI355X."""
import math

import numpy as np
import pytest
import torch

import clustered_sparse_attention_cosine_amd as adc
import oracle
import synth
from gpu_util import dev, host, labels_match, rel_l2, small_workload

pytestmark = pytest.mark.gpu

CASES = {
    "bf16_d64": ("cog17k", dict(H=2, grid=(3, 20, 50), text_tokens=37, q_clusters=40, k_base=24)),
    "bf16_d128": ("wan33k", dict(H=2, grid=(2, 31, 37), q_clusters=24, k_base=18)),
}


def _steps(case, n_steps):
    name, kw = CASES[case]
    w = small_workload(name, **kw)
    return w, [synth.generate(w, seed=0, step=s) for s in range(n_steps)]


def _oracle_cold(w, g):
    """Per head: the oracle's own multi-stage clustering of the step-0 keys."""
    return [oracle.cluster_k(synth.as_f32(g["k"][0, h]), w.k_base, w.k_max, w.iters,
                             adaptive=True, init=w.init, h=h) for h in range(w.H)]


def _state(w, cold):
    """The oracle's cold results as the device-side state a warm call takes."""
    cent = np.stack([c["cent"] for c in cold])[None]
    counts = np.array([[c["n_slots"] for c in cold]], np.int32)
    full = np.array([[c["full"] for c in cold]], np.uint8)
    return dev(cent), dev(counts), dev(full)


@pytest.mark.parametrize("case", list(CASES))
def test_cluster_k_warm_first_round_lockstep(case):
    w, (g0, g1) = _steps(case, 2)
    cold = _oracle_cold(w, g0)
    cent, counts, full = _state(w, cold)
    print(f"{case}: oracle cold counts {host(counts)[0].tolist()} F {host(full)[0].tolist()}")
    K = adc.cluster_k(dev(g1["k"]), dev(g1["v"]), w.k_base, w.k_max, iters=1, adaptive="warm",
                      init_centroids=cent, n_clusters=counts, full=full)
    lab = host(K["assign"])
    assert np.array_equal(host(K["n_clusters"]), host(counts))
    assert np.array_equal(host(K["full"]), host(full))
    st = host(K["stage_sizes"])
    assert np.all(st[..., 0] == w.N) and np.all(st[..., 1:] == -1)
    for h in range(w.H):
        k1 = synth.as_f32(g1["k"][0, h])
        m = cold[h]["n_slots"]
        ref = oracle.assign(k1, cold[h]["cent"][:m])
        bad, diff, ties = labels_match(lab[0, h], *ref)
        print(f"  head {h}: {diff} label differences, {ties} near-ties")
        assert bad == 0
        sizes = np.bincount(lab[0, h], minlength=w.k_max)
        assert np.array_equal(host(K["sizes"])[0, h], sizes)
        assert sizes[m:].sum() == 0
        perm, off = oracle.permute(lab[0, h], w.k_max)
        assert np.array_equal(host(K["perm"])[0, h], perm)
        assert np.array_equal(host(K["offsets"])[0, h], off)
        assert np.array_equal(host(K["k_perm"])[0, h], k1[perm])
        # centres: member means of the GPU labels, untouched where empty
        cm, _ = oracle.update(k1, lab[0, h][:], cold[h]["cent"][:m])
        gc = host(K["centroids"])[0, h]
        ne = sizes[:m] > 0
        assert np.abs(gc[:m][ne] - cm[ne]).max() <= 1e-5 * max(1.0, np.abs(cm).max())
        assert np.array_equal(gc[:m][~ne], cold[h]["cent"][:m][~ne])
        assert np.all(gc[m:] == 0)


@pytest.mark.parametrize("case", list(CASES))
def test_cluster_k_warm_matches_oracle(case):
    w, (g0, g1) = _steps(case, 2)
    cold = _oracle_cold(w, g0)
    cent, counts, full = _state(w, cold)
    K = adc.cluster_k(dev(g1["k"]), dev(g1["v"]), w.k_base, w.k_max, iters=w.iters,
                      adaptive="warm", init_centroids=cent, n_clusters=counts, full=full)
    for h in range(w.H):
        k1 = synth.as_f32(g1["k"][0, h])
        r = oracle.cluster_k_warm(k1, cold[h], w.iters)
        agree = (host(K["assign"])[0, h] == r["lab"]).mean()
        print(f"{case} head {h}: warm label agreement {agree:.4f}")
        assert agree >= 0.98


def test_cluster_k_warm_clamps_counts():
    w, (g0, g1) = _steps("bf16_d64", 2)
    cold = _oracle_cold(w, g0)
    cent, _, full = _state(w, cold)
    counts = dev(np.array([[0, w.k_max + 7]], np.int32))
    K = adc.cluster_k(dev(g1["k"]), dev(g1["v"]), w.k_base, w.k_max, iters=2, adaptive="warm",
                      init_centroids=cent, n_clusters=counts, full=full)
    assert host(K["n_clusters"])[0].tolist() == [1, w.k_max]
    assert host(counts)[0].tolist() == [0, w.k_max + 7]        # the caller's tensor is copied
    lab = host(K["assign"])
    assert np.all(lab[0, 0] == 0)
    assert lab[0, 1].max() < w.k_max
    sz = host(K["sizes"])[0]
    assert sz[0, 0] == w.N and sz[0, 1:].sum() == 0


@pytest.mark.parametrize("case", list(CASES))
def test_layer_warm_chain_close_to_oracle(case):
    # cold step, then two warm steps on drifted inputs, each side free-running
    w, gs = _steps(case, 3)
    cfg = adc.LayerConfig(q_clusters=w.q_clusters, k_base=w.k_base, k_max=w.k_max, top_p=w.top_p,
                          iters=w.iters, init=w.init, adaptive=True, warm_iters=2)
    prev = None
    ora_prev = [None] * w.H
    for s, g in enumerate(gs):
        q, k, v = (dev(g[t]) for t in "qkv")
        out, lse, st = adc.layer(q, k, v, cfg, prev=prev)
        prev = st
        outh = host(out)
        for h in range(w.H):
            qf, kf, vf = (synth.as_f32(g[t][0, h]) for t in "qkv")
            r = oracle.layer_head(qf, kf, vf, cq=w.q_clusters, m0=w.k_base, nmax=w.k_max,
                                  iters=w.iters, top_p=w.top_p, init=w.init, adaptive=True, h=h,
                                  prev=ora_prev[h], warm_iters=2)
            ora_prev[h] = r
            qa = (host(st["Q"]["assign"])[0, h] == r["Q"]["lab"]).mean()
            ka = (host(st["K"]["assign"])[0, h] == r["K"]["lab"]).mean()
            e = rel_l2(outh[0, h], r["out"])
            print(f"{case} step {s} head {h}: slots {host(st['K']['n_clusters'])[0, h]} "
                  f"q-agree {qa:.4f} k-agree {ka:.4f} out rel-L2 {e:.3e}")
            assert host(st["K"]["n_clusters"])[0, h] == r["K"]["n_slots"]
            assert qa >= 0.98 and ka >= 0.98
            assert e <= 5e-2
