"""The layer at the largest configuration (HunyuanVideo-shaped 129-frame 720p:
H=24, N=118800 on a 33x45x80 grid, D=128, 2048 q-clusters, adaptive key
clusters up to 8192 slots, Student-t noise, top-p 0.9), run as the benchmark
runs the headline layer: layouts and counts checked exactly against the
labels, the selection's key counts and top-p rule and the attention checked
against the oracle on sampled rows. Outputs are sampled on the device, so no
full-size tensor is copied to the host. Needs an MI355X."""
import math

import numpy as np
import pytest
import torch

import clustered_sparse_attention_cosine_amd as adc
import oracle
import synth
from gpu_util import dev, host, rel_l2, selection_ok

pytestmark = pytest.mark.gpu

HEADS = (0, 23)


@pytest.fixture(scope="module")
def big():
    w = synth.WORKLOADS["hun119k"]
    g = synth.generate(w, seed=0)
    q, k, v = (dev(g[t]) for t in "qkv")
    Q = adc.cluster_q(q, w.q_clusters, w.iters, w.init, 0)
    K = adc.cluster_k(k, v, w.k_base, w.k_max, w.iters, 1.5, w.k_adaptive, w.init, 0)
    S = adc.select(Q["qrep"], K, w.top_p)
    out, lse = adc.sparse_attn(q, Q["perm"], Q["offsets"], K["k_perm"], K["v_perm"], K["offsets"],
                               S["mask"])
    torch.cuda.synchronize()
    rng = np.random.default_rng(11)
    rows = {h: np.sort(rng.choice(w.N, 64, replace=False)) for h in HEADS}
    res = dict(w=w, g=g,
               Q={n: host(Q[n]) for n in ("assign", "sizes", "offsets", "perm", "qrep")},
               K={n: host(K[n]) for n in ("assign", "sizes", "offsets", "perm", "n_clusters", "full")},
               kmaxmin={h: (host(K["kmax"][0, h]), host(K["kmin"][0, h])) for h in HEADS},
               S={n: host(S[n]) for n in ("mask", "sel_keys")},
               rows=rows,
               out={h: host(out[0, h, torch.from_numpy(rows[h]).long().cuda()]) for h in HEADS},
               lse={h: host(lse[0, h, torch.from_numpy(rows[h]).long().cuda()]) for h in HEADS},
               finite=bool(torch.isfinite(out).all().item()))
    return res


def test_layouts_and_counts(big):
    w, Q, K = big["w"], big["Q"], big["K"]
    for lab, sizes, offsets, perm, m in ((Q["assign"], Q["sizes"], Q["offsets"], Q["perm"], w.q_clusters),
                                         (K["assign"], K["sizes"], K["offsets"], K["perm"], w.k_max)):
        for h in range(w.H):
            assert np.array_equal(sizes[0, h], np.bincount(lab[0, h], minlength=m)[:m])
            assert np.array_equal(offsets[0, h], np.concatenate([[0], np.cumsum(sizes[0, h])]))
            assert np.array_equal(perm[0, h], np.argsort(lab[0, h], kind="stable"))
    ncl = K["n_clusters"][0]
    print("key slots per head:", sorted(set(ncl.tolist())), "full heads:", int(K["full"].sum()))
    assert (ncl >= 1).all() and (ncl <= w.k_max).all()
    assert (K["assign"][0] < ncl[:, None]).all()
    assert big["finite"]


def test_selection_sampled_rows(big):
    w, Q, K, S = big["w"], big["Q"], big["K"], big["S"]
    nmax, scale = w.k_max, 1.0 / math.sqrt(w.D)
    mask = S["mask"].view(np.uint32)
    rng = np.random.default_rng(12)
    for h in range(w.H):
        bits = oracle.mask_bits(mask[0, h], nmax)
        assert np.array_equal(S["sel_keys"][0, h], (bits * K["sizes"][0, h][None]).sum(1))
    for h in HEADS:
        ns = int(K["n_clusters"][0, h])
        sizes = K["sizes"][0, h][:ns]
        kmax, kmin = big["kmaxmin"][h]
        rows = np.sort(rng.choice(w.q_clusters, 32, replace=False))
        Sc = oracle.quest_scores(Q["qrep"][0, h, rows], kmax[:ns], kmin[:ns], sizes)
        sel = oracle.select_topp(Sc, sizes, scale, w.top_p, full=bool(K["full"][0, h]))
        gb = oracle.mask_bits(mask[0, h, rows], nmax)
        assert not gb[:, ns:].any()
        bad, differ = selection_ok(gb[:, :ns], sel, Sc, sizes, scale, w.top_p)
        print(f"head {h}: sampled selection rows differing {differ}, violating {bad}")
        assert bad == 0


def test_attention_sampled_rows(big):
    w, g = big["w"], big["g"]
    mask = big["S"]["mask"].view(np.uint32)
    for h in HEADS:
        rows = big["rows"][h]
        q, k, v = (synth.as_f32(g[t][0, h]) for t in "qkv")
        ref, ref_lse = oracle.sparse_attn_rows(q[rows], big["Q"]["assign"][0, h][rows], k, v,
                                               big["K"]["assign"][0, h], w.q_clusters, w.k_max,
                                               mask[0, h], 1.0 / math.sqrt(w.D))
        got = big["out"][h]
        e, mx = rel_l2(got, ref), float(np.abs(got - ref).max())
        de = float(np.abs(big["lse"][h] - ref_lse).max())
        print(f"head {h}: rel-L2 {e:.2e} max-abs {mx:.2e} lse {de:.2e}")
        assert e <= 1e-2 and mx <= 2e-2 and de <= 1e-2
