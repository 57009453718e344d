"""HIP path vs the CPU oracle, stage by stage (lockstep: each GPU stage is fed
the oracle's inputs to that stage), through the C ABI. Needs an MI355X."""
import math

import numpy as np
import pytest
import torch

import clustered_sparse_attention_cosine_amd as adc
import oracle
import synth
from gpu_util import dev, host, labels_match, rel_l2, selection_ok, small_workload, topk_ok

pytestmark = pytest.mark.gpu

# (workload, overrides): parity sizes span several tiles with ragged tails
CASES = {
    "tiny": ("tiny", {}),
    "bf16_d64": ("cog17k", dict(H=2, grid=(3, 20, 50), text_tokens=37, q_clusters=40, k_base=24)),
    "bf16_d128": ("wan33k", dict(H=2, grid=(2, 31, 37), q_clusters=24, k_base=18)),
}


def _inputs(case, seed=0):
    name, kw = CASES[case]
    w = small_workload(name, **kw)
    g = synth.generate(w, seed=seed)
    return w, g


def _oracle_head(w, g, h, adaptive=None):
    q, k, v = (synth.as_f32(g[t][0, h]) for t in "qkv")
    ad = w.k_adaptive if adaptive is None else adaptive
    return oracle.layer_head(q, k, v, cq=w.q_clusters, m0=w.k_base,
                             nmax=4 * w.k_base if ad else w.k_base, iters=w.iters,
                             top_p=w.top_p, init=w.init, adaptive=ad, h=h)


# ----------------------------------------------------------------- attention (lockstep)
@pytest.mark.parametrize("case", list(CASES))
def test_sparse_attn_matches_oracle(case):
    w, g = _inputs(case)
    _lockstep_attention(case, w, g)


def _lockstep_attention(case, w, g):
    """The HIP attention on the oracle's layouts and selection vs the oracle's layer."""
    H, N, D = w.H, w.N, w.D
    nmax = 4 * w.k_base if w.k_adaptive else w.k_base
    qp = np.zeros((1, H, N), np.int32)
    qo = np.zeros((1, H, w.q_clusters + 1), np.int32)
    kp = np.zeros((1, H, N), np.int32)
    ko = np.zeros((1, H, nmax + 1), np.int32)
    words = (nmax + 31) // 32
    mask = np.zeros((1, H, w.q_clusters, words), np.uint32)
    refs = []
    for h in range(H):
        r = _oracle_head(w, g, h)
        qp[0, h], qo[0, h] = oracle.permute(r["Q"]["lab"], w.q_clusters)
        ns = r["K"]["n_slots"]
        kp[0, h] = r["K"]["perm"]
        ko[0, h] = r["K"]["off"]
        mask[0, h, :, :(ns + 31) // 32] = r["sel"]["mask"]
        refs.append(r)
    kperm = np.take_along_axis(g["k"], kp[..., None].astype(np.int64), axis=2)
    vperm = np.take_along_axis(g["v"], kp[..., None].astype(np.int64), axis=2)
    out, lse = adc.sparse_attn(dev(g["q"]), dev(qp), dev(qo), dev(kperm), dev(vperm), dev(ko),
                               dev(mask.view(np.int32)))
    torch.cuda.synchronize()
    out, lse = host(out), host(lse)
    for h in range(H):
        ref = refs[h]["out"]
        e = rel_l2(out[0, h], ref)
        mx = np.abs(out[0, h] - ref).max()
        print(f"{case} head {h}: rel-L2 {e:.2e} max-abs {mx:.2e}")
        assert e <= 1e-2 and mx <= 2e-2
        assert np.abs(lse[0, h] - refs[h]["lse"]).max() <= 1e-2
    return refs


def test_fixed_65_query_clusters():
    # the pages' experimental setting of 65 query clusters (section 4.1): about
    # 118 queries per cluster, so clusters span one or two 128-row work items
    w = small_workload("cog17k", H=2, grid=(4, 32, 60), text_tokens=11, q_clusters=65, k_base=32)
    g = synth.generate(w, seed=0)
    refs = _lockstep_attention("q65", w, g)
    cfg = adc.LayerConfig(q_clusters=65, k_base=w.k_base, k_max=w.k_max, top_p=w.top_p,
                          iters=w.iters, init=w.init, adaptive=True)
    out, _, st = adc.layer(dev(g["q"]), dev(g["k"]), dev(g["v"]), cfg)
    out = host(out)
    for h in range(w.H):
        r = refs[h]
        qa = (host(st["Q"]["assign"])[0, h] == r["Q"]["lab"]).mean()
        ka = (host(st["K"]["assign"])[0, h] == r["K"]["lab"]).mean()
        e = rel_l2(out[0, h], r["out"])
        big = int((np.bincount(r["Q"]["lab"], minlength=65) > 128).sum())
        print(f"q65 head {h}: {big} clusters over 128 rows; q-agree {qa:.4f} k-agree {ka:.4f} "
              f"out rel-L2 {e:.3e}")
        assert qa >= 0.98 and ka >= 0.98
        assert e <= 5e-2


@pytest.mark.parametrize("D,dtype", [(64, "bf16"), (128, "bf16"), (64, "f32"), (128, "f32")])
def test_select_all_equals_dense(D, dtype):
    # one q-cluster and one key slot holding every token: dense attention,
    # compared with a float64 softmax on the host
    rng = np.random.default_rng(D)
    N, H = 333, 2
    x = rng.standard_normal((3, 1, H, N, D)).astype(np.float32) * 2
    if dtype == "bf16":
        arrs = [synth.f32_to_bf16_bits(t) for t in x]
        xf = [synth.bf16_bits_to_f32(a) for a in arrs]
    else:
        arrs = list(x)
        xf = [a.astype(np.float32) for a in arrs]
    ident = np.tile(np.arange(N, dtype=np.int32), (1, H, 1))
    offs = np.tile(np.array([0, N], np.int32), (1, H, 1))
    mask = np.ones((1, H, 1, 1), np.int32)
    out, lse = adc.sparse_attn(dev(arrs[0]), dev(ident), dev(offs), dev(arrs[1]), dev(arrs[2]),
                               dev(offs), dev(mask))
    out = host(out)
    scale = 1 / math.sqrt(D)
    for h in range(H):
        z = xf[0][0, h].astype(np.float64) @ xf[1][0, h].astype(np.float64).T * scale
        p = np.exp(z - z.max(1, keepdims=True))
        ref = (p @ xf[2][0, h].astype(np.float64)) / p.sum(1, keepdims=True)
        assert rel_l2(out[0, h], ref) <= 1e-2
        assert np.abs(out[0, h] - ref).max() <= 2e-2
        ref_lse = z.max(1) + np.log(p.sum(1))
        assert np.abs(host(lse)[0, h] - ref_lse).max() <= 1e-2


def test_sparse_attn_edge_cases():
    # empty q-clusters, a single-row q-cluster, a 150-row q-cluster (2 chunks of 128 rows), a
    # selection of empty slots only (row gets o = 0, lse = -inf), ragged Ck
    rng = np.random.default_rng(3)
    N, D, Cq, Ck = 200, 64, 5, 37
    q, k, v = (synth.f32_to_bf16_bits(rng.standard_normal((1, 1, N, D)).astype(np.float32)) for _ in range(3))
    qlab = np.concatenate([np.full(150, 0), [2], np.full(49, 4)]).astype(np.int32)
    klab = rng.integers(0, Ck - 5, N).astype(np.int32)   # slots Ck-5.. empty
    qperm, qoff = oracle.permute(qlab, Cq)
    kperm, koff = oracle.permute(klab, Ck)
    words = (Ck + 31) // 32
    mask = np.zeros((Cq, words), np.uint32)
    mask[0, 0] = 0b1011
    mask[2, 0] = 0xFFFFFFFF
    mask[2, 1] = 0x1F
    mask[4, 1] = 1 << (Ck - 1 - 32)   # only an empty slot
    scale = 0.125
    out, lse = adc.sparse_attn(dev(q), dev(qperm[None, None]), dev(qoff[None, None]),
                               dev(k[:, :, kperm]), dev(v[:, :, kperm]), dev(koff[None, None]),
                               dev(mask[None, None].view(np.int32)), scale=scale)
    out, lse = host(out)[0, 0], host(lse)[0, 0]
    ref, ref_lse = oracle.sparse_attn(synth.as_f32(q[0, 0]), synth.as_f32(k[0, 0]),
                                      synth.as_f32(v[0, 0]), qlab, klab, Cq, Ck, mask, scale)
    assert rel_l2(out, ref) <= 1e-2 and np.abs(out - ref).max() <= 2e-2
    assert np.all(out[qlab == 4] == 0) and np.all(np.isneginf(lse[qlab == 4]))
    fin = np.isfinite(ref_lse)
    assert np.abs(lse[fin] - ref_lse[fin]).max() <= 1e-2


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_sparse_attn_many_runs(dtype):
    # one key per slot: an alternating selection gives 1300 separate key ranges
    # (more than the kernel keeps in LDS, so they are read from global memory),
    # next to a full selection (one range) and a random 30% selection
    rng = np.random.default_rng(11)
    Nq, Nk, D, Cq = 300, 2600, 64, 3
    N = Nk
    x = [rng.standard_normal((1, 1, N, D)).astype(np.float32) for _ in range(3)]
    if dtype == "bf16":
        q, k, v = (synth.f32_to_bf16_bits(t) for t in x)
    else:
        q, k, v = x
    qlab = np.concatenate([np.zeros(100), np.ones(100), np.full(100, 2),
                           np.full(N - Nq, Cq)]).astype(np.int32)   # tokens past Nq: no cluster
    qlab = np.minimum(qlab, Cq - 1)
    klab = np.arange(N, dtype=np.int32)
    Ck = N
    qperm, qoff = oracle.permute(qlab, Cq)
    kperm, koff = oracle.permute(klab, Ck)
    words = (Ck + 31) // 32
    bits = np.zeros((Cq, Ck), bool)
    bits[0, ::2] = True
    bits[1, :] = True
    bits[2] = rng.random(Ck) < 0.3
    mask = np.zeros((Cq, words), np.uint32)
    for a in range(Cq):
        for j in np.nonzero(bits[a])[0]:
            mask[a, j // 32] |= np.uint32(1) << np.uint32(j % 32)
    scale = 0.125
    out, lse = adc.sparse_attn(dev(q), dev(qperm[None, None]), dev(qoff[None, None]),
                               dev(k[:, :, kperm]), dev(v[:, :, kperm]), dev(koff[None, None]),
                               dev(mask[None, None].view(np.int32)), scale=scale)
    out, lse = host(out)[0, 0], host(lse)[0, 0]
    ref, ref_lse = oracle.sparse_attn(synth.as_f32(q[0, 0]), synth.as_f32(k[0, 0]),
                                      synth.as_f32(v[0, 0]), qlab, klab, Cq, Ck, mask, scale)
    assert rel_l2(out, ref) <= 1e-2 and np.abs(out - ref).max() <= 2e-2
    assert np.abs(lse - ref_lse).max() <= 1e-2


@pytest.mark.parametrize("D", [64, 128])
def test_sparse_attn_mixed_head_densities(D):
    """Heads of very different selection densities in one call: a head whose
    q-clusters select every slot, a sparse head, a head with one dense
    q-cluster among sparse ones, and random ones. Their items land in both
    halves of the work list (large q-clusters first, judged against the mean
    over all heads) and in several XCD stretches, so workgroups also take
    items of other stretches; every head is compared with the oracle."""
    rng = np.random.default_rng(21 + D)
    H, N, Cq, Ck = 6, 1500, 24, 96
    q, k, v = (synth.f32_to_bf16_bits(rng.standard_normal((1, H, N, D)).astype(np.float32)) for _ in range(3))
    qlab = rng.integers(0, Cq, (H, N)).astype(np.int32)
    klab = rng.integers(0, Ck, (H, N)).astype(np.int32)
    bits = np.zeros((H, Cq, Ck), bool)
    bits[0] = True                                  # every slot
    bits[1] = rng.random((Cq, Ck)) < 0.03           # sparse
    bits[2] = rng.random((Cq, Ck)) < 0.05
    bits[2, 7] = True                               # one dense q-cluster
    bits[3:] = rng.random((H - 3, Cq, Ck)) < rng.uniform(0.2, 0.5, (H - 3, 1, 1))
    words = (Ck + 31) // 32
    mask = np.zeros((H, Cq, words), np.uint32)
    for h in range(H):
        for a in range(Cq):
            for j in np.nonzero(bits[h, a])[0]:
                mask[h, a, j // 32] |= np.uint32(1) << np.uint32(j % 32)
    qperm = np.zeros((1, H, N), np.int32)
    qoff = np.zeros((1, H, Cq + 1), np.int32)
    kperm = np.zeros((1, H, N), np.int32)
    koff = np.zeros((1, H, Ck + 1), np.int32)
    for h in range(H):
        qperm[0, h], qoff[0, h] = oracle.permute(qlab[h], Cq)
        kperm[0, h], koff[0, h] = oracle.permute(klab[h], Ck)
    kp = np.stack([k[0, h, kperm[0, h]] for h in range(H)])[None]
    vp = np.stack([v[0, h, kperm[0, h]] for h in range(H)])[None]
    scale = float(1 / np.sqrt(D))
    out, lse = adc.sparse_attn(dev(q), dev(qperm), dev(qoff), dev(kp), dev(vp), dev(koff),
                               dev(mask[None].view(np.int32)), scale=scale)
    out, lse = host(out)[0], host(lse)[0]
    for h in range(H):
        ref, ref_lse = oracle.sparse_attn(synth.as_f32(q[0, h]), synth.as_f32(k[0, h]), synth.as_f32(v[0, h]),
                                          qlab[h], klab[h], Cq, Ck, mask[h], scale)
        assert rel_l2(out[h], ref) <= 1e-2 and np.abs(out[h] - ref).max() <= 2e-2, h
        fin = np.isfinite(ref_lse)
        assert np.array_equal(fin, np.isfinite(lse[h])), h
        assert np.abs(lse[h][fin] - ref_lse[fin]).max() <= 1e-2, h


# ----------------------------------------------------------------- assignment (lockstep)
@pytest.mark.parametrize("case", list(CASES))
@pytest.mark.parametrize("normalize", [False, True])
def test_assign_matches_oracle(case, normalize):
    w, g = _inputs(case)
    x = g["q" if normalize else "k"]
    M = 2 * w.k_base + 5
    cents = np.zeros((1, w.H, M, w.D), np.float32)
    refs = []
    for h in range(w.H):
        xf = synth.as_f32(x[0, h])
        xo = oracle.normalize(xf) if normalize else xf
        # centres: a Lloyd state (so near-ties are realistic), plus perturbed copies
        c, _, _, _ = oracle.kmeans(xo, M - 5, 2, init="sample", strm=oracle.stream(5, 2, 0, 0, h))
        cents[0, h, :M - 5] = c
        cents[0, h, M - 5:] = c[:5] * 1.01
        refs.append(oracle.assign(xo, cents[0, h]))
    lab = host(adc.assign(dev(x), dev(cents), normalize=normalize))
    for h in range(w.H):
        bad, diff, ties = labels_match(lab[0, h], *refs[h])
        print(f"{case} norm={normalize} head {h}: mismatches {diff}, outside near-ties {bad}, near-ties {ties}")
        assert bad == 0


def test_assign_respects_valid_and_ties():
    rng = np.random.default_rng(4)
    N, D, M = 500, 64, 70
    x = synth.f32_to_bf16_bits(rng.standard_normal((1, 1, N, D)).astype(np.float32))
    c = rng.standard_normal((1, 1, M, D)).astype(np.float32)
    c[0, 0, 50] = c[0, 0, 7]       # duplicate centre: ties go to slot 7
    valid = np.ones((1, 1, M), np.uint8)
    valid[0, 0, 3] = 0
    lab = host(adc.assign(dev(x), dev(c), valid=dev(valid)))[0, 0]
    ref, b1, b2 = oracle.assign(synth.as_f32(x[0, 0]), c[0, 0], valid[0, 0])
    assert labels_match(lab, ref, b1, b2)[0] == 0
    assert not np.any(lab == 3) and not np.any(lab == 50)


# ----------------------------------------------------------------- layout (lockstep)
@pytest.mark.parametrize("case", list(CASES))
def test_permute_matches_oracle(case):
    w, g = _inputs(case)
    M = 3 * w.k_base + 1
    rng = np.random.default_rng(7)
    lab = rng.integers(0, M - 3, (1, w.H, w.N)).astype(np.int32)   # last slots empty
    out = adc.permute(dev(lab), M, dev(g["k"]), dev(g["v"]))
    for h in range(w.H):
        perm, off = oracle.permute(lab[0, h], M)
        assert np.array_equal(host(out["perm"])[0, h], perm)
        assert np.array_equal(host(out["offsets"])[0, h], off)
        assert np.array_equal(host(out["sizes"])[0, h], np.diff(off))
        kf = synth.as_f32(g["k"][0, h])
        kmax, kmin = (np.zeros((M, w.D), np.float32) for _ in range(2))
        oracle.lib()
        cent, sizes = oracle.update(kf, lab[0, h], np.zeros((M, w.D), np.float32))
        ne = sizes > 0
        assert np.abs(host(out["means"])[0, h][ne] - cent[ne]).max() <= 1e-5 * max(1, np.abs(cent).max())
        for j in np.flatnonzero(ne)[:50]:
            assert np.array_equal(host(out["xmax"])[0, h, j], kf[lab[0, h] == j].max(0))
            assert np.array_equal(host(out["xmin"])[0, h, j], kf[lab[0, h] == j].min(0))
        assert np.all(host(out["xmax"])[0, h][~ne] == 0)
        assert np.array_equal(host(out["x_perm"])[0, h], kf[perm])
        assert np.array_equal(host(out["v_perm"])[0, h], synth.as_f32(g["v"][0, h])[perm])


# ----------------------------------------------------------------- selection (lockstep)
@pytest.mark.parametrize("case", list(CASES))
@pytest.mark.parametrize("rule", ["topp", "topk"])
@pytest.mark.parametrize("score", ["quest", "centroid"])
def test_select_matches_oracle(case, rule, score):
    w, g = _inputs(case)
    H, D = w.H, w.D
    nmax = 4 * w.k_base if w.k_adaptive else w.k_base
    Cq = w.q_clusters
    qrep = np.zeros((1, H, Cq, D), np.float32)
    kdt = g["k"].dtype
    kmax = np.zeros((1, H, nmax, D), kdt)
    kmin = np.zeros((1, H, nmax, D), kdt)
    sizes = np.zeros((1, H, nmax), np.int32)
    cent = np.zeros((1, H, nmax, D), np.float32)
    ncl = np.zeros((1, H), np.int32)
    full = np.zeros((1, H), np.uint8)
    refs = []
    scale = 1 / math.sqrt(D)
    for h in range(H):
        r = _oracle_head(w, g, h)
        K = r["K"]
        qrep[0, h] = r["Q"]["qrep"]
        conv = synth.f32_to_bf16_bits if kdt == np.uint16 else (lambda a: a)
        kmax[0, h] = conv(K["kmax"])
        kmin[0, h] = conv(K["kmin"])
        sizes[0, h] = K["sizes"]
        cent[0, h] = K["cent"]
        ncl[0, h] = K["n_slots"]
        full[0, h] = K["full"]
        ns = K["n_slots"]
        if score == "quest":
            S = r["S"]
        else:
            S = oracle.centroid_scores(r["Q"]["qrep"], K["cent"][:ns], K["sizes"][:ns])
        if rule == "topp":
            sel = oracle.select_topp(S, K["sizes"][:ns], scale, w.top_p, full=bool(K["full"]))
        else:
            sel = oracle.select_topk(S, K["sizes"][:ns], 7, full=bool(K["full"]))
        refs.append((S, sel, K))
    Kd = dict(kmax=dev(kmax), kmin=dev(kmin), sizes=dev(sizes), n_clusters=dev(ncl), full=dev(full),
              centroids=dev(cent))
    res = adc.select(dev(qrep), Kd, top_p=w.top_p, score=score, rule=rule, top_k=7)
    mask = host(res["mask"]).view(np.uint32)
    sel_keys = host(res["sel_keys"])
    for h in range(H):
        S, sel, K = refs[h]
        ns = K["n_slots"]
        gbits = oracle.mask_bits(mask[0, h], nmax)
        assert not gbits[:, ns:].any()
        gb = gbits[:, :ns]
        assert np.array_equal(sel_keys[0, h], (gb * K["sizes"][:ns][None]).sum(1))
        if rule == "topp":
            bad, differ = selection_ok(gb, sel, S, K["sizes"], scale, w.top_p)
        else:
            bad, differ = topk_ok(gb, oracle.mask_bits(sel["mask"], ns), S)
        print(f"{case} {score} {rule} head {h}: rows differing {differ}, violating {bad}")
        assert bad == 0


# ----------------------------------------------------------------- query clustering
@pytest.mark.parametrize("case", list(CASES))
def test_cluster_q_first_assignment_and_lockstep(case):
    w, g = _inputs(case)
    H, Cq = w.H, w.q_clusters
    # 1) init + first assignment: one Lloyd round from the seeded init
    Q1 = adc.cluster_q(dev(g["q"]), Cq, iters=1, init=w.init, seed=0)
    lab1 = host(Q1["assign"])
    # 2) lockstep: start from the oracle's centres after 2 rounds, run one round
    c2 = np.zeros((1, H, Cq, w.D), np.float32)
    for h in range(H):
        qh = oracle.normalize(synth.as_f32(g["q"][0, h]))
        strm = oracle.stream(0, oracle.TENSOR_Q, 0, 0, h)
        init_c = (oracle.init_kmeanspp if w.init == "kmeanspp" else oracle.init_sample)(qh, Cq, strm)[0]
        ref1 = oracle.assign(qh, init_c, (np.arange(Cq) < min(Cq, w.N)).astype(np.uint8))
        bad, diff, _ = labels_match(lab1[0, h], *ref1)
        assert bad == 0, f"head {h}: {diff} first-round mismatches"
        c, _, _, _ = oracle.kmeans(qh, Cq, 2, init=w.init, strm=strm)
        c2[0, h] = c
    Q = adc.cluster_q(dev(g["q"]), Cq, iters=1, init="caller", init_centroids=dev(c2))
    lab = host(Q["assign"])
    for h in range(H):
        qf = synth.as_f32(g["q"][0, h])
        qh = oracle.normalize(qf)
        ref = oracle.assign(qh, c2[0, h])
        bad, diff, ties = labels_match(lab[0, h], *ref)
        assert bad == 0
        # centres / representatives: member means of the GPU labels, bit for bit
        # (normalized rows rounded to f32, f64 sums in row order, one rounding)
        cent, sizes = oracle.update(qh, lab[0, h], c2[0, h])
        assert np.array_equal(host(Q["sizes"])[0, h], sizes)
        assert np.array_equal(host(Q["centroids"])[0, h], cent)
        qrep, _ = oracle.update(qf, lab[0, h], np.zeros((Cq, w.D), np.float32))
        assert np.array_equal(host(Q["qrep"])[0, h], qrep)
        perm, off = oracle.permute(lab[0, h], Cq)
        assert np.array_equal(host(Q["perm"])[0, h], perm)
        assert np.array_equal(host(Q["offsets"])[0, h], off)


# ----------------------------------------------------------------- two-stream layer
def test_layer_overlap_matches_sequential_calls():
    """layer() runs the two clusterings on two streams; its outputs equal the
    four calls made one after another on one stream, bit for bit, on two
    layers in a row (the second reuses the side stream and freed memory)."""
    w, g = _inputs("bf16_d64")
    cfg = adc.LayerConfig(q_clusters=w.q_clusters, k_base=w.k_base, k_max=w.k_max, top_p=w.top_p,
                          iters=w.iters, init=w.init, adaptive=w.k_adaptive)
    q, k, v = (dev(g[t]) for t in "qkv")
    Q = adc.cluster_q(q, cfg.q_clusters, cfg.iters, cfg.init, cfg.seed)
    K = adc.cluster_k(k, v, cfg.k_base, cfg.k_max, cfg.iters, cfg.tau_mult, cfg.adaptive, cfg.init, cfg.seed)
    S = adc.select(Q["qrep"], K, cfg.top_p)
    ref, ref_lse = adc.sparse_attn(q, Q["perm"], Q["offsets"], K["k_perm"], K["v_perm"], K["offsets"],
                                   S["mask"])
    for _ in range(2):
        out, lse, st = adc.layer(q, k, v, cfg)
        torch.cuda.synchronize()
        assert torch.equal(out, ref) and torch.equal(lse, ref_lse)
        assert torch.equal(st["Q"]["assign"], Q["assign"]) and torch.equal(st["K"]["assign"], K["assign"])
        assert torch.equal(st["S"]["mask"], S["mask"])


# ----------------------------------------------------------------- every Lloyd round
@pytest.mark.parametrize("case", ["bf16_d64", "bf16_d128"])
@pytest.mark.parametrize("tensor", ["q", "k"])
def test_lloyd_rounds_are_exact_assignments(case, tensor):
    """Rounds 1..5 from the same caller centres: round r's labels are the exact
    assignment (up to near ties) to the member means of round r-1's labels (a
    slot left empty keeps its centre), so no round may keep a label the exact
    assignment would change."""
    w, g = _inputs(case)
    H, D = w.H, w.D
    m = w.q_clusters if tensor == "q" else w.k_base
    rng = np.random.default_rng(3)
    xs = []
    c0 = np.zeros((1, H, m, D), np.float32)
    for h in range(H):
        xf = synth.as_f32(g[tensor][0, h])
        xh = oracle.normalize(xf) if tensor == "q" else xf
        xs.append(xh)
        c0[0, h] = xh[rng.choice(w.N, m, replace=False)]
    cent = [c0[0, h].astype(np.float64) for h in range(H)]
    prev = None
    for r in range(1, 6):
        if tensor == "q":
            out = adc.cluster_q(dev(g["q"]), m, iters=r, init="caller", init_centroids=dev(c0))
        else:
            out = adc.cluster_k(dev(g["k"]), dev(g["v"]), m, iters=r, adaptive=False, init="caller",
                                init_centroids=dev(c0))
        lab = host(out["assign"])
        for h in range(H):
            if prev is not None:
                cent[h] = oracle.update(xs[h], prev[0, h], cent[h])[0]
            bad, diff, ties = labels_match(lab[0, h], *oracle.assign(xs[h], cent[h]))
            print(f"{case} {tensor} round {r} head {h}: differing {diff}, near ties {ties}, violating {bad}")
            assert bad == 0
        prev = lab


# ----------------------------------------------------------------- key clustering
# 4096 rows: the init keeps D^2 and its running sums in LDS; 5120 rows (one head):
# it streams them through LDS in chunks and re-adds the crossing chunk
@pytest.mark.parametrize("grid,H", [(None, None), ((5, 32, 32), 1)])
def test_cluster_k_fixed_first_round_kmeanspp(grid, H):
    if grid is None:
        w, g = _inputs("tiny")
    else:
        w = small_workload("tiny", grid=grid, H=H)
        g = synth.generate(w, seed=0)
    K = adc.cluster_k(dev(g["k"]), dev(g["v"]), w.k_base, iters=1, adaptive=False, init="kmeanspp")
    lab = host(K["assign"])
    for h in range(w.H):
        kf = synth.as_f32(g["k"][0, h])
        c0, _ = oracle.init_kmeanspp(kf, w.k_base, oracle.stream(0, oracle.TENSOR_K, 0, 0, h))
        bad, diff, _ = labels_match(lab[0, h], *oracle.assign(kf, c0))
        assert bad == 0
        assert host(K["n_clusters"])[0, h] == w.k_base and host(K["full"])[0, h] == 0


def _hand_case_tensors(case):
    pts = np.array(case["keys"], np.float32)
    n = len(pts)
    k = np.zeros((1, 1, n, 64), np.float32)
    k[0, 0, :, :2] = pts
    v = np.random.default_rng(0).standard_normal((1, 1, n, 64)).astype(np.float32)
    return k, v


def test_cluster_k_hand_cases_exact():
    import json, os
    with open(os.path.join(os.path.dirname(__file__), "golden", "alg1_hand.json")) as f:
        cases = json.load(f)["cases"]
    for case in cases:
        k, v = _hand_case_tensors(case)
        K = adc.cluster_k(dev(k), dev(v), case["m0"], case["nmax"], iters=case["iters"],
                          tau_mult=case["tau_mult"], adaptive=True, init="sample", seed=11)
        ns = case["n_slots"]
        assert host(K["n_clusters"])[0, 0] == ns, case["name"]
        assert host(K["full"])[0, 0] == case["full"], case["name"]
        assert host(K["tau"])[0, 0] == pytest.approx(case["tau"], abs=1e-6)
        assert host(K["assign"])[0, 0].tolist() == case["labels"], case["name"]
        assert host(K["sizes"])[0, 0][:ns].tolist() == case["sizes"]
        assert host(K["offsets"])[0, 0][:ns + 1].tolist() == case["off"]
        st = host(K["stage_sizes"])[0, 0]
        assert st[st >= 0].tolist() == case["stage_u"], case["name"]


@pytest.mark.parametrize("case", ["bf16_d64", "bf16_d128"])
def test_cluster_k_adaptive_matches_oracle(case):
    w, g = _inputs(case)
    K = adc.cluster_k(dev(g["k"]), dev(g["v"]), w.k_base, 4 * w.k_base, iters=w.iters,
                      adaptive=True, init=w.init)
    for h in range(w.H):
        kf = synth.as_f32(g["k"][0, h])
        r = oracle.cluster_k(kf, w.k_base, 4 * w.k_base, w.iters, adaptive=True, init=w.init, h=h)
        st = host(K["stage_sizes"])[0, h]
        print(f"{case} head {h}: oracle slots {r['n_slots']} F {r['full']} tau {r['tau']:.6f} "
              f"U {r['stage_u'].tolist()} | gpu slots {host(K['n_clusters'])[0, h]} "
              f"F {host(K['full'])[0, h]} tau {host(K['tau'])[0, h]:.6f} U {st[st >= 0].tolist()}")
        assert host(K["tau"])[0, h] == pytest.approx(r["tau"], rel=1e-5)
        assert host(K["n_clusters"])[0, h] == r["n_slots"]
        assert host(K["full"])[0, h] == r["full"]
        gu = st[st >= 0]
        assert len(gu) == len(r["stage_u"])
        assert np.abs(gu - r["stage_u"]).max() <= max(2, 0.002 * w.N)
        agree = (host(K["assign"])[0, h] == r["lab"]).mean()
        print(f"  label agreement {agree:.4f}")
        assert agree >= 0.98
        # outputs consistent with the GPU's own labels
        lab = host(K["assign"])[0, h]
        perm, off = oracle.permute(lab, 4 * w.k_base)
        assert np.array_equal(host(K["perm"])[0, h], perm)
        assert np.array_equal(host(K["k_perm"])[0, h].astype(np.float32), kf[perm])


# ----------------------------------------------------------------- whole layer
def test_layer_tiny_close_to_oracle():
    w, g = _inputs("tiny")
    cfg = adc.LayerConfig(q_clusters=w.q_clusters, k_base=w.k_base, k_max=w.k_base, top_p=w.top_p,
                          iters=w.iters, init=w.init, adaptive=False)
    out, lse, st = adc.layer(dev(g["q"]), dev(g["k"]), dev(g["v"]), cfg)
    out = host(out)
    for h in range(w.H):
        r = _oracle_head(w, g, h)
        qa = (host(st["Q"]["assign"])[0, h] == r["Q"]["lab"]).mean()
        ka = (host(st["K"]["assign"])[0, h] == r["K"]["lab"]).mean()
        e = rel_l2(out[0, h], r["out"])
        print(f"tiny head {h}: q-label agreement {qa:.4f} k-label agreement {ka:.4f} out rel-L2 {e:.3e}")
        assert qa >= 0.98 and ka >= 0.98
        assert e <= 5e-2


def test_layer_full_flag_is_dense():
    # identical keys: tau = 0, F = 1, every slot selected: equals dense attention
    rng = np.random.default_rng(9)
    N, D = 300, 64
    q = synth.f32_to_bf16_bits(rng.standard_normal((1, 1, N, D)).astype(np.float32))
    k = synth.f32_to_bf16_bits(np.tile(rng.standard_normal((1, 1, 1, D)).astype(np.float32), (1, 1, N, 1)))
    v = synth.f32_to_bf16_bits(rng.standard_normal((1, 1, N, D)).astype(np.float32))
    cfg = adc.LayerConfig(q_clusters=8, k_base=4, k_max=16, top_p=0.5, iters=3)
    out, _, st = adc.layer(dev(q), dev(k), dev(v), cfg)
    assert host(st["K"]["full"])[0, 0] == 1
    qf, kf, vf = (synth.as_f32(t[0, 0]).astype(np.float64) for t in (q, k, v))
    z = qf @ kf.T / 8
    p = np.exp(z - z.max(1, keepdims=True))
    ref = p @ vf / p.sum(1, keepdims=True)
    assert rel_l2(host(out)[0, 0], ref) <= 1e-2
