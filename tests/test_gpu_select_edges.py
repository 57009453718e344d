"""Selection at the cut, on constructed scores (AdaCluster section 3.2.3,
Eq. (2)): exact ties at the cut (taken in slot order until the mass or count
is reached), a cut inside a crowd of slots whose l lie within one histogram
bucket (more than the kernel gathers, so it settles the cut by bisection),
slots without members, and capacities that need one, two, four and eight
waves per row. The key statistics hold one nonzero dimension, so every score
q . k is an exact product and l differs between slots only through ln n."""
import math

import numpy as np
import pytest

import clustered_sparse_attention_cosine_amd as adc
import oracle
import synth
from gpu_util import dev, host, selection_ok, topk_ok

pytestmark = pytest.mark.gpu

D = 64
SCALE = 1 / math.sqrt(D)


def _case(Ck, kind, rng):
    """Per-slot score factor s_b and size n_b for one head."""
    s = np.zeros(Ck, np.float32)
    n = np.zeros(Ck, np.int32)
    live = min(Ck, 3000)
    # the low bulk: distinct factors, small sizes
    s[:live] = synth.as_f32(synth.f32_to_bf16_bits(-np.arange(live, dtype=np.float32) / 64.0))
    n[:live] = rng.integers(1, 50, live)
    if kind == "crowd":       # 200 top slots, l apart only by ln n (1e-4 nats)
        s[:200] = 8.0
        n[:200] = 10000 + np.arange(200)
    elif kind == "tie_many":  # 200 top slots with one l: more ties than gathered
        s[:200] = 8.0
        n[:200] = 5000
    elif kind == "tie_few":   # 10 tied slots at the top, a few dozen close below
        s[:10] = 8.0
        n[:10] = 5000
        s[10:40] = 7.0
        n[10:40] = 4000
    n[rng.random(Ck) < 0.05] = 0   # slots without members
    return s, n


@pytest.mark.parametrize("Ck", [700, 2048, 4096, 8192])
@pytest.mark.parametrize("rule", ["topp", "topk"])
def test_select_cut_cases(Ck, rule):
    rng = np.random.default_rng(Ck)
    kinds = ["crowd", "tie_many", "tie_few", "plain"]
    H, Cq = len(kinds), 6
    alphas = np.array([2.0, 1.0, 0.5, 0.25, 16.0, 1.5], np.float32)
    qrep = np.zeros((1, H, Cq, D), np.float32)
    qrep[0, :, :, 0] = alphas[None]
    kstat = np.zeros((1, H, Ck, D), np.float32)
    sizes = np.zeros((1, H, Ck), np.int32)
    for h, kind in enumerate(kinds):
        s, n = _case(Ck, kind, rng)
        kstat[0, h, :, 0] = s
        sizes[0, h] = n
    kb = synth.f32_to_bf16_bits(kstat)
    assert np.array_equal(synth.as_f32(kb), kstat)  # the factors are exact in bf16
    Kd = dict(kmax=dev(kb), kmin=dev(kb), sizes=dev(sizes), centroids=dev(kstat),
              n_clusters=dev(np.full((1, H), Ck, np.int32)), full=dev(np.zeros((1, H), np.uint8)))
    top_p = 0.5 if rule == "topp" else 0.9
    top_k = 5
    res = adc.select(dev(qrep), Kd, top_p=top_p, rule=rule, top_k=top_k)
    mask = host(res["mask"]).view(np.uint32)
    sel_keys = host(res["sel_keys"])
    for h, kind in enumerate(kinds):
        sz = sizes[0, h]
        # S_ab = q+ . kmax + q- . kmin = alpha_a s_b, exactly
        S = (alphas[:, None].astype(np.float64) * kstat[0, h, :, 0][None].astype(np.float64))
        gb = oracle.mask_bits(mask[0, h], Ck)
        assert not (gb & (sz[None] == 0)).any(), (kind, "a slot without members was selected")
        assert np.array_equal(sel_keys[0, h], (gb * sz[None]).sum(1))
        if rule == "topp":
            sel = oracle.select_topp(S, sz, SCALE, top_p)
            bad, differ = selection_ok(gb, sel, S, sz, SCALE, top_p)
        else:
            sel = oracle.select_topk(S, sz, top_k)
            bad, differ = topk_ok(gb, oracle.mask_bits(sel["mask"], Ck), S)
        ob = oracle.mask_bits(sel["mask"], Ck)
        # exact ties at the cut: the GPU takes a prefix of them in slot order
        for a in range(Cq):
            l = S[a] * (SCALE if rule == "topp" else 1.0) + (np.log(np.maximum(sz, 1)) if rule == "topp" else 0)
            sel_l = l[gb[a]]
            if sel_l.size == 0:
                continue
            cut = sel_l.min()
            tied = np.flatnonzero((l == cut) & (sz > 0))
            taken = gb[a, tied]
            assert np.all(taken[:taken.sum()]), (kind, a, "ties not taken in slot order")
        print(f"Ck {Ck} {rule} {kind}: rows differing from the oracle {differ}, violating {bad}, "
              f"selected {gb.sum(1).tolist()} (oracle {ob.sum(1).tolist()})")
        assert bad == 0


def test_select_take_all():
    # full-attention heads and top_p = 1 take every slot with members
    rng = np.random.default_rng(3)
    H, Cq, Ck = 2, 5, 1500
    qrep = rng.standard_normal((1, H, Cq, D)).astype(np.float32)
    kb = synth.f32_to_bf16_bits(rng.standard_normal((1, H, Ck, D)).astype(np.float32))
    sizes = rng.integers(0, 4, (1, H, Ck)).astype(np.int32)
    full = np.array([[1, 0]], np.uint8)
    Kd = dict(kmax=dev(kb), kmin=dev(kb), sizes=dev(sizes), centroids=None,
              n_clusters=dev(np.array([[Ck, 1200]], np.int32)), full=dev(full))
    for p in (0.9, 1.0):
        res = adc.select(dev(qrep), Kd, top_p=p)
        gb = oracle.mask_bits(host(res["mask"]).view(np.uint32)[0], Ck)
        live0 = sizes[0, 0] > 0
        assert np.array_equal(gb[0], np.broadcast_to(live0, (Cq, Ck)))
        if p == 1.0:
            live1 = (sizes[0, 1] > 0) & (np.arange(Ck) < 1200)
            assert np.array_equal(gb[1], np.broadcast_to(live1, (Cq, Ck)))
