"""Helpers shared by the GPU tests: moving seeded inputs to the device and the
parity rules (near-tie exemptions) used to compare with the oracle."""
import numpy as np
import pytest
import torch

import oracle
import synth

NEAR_TIE = 1e-4


def dev(arr):
    """numpy input (uint16 bf16 bits or float32 / int32) -> device tensor."""
    if arr.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16).copy()).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(arr)).cuda()


def host(t):
    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy()
    return t.cpu().numpy()


def labels_match(gpu_lab, ora_lab, b1, b2, tol=NEAR_TIE):
    """Labels equal except rows whose two best oracle distances are within tol."""
    diff = gpu_lab != ora_lab
    tie = (b2 - b1) <= tol * b2
    return int((diff & ~tie).sum()), int(diff.sum()), int(tie.sum())


def rel_l2(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-30))


def selection_ok(gpu_bits, sel, S, sizes, scale, p):
    """Per row: the GPU set may differ from the oracle's only at the cut (near-tie
    logits within 1e-4 * max(1, |l|), or cumulative mass within 1e-4 of p).
    Returns (rows violating, rows differing)."""
    ck = gpu_bits.shape[1]
    ora_bits = oracle.mask_bits(sel["mask"], ck)
    bad = differ = 0
    with np.errstate(divide="ignore"):
        logn = np.log(np.maximum(sizes[:ck], 1).astype(np.float64))
    for a in range(gpu_bits.shape[0]):
        G = set(np.flatnonzero(gpu_bits[a]).tolist())
        O = set(np.flatnonzero(ora_bits[a]).tolist())
        if G == O:
            continue
        differ += 1
        lc = sel["l_cut"][a]
        tol = NEAR_TIE * max(1.0, abs(lc))
        l = S[a] * scale + logn
        ok = True
        for b in G ^ O:
            near_cut = abs(l[b] - lc) <= tol
            near_next = abs(l[b] - sel["l_next"][a]) <= tol
            extra_ok = b in G and (sel["cum_at"][a] - p) <= NEAR_TIE and (near_next or near_cut)
            miss_ok = b in O and (p - sel["cum_before"][a]) <= NEAR_TIE and near_cut
            if not (near_cut and len(G) == len(O)) and not extra_ok and not miss_ok:
                ok = False
        bad += int(not ok)
    return bad, differ


def topk_ok(gpu_bits, ora_bits, S, tol=NEAR_TIE):
    """Per row: the top-k sets may differ only in slots whose oracle score is
    within tol * max(1, |s|) of the row's cut (the k-th largest score), with the
    same set size. Returns (rows violating, rows differing)."""
    bad = differ = 0
    for a in range(gpu_bits.shape[0]):
        G, O = gpu_bits[a], ora_bits[a]
        if np.array_equal(G, O):
            continue
        differ += 1
        cut = S[a][O].min()
        near = np.abs(S[a] - cut) <= tol * max(1.0, abs(cut))
        bad += int(G.sum() != O.sum() or not np.all(near[G != O]))
    return bad, differ


def small_workload(name, **kw):
    return synth.scaled(synth.WORKLOADS[name], **kw)


def check_alg1_head(kf, K, tr, h, m0, nmax, tau_mult=1.5, tag=""):
    """Every decision of Algorithm 1 (AdaCluster section 3.2.2, tau from section
    4.1) for head h of a traced STAGED key clustering, recomputed from the
    values it was taken on:
      - each stage's labels are the exact assignment (oracle.assign) of the
        keys of U to the centres that stage's last assignment measured
        against, except near ties (two best distances within 1e-4 relative);
      - each stage's centres are the member means of those labels (rel-L2
        1e-5 per centre; a slot with no member keeps its centre);
      - tau = tau_mult x the mean distance of all keys to their stage-0 centre
        (rel 1e-5);
      - U after stage t is {i in U_t : d_i >= tau} except keys with
        |d_i - tau| <= 1e-4 tau, and the loop runs, stops and sets F exactly as
        those sets say (counts and F exact when no such key exists);
      - the final labels are the exact assignment to every slot holding a
        centre, before the refresh, except near ties.
    kf: the head's keys as float32 [N, D]; K / tr: host copies of the
    cluster_k outputs and of its record. Returns a short summary dict."""
    N = kf.shape[0]
    kd = kf.astype(np.float64)
    base = tr["stage_base"][0, h]
    labs = tr["stage_labels"][0, h]
    last = tr["last_centroids"][0, h]
    cent = tr["stage_centroids"][0, h]
    valid = tr["slot_valid"][0, h].astype(bool)
    st = K["stage_sizes"][0, h]
    tau = float(K["tau"][0, h])
    n_stages = int((base >= 0).sum())
    assert n_stages >= 1 and np.all(base[:n_stages] >= 0) and np.all(base[n_stages:] == -1)
    U = np.arange(N)
    slots = 0
    near_total = 0
    summary = dict(stages=n_stages, U=[], near_tau=0, label_ties=0)
    for t in range(n_stages):
        mt = m0 if t == 0 else m0 << (t - 1)
        mt = min(mt, nmax - slots)
        assert base[t] == slots, (tag, h, t)
        Ut = np.flatnonzero(labs[t] >= 0)
        assert np.array_equal(Ut, U), (tag, h, t, "U differs from the previous stage's decision")
        assert st[t] == len(Ut)
        summary["U"].append(len(Ut))
        lab = labs[t][Ut] - slots
        assert lab.min() >= 0 and lab.max() < mt
        sl = slice(slots, slots + mt)
        # labels: exact assignment to the centres the last round measured against
        lo, b1, b2 = oracle.assign(kf[Ut], last[sl], valid[sl])
        bad, diff, ties = labels_match(lab, lo, b1, b2)
        summary["label_ties"] += diff
        assert bad == 0, (tag, h, t, "stage labels", bad)
        # centres: member means (f32 sums in a fixed order vs the f64 mean)
        ref, sizes = oracle.update(kf[Ut], lab, last[sl])
        for j in np.flatnonzero(sizes):
            assert rel_l2(cent[slots + j], ref[j]) <= 1e-5, (tag, h, t, j)
        empty = np.flatnonzero(sizes == 0)
        assert np.array_equal(cent[slots + empty], last[sl][empty])
        # the threshold test of every key of U against its stage centre
        d = np.sqrt(((kd[Ut] - cent[slots + lab].astype(np.float64)) ** 2).sum(1))
        if t == 0:
            assert tau == pytest.approx(tau_mult * d.mean(), rel=1e-5), (tag, h)
        keep = d >= tau
        near = np.abs(d - tau) <= 1e-4 * tau
        near_total += int(near.sum())
        slots += mt
        if t + 1 < n_stages:
            Un = np.flatnonzero(labs[t + 1] >= 0)
            assert np.all(np.isin(Un, Ut)), (tag, h, t, "a removed key came back")
            inn = np.isin(Ut, Un)
            assert np.array_equal(inn[~near], keep[~near]), (tag, h, t, "threshold test")
            assert len(Un) > 0 and slots < nmax  # the loop went on
            U = Un
        else:
            left = int(st[t + 1]) if t + 1 < len(st) else None
            if left is not None:
                assert abs(left - int(keep.sum())) <= int(near.sum()), (tag, h, "U after the last stage")
            # the loop ended: U empty, or Nmax slots with U left (F = 1)
            full = int(K["full"][0, h])
            if near.sum() == 0:
                assert full == int(keep.sum() > 0 and slots >= nmax), (tag, h, "F")
                assert keep.sum() == 0 or slots >= nmax
            assert full in (0, 1)
    summary["near_tau"] = near_total
    assert int(K["n_clusters"][0, h]) == slots
    # final assignment over every slot holding a centre, before the refresh
    lo, b1, b2 = oracle.assign(kf, cent[:slots], valid[:slots])
    bad, diff, ties = labels_match(K["assign"][0, h], lo, b1, b2)
    summary["final_ties"] = diff
    assert bad == 0, (tag, h, "final labels", bad)
    return summary
