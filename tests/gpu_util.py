"""Helpers shared by the GPU tests: moving seeded inputs to the device and the
parity rules (near-tie exemptions) used to compare with the oracle."""
import numpy as np
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
