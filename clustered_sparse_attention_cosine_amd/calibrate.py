"""Per-layer key-cluster counts and the Nmax calibration over a stack of layers.

AdaCluster (section 3.2.1) measures how compact each layer's keys are (the mean
squared reconstruction error at a uniform cluster count, Comp_l = 1 / MSE_l,
Fig. 4) and argues that scattered layers need more clusters; Algorithm 1
finds each head's count, and section 4.1 sets the cap so that the top 15 % of
layers (those that would need the most clusters) fall back to full attention.

This module runs that study on the GPU: every step is a call of the library
(adaptive and fixed key clustering, compactness); only the bookkeeping over
layers is done here. A layer's required count is the largest count any of its
heads reaches with a generous cap (a head that still has unassigned keys at
the cap counts as needing more than the cap).
"""
from __future__ import annotations

import numpy as np

from . import cluster_k, compactness


def profile_layer(k, v, m0, probe_max, iters=5, tau_mult=1.5, init="sample", seed=0,
                  comp_clusters=400):
    """Algorithm 1 with cap probe_max on every head of one layer, and the
    layer's compactness at comp_clusters centres (one k-means per head)."""
    K = cluster_k(k, v, m0, probe_max, iters, tau_mult, True, init, seed)
    Kc = cluster_k(k, v, comp_clusters, comp_clusters, iters, adaptive=False, init=init, seed=seed)
    C = compactness(Kc["k_perm"], Kc["offsets"], Kc["centroids"])
    counts = K["n_clusters"].cpu().numpy().reshape(-1)
    full = K["full"].cpu().numpy().reshape(-1).astype(bool)
    need = np.where(full, probe_max + 1, counts)
    return dict(head_counts=counts, head_full=full, required=int(need.max()),
                mse=C["mse"].cpu().numpy().reshape(-1), comp=float(C["comp"].cpu()[0]))


def choose_kmax(required, m0, probe_max, top_frac=0.15):
    """Smallest stage boundary (m0, 2 m0, 4 m0, ... up to probe_max) that at
    most top_frac of the layers need more than; probe_max if none does."""
    req = np.asarray(required)
    c = m0
    while c <= probe_max:
        if np.mean(req > c) <= top_frac + 1e-12:
            return c
        c *= 2
    return probe_max


def calibrate_stack(layers, m0, probe_max, top_frac=0.15, iters=5, tau_mult=1.5, init="sample",
                    seed=0, comp_clusters=400):
    """layers: list of (k, v) device tensors [B,H,N,D]. Profiles every layer,
    picks Nmax, and re-runs Algorithm 1 with that cap to report which heads
    (and layers) then take full attention."""
    prof = [profile_layer(k, v, m0, probe_max, iters, tau_mult, init, seed, comp_clusters)
            for k, v in layers]
    kmax = choose_kmax([p["required"] for p in prof], m0, probe_max, top_frac)
    for p, (k, v) in zip(prof, layers):
        K = cluster_k(k, v, m0, kmax, iters, tau_mult, True, init, seed)
        p["full_at_kmax"] = K["full"].cpu().numpy().reshape(-1).astype(bool)
    return dict(kmax=kmax, layers=prof)
