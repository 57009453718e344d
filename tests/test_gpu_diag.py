"""Compactness diagnostics (section 3.2.1 MSE and Comp, Fig. 10 mean distance
and Davies-Bouldin index): the HIP kernels on the oracle's clusterings vs the
oracle, through the C ABI. Needs an MI355X."""
import numpy as np
import pytest
import torch

import clustered_sparse_attention_cosine_amd as adc
import oracle
import synth
from gpu_util import dev, host, small_workload

pytestmark = pytest.mark.gpu

CASES = {
    "f32_d64": ("tiny", {}),
    "bf16_d64": ("cog17k", dict(H=2, grid=(3, 20, 50), text_tokens=37, q_clusters=40, k_base=24)),
    "bf16_d128": ("wan33k", dict(H=2, grid=(2, 31, 37), q_clusters=24, k_base=18)),
}


def _gpu_compactness(x, labs, cents):
    """x [1,H,N,D] (generator dtype), per-head labels and centres from the oracle."""
    H = x.shape[1]
    M = cents[0].shape[0]
    xp = np.empty_like(x)
    off = np.zeros((1, H, M + 1), np.int32)
    for h in range(H):
        perm, off[0, h] = oracle.permute(labs[h], M)
        xp[0, h] = x[0, h][perm]
    return adc.compactness(dev(xp), dev(off), dev(np.stack(cents)[None].astype(np.float32)))


@pytest.mark.parametrize("case", list(CASES))
def test_compactness_matches_oracle(case):
    name, kw = CASES[case]
    w = small_workload(name, **kw)
    g = synth.generate(w, seed=0)
    labs, cents, refs = [], [], []
    for h in range(w.H):
        kf = synth.as_f32(g["k"][0, h])
        r = oracle.cluster_k(kf, w.k_base, w.k_max, w.iters, adaptive=w.k_adaptive, init=w.init, h=h)
        labs.append(r["lab"])
        cents.append(r["cent"])
        refs.append(oracle.compactness(kf, r["lab"], r["cent"]))
    out = {n: host(t) for n, t in _gpu_compactness(g["k"], labs, cents).items()}
    for h in range(w.H):
        ref = refs[h]
        print(f"{case} head {h}: mse {out['mse'][0, h]:.6e}/{ref['mse']:.6e} "
              f"dist {out['mean_dist'][0, h]:.6e}/{ref['mean_dist']:.6e} "
              f"db {out['db'][0, h]:.6e}/{ref['db']:.6e}")
        assert out["mse"][0, h] == pytest.approx(ref["mse"], rel=1e-5)
        assert out["mean_dist"][0, h] == pytest.approx(ref["mean_dist"], rel=1e-5)
        assert out["db"][0, h] == pytest.approx(ref["db"], rel=1e-4)
    comp = oracle.layer_compactness([r["mse"] for r in refs])
    assert out["comp"][0] == pytest.approx(comp, rel=1e-5)


def test_compactness_hand_cases():
    # head 0: pairs {0, 2} and {10, 12} around 1 and 11 with an empty slot between
    # (DB = 2/10); head 1: two clusters with one centre (no partner: DB = 0);
    # head 2: one cluster holds every row (DB = 0)
    N, M, D = 4, 3, 64
    x = np.zeros((1, 3, N, D), np.float32)
    cent = np.zeros((3, M, D), np.float32)
    x[0, 0, :, 0] = [0, 2, 10, 12]
    cent[0, 0, 0], cent[0, 2, 0] = 1, 11
    x[0, 1, :, 0] = [-1, 1, -2, 2]
    x[0, 2, :, 0] = [1, 2, 3, 6]
    cent[2, 1, 0] = 3
    labs = [np.array([0, 0, 2, 2]), np.array([0, 0, 1, 1]), np.array([1, 1, 1, 1])]
    out = {n: host(t) for n, t in _gpu_compactness(x, labs, list(cent)).items()}
    assert out["mse"][0].tolist() == pytest.approx([1.0, 2.5, 14 / 4], rel=1e-12)
    assert out["mean_dist"][0].tolist() == pytest.approx([1.0, 1.5, 1.5], rel=1e-12)
    assert out["db"][0].tolist() == pytest.approx([0.2, 0.0, 0.0], rel=1e-6)
    assert out["comp"][0] == pytest.approx(3 / (1.0 + 2.5 + 3.5), rel=1e-12)
