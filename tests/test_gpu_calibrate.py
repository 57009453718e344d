"""Per-layer counts and the Nmax calibration over a synthetic stack of layers
(sections 3.2.1, 3.2.2 and 4.1), HIP path vs the oracle. Needs an MI355X."""
import numpy as np
import pytest

import clustered_sparse_attention_cosine_amd as adc
from clustered_sparse_attention_cosine_amd import calibrate
import oracle
import synth
from gpu_util import dev, small_workload

pytestmark = pytest.mark.gpu

M0, PROBE, COMP = 16, 256, 40


def test_stack_calibration_matches_oracle():
    w = small_workload("cog17k", H=2, grid=(3, 20, 30), text_tokens=11)
    stack = synth.layer_stack(w, 8)
    gens = [synth.generate(lw, seed=seed) for lw, seed in stack]
    res = calibrate.calibrate_stack([(dev(g["k"]), dev(g["v"])) for g in gens], M0, PROBE,
                                    top_frac=0.15, comp_clusters=COMP)
    req_o = []
    for li, g in enumerate(gens):
        ks = [synth.as_f32(g["k"][0, h]) for h in range(w.H)]
        req_o.append(oracle.layer_required_count(ks, M0, PROBE))
        mse_o = []
        for h, k in enumerate(ks):
            r = oracle.cluster_k(k, COMP, COMP, 5, adaptive=False, h=h)
            mse_o.append(oracle.compactness(k, r["lab"], r["cent"])["mse"])
        p = res["layers"][li]
        print(f"layer {li}: gpu heads {p['head_counts'].tolist()} required {p['required']} "
              f"| oracle {req_o[-1]}; Comp gpu {p['comp']:.5f} oracle {oracle.layer_compactness(mse_o):.5f}")
        assert p["required"] == req_o[-1]
        assert p["comp"] == pytest.approx(oracle.layer_compactness(mse_o), rel=2e-2)
    kmax = oracle.kmax_for_top_fraction(req_o, M0, PROBE, 0.15)
    assert res["kmax"] == kmax
    # at the chosen cap, exactly the layers that need more than it have heads
    # on full attention, and no more than 15 % of the layers do
    over = [r > kmax for r in req_o]
    got = [bool(p["full_at_kmax"].any()) for p in res["layers"]]
    assert got == over
    assert np.mean(got) <= 0.15 + 1e-9
