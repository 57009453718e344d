"""The graph-captured layer (LayerGraph) against eager layer() calls: three
replays on three different inputs written into the graph's input buffers, each
followed by an eager layer on the same inputs and a synchronization, and every
replay's outputs equal to the eager ones bit for bit (every kernel of the path
is deterministic)."""
import pytest
import torch

import clustered_sparse_attention_cosine_amd as adc
import synth
from gpu_util import dev
from test_gpu_parity import _inputs

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("case", ["bf16_d64", "bf16_d128"])
def test_layer_graph_replays_match_eager(case):
    w, g = _inputs(case, seed=0)
    cfg = adc.LayerConfig(q_clusters=w.q_clusters, k_base=w.k_base, k_max=w.k_max, top_p=w.top_p,
                          iters=w.iters, init=w.init, adaptive=w.k_adaptive)
    q, k, v = (dev(g[t]) for t in "qkv")
    lg = adc.LayerGraph(q, k, v, cfg)
    for seed in (1, 2, 3):
        g2 = synth.generate(w, seed=seed)
        for name, t in zip("qkv", (lg.q, lg.k, lg.v)):
            t.copy_(dev(g2[name]))
        out, lse, st = lg.replay()
        torch.cuda.synchronize()
        got = (out.clone(), lse.clone(), st["Q"]["assign"].clone(), st["K"]["assign"].clone(),
               st["K"]["n_clusters"].clone(), st["S"]["mask"].clone())
        ref_out, ref_lse, ref_st = adc.layer(lg.q, lg.k, lg.v, cfg)
        torch.cuda.synchronize()
        ref = (ref_out, ref_lse, ref_st["Q"]["assign"], ref_st["K"]["assign"], ref_st["K"]["n_clusters"],
               ref_st["S"]["mask"])
        names = ["out", "lse", "q assign", "k assign", "k counts", "mask"]
        for n, a, b in zip(names, got, ref):
            assert torch.equal(a, b), (case, seed, n)
