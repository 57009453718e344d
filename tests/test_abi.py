"""The C-ABI library loads and exports every entry point the header declares;
argument checks reject bad calls before any launch. CPU only: no call here
reaches a kernel or any HIP runtime function."""
import ctypes

import pytest

import clustered_sparse_attention_cosine_amd as adc

EXPECTED = {
    "adacluster_abi_version", "adacluster_last_error",
    "adacluster_cluster_q_workspace", "adacluster_cluster_q",
    "adacluster_cluster_k_workspace", "adacluster_cluster_k", "adacluster_cluster_k_trace",
    "adacluster_select_workspace", "adacluster_select",
    "adacluster_sparse_attn_workspace", "adacluster_sparse_attn", "adacluster_sparse_attn_noalloc",
    "adacluster_assign_workspace", "adacluster_assign",
    "adacluster_permute_workspace", "adacluster_permute",
    "adacluster_compactness_workspace", "adacluster_compactness",
}


def test_header_declares_expected_entry_points():
    assert set(adc.header_symbols()) == EXPECTED


def test_library_exports_every_header_symbol():
    L = adc.lib()
    for name in adc.header_symbols():
        assert hasattr(L, name), name


def test_abi_version():
    assert adc.lib().adacluster_abi_version() == 3


def _shape(B=1, H=2, N=1000, D=64, dt=adc.ADC_BF16):
    return adc.Shape(B, H, N, D, dt)


def test_workspace_queries_positive_and_scale():
    L = adc.lib()
    sh = _shape()
    qp = adc.QParams(32, 5, 1, 0, 0)
    kp = adc.KParams(16, 64, 5, 1.5, 1, 1, 0)
    assert L.adacluster_cluster_q_workspace(ctypes.byref(sh), ctypes.byref(qp)) > 0
    a = L.adacluster_cluster_k_workspace(ctypes.byref(sh), ctypes.byref(kp))
    kp2 = adc.KParams(16, 64, 5, 1.5, 0, 1, 0)
    b = L.adacluster_cluster_k_workspace(ctypes.byref(sh), ctypes.byref(kp2))
    assert a > b > 0  # the multi-stage state is only needed when adaptive
    assert L.adacluster_select_workspace(ctypes.byref(sh), 32, 64) >= 2 * 32 * 64 * 4
    assert L.adacluster_sparse_attn_workspace(ctypes.byref(sh), 32, 64) > 0
    assert L.adacluster_assign_workspace(ctypes.byref(sh), 64) > 0
    assert L.adacluster_permute_workspace(ctypes.byref(sh), 64) > 0


@pytest.mark.parametrize("bad", [
    dict(D=96), dict(N=0), dict(H=0), dict(dt=7), dict(N=1 << 22)])
def test_workspace_query_rejects_bad_shape(bad):
    kw = dict(B=1, H=2, N=1000, D=64, dt=adc.ADC_BF16)
    kw.update(bad)
    sh = _shape(**kw)
    qp = adc.QParams(32, 5, 1, 0, 0)
    assert adc.lib().adacluster_cluster_q_workspace(ctypes.byref(sh), ctypes.byref(qp)) == 0
    assert adc.lib().adacluster_last_error()


def _q_call(sh, qp, ptrs=None, ws_bytes=1 << 40):
    L = adc.lib()
    p = ptrs if ptrs is not None else [ctypes.c_void_p(16)] * 8
    return L.adacluster_cluster_q(ctypes.byref(sh), ctypes.byref(qp), *p,
                                  ctypes.c_void_p(16), ws_bytes, None)


def test_error_codes_before_launch():
    L = adc.lib()
    sh = _shape()
    # null output pointer
    ptrs = [ctypes.c_void_p(16)] * 8
    ptrs[2] = None
    assert _q_call(sh, adc.QParams(32, 5, 1, 0, 0), ptrs) == -1
    assert b"assign" in L.adacluster_last_error()
    # bad cluster count, bad iteration count, unknown init
    assert _q_call(sh, adc.QParams(0, 5, 1, 0, 0)) == -2
    assert _q_call(sh, adc.QParams(9000, 5, 1, 0, 0)) == -2
    assert _q_call(sh, adc.QParams(32, 0, 1, 0, 0)) == -1
    assert _q_call(sh, adc.QParams(32, 5, 9, 0, 0)) == -1
    # caller init without centres
    ptrs = [ctypes.c_void_p(16)] * 8
    ptrs[1] = None
    assert _q_call(sh, adc.QParams(32, 5, 2, 0, 0), ptrs) == -1
    # workspace too small
    assert _q_call(sh, adc.QParams(32, 5, 1, 0, 0), ws_bytes=10) == -4
    # bad dtype / head dim
    assert _q_call(_shape(dt=3), adc.QParams(32, 5, 1, 0, 0)) == -3
    assert _q_call(_shape(D=80), adc.QParams(32, 5, 1, 0, 0)) == -2


def test_cluster_k_parameter_checks():
    L = adc.lib()
    sh = _shape()
    ptr = [ctypes.c_void_p(16)] * 16

    def call(kp):
        return L.adacluster_cluster_k(ctypes.byref(sh), ctypes.byref(kp), *ptr,
                                      ctypes.c_void_p(16), 1 << 40, None)
    assert call(adc.KParams(64, 32, 5, 1.5, 1, 1, 0)) == -2          # Nmax < m0
    assert call(adc.KParams(16, 64, 5, float("nan"), 1, 1, 0)) == -1  # tau_mult
    assert call(adc.KParams(16, 64, 5, 1.5, 1, 2, 0)) == -6          # caller + adaptive
    assert call(adc.KParams(16, 64, 5, 1.5, 2, 1, 0)) == -1          # warm without caller init
    assert call(adc.KParams(16, 64, 5, 1.5, 3, 2, 0)) == -1          # unknown mode
    no_init = list(ptr)
    no_init[2] = None                                                # init_centroids
    assert L.adacluster_cluster_k(ctypes.byref(sh), ctypes.byref(adc.KParams(16, 64, 5, 1.5, 2, 2, 0)),
                                  *no_init, ctypes.c_void_p(16), 1 << 40, None) == -1
    # the warm mode needs no multi-stage state
    ws = L.adacluster_cluster_k_workspace
    assert 0 < ws(ctypes.byref(sh), ctypes.byref(adc.KParams(16, 64, 5, 1.5, 2, 2, 0))) \
        < ws(ctypes.byref(sh), ctypes.byref(adc.KParams(16, 64, 5, 1.5, 1, 1, 0)))


def test_select_and_attn_parameter_checks():
    L = adc.lib()
    sh = _shape()
    P = ctypes.c_void_p(16)

    def sel(score=0, rule=0, top_p=0.9, top_k=4, scale=0.125, q_off=P, pairs=P):
        return L.adacluster_select(ctypes.byref(sh), 32, 64, P, q_off, P, P, P, P, P, P, score, rule,
                                   top_p, top_k, scale, P, P, pairs, P, 1 << 40, None)
    assert sel(q_off=None) == -1          # sel_pairs needs q_offsets
    assert sel(top_p=0.0) == -1
    assert sel(top_p=1.5) == -1
    assert sel(rule=1, top_k=0) == -1
    assert sel(score=5) == -1
    assert sel(scale=-1.0) == -1

    def attn(Cq=32, Ck=64, scale=0.125, ws=1 << 40, odt=0, shape=sh):
        return L.adacluster_sparse_attn(ctypes.byref(shape), Cq, Ck, P, P, P, P, P, P, P, scale, P,
                                        odt, P, P, ws, None)
    assert attn(Cq=0) == -2
    assert attn(Ck=10000) == -2
    assert attn(scale=float("inf")) == -1
    assert attn(ws=1) == -4
    assert attn(odt=5) == -3
    assert attn(odt=adc.ADC_BF16, shape=_shape(dt=adc.ADC_F32)) == -3


def test_cluster_k_trace_checks():
    L = adc.lib()
    sh = _shape()
    P = ctypes.c_void_p(16)
    rec = adc.KTrace(16, 16, 16, 16, 16)

    def call(kp, trace=True):
        return L.adacluster_cluster_k_trace(ctypes.byref(sh), ctypes.byref(kp), *([P] * 15),
                                            ctypes.byref(rec) if trace else None, P, 1 << 40, None)
    assert call(adc.KParams(16, 64, 5, 1.5, 1, 1, 0), trace=False) == -1  # no record
    assert call(adc.KParams(16, 64, 5, 1.5, 0, 1, 0)) == -6               # FIXED has no stages
    assert call(adc.KParams(64, 32, 5, 1.5, 1, 1, 0)) == -2               # Nmax < m0


def test_binding_refuses_cpu_tensors():
    import torch
    q = torch.zeros(1, 1, 128, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        adc.cluster_q(q, 4)
