"""The full-size references (tests/fullsize_ref.py) against the oracle called
directly, on small problems: composing the oracle over key pieces with the exact
LSE merge, skipping pieces whose mask is empty, gives the same O, LSE, dQ, dK and
dV as the dense oracle over every key (BDLM rank shares, varlen documents and
core-attention tasks), with pieces smaller than the problems so that every path
of the composition runs."""
import numpy as np
import pytest

import fullsize_ref as fr
import oracle
from masked_long_context_amd import workloads as wl

TOL = 1e-12


def _direct(v):
    o, lse = oracle.attention_fwd(v["q"], v["k"], v["v"], v["mask"], v["scale"])
    D = oracle.delta_rows(o, v["dout"])
    dq, dk, dv = oracle.attention_bwd(v["q"], v["k"], v["v"], v["dout"], lse, D, v["mask"], v["scale"])
    return o, lse, D, dq, dk, dv


def _close(a, b):
    a, b = np.asarray(a), np.asarray(b)
    assert np.array_equal(np.isneginf(a), np.isneginf(b))
    fin = np.isfinite(b)
    assert np.abs(a[fin] - b[fin]).max() <= TOL


def _views():
    bd = wl.small_bdlm_config(1024, 16, 4, 1, 8, 2, 64, 4)
    yield "bdlm", fr.bdlm_group0(bd, wl.bdlm_inputs(bd, seed=0))
    vc = wl.VarlenConfig("v", (0, 70, 1, 300, 129), 4, 2, 64, True, 1.0, "")
    yield "varlen", fr.varlen_group0(vc, wl.varlen_inputs(vc, seed=1))
    q_cu, k_cu = [0, 40, 45, 200], [0, 90, 95, 260]
    inp = wl.task_inputs(200, 260, 4, 2, 64, seed=2)
    v = dict(q=fr.f64(inp["q"][:, :2]), dout=fr.f64(inp["dout"][:, :2]), k=fr.f64(inp["k"][:, :1]),
             v=fr.f64(inp["v"][:, :1]), mask=oracle.task_mask_fn(q_cu, k_cu, True), scale=0.125, G=2)
    yield "tasks", v


@pytest.mark.parametrize("name,view", list(_views()), ids=lambda x: x if isinstance(x, str) else "")
def test_piecewise_references_equal_the_dense_oracle(name, view):
    v = view
    o, lse, D, dq, dk, dv = _direct(v)
    n = v["q"].shape[0]
    for piece in (37, 100):
        rows = np.arange(0, n, 3)
        r, o2, l2, dq2 = fr.rows_reference(v["q"], v["k"], v["v"], v["dout"], v["mask"], v["scale"], rows, piece=piece)
        _close(o2, o[r]); _close(l2, lse[:, r]); _close(dq2, dq[r])
        L2, D2 = fr.lse_delta_all_rows(v["q"], v["k"], v["v"], v["dout"], v["mask"], v["scale"], n, piece=piece)
        _close(L2, lse); _close(D2, D)
        O3, L3, DQ3, DK3, DV3 = fr.group_reference(v["q"], v["k"], v["v"], v["dout"], v["mask"], v["scale"],
                                                   piece=piece)
        for a, b in ((O3, o), (L3, lse), (DQ3, dq), (DK3, dk), (DV3, dv)):
            _close(a, b)
        keys = np.unique(np.r_[0, v["k"].shape[0] - 1, np.arange(3, v["k"].shape[0], 11)])
        DK4, DV4 = fr.keys_reference(v["q"], v["k"], v["v"], v["dout"], lse, D, v["mask"], v["scale"], keys)
        _close(DK4, dk[keys]); _close(DV4, dv[keys])


def test_spread_keys_cover_every_stratum():
    k = fr.spread_keys(100, 1100, 50, seed=3)
    assert k.size == 50 and k.min() >= 100 and k.max() < 1100
    edges = np.linspace(100, 1100, 51)
    assert np.all(np.histogram(k, edges)[0] == 1)
