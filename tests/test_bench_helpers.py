"""bench.py's host-side helpers (CPU): the parity report's tolerance rule against the
oracle's values, and the achieved-bandwidth arithmetic of the bandwidth-bound calls."""
import os
import sys

import numpy as np
import torch

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import bench  # noqa: E402


def _case(seed=0, n=64, hq=4, d=32, whole=True):
    rng = np.random.default_rng(seed)
    rows = np.sort(rng.choice(n, 16, replace=False)) if not whole else np.arange(n)
    G = 2
    ref = dict(rows=rows, G=G, o=rng.standard_normal((rows.size, G, d)), lse=rng.standard_normal((G, rows.size)),
               dq=rng.standard_normal((rows.size, G, d)), dk=None, dv=None)
    if whole:
        ref["dk"] = rng.standard_normal((n, 1, d))
        ref["dv"] = rng.standard_normal((n, 1, d))
    # "GPU" outputs holding the reference values exactly in the sampled rows / group
    o = torch.zeros((n, hq, d), dtype=torch.float64)
    dq = torch.zeros_like(o)
    lse = torch.zeros((hq, n), dtype=torch.float64)
    o[rows, :G] = torch.from_numpy(ref["o"])
    dq[rows, :G] = torch.from_numpy(ref["dq"])
    lse[:G, rows] = torch.from_numpy(ref["lse"])
    dk = torch.from_numpy(ref["dk"]).clone() if whole else None
    dv = torch.from_numpy(ref["dv"]).clone() if whole else None
    return ref, o, lse, dq, dk, dv


def test_exact_outputs_are_within_tolerance():
    for whole in (True, False):
        ref, o, lse, dq, dk, dv = _case(whole=whole)
        rep = bench.parity_report(ref, o, lse, dq, dk, dv)
        assert rep["within_tolerance"], rep
        assert rep["o"]["max_abs"] == 0.0 and rep["o"]["element_bound_ratio"] == 0.0
        assert ("dk" in rep) == whole


def test_one_element_beyond_either_bound_fails():
    ref, o, lse, dq, dk, dv = _case()
    r, h = int(ref["rows"][3]), 1
    # 2.5e-2 on an element of magnitude <= 4: inside 2e-2 + 5e-3 |x| for |x| >= 1, but
    # above the plain 2e-2 that elements with |x| <= 4 are held to
    x = float(o[r, h, 5])
    assert abs(x) <= 4.0
    o[r, h, 5] += 2.5e-2
    rep = bench.parity_report(ref, o, lse, dq, dk, dv)
    assert rep["o"]["max_abs_where_abs_ref_le_4"] >= 2.4e-2 and not rep["within_tolerance"]
    # a large element off by 0.045: within 2e-2 + 5e-3 |x| only when |x| >= 5
    ref, o, lse, dq, dk, dv = _case()
    dk[7, 0, 3] = torch.tensor(6.0, dtype=torch.float64)
    ref["dk"][7, 0, 3] = 6.0
    dk[7, 0, 3] += 0.045
    rep = bench.parity_report(ref, o, lse, dq, dk, dv)
    assert rep["within_tolerance"], rep   # 0.045 <= 2e-2 + 3e-2
    dk[7, 0, 3] += 0.02
    assert not bench.parity_report(ref, o, lse, dq, dk, dv)["within_tolerance"]
    # the LSE bound and the -inf pattern
    ref, o, lse, dq, dk, dv = _case()
    lse[0, int(ref["rows"][0])] += 2e-5
    assert not bench.parity_report(ref, o, lse, dq, dk, dv)["within_tolerance"]
    ref, o, lse, dq, dk, dv = _case()
    ref["lse"][1, 2] = -np.inf
    assert not bench.parity_report(ref, o, lse, dq, dk, dv)["lse_neginf_match"]


def test_aux_bandwidth_arithmetic():
    tot = {"prepare": (2.0, 4), "cast": (1.0, 4)}
    out = bench.aux_bandwidth(tot, steps=2, rows=1000, h=8, d=128)
    # preprocess: 10d + 4 bytes per (row, head) in 1 ms per step
    assert out["prepare_ms"] == 1.0
    assert abs(out["prepare_gbs"] - 1000 * 8 * (10 * 128 + 4) / 1e-3 / 1e9) < 0.1
    assert abs(out["cast_gbs"] - 1000 * 8 * 6 * 128 / 0.5e-3 / 1e9) < 0.1
    assert out["finalize_ms"] == 0.0 and "finalize_gbs" not in out
