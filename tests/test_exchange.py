"""Per-rank exchange and work accounting of CSBP and conventional context
parallelism against the oracle's mask over the whole combined sequence (CPU)."""
import numpy as np
import pytest

import oracle
from masked_long_context_amd import exchange as E
from masked_long_context_amd import workloads as wl


def _rows(L, B, R, r, scheme):
    n, nb = L // R, L // B
    owned = wl.zigzag_owned_blocks(nb, R, r) if scheme == "csbp" else wl.cp_owned_blocks(nb, R, r)
    corr = (L + owned[:, None] * B + np.arange(B)[None, :]).reshape(-1)
    return np.concatenate([r * n + np.arange(n), corr])


@pytest.mark.parametrize("L,B,R", [(96, 4, 2), (128, 8, 4), (256, 2, 8), (64, 1, 4)])
@pytest.mark.parametrize("scheme", ["csbp", "cp"])
def test_exchange_matches_combined_mask(L, B, R, scheme):
    full = oracle.combined_mask(L, B)
    n = L // R
    h_kv, d = 2, 64
    chunk = n * h_kv * d * 2 * 2
    total = 0
    for r in range(R):
        x = E.rank_exchange(L, B, R, r, h_kv, d, scheme)
        rows = _rows(L, B, R, r, scheme)
        m = full[rows]
        assert x.pairs == int(m.sum())
        total += x.pairs
        clean_needed = [s for s in range(R) if s != r and m[:, s * n:(s + 1) * n].any()]
        # the only corrupted keys a rank attends are those of its own blocks (local in both schemes)
        attended_corr = L + np.nonzero(m[:, L:].any(axis=0))[0]
        assert set(attended_corr.tolist()) <= set(rows[n:].tolist())
        assert x.remote_clean_needed == len(clean_needed)
        assert x.kv_bytes_needed == len(clean_needed) * chunk
        if scheme == "csbp":
            assert x.kv_bytes_received == x.kv_bytes_needed
        else:                                         # every remote chunk of both copies
            assert x.kv_bytes_received == (R - 1) * 2 * chunk
    assert total == int(full.sum())


def test_compare_schemes_summary():
    c = E.compare_schemes(128, 8, 4, 2, 64)
    for scheme in ("csbp", "cp"):
        rs = c["ranks"][scheme]
        s = c["summary"][scheme]
        pr = np.array([x.pairs for x in rs])
        assert s["busiest_rank"] == int(pr.argmax())
        assert s["kv_bytes_received_total"] == sum(x.kv_bytes_received for x in rs)
    assert c["summary"]["cp"]["kv_bytes_received_total"] > c["summary"]["csbp"]["kv_bytes_received_total"]


def test_rank_exchange_rejects_ragged_chunks():
    with pytest.raises(ValueError):
        E.rank_exchange(100, 8, 4, 0, 1, 64, "cp")
    with pytest.raises(ValueError):
        E.rank_exchange(128, 8, 4, 0, 1, 64, "ring")
