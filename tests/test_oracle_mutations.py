"""The oracle's pins have teeth: plausible mistakes planted in a COPY of the
oracle's source (on the CPU) must each make at least one pin fail."""
import inspect
import os
import types

import numpy as np
import pytest

import oracle.bdlm_attention as real
import test_oracle as pins

SRC = inspect.getsource(real)

# (name, text in the oracle, planted replacement)
MUTATIONS = [
    ("corrupted_sees_own_clean_block", "corr_clean = (~rc) & kc & (key_block[None, :] < row_block[:, None])",
     "corr_clean = (~rc) & kc & (key_block[None, :] <= row_block[:, None])"),
    ("clean_excludes_own_block", "clean_clean = rc & kc & (key_block[None, :] <= row_block[:, None])",
     "clean_clean = rc & kc & (key_block[None, :] < row_block[:, None])"),
    ("corrupted_sees_all_corrupted", "corr_corr = (~rc) & (~kc) & (key_slot[None, :] == row_slot[:, None])",
     "corr_corr = (~rc) & (~kc)"),
    ("query_offset_dropped", "(q_clean_offset + rows) // B", "rows // B"),
    ("kv_offset_dropped", "(kv_clean_offset + keys) // B", "keys // B"),
    ("gqa_mapping_modulo", "g = h // G", "g = h % hkv"),
    ("fwd_scale_dropped", "s = scale * (q[rr, h, :] @ k[:, g, :].T)", "s = (q[rr, h, :] @ k[:, g, :].T)"),
    ("lse_max_dropped", "l = np.where(has, mx_safe + np.log(", "l = np.where(has, 0.0 + np.log("),
    ("delta_dropped", "ds = p * (dp - delta[h, sl][:, None])", "ds = p * dp"),
    ("dk_scale_dropped", "dk[:, g, :] += scale * (ds.T @ q[rr, h, :])", "dk[:, g, :] += (ds.T @ q[rr, h, :])"),
    ("dv_wrong_operand", "dv[:, g, :] += p.T @ dout[rr, h, :]", "dv[:, g, :] += ds.T @ dout[rr, h, :]"),
    ("dq_wrong_sign", "dq[sl, h, :] = scale * (ds @ kk[:, g, :])", "dq[sl, h, :] = -scale * (ds @ kk[:, g, :])"),
    ("merge_unnormalised", "coef = np.where(has[None], np.exp(lse_parts - np.where(has, lse, 0.0)[None]), 0.0)",
     "coef = np.where(has[None], np.exp(lse_parts - m_safe[None]), 0.0)"),
    ("merge_lse_max_dropped", "lse = np.where(has, m_safe + np.log(np.where(has, tot, 1.0)), NEG_INF)",
     "lse = np.where(has, np.log(np.where(has, tot, 1.0)), NEG_INF)"),
    ("varlen_strict_causal", "m &= keys[None, :] <= rows[:, None]", "m &= keys[None, :] < rows[:, None]"),
    ("delta_transposed_heads", 'np.einsum("nhd,nhd->hn"', 'np.einsum("nhd,nhd->nh"'),
    ("combined_corrupted_sees_own_clean_block", "xc = ~rc[:, None] & kc[None, :] & (kb[None, :] < rb[:, None])",
     "xc = ~rc[:, None] & kc[None, :] & (kb[None, :] <= rb[:, None])"),
    ("combined_corrupted_sees_earlier_corrupted", "xx = ~rc[:, None] & ~kc[None, :] & (kb[None, :] == rb[:, None])",
     "xx = ~rc[:, None] & ~kc[None, :] & (kb[None, :] <= rb[:, None])"),
    ("combined_position_not_wrapped", "rb, kb = (rows % L) // B, (keys % L) // B", "rb, kb = rows // B, keys // B"),
    ("task_top_left_causal", "limit = kc[tr] + k_len - q_len + (rows - qc[tr]) + 1",
     "limit = kc[tr] + (rows - qc[tr]) + 1"),
    ("task_strict_causal", "limit = kc[tr] + k_len - q_len + (rows - qc[tr]) + 1",
     "limit = kc[tr] + k_len - q_len + (rows - qc[tr])"),
    ("task_keys_not_offset", "limit = kc[tr] + k_len - q_len + (rows - qc[tr]) + 1",
     "limit = k_len - q_len + (rows - qc[tr]) + 1"),
]

PIN_FUNCS = [(n, f) for n, f in vars(pins).items() if n.startswith("test_") and callable(f)]


def _mutant(old, new):
    assert SRC.count(old) >= 1, old
    mod = types.ModuleType("oracle_mutant")
    mod.__file__ = real.__file__
    exec(compile(SRC.replace(old, new), "oracle_mutant", "exec"), mod.__dict__)
    return mod


def _run_pin(fn, mod):
    params = inspect.signature(fn).parameters
    marks = getattr(fn, "pytestmark", [])
    calls = [dict()]
    for mk in marks:
        if mk.name == "parametrize":
            names = [s.strip() for s in mk.args[0].split(",")]
            calls = [dict(zip(names, v if isinstance(v, tuple) else (v,))) for v in mk.args[1]]
    for kw in calls:
        fn(orc=mod, **{k: v for k, v in kw.items() if k in params})


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistake_is_caught(name, old, new):
    mod = _mutant(old, new)
    caught = []
    for pin_name, fn in PIN_FUNCS:
        if pin_name in ("test_pair_count_large_configs_sampled_rows",):
            continue   # slow; the small-config count pins cover the same code
        try:
            with np.errstate(all="ignore"):
                _run_pin(fn, mod)
        except Exception:       # AssertionError or a shape error both count as caught
            caught.append(pin_name)
            break
    assert caught, f"planted mistake {name!r} passed every pin"


def test_unmutated_copy_passes_every_pin():
    mod = _mutant("NEG_INF = -np.inf", "NEG_INF = -np.inf")
    for pin_name, fn in PIN_FUNCS:
        if pin_name == "test_pair_count_large_configs_sampled_rows":
            continue
        _run_pin(fn, mod)
