"""Pins of the fp64 oracle to facts other than itself.

Each test ties one part of the oracle to something it does not compute: a
hand-derived mask fixture, closed-form counts and values, textbook/library
routines in special cases, finite differences, exactness of the LSE merge
and the separability of the BDLM objective over target blocks.
"""
import math
import os

import numpy as np
import pytest
import torch

import oracle as _oracle_module
from masked_long_context_amd import workloads as wl

@pytest.fixture
def orc():
    return _oracle_module


GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "bdlm_mask_small.txt")


def _parse_golden():
    cases, cur, in_mask = [], None, False
    for raw in open(GOLDEN):
        line = raw.strip()
        if not line or line.startswith("#"):
            continue
        if line.startswith("case "):
            cur = {"name": line.split()[1], "rows": []}
            continue
        if line == "mask":
            in_mask = True
            continue
        if line == "end":
            cur["mask"] = np.array([[c == "1" for c in r] for r in cur.pop("rows")])
            cases.append(cur)
            cur, in_mask = None, False
            continue
        if in_mask:
            cur["rows"].append(line)
        else:
            key, *vals = line.split()
            cur[key] = [int(v) for v in vals] if key == "owned_blocks" else int(vals[0])
    return cases


@pytest.mark.parametrize("case", _parse_golden(), ids=lambda c: c["name"])
def test_mask_matches_hand_derived_fixture(case, orc):
    m = orc.bdlm_mask(case["clean_len"], case["block_size"], case["q_clean_offset"],
                         case["q_clean_len"], case["owned_blocks"], case["kv_clean_offset"],
                         case["kv_clean_len"], bool(case["with_local_corrupt"]))
    assert m.shape == case["mask"].shape
    assert np.array_equal(m, case["mask"])


# ----------------------------------------------------------------------------- helpers

def _np(t):
    return t.to(torch.float64).numpy()


def _rand_problem(rng, L=None, B=None):
    B = B or int(rng.choice([1, 2, 4, 8]))
    nb = int(L // B) if L else int(rng.integers(2, 9))
    L = nb * B
    q0b = int(rng.integers(0, nb))
    qnb = int(rng.integers(0, nb - q0b + 1))
    owned = rng.permutation(nb)[: int(rng.integers(0, nb + 1))]
    k0b = int(rng.integers(0, nb))
    knb = int(rng.integers(0, nb - k0b + 1))
    return dict(clean_len=L, block_size=B, q_clean_offset=q0b * B, q_clean_len=qnb * B,
                owned_blocks=[int(x) for x in owned], kv_clean_offset=k0b * B,
                kv_clean_len=knb * B, with_local_corrupt=bool(rng.integers(0, 2)))


def _legal_keys_prefix_form(p, row):
    """Legal keys of one row written as index ranges (not as the block predicate):
    a clean row at position x sees clean keys up to the end of its block; a corrupted
    block b sees clean keys below b*B and its own B corrupted rows."""
    B = p["block_size"]
    lo, n = p["kv_clean_offset"], p["kv_clean_len"]
    if row < p["q_clean_len"]:
        hi = (p["q_clean_offset"] + row) // B * B + B
        own = []
    else:
        slot = (row - p["q_clean_len"]) // B
        hi = p["owned_blocks"][slot] * B
        own = list(range(n + slot * B, n + slot * B + B)) if p["with_local_corrupt"] else []
    clean = list(range(0, max(0, min(hi, lo + n) - lo)))
    return clean + own


def _mask_of(p, orc):
    return orc.bdlm_mask(p["clean_len"], p["block_size"], p["q_clean_offset"], p["q_clean_len"],
                            p["owned_blocks"], p["kv_clean_offset"], p["kv_clean_len"],
                            p["with_local_corrupt"])


def _mask_fn_of(p, orc):
    return orc.bdlm_mask_fn(p["clean_len"], p["block_size"], p["q_clean_offset"],
                               p["q_clean_len"], p["owned_blocks"], p["kv_clean_offset"],
                               p["kv_clean_len"], p["with_local_corrupt"])


def test_mask_equals_prefix_ranges_random(orc):
    rng = np.random.default_rng(1)
    for _ in range(200):
        p = _rand_problem(rng)
        m = _mask_of(p, orc)
        for r in range(m.shape[0]):
            want = np.zeros(m.shape[1], bool)
            want[_legal_keys_prefix_form(p, r)] = True
            assert np.array_equal(m[r], want), (p, r)


def _closed_form_pairs(L, B, q_off, q_len, owned):
    """Clean block c (B rows) sees (c+1)B keys; corrupted block b sees bB + B keys."""
    tot = 0
    for c in range(q_off // B, (q_off + q_len) // B):
        tot += B * (c + 1) * B
    for b in owned:
        tot += B * b * B + B * B
    return tot


@pytest.mark.parametrize("idx,expected", [(1, 73728), (2, 17039360)])
def test_pair_count_small_configs(idx, expected, orc):
    p = wl.config(idx).problem
    mf = orc.bdlm_mask_fn(p.clean_len, p.block_size, p.q_clean_offset, p.q_clean_len,
                             p.owned_blocks, 0, p.clean_len, True)
    n = orc.count_pairs(mf, p.n_q, p.clean_len + p.n_corr)
    assert n == expected
    assert n == _closed_form_pairs(p.clean_len, p.block_size, p.q_clean_offset, p.q_clean_len,
                                   p.owned_blocks)


@pytest.mark.parametrize("idx,expected", [(3, 4429709312), (5, 146030985216)])
def test_pair_count_large_configs_sampled_rows(idx, expected, orc):
    """Closed form of the whole rank share, and the mask's per-row count on sampled rows."""
    p = wl.config(idx).problem
    B = p.block_size
    assert _closed_form_pairs(p.clean_len, B, p.q_clean_offset, p.q_clean_len,
                              p.owned_blocks) == expected
    rng = np.random.default_rng(idx)
    rows = np.sort(rng.choice(p.n_q, 24, replace=False))
    m = orc.bdlm_mask(p.clean_len, B, p.q_clean_offset, p.q_clean_len, p.owned_blocks,
                         0, p.clean_len, True, rows=rows)
    for r, cnt in zip(rows, m.sum(axis=1)):
        if r < p.q_clean_len:
            want = ((p.q_clean_offset + r) // B + 1) * B
        else:
            want = p.owned_blocks[(r - p.q_clean_len) // B] * B + B
        assert cnt == want


def test_zigzag_balances_work(orc):
    """Early+late pairing gives every rank the same number of useful pairs."""
    L, B, R = 4096, 16, 8
    nb = L // B
    works = []
    for r in range(R):
        owned = wl.zigzag_owned_blocks(nb, R, r)
        works.append(sum(B * b * B + B * B for b in owned))
    assert len(set(works)) == 1
    allb = np.sort(np.concatenate([wl.zigzag_owned_blocks(nb, R, r) for r in range(R)]))
    assert np.array_equal(allb, np.arange(nb))


# ----------------------------------------------------------------------------- values

def _rand_qkv(rng, nq, nk, hq, hkv, d, scale=1.0):
    q = rng.standard_normal((nq, hq, d)) * scale
    k = rng.standard_normal((nk, hkv, d)) * scale
    v = rng.standard_normal((nk, hkv, d))
    return q, k, v


def test_zero_query_gives_uniform_average(orc):
    """Q = 0: softmax is uniform over the legal keys -> LSE = ln n_i, O = mean of legal V."""
    rng = np.random.default_rng(2)
    for _ in range(30):
        p = _rand_problem(rng)
        nq = p["q_clean_len"] + len(p["owned_blocks"]) * p["block_size"]
        nk = p["kv_clean_len"] + (len(p["owned_blocks"]) * p["block_size"] if p["with_local_corrupt"] else 0)
        if nq == 0:
            continue
        _, k, v = _rand_qkv(rng, nq, nk, 2, 1, 3)
        q = np.zeros((nq, 2, 3))
        o, lse = orc.attention_fwd(q, k, v, _mask_fn_of(p, orc), 0.7)
        for r in range(nq):
            keys = _legal_keys_prefix_form(p, r)
            for h in range(2):
                if not keys:
                    assert lse[h, r] == -np.inf and np.all(o[r, h] == 0)
                else:
                    assert abs(lse[h, r] - math.log(len(keys))) < 1e-12
                    assert np.allclose(o[r, h], v[keys, 0].mean(axis=0), atol=1e-12)


def test_constant_values_pass_through(orc):
    rng = np.random.default_rng(3)
    p = _rand_problem(rng, L=32, B=4)
    p["owned_blocks"] = [5, 2, 7]
    p["with_local_corrupt"] = True
    nq = p["q_clean_len"] + 12
    nk = p["kv_clean_len"] + 12
    q, k, _ = _rand_qkv(rng, nq, nk, 4, 2, 8)
    c = rng.standard_normal(8)
    v = np.broadcast_to(c, (nk, 2, 8)).copy()
    o, lse = orc.attention_fwd(q, k, v, _mask_fn_of(p, orc), 0.35)
    for r in range(nq):
        for h in range(4):
            if np.isfinite(lse[h, r]):
                assert np.allclose(o[r, h], c, atol=1e-12)


def _sdpa(q, k, v, causal, scale):
    """Library reference: torch CPU fp64 scaled_dot_product_attention, [N,H,d] layout."""
    G = q.shape[1] // k.shape[1]
    qt = torch.from_numpy(q).permute(1, 0, 2).contiguous()
    kt = torch.from_numpy(np.repeat(k, G, axis=1)).permute(1, 0, 2).contiguous()
    vt = torch.from_numpy(np.repeat(v, G, axis=1)).permute(1, 0, 2).contiguous()
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=causal, scale=scale)
    return o.permute(1, 0, 2).numpy()


def test_block_size_one_is_token_causal_attention(orc):
    rng = np.random.default_rng(4)
    L, hq, hkv, d = 40, 4, 2, 16
    q, k, v = _rand_qkv(rng, L + 5, L + 5, hq, hkv, d)
    mf = orc.bdlm_mask_fn(L, 1, 0, L, [3, 17, 30, 31, 9], 0, L, True)
    o, _ = orc.attention_fwd(q, k, v, mf, 0.25)
    ref = _sdpa(q[:L], k[:L], v[:L], True, 0.25)
    assert np.allclose(o[:L], ref, atol=1e-12)


def test_block_size_L_is_full_attention_and_block0_sees_only_itself(orc):
    rng = np.random.default_rng(5)
    L, hq, hkv, d = 24, 2, 2, 8
    q, k, v = _rand_qkv(rng, 2 * L, 2 * L, hq, hkv, d)
    mf = orc.bdlm_mask_fn(L, L, 0, L, [0], 0, L, True)
    o, _ = orc.attention_fwd(q, k, v, mf, 0.3)
    assert np.allclose(o[:L], _sdpa(q[:L], k[:L], v[:L], False, 0.3), atol=1e-12)
    assert np.allclose(o[L:], _sdpa(q[L:], k[L:], v[L:], False, 0.3), atol=1e-12)


def test_softmax_rows_sum_to_one_and_vanish_off_mask(orc):
    rng = np.random.default_rng(6)
    for _ in range(20):
        p = _rand_problem(rng)
        nq = p["q_clean_len"] + len(p["owned_blocks"]) * p["block_size"]
        nk = p["kv_clean_len"] + (len(p["owned_blocks"]) * p["block_size"] if p["with_local_corrupt"] else 0)
        if nq == 0:
            continue
        q, k, _ = _rand_qkv(rng, nq, nk, 2, 2, 4, scale=2.0)
        m = _mask_of(p, orc)
        for h in range(2):
            P = orc.softmax_probs(q, k, _mask_fn_of(p, orc), 0.5, h)
            has = m.any(axis=1)
            assert np.all(np.abs(P.sum(axis=1)[has] - 1.0) < 1e-12)
            assert np.all(P[~m] == 0.0)


def _brute_force(q, k, v, dout, mask, scale):
    """Scalar loops over the definitions (math module only)."""
    nq, hq, d = q.shape
    nk, hkv, _ = k.shape
    G = hq // hkv
    O = np.zeros_like(q)
    LSE = np.full((hq, nq), -np.inf)
    dQ = np.zeros_like(q)
    dK = np.zeros_like(k)
    dV = np.zeros_like(v)
    for h in range(hq):
        g = h // G
        for i in range(nq):
            legal = [j for j in range(nk) if mask[i, j]]
            if not legal:
                continue
            s = {j: scale * sum(q[i, h, c] * k[j, g, c] for c in range(d)) for j in legal}
            mx = max(s.values())
            z = sum(math.exp(s[j] - mx) for j in legal)
            LSE[h, i] = mx + math.log(z)
            p = {j: math.exp(s[j] - LSE[h, i]) for j in legal}
            for c in range(d):
                O[i, h, c] = sum(p[j] * v[j, g, c] for j in legal)
            Di = sum(dout[i, h, c] * O[i, h, c] for c in range(d))
            for j in legal:
                dp = sum(dout[i, h, c] * v[j, g, c] for c in range(d))
                ds = p[j] * (dp - Di)
                for c in range(d):
                    dV[j, g, c] += p[j] * dout[i, h, c]
                    dQ[i, h, c] += scale * ds * k[j, g, c]
                    dK[j, g, c] += scale * ds * q[i, h, c]
    return O, LSE, dQ, dK, dV


def test_vectorized_equals_scalar_loops(orc):
    rng = np.random.default_rng(7)
    p = dict(clean_len=12, block_size=3, q_clean_offset=3, q_clean_len=6, owned_blocks=[2, 0, 3],
             kv_clean_offset=0, kv_clean_len=12, with_local_corrupt=True)
    nq, nk = 6 + 9, 12 + 9
    q, k, v = _rand_qkv(rng, nq, nk, 4, 2, 5)
    dout = rng.standard_normal(q.shape)
    m = _mask_of(p, orc)
    O, LSE, dQ, dK, dV = _brute_force(q, k, v, dout, m, 0.6)
    o, lse = orc.attention_fwd(q, k, v, _mask_fn_of(p, orc), 0.6, row_block=4)
    D = orc.delta_rows(o, dout)
    dq, dk, dv = orc.attention_bwd(q, k, v, dout, lse, D, _mask_fn_of(p, orc), 0.6, row_block=4)
    for a, b in [(o, O), (lse, LSE), (dq, dQ), (dk, dK), (dv, dV)]:
        assert np.allclose(a, b, atol=1e-12, rtol=1e-12)


def test_gradients_match_central_finite_differences(orc):
    rng = np.random.default_rng(8)
    p = dict(clean_len=8, block_size=2, q_clean_offset=2, q_clean_len=4, owned_blocks=[3, 1],
             kv_clean_offset=0, kv_clean_len=8, with_local_corrupt=True)
    nq, nk = 8, 12
    q, k, v = _rand_qkv(rng, nq, nk, 2, 1, 3)
    dout = rng.standard_normal(q.shape)
    mf = _mask_fn_of(p, orc)
    scale = 0.8

    def loss(q_, k_, v_):
        o_, _ = orc.attention_fwd(q_, k_, v_, mf, scale)
        return float((o_ * dout).sum())

    o, lse = orc.attention_fwd(q, k, v, mf, scale)
    dq, dk, dv = orc.attention_bwd(q, k, v, dout, lse, orc.delta_rows(o, dout), mf, scale)
    eps = 1e-6
    for arr, grad, which in [(q, dq, 0), (k, dk, 1), (v, dv, 2)]:
        num = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            ap = arr.copy(); ap[idx] += eps
            am = arr.copy(); am[idx] -= eps
            args_p = [q, k, v]; args_p[which] = ap
            args_m = [q, k, v]; args_m[which] = am
            num[idx] = (loss(*args_p) - loss(*args_m)) / (2 * eps)
        err = np.linalg.norm(num - grad) / max(np.linalg.norm(grad), 1e-30)
        assert err < 1e-6, (which, err)


# ----------------------------------------------------------------------------- merge

def test_merge_closed_forms(orc):
    rng = np.random.default_rng(9)
    o1 = rng.standard_normal((5, 2, 4))
    o2 = rng.standard_normal((5, 2, 4))
    l = rng.uniform(0, 10, (2, 5))
    o, lse = orc.lse_merge(np.stack([o1, o2]), np.stack([l, l]))
    assert np.allclose(lse, l + math.log(2), atol=1e-13)
    assert np.allclose(o, (o1 + o2) / 2, atol=1e-13)
    ninf = np.full((2, 5), -np.inf)
    o, lse = orc.lse_merge(np.stack([o1, o2]), np.stack([l, ninf]))
    assert np.allclose(o, o1, atol=1e-13) and np.allclose(lse, l, atol=1e-13)
    o, lse = orc.lse_merge(np.stack([o1, o2]), np.stack([ninf, ninf]))
    assert np.all(o == 0) and np.all(lse == -np.inf)


def _split_points(rng, nb, B, n_parts):
    cuts = np.sort(rng.integers(0, nb + 1, n_parts - 1)) * B
    return np.concatenate([[0], cuts, [nb * B]])


def test_sharded_merge_equals_unsharded_fwd_and_bwd(orc):
    rng = np.random.default_rng(10)
    for trial in range(6):
        B = int(rng.choice([2, 4]))
        nb = 10
        L = nb * B
        owned = [int(x) for x in rng.permutation(nb)[:4]]
        prob = dict(clean_len=L, block_size=B, q_clean_offset=4 * B, q_clean_len=3 * B,
                    owned_blocks=owned, scale=0.4)
        nq = 3 * B + 4 * B
        q, _, _ = _rand_qkv(rng, nq, 1, 4, 2, 6)
        kc, vc = rng.standard_normal((L, 2, 6)), rng.standard_normal((L, 2, 6))
        kx, vx = rng.standard_normal((4 * B, 2, 6)), rng.standard_normal((4 * B, 2, 6))
        dout = rng.standard_normal(q.shape)
        full = dict(prob, kv_clean_offset=0, kv_clean_len=L, with_local_corrupt=True)
        o_ref, lse_ref = orc.bdlm_fwd(full, q, kc, vc, kx, vx)
        D = orc.delta_rows(o_ref, dout)
        dq_ref, dk_ref, dv_ref = orc.bdlm_bwd(full, q, kc, vc, kx, vx, dout, lse_ref, D)

        cuts = _split_points(rng, nb, B, 4)          # may contain empty shards
        local = int(rng.integers(0, 4))
        parts_o, parts_l = [], []
        dq = np.zeros_like(q)
        dk = np.zeros((L + 4 * B, 2, 6))
        dv = np.zeros_like(dk)
        for s in range(4):
            a, b = int(cuts[s]), int(cuts[s + 1])
            pr = dict(prob, kv_clean_offset=a, kv_clean_len=b - a, with_local_corrupt=(s == local))
            o_s, l_s = orc.bdlm_fwd(pr, q, kc[a:b], vc[a:b], kx, vx)
            parts_o.append(o_s)
            parts_l.append(l_s)
        o_m, lse_m = orc.lse_merge(np.stack(parts_o), np.stack(parts_l))
        assert np.allclose(o_m, o_ref, atol=1e-12)
        assert np.allclose(lse_m, lse_ref, atol=1e-12)
        Dm = orc.delta_rows(o_m, dout)
        for s in range(4):
            a, b = int(cuts[s]), int(cuts[s + 1])
            pr = dict(prob, kv_clean_offset=a, kv_clean_len=b - a, with_local_corrupt=(s == local))
            dq_s, dk_s, dv_s = orc.bdlm_bwd(pr, q, kc[a:b], vc[a:b], kx, vx, dout, lse_m, Dm)
            dq += dq_s
            dk[a:b] = dk_s[: b - a]
            dv[a:b] = dv_s[: b - a]
            if s == local:
                dk[L:] = dk_s[b - a:]
                dv[L:] = dv_s[b - a:]
        for a_, b_ in [(dq, dq_ref), (dk, dk_ref), (dv, dv_ref)]:
            assert np.allclose(a_, b_, atol=1e-12)


def test_objective_separates_over_target_blocks(orc):
    """Block parallelism: each corrupted block computed alone equals its rows of the joint
    run, and the clean K/V gradients are the sum over the clean stream and every block."""
    rng = np.random.default_rng(11)
    B, nb = 4, 8
    L = nb * B
    owned = [6, 1, 4]
    prob = dict(clean_len=L, block_size=B, q_clean_offset=2 * B, q_clean_len=3 * B, scale=0.5,
                kv_clean_offset=0, kv_clean_len=L, with_local_corrupt=True)
    nq = 3 * B + 3 * B
    q = rng.standard_normal((nq, 2, 5))
    kc, vc = rng.standard_normal((L, 1, 5)), rng.standard_normal((L, 1, 5))
    kx, vx = rng.standard_normal((3 * B, 1, 5)), rng.standard_normal((3 * B, 1, 5))
    dout = rng.standard_normal(q.shape)
    joint = dict(prob, owned_blocks=owned)
    o, lse = orc.bdlm_fwd(joint, q, kc, vc, kx, vx)
    D = orc.delta_rows(o, dout)
    dq, dk, dv = orc.bdlm_bwd(joint, q, kc, vc, kx, vx, dout, lse, D)

    # clean stream alone (no corrupted blocks)
    cs = dict(prob, owned_blocks=[])
    rows_c = slice(0, 3 * B)
    o_c, l_c = orc.bdlm_fwd(cs, q[rows_c], kc, vc, kx[:0], vx[:0])
    dq_c, dk_c, dv_c = orc.bdlm_bwd(cs, q[rows_c], kc, vc, kx[:0], vx[:0], dout[rows_c], l_c,
                                       orc.delta_rows(o_c, dout[rows_c]))
    assert np.allclose(o_c, o[rows_c], atol=1e-12) and np.allclose(dq_c, dq[rows_c], atol=1e-12)
    dk_sum = dk_c[:L].copy()
    dv_sum = dv_c[:L].copy()
    for m, b in enumerate(owned):
        rr = slice(3 * B + m * B, 3 * B + (m + 1) * B)
        one = dict(prob, owned_blocks=[b], q_clean_len=0)
        kxm, vxm = kx[m * B:(m + 1) * B], vx[m * B:(m + 1) * B]
        o_b, l_b = orc.bdlm_fwd(one, q[rr], kc, vc, kxm, vxm)
        assert np.allclose(o_b, o[rr], atol=1e-12) and np.allclose(l_b, lse[:, rr], atol=1e-12)
        dq_b, dk_b, dv_b = orc.bdlm_bwd(one, q[rr], kc, vc, kxm, vxm, dout[rr], l_b,
                                           orc.delta_rows(o_b, dout[rr]))
        assert np.allclose(dq_b, dq[rr], atol=1e-12)
        # corrupted K/V gradients stay with their block
        assert np.allclose(dk_b[L:], dk[L + m * B:L + (m + 1) * B], atol=1e-12)
        assert np.allclose(dv_b[L:], dv[L + m * B:L + (m + 1) * B], atol=1e-12)
        dk_sum += dk_b[:L]
        dv_sum += dv_b[:L]
    assert np.allclose(dk_sum, dk[:L], atol=1e-12) and np.allclose(dv_sum, dv[:L], atol=1e-12)


# ----------------------------------------------------------------------------- varlen

def test_varlen_equals_per_shard_causal_sdpa(orc):
    rng = np.random.default_rng(12)
    lens = [5, 1, 17, 9]
    cu = np.concatenate([[0], np.cumsum(lens)])
    T = int(cu[-1])
    q, k, v = _rand_qkv(rng, T, T, 4, 2, 8)
    o, lse = orc.varlen_fwd(q, k, v, cu, True, 0.3)
    for s in range(len(lens)):
        a, b = cu[s], cu[s + 1]
        assert np.allclose(o[a:b], _sdpa(q[a:b], k[a:b], v[a:b], True, 0.3), atol=1e-12)
    assert orc.varlen_mask(cu, True).sum() == sum(n * (n + 1) // 2 for n in lens)
    assert orc.varlen_mask(cu, False).sum() == sum(n * n for n in lens)


def test_varlen_config_lengths(orc):
    cfg = wl.config(4)
    assert cfg.total == 262144 and len(cfg.seqlens) == 27
    assert min(cfg.seqlens) >= 128 and max(cfg.seqlens) <= 65536
    assert sum(n * (n + 1) // 2 for n in cfg.seqlens) == 3214974270


# ----------------------------------------------------------------------------- core-attention tasks

def _chunk_tasks(doc_lens, chunk):
    """Documents split into query chunks of `chunk` rows; each task's keys are its
    document's prefix up to the chunk's end (built here, independent of any library
    scheduler).  Returns q_cu, k_cu and, per task key row, the document row it copies."""
    q_cu, k_cu, src = [0], [0], []
    start = 0
    for n in doc_lens:
        for c0 in range(0, n, chunk):
            c1 = min(n, c0 + chunk)
            q_cu.append(q_cu[-1] + (c1 - c0))
            k_cu.append(k_cu[-1] + c1)
            src.extend(range(start, start + c1))
        start += n
    return np.array(q_cu), np.array(k_cu), np.array(src, dtype=np.int64)


def test_task_mask_reduces_to_varlen(orc):
    cu = np.array([0, 3, 3, 10, 11, 30])
    for causal in (True, False):
        assert np.array_equal(orc.task_mask(cu, cu, causal), orc.varlen_mask(cu, causal))


def test_task_prefix_chunks_reproduce_document_causal_attention(orc):
    """Splitting each document into query chunks, each attending its document's
    prefix (bottom-right causal), composes to plain causal attention per document:
    O, LSE and dQ agree, and dK/dV summed back over the prefix copies agree."""
    rng = np.random.default_rng(21)
    doc_lens = [7, 13, 1, 20]
    cu = np.concatenate([[0], np.cumsum(doc_lens)])
    T = int(cu[-1])
    hq, hkv, d, scale = 4, 2, 8, 0.3
    q, k, v = _rand_qkv(rng, T, T, hq, hkv, d)
    dout = rng.standard_normal((T, hq, d))
    o_ref, lse_ref = orc.varlen_fwd(q, k, v, cu, True, scale)
    D = orc.delta_rows(o_ref, dout)
    dq_ref, dk_ref, dv_ref = orc.varlen_bwd(q, k, v, dout, lse_ref, D, cu, True, scale)
    for chunk in (1, 4, 6, 64):
        q_cu, k_cu, src = _chunk_tasks(doc_lens, chunk)
        kt, vt = k[src], v[src]
        o, lse = orc.task_fwd(q, kt, vt, q_cu, k_cu, True, scale)
        assert np.allclose(o, o_ref, atol=1e-12) and np.allclose(lse, lse_ref, atol=1e-12)
        dq, dkt, dvt = orc.task_bwd(q, kt, vt, dout, lse, D, q_cu, k_cu, True, scale)
        assert np.allclose(dq, dq_ref, atol=1e-12)
        dk = np.zeros_like(dk_ref)
        dv = np.zeros_like(dv_ref)
        np.add.at(dk, src, dkt)
        np.add.at(dv, src, dvt)
        assert np.allclose(dk, dk_ref, atol=1e-12) and np.allclose(dv, dv_ref, atol=1e-12)


def test_task_noncausal_is_full_attention_per_task(orc):
    rng = np.random.default_rng(22)
    q_lens, k_lens = [3, 9, 1, 5], [11, 2, 7, 5]
    q_cu = np.concatenate([[0], np.cumsum(q_lens)])
    k_cu = np.concatenate([[0], np.cumsum(k_lens)])
    q, k, v = _rand_qkv(rng, int(q_cu[-1]), int(k_cu[-1]), 4, 2, 8)
    o, _ = orc.task_fwd(q, k, v, q_cu, k_cu, False, 0.2)
    for t in range(len(q_lens)):
        a, b, c, e = q_cu[t], q_cu[t + 1], k_cu[t], k_cu[t + 1]
        assert np.allclose(o[a:b], _sdpa(q[a:b], k[c:e], v[c:e], False, 0.2), atol=1e-12)


def test_task_context_shorter_than_queries_leaves_leading_rows_empty(orc):
    """Bottom-right alignment with k_len < q_len: the first q_len - k_len rows see
    no key (O = 0, LSE = -inf); row q_len - k_len + i sees keys 0..i."""
    rng = np.random.default_rng(23)
    q_cu, k_cu = np.array([0, 6]), np.array([0, 4])
    q, k, v = _rand_qkv(rng, 6, 4, 2, 1, 8)
    m = orc.task_mask(q_cu, k_cu, True)
    assert not m[:2].any()
    for i in range(4):
        assert np.array_equal(m[2 + i], np.arange(4) <= i)
    o, lse = orc.task_fwd(q, k, v, q_cu, k_cu, True, 0.5)
    assert np.all(o[:2] == 0) and np.all(np.isneginf(lse[:, :2]))
    assert np.allclose(o[5], _sdpa(q[5:6], k, v, False, 0.5)[0], atol=1e-12)


def test_task_mask_matches_scalar_definition(orc):
    q_cu, k_cu = [0, 2, 2, 7, 8], [0, 5, 9, 12, 20]
    m = orc.task_mask(q_cu, k_cu, True)
    for i in range(q_cu[-1]):
        t = max(x for x in range(len(q_cu) - 1) if q_cu[x] <= i < q_cu[x + 1])
        ql, kl = q_cu[t + 1] - q_cu[t], k_cu[t + 1] - k_cu[t]
        for j in range(k_cu[-1]):
            legal = k_cu[t] <= j < k_cu[t + 1] and (j - k_cu[t]) <= kl - ql + (i - q_cu[t])
            assert m[i, j] == legal, (i, j)


# ----------------------------------------------------------------------------- combined sequence

COMBINED = os.path.join(os.path.dirname(__file__), "golden", "combined_mask_L6_B2.txt")


def test_combined_mask_matches_hand_derived_fixture(orc):
    rows = [ln.strip() for ln in open(COMBINED) if ln.strip() and not ln.startswith("#")]
    want = np.array([[c == "1" for c in r] for r in rows])
    assert want.shape == (12, 12)
    assert np.array_equal(orc.combined_mask(6, 2), want)


@pytest.mark.parametrize("L,B", [(6, 2), (64, 1), (96, 8), (120, 40), (128, 128)])
def test_combined_mask_counts_closed_form(L, B, orc):
    """A clean row of block b sees (b+1)B clean keys; a corrupted row of block b sees
    bB clean keys and its B own corrupted keys; all pairs: B^2 n_b (n_b + 1)."""
    m = orc.combined_mask(L, B)
    blk = np.arange(L) // B
    assert np.array_equal(m[:L].sum(axis=1), (blk + 1) * B)
    assert np.array_equal(m[L:, :L].sum(axis=1), blk * B)
    assert np.array_equal(m[L:, L:].sum(axis=1), np.full(L, B))
    nb = L // B
    assert int(m.sum()) == B * B * nb * (nb + 1)


def _rank_rows_keys(L, B, q_off, q_len, owned, kv_off, kv_len, local):
    """Combined-sequence indices of a rank's rows and of one call's keys."""
    owned = np.asarray(owned, dtype=np.int64)
    corr = (L + owned[:, None] * B + np.arange(B)[None, :]).reshape(-1)
    rows = np.concatenate([q_off + np.arange(q_len), corr]).astype(np.int64)
    keys = np.concatenate([kv_off + np.arange(kv_len), corr if local else np.zeros(0, np.int64)]).astype(np.int64)
    return rows, keys


@pytest.mark.parametrize("L,B,R", [(96, 4, 2), (128, 8, 4), (64, 1, 4)])
def test_rank_shares_partition_the_combined_mask(L, B, R, orc):
    """Both position shardings -- CSBP (clean shard r, zigzag corrupted blocks) and
    conventional CP (clean and corrupted positions of chunk r) -- give every row of
    the combined sequence to exactly one rank; each rank's call against clean shard s
    (plus its own corrupted K/V) is the combined mask restricted to those rows and
    keys; and no rank's row may attend another rank's corrupted keys."""
    full = orc.combined_mask(L, B)
    nb, n = L // B, L // R
    for scheme in ("csbp", "cp"):
        seen = np.zeros(2 * L, dtype=int)
        for r in range(R):
            owned = (wl.zigzag_owned_blocks(nb, R, r) if scheme == "csbp"
                     else np.arange(r * nb // R, (r + 1) * nb // R))
            rows, own_keys = _rank_rows_keys(L, B, r * n, n, owned, 0, 0, True)
            seen[rows] += 1
            for s in range(R):
                local = s == r
                m = orc.bdlm_mask(L, B, r * n, n, owned, s * n, n, local)
                _, keys = _rank_rows_keys(L, B, r * n, n, owned, s * n, n, local)
                assert np.array_equal(m, full[np.ix_(rows, keys)]), (scheme, r, s)
            other_corr = np.setdiff1d(np.arange(L, 2 * L), own_keys)
            assert not full[np.ix_(rows, other_corr)].any(), (scheme, r)
        assert np.all(seen == 1), scheme
