"""Host tile scheduler against the oracle's explicit mask (CPU only).

Checks that the per-row key ranges equal the mask, that the scheduled tiles
cover every legal pair, that tiles marked full hold no masked pair, that no
scheduled tile is empty, the useful-pair counts (closed forms of the
workloads), and the longest-first ordering."""
import numpy as np
import pytest

import oracle
from masked_long_context_amd import bdattn as B
from masked_long_context_amd import workloads as wl

FWD_BN, BWD_BN = 64, 128


def _mask_and_plan(p):
    plan = B.Plan.from_problem(p)
    m = oracle.bdlm_mask(p.clean_len, p.block_size, p.q_clean_offset, p.q_clean_len, p.owned_blocks,
                         p.kv_clean_offset, p.kv_clean_len, p.with_local_corrupt)
    return plan, m


def _check_plan(plan, m, n0, n1):
    rows = plan.export(0)
    nq = m.shape[0]
    assert rows.shape == (nq, 4)
    # 1. per-row ranges reproduce the mask exactly
    rebuilt = np.zeros_like(m)
    for r in range(nq):
        lo0, hi0, lo1, hi1 = rows[r]
        if hi0 > lo0:
            rebuilt[r, lo0:hi0] = True
        if hi1 > lo1:
            rebuilt[r, n0 + lo1:n0 + hi1] = True
    assert np.array_equal(rebuilt, m)
    assert plan.useful_pairs == int(m.sum())

    def seg_cols(s, k0, k1):
        base = 0 if s == 0 else n0
        n = n0 if s == 0 else n1
        return base + k0, base + min(k1, n)

    # 2. forward items: every row once; visited tiles cover the mask; full tiles are all legal
    items = plan.export(1)
    seen = np.zeros(nq, int)
    covered = np.zeros_like(m)
    costs = []
    for it in items:
        q0, nr = it[0], it[1]
        seen[q0:q0 + nr] += 1
        costs.append(it[10])
        for s in range(2):
            lo_min, lo_max, hi_min, hi_max = it[2 + 4 * s: 6 + 4 * s]
            if hi_max <= lo_min:
                assert not m[q0:q0 + nr, seg_cols(s, 0, n0 if s == 0 else n1)[0]:
                             seg_cols(s, 0, n0 if s == 0 else n1)[1]].any()
                continue
            for k0 in range(lo_min // FWD_BN * FWD_BN, hi_max, FWD_BN):
                a, b = seg_cols(s, k0, k0 + FWD_BN)
                covered[q0:q0 + nr, a:b] = True
                full = lo_max <= k0 and k0 + FWD_BN <= hi_min
                if full:
                    assert m[q0:q0 + nr, a:b].all()
                    assert b - a == FWD_BN
    assert np.all(seen == 1)
    assert not (m & ~covered).any()
    assert costs == sorted(costs, reverse=True)

    # 3. backward: k-tiles cover every key once, lists cover the mask, full entries all legal,
    #    no entry without a legal pair, longest list first
    bq = plan.export(2)
    kts = plan.export(3)
    lst = plan.export(4)
    cov_b = np.zeros_like(m)
    keys_seen = {0: set(), 1: set()}
    lens = []
    for s, k0, beg, end in kts:
        keys_seen[s].add(k0)
        lens.append(end - beg)
        a, b = seg_cols(s, k0, k0 + BWD_BN)
        for e in lst[beg:end]:
            full = e < 0
            qi = e & 0x7FFFFFFF
            q0, nr = bq[qi][0], bq[qi][1]
            blk = m[q0:q0 + nr, a:b]
            assert blk.any()
            cov_b[q0:q0 + nr, a:b] = True
            if full:
                assert blk.all() and b - a == BWD_BN
    assert keys_seen[0] == set(range(0, n0, BWD_BN))
    assert keys_seen[1] == set(range(0, n1, BWD_BN))
    assert not (m & ~cov_b).any()
    assert lens == sorted(lens, reverse=True)
    # backward q-tiles cover every row once
    seen = np.zeros(nq, int)
    for t in bq:
        seen[t[0]:t[0] + t[1]] += 1
    assert np.all(seen == 1)


SMALL = [
    wl.small_bdlm_config(512, 16, 4, 1, 4, 2, 128, 4),
    wl.small_bdlm_config(768, 32, 2, 1, 2, 1, 64, 3),
    wl.small_bdlm_config(384, 24, 2, 0, 2, 2, 128, 2),
    wl.small_bdlm_config(64, 1, 2, 1, 1, 1, 64, 2),
    wl.small_bdlm_config(1024, 128, 2, 1, 2, 1, 128, 2),
    wl.small_bdlm_config(1600, 200, 2, 1, 2, 2, 64, 4),
    wl.config(1),
    wl.config(2),
]


@pytest.mark.parametrize("cfg", SMALL, ids=lambda c: c.name)
def test_bdlm_plans_match_mask(cfg):
    total = 0
    for p in cfg.shard_problems() + [cfg.problem]:
        plan, m = _mask_and_plan(p)
        _check_plan(plan, m, p.kv_clean_len, p.n_corr if p.with_local_corrupt else 0)
    for p in cfg.shard_problems():
        total += B.Plan.from_problem(p).useful_pairs
    assert total == B.Plan.from_problem(cfg.problem).useful_pairs


def test_random_bdlm_plans_match_mask():
    rng = np.random.default_rng(0)
    for _ in range(40):
        Bs = int(rng.choice([1, 2, 5, 16, 32, 48]))
        nb = int(rng.integers(2, 12))
        L = nb * Bs
        q0 = int(rng.integers(0, nb)) * Bs
        ql = int(rng.integers(0, nb - q0 // Bs + 1)) * Bs
        owned = [int(x) for x in rng.permutation(nb)[:int(rng.integers(0, nb + 1))]]
        k0 = int(rng.integers(0, nb)) * Bs
        kl = int(rng.integers(0, nb - k0 // Bs + 1)) * Bs
        local = bool(rng.integers(0, 2))
        p = wl.BdlmProblem(L, Bs, q0, ql, tuple(owned), k0, kl, local, 2, 1, 64)
        plan, m = _mask_and_plan(p)
        _check_plan(plan, m, kl, p.n_corr if local else 0)


@pytest.mark.parametrize("lens,causal", [([1, 5, 130, 64, 257, 300], True), ([7, 129, 128, 1], False),
                                         ([0, 70, 0, 200], True)])
def test_varlen_plans_match_mask(lens, causal):
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    plan = B.Plan.varlen(cu, causal, 4, 2, 128)
    m = oracle.varlen_mask(cu, causal)
    _check_plan(plan, m, int(cu[-1]), 0)


@pytest.mark.parametrize("idx,expected", [(1, 73728), (2, 17039360), (3, 4429709312), (5, 146030985216)])
def test_useful_pairs_of_workloads(idx, expected):
    cfg = wl.config(idx)
    assert sum(B.Plan.from_problem(p).useful_pairs for p in cfg.shard_problems()) == expected


def test_varlen_workload_pairs():
    cfg = wl.config(4)
    assert B.Plan.varlen(cfg.cu_seqlens, True, 32, 8, 128).useful_pairs == 3214974270


@pytest.mark.parametrize("q_lens,k_lens,causal", [
    ([3, 130, 64, 1, 257], [3, 200, 64, 900, 257], True),      # prefix contexts, k_len >= q_len
    ([70, 5, 300], [10, 0, 129], True),                         # k_len < q_len: leading rows see nothing
    ([0, 40, 0, 65], [12, 40, 0, 300], True),                   # empty tasks on either side
    ([7, 129, 128, 1], [300, 5, 128, 64], False),
])
def test_task_plans_match_mask(q_lens, k_lens, causal):
    q_cu = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32)
    k_cu = np.concatenate([[0], np.cumsum(k_lens)]).astype(np.int32)
    plan = B.Plan.tasks(q_cu, k_cu, causal, 4, 2, 128)
    m = oracle.task_mask(q_cu, k_cu, causal)
    assert plan.n_q == int(q_cu[-1]) and plan.n_kv(0) == int(k_cu[-1]) and plan.n_kv(1) == 0
    _check_plan(plan, m, int(k_cu[-1]), 0)


def test_random_task_plans_match_mask():
    rng = np.random.default_rng(1)
    for _ in range(30):
        n = int(rng.integers(1, 6))
        q_lens = rng.integers(0, 300, n)
        k_lens = np.where(rng.random(n) < 0.7, q_lens + rng.integers(0, 300, n), rng.integers(0, 300, n))
        causal = bool(rng.integers(0, 2))
        q_cu = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32)
        k_cu = np.concatenate([[0], np.cumsum(k_lens)]).astype(np.int32)
        plan = B.Plan.tasks(q_cu, k_cu, causal, 2, 1, 64)
        _check_plan(plan, oracle.task_mask(q_cu, k_cu, causal), int(k_cu[-1]), 0)


def _check_cad_split(cu, max_pairs):
    cu = np.asarray(cu, np.int64)
    q_cu, k_cu, src = B.cad_split(cu, max_pairs)
    n = src.size
    assert q_cu.size == n + 1 and k_cu.size == n + 1 and q_cu[0] == 0 and k_cu[0] == 0
    # the task queries are the packed document rows, in order, each exactly once
    assert q_cu[-1] == cu[-1] and np.all(np.diff(q_cu) >= 1)
    doc = np.searchsorted(cu, q_cu[:-1], side="right") - 1
    for t in range(n):
        q0, q1, kl = int(q_cu[t]), int(q_cu[t + 1]), int(k_cu[t + 1] - k_cu[t])
        d = int(doc[t])
        assert src[t] == cu[d] and q1 <= cu[d + 1]           # one document, context from its start
        assert kl == q1 - cu[d]                               # context = prefix up to the run's end
        x0 = q0 - int(cu[d])                                  # first row's index in the document
        pairs = sum(x + 1 for x in range(x0, x0 + (q1 - q0)))
        assert pairs <= max_pairs or q1 - q0 == 1
        if q1 < cu[d + 1]:                                    # greedy: one more row would break the bound
            assert pairs + (x0 + q1 - q0) + 1 > max_pairs
    return q_cu, k_cu, src


@pytest.mark.parametrize("lens,max_pairs", [([5, 0, 7], 10), ([1, 300, 64, 1000], 4096), ([1000], 1),
                                            ([257, 129], 100000), ([], 5)])
def test_cad_split_tasks_are_bounded_prefix_chunks(lens, max_pairs):
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    _check_cad_split(cu, max_pairs)


def test_cad_split_reproduces_document_causal_attention():
    """Gathering each task's context from its document makes the task mask equal the
    documents' causal mask row by row, with the same useful-pair count."""
    rng = np.random.default_rng(2)
    for _ in range(10):
        lens = rng.integers(0, 200, int(rng.integers(1, 5)))
        cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
        max_pairs = int(rng.integers(1, 6000))
        q_cu, k_cu, src = _check_cad_split(cu, max_pairs)
        kv_rows = np.concatenate([np.arange(s, s + k_cu[t + 1] - k_cu[t]) for t, s in enumerate(src)]
                                 + [np.zeros(0, np.int64)]).astype(np.int64)
        mt = oracle.task_mask(q_cu, k_cu, True)
        mv = oracle.varlen_mask(cu, True)
        mapped = np.zeros_like(mv)
        for r, j in zip(*np.nonzero(mt)):
            assert not mapped[r, kv_rows[j]]
            mapped[r, kv_rows[j]] = True
        assert np.array_equal(mapped, mv)
        if cu[-1]:
            tp = B.Plan.tasks(q_cu, k_cu, True, 2, 1, 64).useful_pairs
            assert tp == B.Plan.varlen(cu, True, 2, 1, 64).useful_pairs == int(mv.sum())


def test_dkdv_split_follows_the_occupancy_rule():
    """Automatic dK/dV split: F = min(8, ceil(1024 / workgroups), longest walk / 8),
    and 1 when the plan already has 512 or more workgroups (key tiles x KV heads)."""
    from masked_long_context_amd import bdattn as B
    from masked_long_context_amd import workloads as wl
    cfg2 = wl.config(2)
    got = []
    for sh in cfg2.shards:
        pl = B.Plan.from_problem(cfg2.problem.with_kv(*sh))
        kt = pl.export(3)
        n_wg = len(kt) * cfg2.problem.h_kv
        longest = int((kt[:, 3] - kt[:, 2]).max()) * (cfg2.problem.h_q // cfg2.problem.h_kv)
        want = 1 if n_wg >= 512 else max(1, min(8, -(-1024 // n_wg), longest // 8))
        assert pl.dkdv_split == want, (sh, pl.dkdv_split, want)
        got.append(pl.dkdv_split)
    assert got[0] == 7 and all(f == 8 for f in got[1:]), got
    cfg3 = wl.config(3)
    for sh in list(cfg3.shards)[:3]:
        assert B.Plan.from_problem(cfg3.problem.with_kv(*sh)).dkdv_split == 1
