"""GPU parity at the workloads' full sizes, in the launch configuration that
bench.py times (every head, every clean shard, merge, backward per shard).

The fp64 oracle cannot run these whole, so it checks what it can compute one
by one, plus identities that hold at any size:
  * sampled query rows (KV-head group 0): O, LSE and dQ are row-local and exact;
  * keys attended by few rows (the corrupted-self keys of a block, the highest
    attended clean keys, whole short varlen shards): dK and dV are exact once the
    attending rows' LSE and delta come from the oracle;
  * every key: for each KV head g, sum_j dV_j = sum_{rows i, q-heads h of g} dO_ih
    (each row's probabilities sum to 1), and sum_j dK_j = 0 (each row of dS sums
    to 0: sum_j P_ij (dP_ij - delta_i) = delta_i - delta_i).
"""
import time

import numpy as np
import pytest
import torch

import oracle
from masked_long_context_amd import workloads as wl
from masked_long_context_amd import bdattn as B
from masked_long_context_amd.rank_step import BdlmRankStep, TaskStep, VarlenStep
from gpu_util import TOL_REL_L2, check_close, check_lse, need_gpu, poison_, to64

pytestmark = pytest.mark.gpu


def log(msg):
    print(f"[{time.strftime('%H:%M:%S')}] {msg}", flush=True)


def _f64(t):
    return t.to(torch.float64).numpy()


def check_sum_identities(dk, dv, dout, G, label):
    """sum_j dV_j = sum over rows and the group's q-heads of dO; sum_j dK_j = 0 (per KV head)."""
    dk = dk.double()
    dv = dv.double()
    do = dout.double()
    h_kv = dk.shape[1]
    for g in range(h_kv):
        sv = dv[:, g].sum(0)
        want = do[:, g * G:(g + 1) * G].sum((0, 1))
        rel = float((sv - want).norm() / want.norm())
        sk = dk[:, g].sum(0)
        scale = float(dk[:, g].norm())
        relk = float(sk.norm()) / scale
        assert rel <= TOL_REL_L2, f"{label}: sum dV != sum dO (kv head {g}): {rel:.2e}"
        assert relk <= TOL_REL_L2, f"{label}: sum dK != 0 (kv head {g}): {relk:.2e}"
    log(f"{label}: gradient-sum identities hold on every KV head (last: dV {rel:.1e}, dK {relk:.1e})")


def bdlm_oracle_group0(cfg, inp):
    """Oracle callables on KV-head group 0 (q-heads 0..G-1, KV head 0) over all keys."""
    p = cfg.problem
    G = p.h_q // p.h_kv
    q = _f64(inp["q"][:, :G])
    do = _f64(inp["dout"][:, :G])
    kc, vc = _f64(inp["k_clean"][:, :1]), _f64(inp["v_clean"][:, :1])
    kx, vx = _f64(inp["k_corr"][:, :1]), _f64(inp["v_corr"][:, :1])
    prob = dict(clean_len=p.clean_len, block_size=p.block_size, q_clean_offset=p.q_clean_offset,
                q_clean_len=p.q_clean_len, owned_blocks=list(p.owned_blocks), kv_clean_offset=0,
                kv_clean_len=p.clean_len, with_local_corrupt=True, scale=p.scale)

    def rows_fwd_bwd(rows, keys=None):
        o, lse = oracle.bdlm_fwd(prob, q, kc, vc, kx, vx, rows=rows)
        D = oracle.delta_rows(o, do[rows])
        dq, dk, dv = oracle.bdlm_bwd(prob, q, kc, vc, kx, vx, do, lse, D, rows=rows, keys=keys)
        return o, lse, dq, dk, dv

    def attending_rows(keys):
        m = oracle.bdlm_mask(p.clean_len, p.block_size, p.q_clean_offset, p.q_clean_len, p.owned_blocks,
                             0, p.clean_len, True, keys=np.asarray(keys))
        return np.nonzero(m.any(axis=1))[0]

    return G, rows_fwd_bwd, attending_rows


def run_bdlm_fullsize(idx, n_rows, n_slots, n_tail_keys, fused=False):
    need_gpu()
    cfg = wl.config(idx)
    p = cfg.problem
    log(f"{cfg.name}: generating inputs")
    inp = wl.bdlm_inputs(cfg, seed=0)
    g = {k: v.cuda() for k, v in inp.items()}
    shards = [(0, p.clean_len, True)] if fused else cfg.shards
    step = BdlmRankStep(p, shards)
    assert step.direct == fused
    poison_(step.o_parts, step.lse_parts, step.o, step.lse, step.dq, step.dk_clean, step.dv_clean,
            step.dk_corr, step.dv_corr)
    log(f"{cfg.name}: GPU step ({len(shards)} clean K/V range(s))")
    step.step(g["q"], g["k_clean"], g["v_clean"], g["k_corr"], g["v_corr"], g["dout"])
    torch.cuda.synchronize()
    o, lse, dq = step.o.cpu(), step.lse.cpu(), step.dq.cpu()
    dk = torch.cat([step.dk_clean, step.dk_corr]).cpu()
    dv = torch.cat([step.dv_clean, step.dv_corr]).cpu()
    del g
    for t in (o, lse, dq, dk, dv):
        assert not torch.isnan(t.float()).any(), "unwritten output"
    G = p.h_q // p.h_kv
    check_sum_identities(dk, dv, inp["dout"], G, cfg.name)

    G, rows_fwd_bwd, attending_rows = bdlm_oracle_group0(cfg, inp)
    rng = np.random.default_rng(idx)
    rows = np.sort(rng.choice(p.n_q, n_rows, replace=False))
    log(f"{cfg.name}: oracle on {len(rows)} sampled rows x {G} q-heads")
    o_r, lse_r, dq_r, _, _ = rows_fwd_bwd(rows)
    check_lse("lse[rows]", lse[:G, rows], lse_r)
    check_close("o[rows]", o[rows, :G], o_r)
    check_close("dq[rows]", dq[rows, :G], dq_r)

    # keys whose attending rows are few: whole corrupted-self blocks and the top clean keys
    B = p.block_size
    slots = rng.choice(p.n_owned, n_slots, replace=False)
    self_keys = np.concatenate([p.clean_len + np.arange(m * B, (m + 1) * B) for m in slots])
    top = max(b for b in p.owned_blocks) * B          # highest clean key any row attends, + 1
    tail_keys = np.arange(top - n_tail_keys, top)
    keys = np.concatenate([tail_keys, self_keys])
    arows = attending_rows(keys)
    log(f"{cfg.name}: oracle dK/dV on {len(keys)} keys ({len(arows)} attending rows)")
    _, _, _, dk_r, dv_r = rows_fwd_bwd(arows, keys=keys)
    check_close("dk[keys]", dk[keys, :1], dk_r)
    check_close("dv[keys]", dv[keys, :1], dv_r)


def test_csbp_256k_rank_share_fullsize():
    run_bdlm_fullsize(3, n_rows=48, n_slots=2, n_tail_keys=64)


def test_csbp_256k_rank_share_fused_fullsize():
    """All sixteen clean shards resident and passed as one range (no partials, no merge)."""
    run_bdlm_fullsize(3, n_rows=48, n_slots=2, n_tail_keys=64, fused=True)


def test_cp_256k_rank_share_fullsize():
    """Conventional context parallelism's share of the same sequence (rank 8's position chunk)."""
    run_bdlm_fullsize(7, n_rows=48, n_slots=2, n_tail_keys=64)


def test_csbp_1m_rank_share_fullsize():
    run_bdlm_fullsize(5, n_rows=16, n_slots=2, n_tail_keys=32)


def test_varlen_262k_fullsize():
    need_gpu()
    cfg = wl.config(4)
    cu = cfg.cu_seqlens
    log(f"{cfg.name}: generating inputs")
    inp = wl.varlen_inputs(cfg, seed=0)
    g = {k: v.cuda() for k, v in inp.items()}
    step = VarlenStep(cu, True, cfg.h_q, cfg.h_kv, cfg.head_dim)
    poison_(step.o, step.lse, step.dq, step.dk, step.dv)
    log(f"{cfg.name}: GPU step")
    step.step(g["q"], g["k"], g["v"], g["dout"])
    torch.cuda.synchronize()
    o, lse, dq, dk, dv = (t.cpu() for t in (step.o, step.lse, step.dq, step.dk, step.dv))
    del g
    G = cfg.h_q // cfg.h_kv
    # per-shard identities: every shard is an independent attention problem
    for s in range(len(cfg.seqlens)):
        a, b = int(cu[s]), int(cu[s + 1])
        check_sum_identities(dk[a:b], dv[a:b], inp["dout"][a:b], G, f"shard {s} (len {b - a})")

    q = _f64(inp["q"][:, :G])
    do = _f64(inp["dout"][:, :G])
    k, v = _f64(inp["k"][:, :1]), _f64(inp["v"][:, :1])
    rng = np.random.default_rng(4)
    rows = np.sort(rng.choice(cfg.total, 48, replace=False))
    log(f"{cfg.name}: oracle on {len(rows)} sampled rows")
    o_r, lse_r = oracle.varlen_fwd(q, k, v, cu, True, cfg.scale, rows=rows)
    D = oracle.delta_rows(o_r, do[rows])
    dq_r, _, _ = oracle.varlen_bwd(q, k, v, do, lse_r, D, cu, True, cfg.scale, rows=rows)
    check_lse("lse[rows]", lse[:G, rows], lse_r)
    check_close("o[rows]", o[rows, :G], o_r)
    check_close("dq[rows]", dq[rows, :G], dq_r)
    # whole short shards, and the last keys of the longest shard
    order = np.argsort(cfg.seqlens)
    keys = [np.arange(cu[s], cu[s + 1]) for s in order[:2]]
    longest = order[-1]
    keys.append(np.arange(cu[longest + 1] - 48, cu[longest + 1]))
    keys = np.concatenate(keys)
    m = oracle.varlen_mask(cu, True, keys=keys)
    arows = np.nonzero(m.any(axis=1))[0]
    log(f"{cfg.name}: oracle dK/dV on {len(keys)} keys ({len(arows)} attending rows)")
    o_a, lse_a = oracle.varlen_fwd(q, k, v, cu, True, cfg.scale, rows=arows)
    D = oracle.delta_rows(o_a, do[arows])
    _, dk_r, dv_r = oracle.varlen_bwd(q, k, v, do, lse_a, D, cu, True, cfg.scale, rows=arows, keys=keys)
    check_close("dk[keys]", dk[keys, :1], dk_r)
    check_close("dv[keys]", dv[keys, :1], dv_r)


def test_cad_tasks_262k_fullsize():
    """Workload 4's documents as core-attention tasks with gathered prefix contexts, at full size."""
    need_gpu()
    cfg = wl.config(6)
    docs = cfg.docs
    cu = docs.cu_seqlens
    q_cu, k_cu, src = B.cad_split(cu, cfg.max_pairs)
    rows = wl.task_context_rows(k_cu, src)
    log(f"{cfg.name}: {len(src)} tasks, {len(rows)} context rows; generating inputs")
    inp = wl.varlen_inputs(docs, seed=0)
    g = {k: v.cuda() for k, v in inp.items()}
    idx = torch.from_numpy(rows).cuda()
    kt, vt = g["k"].index_select(0, idx), g["v"].index_select(0, idx)
    step = TaskStep(q_cu, k_cu, True, cfg.h_q, cfg.h_kv, cfg.head_dim)
    poison_(step.o, step.lse, step.dq, step.dk, step.dv)
    log(f"{cfg.name}: GPU step")
    step.step(g["q"], kt, vt, g["dout"])
    torch.cuda.synchronize()
    G = cfg.h_q // cfg.h_kv
    # every task is an independent attention problem over its own context copy
    for t in range(len(src)):
        a, b, c, e = int(q_cu[t]), int(q_cu[t + 1]), int(k_cu[t]), int(k_cu[t + 1])
        check_sum_identities(step.dk[c:e], step.dv[c:e], g["dout"][a:b], G, f"task {t} (q {b - a}, ctx {e - c})")
    o, lse, dq, dk, dv = (t.cpu() for t in (step.o, step.lse, step.dq, step.dk, step.dv))
    del g, kt, vt, idx, step

    # sampled rows: a task's queries are its document's rows, so O, LSE, dQ are the documents'
    q = _f64(inp["q"][:, :G])
    do = _f64(inp["dout"][:, :G])
    k, v = _f64(inp["k"][:, :1]), _f64(inp["v"][:, :1])
    rng = np.random.default_rng(6)
    rs = np.sort(rng.choice(docs.total, 48, replace=False))
    log(f"{cfg.name}: oracle on {len(rs)} sampled rows")
    o_r, lse_r = oracle.varlen_fwd(q, k, v, cu, True, cfg.scale, rows=rs)
    D = oracle.delta_rows(o_r, do[rs])
    dq_r, _, _ = oracle.varlen_bwd(q, k, v, do, lse_r, D, cu, True, cfg.scale, rows=rs)
    check_lse("lse[rows]", lse[:G, rs], lse_r)
    check_close("o[rows]", o[rs, :G], o_r)
    check_close("dq[rows]", dq[rs, :G], dq_r)

    # dK/dV copies of two tasks, each against the oracle of that task alone: every key of the
    # smallest task, and the last 48 context keys of the task with the longest context
    ql, kl = np.diff(q_cu), np.diff(k_cu)
    for t, nk in ((int(np.argmin(ql * kl)), None), (int(np.argmax(kl)), 48)):
        a, b, c, e = int(q_cu[t]), int(q_cu[t + 1]), int(k_cu[t]), int(k_cu[t + 1])
        tq, tdo = q[a:b], do[a:b]
        tk, tv = k[rows[c:e]], v[rows[c:e]]
        one_q, one_k = [0, b - a], [0, e - c]
        keys = np.arange(e - c) if nk is None else np.arange(e - c - nk, e - c)
        arows = np.nonzero(oracle.task_mask(one_q, one_k, True, keys=keys).any(axis=1))[0]
        log(f"{cfg.name}: task {t} (q {b - a}, ctx {e - c}): oracle dK/dV on {len(keys)} keys "
            f"({len(arows)} attending rows)")
        o_a, lse_a = oracle.task_fwd(tq, tk, tv, one_q, one_k, True, cfg.scale, rows=arows)
        D = oracle.delta_rows(o_a, tdo[arows])
        _, dk_r, dv_r = oracle.task_bwd(tq, tk, tv, tdo, lse_a, D, one_q, one_k, True, cfg.scale,
                                        rows=arows, keys=keys)
        check_close(f"dk[task {t}]", dk[c + keys, :1], dk_r)
        check_close(f"dv[task {t}]", dv[c + keys, :1], dv_r)
