"""GPU parity at the workloads' full sizes, in the launch configuration that
bench.py times (every head, every clean shard, merge, backward per shard).

KV-head group 0 (q-heads 0..G-1, KV head 0) is compared with the fp64 oracle
element by element.  At the 256K rank share (sharded) and the varlen workload
that is every element of the group: all rows' O, LSE and dQ and all keys' dK
and dV (tests/fullsize_ref.group_reference, about 10^10 score elements each, a
minute or two on the host's cores).  Elsewhere:
  * sampled query rows (1024; 4096 at the 1M rank share): O, LSE and dQ, each
    row exact on its own (tests/fullsize_ref.py composes the oracle over key
    pieces with the exact LSE merge);
  * keys spread over the whole attended key range (512; 1024 at the 1M rank
    share), including the bulk clean keys that nearly every row attends and
    the corrupted self-blocks: dK and dV against fp64 references that need the
    LSE and delta of every attending row.  That is a forward of the whole
    group, so tests/golden/make_fullsize_fixtures.py computes the references
    once from the oracle and stores them; the test checks that it draws the
    same inputs (fingerprint) before comparing;
  * LSE of every row of the group (256K rank shares);
  * keys past the last attended one: dK = dV = 0 exactly.
Identities that hold at any size are checked on every KV head as well:
sum_j dV_j = sum over rows and the group's q-heads of dO (each row's
probabilities sum to 1), and sum_j dK_j = 0 (each row of dS sums to 0).
"""
import os
import time

import numpy as np
import pytest
import torch

import fullsize_ref as fr
import oracle
from masked_long_context_amd import workloads as wl
from masked_long_context_amd import bdattn as B
from masked_long_context_amd.rank_step import BdlmRankStep, ResidentShardsStep, TaskStep, VarlenStep
from gpu_util import TOL_REL_L2, check_close, check_lse, need_gpu, poison_

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(900)]

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
# per-key relative L2 bound: a key whose gradient went to another key, or was
# dropped, has a relative error near 1; bf16 output rounding alone gives ~2e-3
TOL_PER_KEY = 5 * TOL_REL_L2


def log(msg):
    print(f"[{time.strftime('%H:%M:%S')}] {msg}", flush=True)


def load_fixture(idx, view):
    path = os.path.join(GOLDEN, f"fullsize_w{idx}.npz")
    z = np.load(path, allow_pickle=False)
    fp = fr.fingerprint(view)
    assert str(z["fingerprint"]) == fp, (f"{path} was made from other inputs than the ones drawn now: "
                                         "rerun tests/golden/make_fullsize_fixtures.py")
    return {k: z[k] for k in z.files}


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


def check_keys(name, got, want, per_key_bound=True):
    """Element-wise dK or dV of a set of keys: the stated tensor bounds, a per-key
    relative bound (or, with per_key_bound=False, its worst value printed only),
    and exact zeros where the reference is exactly zero."""
    got = got.double().numpy() if isinstance(got, torch.Tensor) else np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    zero = np.all(want == 0, axis=1)
    if zero.any():
        assert np.all(got[zero] == 0), f"{name}: keys no row attends have non-zero gradients"
    nz = ~zero
    check_close(name, got[nz], want[nz])
    per = np.linalg.norm(got[nz] - want[nz], axis=1) / np.linalg.norm(want[nz], axis=1)
    worst = int(np.argmax(per))
    print(f"  {name}: {int(nz.sum())} keys, per-key relative L2 max {per.max():.2e} (key #{worst}), "
          f"median {np.median(per):.2e}; {int(zero.sum())} exact zeros", flush=True)
    if per_key_bound:
        assert per.max() <= TOL_PER_KEY, f"{name}: key #{worst} relative error {per.max():.2e}"


def check_rows(label, view, rows, o, lse, dq):
    G = view["G"]
    log(f"{label}: oracle on {len(rows)} sampled rows x {G} q-heads")
    r, o_r, lse_r, dq_r = fr.rows_reference(view["q"], view["k"], view["v"], view["dout"], view["mask"],
                                           view["scale"], rows)
    check_lse("lse[rows]", lse[:G, r], lse_r)
    check_close("o[rows]", o[r, :G], o_r)
    check_close("dq[rows]", dq[r, :G], dq_r)


def check_every_element(label, view, o, lse, dq, dk, dv):
    """Every output of KV-head group 0 (q-heads 0..G-1, KV head 0) against the oracle."""
    G = view["G"]
    t0 = time.time()
    log(f"{label}: oracle on every row and key of KV-head group 0 "
        f"({view['q'].shape[0]} rows x {G} q-heads, {view['k'].shape[0]} keys)")
    O, L, DQ, DK, DV = fr.group_reference(view["q"], view["k"], view["v"], view["dout"], view["mask"], view["scale"])
    log(f"{label}: reference done in {time.time() - t0:.0f} s")
    check_lse("lse[group 0, every row]", lse[:G], L)
    check_close("o[group 0, every row]", o[:, :G], O)
    check_close("dq[group 0, every row]", dq[:, :G], DQ)
    check_keys("dk[kv head 0, every key]", dk[:, 0], DK[:, 0], per_key_bound=False)
    check_keys("dv[kv head 0, every key]", dv[:, 0], DV[:, 0], per_key_bound=False)


def run_bdlm_fullsize(idx, n_rows, fused=False, every_element=False):
    need_gpu()
    cfg = wl.config(idx)
    p = cfg.problem
    log(f"{cfg.name}: generating inputs")
    inp = wl.bdlm_inputs(cfg, seed=0)
    g = {k: v.cuda() for k, v in inp.items()}
    if fused:
        # every clean shard resident in a buffer of its own, one launch per kernel
        step = ResidentShardsStep(p, cfg.shards)
        k_sh = [g["k_clean"][o_:o_ + n_].clone() for (o_, n_, _) in cfg.shards]
        v_sh = [g["v_clean"][o_:o_ + n_].clone() for (o_, n_, _) in cfg.shards]
        poison_(step.o, step.o32, step.lse, step.dq, *step.dk_shards, *step.dv_shards, step.dk_corr, step.dv_corr)
        log(f"{cfg.name}: GPU step ({len(k_sh)} resident shard buffers, one launch per kernel)")
        step.step(g["q"], k_sh, v_sh, g["k_corr"], g["v_corr"], g["dout"])
        torch.cuda.synchronize()
        o, lse, dq = step.o.cpu(), step.lse.cpu(), step.dq.cpu()
        dk = torch.cat(step.dk_shards + [step.dk_corr]).cpu()
        dv = torch.cat(step.dv_shards + [step.dv_corr]).cpu()
        del step, k_sh, v_sh
        # the same plan with the clean K/V in one buffer: the same bits
        one = BdlmRankStep(p, [(0, p.clean_len, True)])
        assert one.direct
        poison_(one.o, one.o32, one.lse, one.dq, one.dk_clean, one.dv_clean, one.dk_corr, one.dv_corr)
        log(f"{cfg.name}: GPU step (one buffer, the same plan)")
        one.step(g["q"], g["k_clean"], g["v_clean"], g["k_corr"], g["v_corr"], g["dout"])
        torch.cuda.synchronize()
        for name, a_, b_ in (("o", o, one.o), ("lse", lse, one.lse), ("dq", dq, one.dq),
                             ("dk", dk, torch.cat([one.dk_clean, one.dk_corr])),
                             ("dv", dv, torch.cat([one.dv_clean, one.dv_corr]))):
            assert torch.equal(a_, b_.cpu()), f"resident shards vs one buffer: {name} differs"
        log(f"{cfg.name}: resident shards and one buffer agree bit for bit")
        del one
    else:
        step = BdlmRankStep(p, cfg.shards)
        assert not step.direct
        poison_(step.o_parts, step.lse_parts, step.o, step.o32, step.lse, step.dq, step.dk_clean, step.dv_clean,
                step.dk_corr, step.dv_corr)
        log(f"{cfg.name}: GPU step ({len(cfg.shards)} clean K/V ranges)")
        step.step(g["q"], g["k_clean"], g["v_clean"], g["k_corr"], g["v_corr"], g["dout"])
        torch.cuda.synchronize()
        o, lse, dq = step.o.cpu(), step.lse.cpu(), step.dq.cpu()
        dk = torch.cat([step.dk_clean, step.dk_corr]).cpu()
        dv = torch.cat([step.dv_clean, step.dv_corr]).cpu()
        del step
    del g
    for t in (o, lse, dq, dk, dv):
        assert not torch.isnan(t.float()).any(), "unwritten output"
    G = p.h_q // p.h_kv
    check_sum_identities(dk, dv, inp["dout"], G, cfg.name)

    view = fr.bdlm_group0(cfg, inp)
    fx = load_fixture(idx, view)
    if "lse" in fx:
        check_lse("lse[every row of group 0]", lse[:G], fx["lse"])
    keys = fx["keys"]
    L = p.clean_len
    log(f"{cfg.name}: dK/dV on {len(keys)} keys against the stored fp64 references")
    clean = keys < L
    check_keys("dk[clean keys]", dk[keys[clean], 0], fx["dk"][clean])
    check_keys("dv[clean keys]", dv[keys[clean], 0], fx["dv"][clean])
    check_keys("dk[corrupted self-block keys]", dk[keys[~clean], 0], fx["dk"][~clean])
    check_keys("dv[corrupted self-block keys]", dv[keys[~clean], 0], fx["dv"][~clean])

    if every_element:
        check_every_element(cfg.name, view, o, lse, dq, dk, dv)
        return
    rng = np.random.default_rng(idx)
    rows = np.sort(rng.choice(p.n_q, n_rows, replace=False))
    check_rows(cfg.name, view, rows, o, lse, dq)


def test_csbp_256k_rank_share_fullsize():
    """The headline workload: every element of KV-head group 0 (all 32768 rows x 4
    q-heads and all 278528 keys of KV head 0), plus the stored spread keys."""
    run_bdlm_fullsize(3, n_rows=1024, every_element=True)


def test_csbp_256k_rank_share_fused_fullsize():
    """All sixteen clean shards resident, each in a buffer of its own, and one launch per
    kernel over all of them (no partials, no merge); bit for bit the same plan run with
    the clean K/V in one buffer."""
    run_bdlm_fullsize(3, n_rows=1024, fused=True)


def test_cp_256k_rank_share_fullsize():
    """Conventional context parallelism's share of the same sequence (rank 8's position chunk)."""
    run_bdlm_fullsize(7, n_rows=1024)


def test_csbp_1m_rank_share_fullsize():
    run_bdlm_fullsize(5, n_rows=4096)


def test_csbp_1m_resident_shards_match_one_buffer():
    """The 1M-context rank share with its 8 clean shards resident in buffers of 131072
    positions, one launch per kernel: bit for bit the same plan over one buffer (the
    split-buffer kernels at their largest in-buffer offsets)."""
    need_gpu()
    cfg = wl.config(5)
    p = cfg.problem
    log(f"{cfg.name}: generating inputs")
    g = {k: v.cuda() for k, v in wl.bdlm_inputs(cfg, seed=0).items()}
    step = ResidentShardsStep(p, cfg.shards)
    k_sh = [g["k_clean"][o_:o_ + n_].clone() for (o_, n_, _) in cfg.shards]
    v_sh = [g["v_clean"][o_:o_ + n_].clone() for (o_, n_, _) in cfg.shards]
    assert step.shard_lens == [131072] * 8
    log(f"{cfg.name}: GPU step (8 resident shard buffers)")
    step.step(g["q"], k_sh, v_sh, g["k_corr"], g["v_corr"], g["dout"])
    torch.cuda.synchronize()
    got = [step.o.cpu(), step.lse.cpu(), step.dq.cpu(), torch.cat(step.dk_shards + [step.dk_corr]).cpu(),
           torch.cat(step.dv_shards + [step.dv_corr]).cpu()]
    del step, k_sh, v_sh
    one = BdlmRankStep(p, [(0, p.clean_len, True)])
    log(f"{cfg.name}: GPU step (one buffer, the same plan)")
    one.step(g["q"], g["k_clean"], g["v_clean"], g["k_corr"], g["v_corr"], g["dout"])
    torch.cuda.synchronize()
    want = [one.o, one.lse, one.dq, torch.cat([one.dk_clean, one.dk_corr]), torch.cat([one.dv_clean, one.dv_corr])]
    for name, a_, b_ in zip(("o", "lse", "dq", "dk", "dv"), got, want):
        assert not torch.isnan(a_.float()).any(), f"{name}: unwritten values"
        assert torch.equal(a_, b_.cpu()), f"resident shards vs one buffer: {name} differs"
    log(f"{cfg.name}: resident shards and one buffer agree bit for bit")


def test_varlen_262k_fullsize():
    need_gpu()
    cfg = wl.config(4)
    cu = cfg.cu_seqlens
    log(f"{cfg.name}: generating inputs")
    inp = wl.varlen_inputs(cfg, seed=0)
    g = {k: v.cuda() for k, v in inp.items()}
    step = VarlenStep(cu, True, cfg.h_q, cfg.h_kv, cfg.head_dim)
    poison_(step.o, step.o32, step.lse, step.dq, step.dk, step.dv)
    log(f"{cfg.name}: GPU step")
    step.step(g["q"], g["k"], g["v"], g["dout"])
    torch.cuda.synchronize()
    o, lse, dq, dk, dv = (t.cpu() for t in (step.o, step.lse, step.dq, step.dk, step.dv))
    del g, step
    G = cfg.h_q // cfg.h_kv
    # per-shard identities: every shard is an independent attention problem
    for s in range(len(cfg.seqlens)):
        a, b = int(cu[s]), int(cu[s + 1])
        check_sum_identities(dk[a:b], dv[a:b], inp["dout"][a:b], G, f"shard {s} (len {b - a})")

    view = fr.varlen_group0(cfg, inp)
    fx = load_fixture(4, view)
    keys = fx["keys"]
    longest = int(np.argmax(cfg.seqlens))
    log(f"{cfg.name}: dK/dV on {len(keys)} keys against the stored fp64 references "
        f"({int(((keys >= cu[longest]) & (keys < cu[longest + 1])).sum())} in the longest document)")
    check_keys("dk[keys]", dk[keys, 0], fx["dk"])
    check_keys("dv[keys]", dv[keys, 0], fx["dv"])
    check_every_element(cfg.name, view, o, lse, dq, dk, dv)


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
    poison_(step.o, step.o32, step.lse, step.dq, step.dk, step.dv)
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
    view = fr.varlen_group0(docs, inp)
    rng = np.random.default_rng(6)
    rs = np.sort(rng.choice(docs.total, 1024, replace=False))
    check_rows(cfg.name, view, rs, o, lse, dq)

    # dK/dV copies of three tasks, each against the oracle of that task alone, on keys
    # spread over its whole context: the smallest task (every key), the task with the
    # longest context and the task with the most causal pairs
    ql, kl = np.diff(q_cu), np.diff(k_cu)
    pairs = ql * kl - ql * (ql - 1) // 2
    picks = {int(np.argmin(ql * kl)): None, int(np.argmax(kl)): 512, int(np.argmax(pairs)): 512}
    for t, nk in picks.items():
        a, b, c, e = int(q_cu[t]), int(q_cu[t + 1]), int(k_cu[t]), int(k_cu[t + 1])
        tq, tdo = view["q"][a:b], view["dout"][a:b]
        tk, tv = view["k"][rows[c:e]], view["v"][rows[c:e]]
        mask = oracle.task_mask_fn([0, b - a], [0, e - c], True)
        keys = np.arange(e - c) if nk is None else fr.spread_keys(0, e - c, nk, seed=600 + t)
        log(f"{cfg.name}: task {t} (q {b - a}, ctx {e - c}): oracle dK/dV on {len(keys)} keys")
        lse_t, delta_t = fr.lse_delta_all_rows(tq, tk, tv, tdo, mask, cfg.scale, b - a)
        dk_r, dv_r = fr.keys_reference(tq, tk, tv, tdo, lse_t, delta_t, mask, cfg.scale, keys)
        check_keys(f"dk[task {t}]", dk[c + keys, 0], dk_r[:, 0])
        check_keys(f"dv[task {t}]", dv[c + keys, 0], dv_r[:, 0])
