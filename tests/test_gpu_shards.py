"""GPU parity of the resident-shards step: the clean K/V of a rank share held in
one buffer per shard, and each kernel launched once over all of them (the
shards merged online in registers).  Checked element by element against the
fp64 oracle, and bit for bit against the same plan run with the clean range in
one buffer (the kernels read the same values in the same order)."""
import pytest
import torch

from masked_long_context_amd import workloads as wl
from masked_long_context_amd.rank_step import ResidentShardsStep, StepGraph
from gpu_util import compare_bdlm, need_gpu, oracle_bdlm_full, poison_, run_gpu_bdlm

pytestmark = pytest.mark.gpu

OUT = ("o", "lse", "dq", "dk_clean", "dv_clean", "dk_corr", "dv_corr")


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


def run_resident(cfg, inp, shards, split=0):
    g = {k: v.to("cuda") for k, v in inp.items()}
    step = ResidentShardsStep(cfg.problem, shards, dkdv_split=split)
    # one separately allocated buffer per shard, as a rank would receive them
    k_sh = [g["k_clean"][o:o + n].clone() for (o, n, _) in shards]
    v_sh = [g["v_clean"][o:o + n].clone() for (o, n, _) in shards]
    poison_(step.o, step.o32, step.lse, step.delta, step.dq_acc, step.dq, step.dk_corr, step.dv_corr,
            *step.dk_shards, *step.dv_shards)
    args = (g["q"], k_sh, v_sh, g["k_corr"], g["v_corr"], g["dout"])
    step.step(*args)
    torch.cuda.synchronize()
    return dict(o=step.o, lse=step.lse, dq=step.dq, dk_clean=torch.cat(step.dk_shards),
                dv_clean=torch.cat(step.dv_shards), dk_corr=step.dk_corr, dv_corr=step.dv_corr,
                step=step, args=args)


def same_bits(a, b, label):
    for k in OUT:
        assert torch.equal(a[k], b[k]), f"{label}: {k} differs from the one-buffer run"


SPECS = [
    # L, B, ranks, rank, h_q, h_kv, d, clean shards (L / shards a multiple of 128)
    (512, 16, 4, 1, 4, 2, 128, 4),
    (2048, 32, 8, 5, 8, 2, 128, 8),
    (768, 16, 2, 1, 16, 2, 64, 3),
    (1024, 32, 4, 2, 8, 1, 128, 4),
]


@pytest.mark.parametrize("spec", SPECS, ids=lambda s: "L{}_B{}_R{}_r{}_h{}x{}_d{}_s{}".format(*s))
def test_resident_shards_small(spec):
    L, Bs, R, rank, hq, hkv, d, ns = spec
    cfg = wl.small_bdlm_config(L, Bs, R, rank, hq, hkv, d, ns)
    inp = wl.bdlm_inputs(cfg, seed=5)
    got = run_resident(cfg, inp, list(cfg.shards))
    compare_bdlm(got, oracle_bdlm_full(cfg, inp), cfg.name + " resident shards")
    same_bits(got, run_gpu_bdlm(cfg, inp, shards=[(0, L, True)]), cfg.name)


def test_resident_shards_gqa_4k():
    """The 4K GQA workload's four shards in four buffers (the plan splits its dK/dV
    key tiles over several workgroups, so the split reduction writes through the
    buffer table too)."""
    cfg = wl.config(2)
    inp = wl.bdlm_inputs(cfg, seed=0)
    got = run_resident(cfg, inp, list(cfg.shards))
    assert got["step"].plan.dkdv_split > 1
    compare_bdlm(got, oracle_bdlm_full(cfg, inp), cfg.name + " resident shards")
    same_bits(got, run_gpu_bdlm(cfg, inp, shards=[(0, cfg.problem.clean_len, True)]), cfg.name)


@pytest.mark.parametrize("split", [1, 3])
def test_resident_shards_ragged_last_buffer(split):
    """Buffers of 512, 512, 512 and 64 positions; the split factor forced to 1 and 3."""
    cfg = wl.small_bdlm_config(1600, 200, 2, 1, 2, 2, 64, 4)
    inp = wl.bdlm_inputs(cfg, seed=6)
    shards = [(0, 512, False), (512, 512, False), (1024, 512, False), (1536, 64, True)]
    got = run_resident(cfg, inp, shards, split=split)
    assert got["step"].shard_lens == [512, 512, 512, 64]
    compare_bdlm(got, oracle_bdlm_full(cfg, inp), f"{cfg.name} ragged split {split}")
    same_bits(got, run_gpu_bdlm(cfg, inp, shards=[(0, 1600, True)], dkdv_split=split), f"ragged split {split}")


def test_resident_shards_partial_span():
    """Shards covering positions 256 .. 1024 only (the plan's range does not start at
    0): bit for bit the one-buffer call over the same range."""
    cfg = wl.small_bdlm_config(1024, 32, 4, 2, 8, 1, 128, 4)
    inp = wl.bdlm_inputs(cfg, seed=7)
    shards = [(256, 256, False), (512, 256, True), (768, 256, False)]
    got = run_resident(cfg, inp, shards)
    one = run_gpu_bdlm(cfg, inp, shards=[(256, 768, True)])
    for k in ("o", "lse", "dq", "dk_corr", "dv_corr"):
        assert torch.equal(got[k], one[k]), k
    assert torch.equal(got["dk_clean"], one["dk_clean"][256:1024])
    assert torch.equal(got["dv_clean"], one["dv_clean"][256:1024])


def test_resident_shards_replayed_from_a_hip_graph():
    """The step captured once and replayed three times, with eager work between the
    replays: every replay gives the eager result bit for bit."""
    cfg = wl.config(2)
    inp = wl.bdlm_inputs(cfg, seed=0)
    eager = run_resident(cfg, inp, list(cfg.shards))
    want = {k: eager[k].clone() for k in OUT}
    step, args = eager["step"], eager["args"]
    sg = StepGraph(step, *args)
    for r in range(3):
        poison_(step.o, step.lse, step.dq, *step.dk_shards, *step.dv_shards, step.dk_corr, step.dv_corr)
        torch.cuda.synchronize()
        sg.replay()
        torch.cuda.synchronize()
        got = dict(o=step.o, lse=step.lse, dq=step.dq, dk_clean=torch.cat(step.dk_shards),
                   dv_clean=torch.cat(step.dv_shards), dk_corr=step.dk_corr, dv_corr=step.dv_corr)
        for k in OUT:
            assert torch.equal(got[k], want[k]), f"replay {r}: {k}"
        torch.randn(1 << 20, device="cuda").sum().item()   # eager work between replays


@pytest.mark.parametrize("lens,causal,split,tasks", [
    ([1, 5, 130, 64, 257, 300, 40], True, 0, False),
    ([600, 7, 129], False, 3, False),
    ([2000, 37], True, 0, False),              # 2037 keys: the full table of 16 buffers
    ([130, 64, 257, 900], True, 0, True),      # core-attention tasks with prefix contexts
])
def test_varlen_plan_over_shard_buffers(lens, causal, split, tasks):
    """A varlen (or task) plan whose packed K/V sit in buffers of 128 positions or more
    (the last holding the rest; documents span buffer boundaries): bit for bit the
    one-buffer calls."""
    from masked_long_context_amd import bdattn as B
    import numpy as np
    hq, hkv, d = 4, 2, 128
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    cfg = wl.VarlenConfig("t", tuple(lens), hq, hkv, d, causal, 1.0, "")
    g = {k: v.cuda() for k, v in wl.varlen_inputs(cfg, seed=9).items()}
    T = int(cu[-1])
    if tasks:
        # the documents as bounded tasks, each carrying its prefix context (gathered keys)
        q_cu, k_cu, src = B.cad_split(cu, 20000)
        rows = wl.task_context_rows(k_cu, src)
        g["k"], g["v"] = g["k"][torch.from_numpy(rows).long().cuda()], g["v"][torch.from_numpy(rows).long().cuda()]
        assert int(q_cu[-1]) == T and len(q_cu) > len(cu)
    n_keys = int(g["k"].shape[0])
    # buffers of 128 positions, or the smallest multiple of 128 that needs at most 16
    blen = max(128, -(-n_keys // (B.MAX_SHARDS * 128)) * 128)
    lens_b = B.shard_split(n_keys, -(-n_keys // blen), blen)
    starts = np.concatenate([[0], np.cumsum(lens_b)])
    ks = [g["k"][a:b].clone() for a, b in zip(starts[:-1], starts[1:])]
    vs = [g["v"][a:b].clone() for a, b in zip(starts[:-1], starts[1:])]
    outs = []
    for sharded in (False, True):
        plan = B.Plan.tasks(q_cu, k_cu, causal, hq, hkv, d) if tasks else B.Plan.varlen(cu, causal, hq, hkv, d)
        if split:
            plan.set_dkdv_split(split)
        ws = B.workspace(plan.workspace_bytes)
        o = torch.full((T, hq, d), float("nan"), dtype=torch.float32, device="cuda")
        lse = torch.full((hq, T), float("nan"), dtype=torch.float32, device="cuda")
        delta = torch.empty((hq, T), dtype=torch.float32, device="cuda")
        dq = torch.empty((T, hq, d), dtype=torch.float32, device="cuda")
        if sharded:
            dks = [torch.full_like(k, float("nan")) for k in ks]
            dvs = [torch.full_like(v, float("nan")) for v in vs]
            B.bdattn_fwd_shards(plan, g["q"], ks, vs, None, None, o, lse, ws)
            B.bdattn_bwd_prepare(plan, o, g["dout"], delta, dq)
            B.bdattn_bwd_shards(plan, g["q"], ks, vs, None, None, g["dout"], lse, delta, dq, dks, dvs, None, None, ws)
            dk, dv = torch.cat(dks), torch.cat(dvs)
        else:
            dk = torch.full_like(g["k"], float("nan"))
            dv = torch.full_like(g["v"], float("nan"))
            assert plan.n_kv(0) == n_keys
            B.bdattn_varlen_fwd(plan, g["q"], g["k"], g["v"], o, lse, ws)
            B.bdattn_bwd_prepare(plan, o, g["dout"], delta, dq)
            B.bdattn_varlen_bwd(plan, g["q"], g["k"], g["v"], g["dout"], lse, delta, dq, dk, dv, ws)
        torch.cuda.synchronize()
        outs.append((o, lse, dq, dk, dv))
    for name, a, b in zip(("o", "lse", "dq", "dk", "dv"), *outs):
        assert not torch.isnan(b.float()).any(), f"{name}: unwritten values"
        assert torch.equal(a, b), name
