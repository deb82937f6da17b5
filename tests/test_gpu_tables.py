"""Plan tables kept in a workspace (bdattn_plan_keep_tables): calls of that plan
with that workspace skip their upload and give the same bits as calls that
upload, and an upload of another plan's tables into the workspace ends the first
plan's claim (its next call uploads again)."""
import pytest
import torch

from masked_long_context_amd import bdattn as B
from masked_long_context_amd import workloads as wl
from masked_long_context_amd.rank_step import BdlmRankStep, ResidentShardsStep
from gpu_util import need_gpu, poison_

pytestmark = pytest.mark.gpu

OUT = ("o", "lse", "dq", "dk_clean", "dv_clean", "dk_corr", "dv_corr")


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


def _run(step, g):
    poison_(step.o, step.lse, step.dq, step.dk_clean, step.dv_clean, step.dk_corr, step.dv_corr)
    step.step(g["q"], g["k_clean"], g["v_clean"], g["k_corr"], g["v_corr"], g["dout"])
    torch.cuda.synchronize()
    return {k: getattr(step, k).clone() for k in OUT}


@pytest.mark.parametrize("streams", [1, 3])
def test_kept_tables_give_the_same_bits(streams):
    cfg = wl.small_bdlm_config(2048, 32, 8, 5, 8, 2, 128, 8)
    g = {k: v.cuda() for k, v in wl.bdlm_inputs(cfg, seed=11).items()}
    kept = BdlmRankStep(cfg.problem, cfg.shards, streams=streams)
    plain = BdlmRankStep(cfg.problem, cfg.shards, streams=streams, keep_tables=False)
    assert kept.ws_plan is not None and plain.ws_plan is None
    a, b = _run(kept, g), _run(plain, g)
    a2 = _run(kept, g)   # second step: no upload at all
    for k in OUT:
        assert torch.equal(a[k], b[k]), k
        assert torch.equal(a2[k], b[k]), k


def test_another_plans_upload_ends_the_claim():
    """Plan A keeps its tables in ws; plan B's forward through the same ws uploads B's
    tables there; A's next forward through ws must upload A's tables again."""
    cfg = wl.small_bdlm_config(1024, 32, 4, 2, 8, 1, 128, 4)
    p = cfg.problem
    g = {k: v.cuda() for k, v in wl.bdlm_inputs(cfg, seed=12).items()}
    pa = B.Plan.from_problem(p.with_kv(0, 512, True))
    pb = B.Plan.from_problem(p.with_kv(512, 512, False))
    ws = B.workspace(max(pa.workspace_bytes, pb.workspace_bytes) + 256)
    pa.keep_tables(ws)

    def fwd_a():
        o = torch.full(pa.q_shape(), float("nan"), dtype=torch.float32, device="cuda")
        lse = torch.full(pa.lse_shape(), float("nan"), dtype=torch.float32, device="cuda")
        B.bdattn_fwd(pa, g["q"], g["k_clean"][:512], g["v_clean"][:512], g["k_corr"], g["v_corr"], o, lse, ws)
        torch.cuda.synchronize()
        return o, lse

    o1, l1 = fwd_a()
    ob = torch.empty(pb.q_shape(), dtype=torch.float32, device="cuda")
    lb = torch.empty(pb.lse_shape(), dtype=torch.float32, device="cuda")
    B.bdattn_fwd(pb, g["q"], g["k_clean"][512:], g["v_clean"][512:], None, None, ob, lb, ws)
    o2, l2 = fwd_a()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    # B's tables written 256 bytes into A's kept bytes (another start address) end
    # A's claim as well
    pa.keep_tables(ws)
    inner = ws[256:]
    assert inner.data_ptr() % 256 == 0 and inner.numel() >= pb.workspace_bytes
    B.bdattn_fwd(pb, g["q"], g["k_clean"][512:], g["v_clean"][512:], None, None, ob, lb, inner)
    o4, l4 = fwd_a()
    assert torch.equal(o1, o4) and torch.equal(l1, l4)
    # and a fresh workspace (no claim) gives the same bits
    ws2 = B.workspace(pa.workspace_bytes)
    o3 = torch.empty_like(o1)
    l3 = torch.empty_like(l1)
    B.bdattn_fwd(pa, g["q"], g["k_clean"][:512], g["v_clean"][:512], g["k_corr"], g["v_corr"], o3, l3, ws2)
    torch.cuda.synchronize()
    assert torch.equal(o1, o3) and torch.equal(l1, l3)
    pa.keep_tables(None)


def test_resident_shards_step_keeps_its_tables():
    cfg = wl.config(2)
    g = {k: v.cuda() for k, v in wl.bdlm_inputs(cfg, seed=0).items()}
    ks = [g["k_clean"][o:o + n].clone() for (o, n, _) in cfg.shards]
    vs = [g["v_clean"][o:o + n].clone() for (o, n, _) in cfg.shards]
    outs = []
    for keep in (True, False):
        st = ResidentShardsStep(cfg.problem, cfg.shards, keep_tables=keep)
        st.step(g["q"], ks, vs, g["k_corr"], g["v_corr"], g["dout"])
        torch.cuda.synchronize()
        outs.append([st.o.clone(), st.dq.clone(), torch.cat(st.dk_shards), torch.cat(st.dv_shards)])
    for a, b in zip(*outs):
        assert torch.equal(a, b)
