"""bdattn_fwd_static (the forward that allocates nothing: its tables live in a
static per-GPU device array) against bdattn_fwd (tables in a caller workspace):
the same kernel on the same inputs gives the same bits, on two calls in a row,
the second on a smaller problem (the array keeps the first call's tables, which
the second must overwrite where it reads them)."""
import ctypes

import pytest
import torch

from masked_long_context_amd import bdattn as B
from masked_long_context_amd import workloads as wl
from gpu_util import need_gpu

pytestmark = pytest.mark.gpu


def _run_both(cfg, shard):
    """One shard's forward through both entry points; returns (o, lse) of each."""
    off, n, local = cfg.shards[shard]
    p = cfg.problem.with_kv(off, n, local)
    plan = B.Plan.from_problem(p)
    inp = wl.bdlm_inputs(cfg, seed=11)
    g = {k: v.cuda() for k, v in inp.items()}
    kc, vc = g["k_clean"][off:off + n], g["v_clean"][off:off + n]
    kx, vx = (g["k_corr"], g["v_corr"]) if local else (None, None)
    outs = []
    for static in (False, True):
        o = torch.full(plan.q_shape(), float("nan"), dtype=torch.float32, device="cuda")
        lse = torch.full(plan.lse_shape(), float("nan"), dtype=torch.float32, device="cuda")
        if static:
            # through the C ABI directly: no workspace argument exists
            st = torch.cuda.current_stream().cuda_stream
            ptr = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())
            rc = B.lib().bdattn_fwd_static(plan.handle, ptr(g["q"]), ptr(kc), ptr(vc), ptr(kx), ptr(vx), ptr(o),
                                           B.F32, ptr(lse), ctypes.c_void_p(st))
            assert rc == B.OK, B.last_error()
        else:
            ws = B.workspace(plan.workspace_bytes)
            B.bdattn_fwd(plan, g["q"], kc, vc, kx, vx, o, lse, ws)
        torch.cuda.synchronize()
        outs.append((o, lse))
    return plan, outs


def test_static_forward_equals_workspace_forward_on_two_calls():
    need_gpu()
    big = wl.small_bdlm_config(4096, 32, 8, 5, 8, 2, 128, 4)       # 1024 rows, shard 2 holds the local keys
    small = wl.small_bdlm_config(1024, 16, 4, 1, 4, 2, 64, 4)      # 384 rows, d = 64
    for cfg, shard in ((big, 2), (small, 1)):
        plan, ((o_ws, l_ws), (o_st, l_st)) = _run_both(cfg, shard)
        assert plan.useful_pairs > 0
        assert not torch.isnan(o_st).any() and not torch.isnan(l_st).any(), cfg.name
        assert torch.equal(o_st, o_ws), cfg.name
        assert torch.equal(l_st, l_ws), cfg.name


def test_static_forward_binding_and_limit():
    """The binding form gives the same bits; a plan whose tables exceed the static
    array is rejected before any HIP call (8 MiB: about 500K query rows)."""
    need_gpu()
    cfg = wl.small_bdlm_config(2048, 32, 8, 5, 8, 2, 128, 8)
    plan, ((o_ws, l_ws), _) = _run_both(cfg, 5)
    off, n, local = cfg.shards[5]
    inp = wl.bdlm_inputs(cfg, seed=11)
    g = {k: v.cuda() for k, v in inp.items()}
    o = torch.empty(plan.q_shape(), dtype=torch.float32, device="cuda")
    lse = torch.empty(plan.lse_shape(), dtype=torch.float32, device="cuda")
    B.bdattn_fwd_static(plan, g["q"], g["k_clean"][off:off + n], g["v_clean"][off:off + n],
                        g["k_corr"] if local else None, g["v_corr"] if local else None, o, lse)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ws) and torch.equal(lse, l_ws)
    huge = B.Plan.bdlm(clean_len=1 << 20, block_size=64, q_clean_offset=0, q_clean_len=1 << 20, owned_blocks=[],
                       kv_clean_offset=0, kv_clean_len=64, with_local_corrupt=False, h_q=1, h_kv=1, head_dim=64)
    p_ = ctypes.c_void_p(1 << 20)
    assert B.lib().bdattn_fwd_static(huge.handle, p_, p_, p_, None, None, p_, B.F32, p_, None) == B.EWORKSPACE
