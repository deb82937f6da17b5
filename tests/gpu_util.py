"""Shared helpers of the GPU parity tests: run the HIP path through the C ABI,
run the oracle on the same seeded inputs, compare at the stated tolerances."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from masked_long_context_amd import workloads as wl
from masked_long_context_amd.rank_step import BdlmRankStep, TaskStep, VarlenStep

# bf16 outputs O, dQ, dK, dV: every element within TOL_MAX_ABS + TOL_REL_L2 |x| of the
# oracle's x (an absolute and a relative tolerance combined per element, as
# numpy.allclose does: a plain absolute 2e-2 cannot hold for large |x| in bf16, whose
# correct rounding alone is up to |x| 2^-9 away, 3e-2 at |x| = 9.6), and the
# tensor's relative L2 error within TOL_REL_L2; fp32 LSE: max abs error.
TOL_MAX_ABS = 2e-2
TOL_REL_L2 = 5e-3
TOL_LSE = 1e-5
SMALL_X = 4.0   # elements up to this magnitude are also held to TOL_MAX_ABS itself


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def to64(t) -> np.ndarray:
    if isinstance(t, np.ndarray):
        return t.astype(np.float64)
    return t.detach().to("cpu", torch.float64).numpy()


def check_close(name, got, want, max_abs=TOL_MAX_ABS, rel=TOL_REL_L2):
    g = to64(got)
    want = np.asarray(want, dtype=np.float64)
    assert g.shape == want.shape, (name, g.shape, want.shape)
    assert np.isfinite(g).all(), f"{name}: non-finite values (unwritten or overflow)"
    if g.size == 0:
        return 0.0, 0.0
    diff = g - want
    ma = float(np.abs(diff).max())
    nrm = float(np.linalg.norm(want))
    rl = float(np.linalg.norm(diff) / nrm) if nrm > 0 else float(np.linalg.norm(diff))
    floor = float(np.abs(torch.from_numpy(want).to(torch.bfloat16).double().numpy() - want).max())
    # each element against max_abs + rel |x|: the ratio must stay <= 1
    ratio = np.abs(diff) / (max_abs + rel * np.abs(want))
    worst = int(np.argmax(ratio))
    r_max = float(ratio.reshape(-1)[worst])
    print(f"  {name}: max_abs={ma:.3e} rel_l2={rl:.3e} element bound ratio={r_max:.3f} "
          f"(at |ref|={np.abs(want).reshape(-1)[worst]:.3e}; |ref|max={np.abs(want).max():.3e}, "
          f"bf16 rounding of ref alone: {floor:.3e})", flush=True)
    assert r_max <= 1.0, (f"{name}: element error {np.abs(diff).reshape(-1)[worst]:.3e} above "
                          f"{max_abs} + {rel} |ref| at |ref|={np.abs(want).reshape(-1)[worst]:.3e}")
    assert rl <= rel, f"{name}: relative L2 error {rl:.3e} > {rel}"
    # the plain absolute bound, wherever |x| <= 4 (there a bf16 value is within
    # 2^-8 of x, so the bound leaves room for the arithmetic)
    small = np.abs(want) <= SMALL_X
    if small.any():
        ma_small = float(np.abs(diff[small]).max())
        assert ma_small <= max_abs, f"{name}: max abs error {ma_small:.3e} > {max_abs} where |ref| <= {SMALL_X}"
    return ma, rl


def check_lse(name, got, want, tol=TOL_LSE):
    g = to64(got)
    want = np.asarray(want, dtype=np.float64)
    assert g.shape == want.shape
    assert not np.isnan(g).any(), f"{name}: NaN"
    gi, wi = np.isneginf(g), np.isneginf(want)
    assert np.array_equal(gi, wi), f"{name}: -inf pattern differs ({gi.sum()} vs {wi.sum()})"
    fin = ~wi
    ma = float(np.abs(g[fin] - want[fin]).max()) if fin.any() else 0.0
    print(f"  {name}: max_abs={ma:.3e} ({int(wi.sum())} rows -inf)", flush=True)
    assert ma <= tol, f"{name}: max abs error {ma:.3e} > {tol}"
    return ma


def oracle_prob(p, kv_offset=None, kv_len=None, local=None):
    return dict(clean_len=p.clean_len, block_size=p.block_size, q_clean_offset=p.q_clean_offset,
                q_clean_len=p.q_clean_len, owned_blocks=list(p.owned_blocks),
                kv_clean_offset=p.kv_clean_offset if kv_offset is None else kv_offset,
                kv_clean_len=p.kv_clean_len if kv_len is None else kv_len,
                with_local_corrupt=p.with_local_corrupt if local is None else local, scale=p.scale)


def oracle_bdlm_full(cfg: wl.BdlmConfig, inp) -> dict:
    """Unsharded fp64 reference of the whole rank share (all clean keys + local corrupted)."""
    p = cfg.problem
    prob = oracle_prob(p, 0, p.clean_len, True)
    q, kc, vc, kx, vx, do = (to64(inp[n]) for n in ("q", "k_clean", "v_clean", "k_corr", "v_corr", "dout"))
    o, lse = oracle.bdlm_fwd(prob, q, kc, vc, kx, vx)
    D = oracle.delta_rows(o, do)
    dq, dk, dv = oracle.bdlm_bwd(prob, q, kc, vc, kx, vx, do, lse, D)
    L = p.clean_len
    return dict(o=o, lse=lse, dq=dq, dk_clean=dk[:L], dv_clean=dv[:L], dk_corr=dk[L:], dv_corr=dv[L:])


def poison_(*ts):
    for t in ts:
        if t is not None and t.numel():
            t.fill_(float("nan"))


def run_gpu_bdlm(cfg: wl.BdlmConfig, inp, shards=None, poison=True, dkdv_split=0, exact_delta=True) -> dict:
    g = {k: v.to("cuda") for k, v in inp.items()}
    step = BdlmRankStep(cfg.problem, shards if shards is not None else cfg.shards, dkdv_split=dkdv_split,
                        exact_delta=exact_delta)
    if poison:
        poison_(step.o_parts, step.lse_parts, step.o, step.o32, step.lse, step.delta, step.dq_acc, step.dq,
                step.dk_clean, step.dv_clean, step.dk_corr, step.dv_corr)
    step.step(g["q"], g["k_clean"], g["v_clean"], g["k_corr"], g["v_corr"], g["dout"])
    torch.cuda.synchronize()
    return dict(o=step.o, lse=step.lse, dq=step.dq, dk_clean=step.dk_clean, dv_clean=step.dv_clean,
                dk_corr=step.dk_corr, dv_corr=step.dv_corr, step=step)


def compare_bdlm(got: dict, want: dict, label=""):
    print(f"[{label}]", flush=True)
    check_lse("lse", got["lse"], want["lse"])
    for k in ("o", "dq", "dk_clean", "dv_clean", "dk_corr", "dv_corr"):
        check_close(k, got[k], want[k])


def run_gpu_varlen(cu, causal, h_q, h_kv, d, inp, poison=True) -> dict:
    g = {k: v.to("cuda") for k, v in inp.items()}
    step = VarlenStep(cu, causal, h_q, h_kv, d)
    if poison:
        poison_(step.o, step.o32, step.lse, step.delta, step.dq_acc, step.dq, step.dk, step.dv)
    step.step(g["q"], g["k"], g["v"], g["dout"])
    torch.cuda.synchronize()
    return dict(o=step.o, lse=step.lse, dq=step.dq, dk=step.dk, dv=step.dv, step=step)


def oracle_varlen(cu, causal, scale, inp) -> dict:
    q, k, v, do = (to64(inp[n]) for n in ("q", "k", "v", "dout"))
    o, lse = oracle.varlen_fwd(q, k, v, cu, causal, scale)
    D = oracle.delta_rows(o, do)
    dq, dk, dv = oracle.varlen_bwd(q, k, v, do, lse, D, cu, causal, scale)
    return dict(o=o, lse=lse, dq=dq, dk=dk, dv=dv)


def run_gpu_tasks(q_cu, k_cu, causal, h_q, h_kv, d, inp, poison=True) -> dict:
    g = {k: v.to("cuda") for k, v in inp.items()}
    step = TaskStep(q_cu, k_cu, causal, h_q, h_kv, d)
    if poison:
        poison_(step.o, step.o32, step.lse, step.delta, step.dq_acc, step.dq, step.dk, step.dv)
    step.step(g["q"], g["k"], g["v"], g["dout"])
    torch.cuda.synchronize()
    return dict(o=step.o, lse=step.lse, dq=step.dq, dk=step.dk, dv=step.dv, step=step)


def oracle_tasks(q_cu, k_cu, causal, scale, inp) -> dict:
    q, k, v, do = (to64(inp[n]) for n in ("q", "k", "v", "dout"))
    o, lse = oracle.task_fwd(q, k, v, q_cu, k_cu, causal, scale)
    D = oracle.delta_rows(o, do)
    dq, dk, dv = oracle.task_bwd(q, k, v, do, lse, D, q_cu, k_cu, causal, scale)
    return dict(o=o, lse=lse, dq=dq, dk=dk, dv=dv)
