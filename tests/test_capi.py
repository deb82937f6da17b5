"""C ABI: the library loads, exports every symbol the header declares, and
rejects bad arguments with the documented status codes before any HIP call
(so these run on a machine without a GPU)."""
import ctypes
import os
import re

import numpy as np
import pytest

from masked_long_context_amd import bdattn as B

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "bdattn.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(bdattn_\w+)\s*\(", src)))


def test_header_declares_the_entry_points():
    names = _declared()
    for n in ["bdattn_fwd", "bdattn_bwd", "bdattn_lse_merge", "bdattn_varlen_fwd", "bdattn_varlen_bwd",
              "bdattn_plan_create", "bdattn_plan_create_varlen", "bdattn_bwd_prepare", "bdattn_dq_finalize",
              "bdattn_plan_create_tasks", "bdattn_cad_split", "bdattn_cast_f32_bf16", "bdattn_plan_heads"]:
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = B.lib()
    missing = [n for n in _declared() if not hasattr(lib, n)]
    assert not missing, missing


def _problem(**kw):
    d = dict(clean_len=256, block_size=32, q_clean_offset=64, q_clean_len=64, owned_blocks=[3, 1],
             kv_clean_offset=0, kv_clean_len=128, with_local_corrupt=True, h_q=4, h_kv=2, head_dim=128)
    d.update(kw)
    return d


def _status(fn):
    with pytest.raises(B.BdattnError) as e:
        fn()
    assert B.last_error()
    return e.value.status


@pytest.mark.parametrize("kw,code", [
    (dict(block_size=0), B.EINVAL),
    (dict(clean_len=250), B.EALIGN),
    (dict(q_clean_offset=16), B.EALIGN),
    (dict(q_clean_len=48), B.EALIGN),
    (dict(kv_clean_offset=8), B.EALIGN),
    (dict(kv_clean_len=300), B.EINVAL),
    (dict(owned_blocks=[8]), B.EINVAL),
    (dict(owned_blocks=[-1]), B.EINVAL),
    (dict(h_q=3, h_kv=2), B.EINVAL),
    (dict(h_q=0), B.EINVAL),
    (dict(head_dim=96), B.EUNSUPPORTED),
    (dict(head_dim=256), B.EUNSUPPORTED),
])
def test_plan_create_rejects(kw, code):
    assert _status(lambda: B.Plan.bdlm(**_problem(**kw))) == code


def test_varlen_plan_rejects():
    assert _status(lambda: B.Plan.varlen([1, 5], True, 4, 2, 128)) == B.EINVAL
    assert _status(lambda: B.Plan.varlen([0, 5, 3], True, 4, 2, 128)) == B.EINVAL
    assert _status(lambda: B.Plan.varlen([0, 5], True, 4, 2, 80)) == B.EUNSUPPORTED


def test_task_plan_rejects():
    assert _status(lambda: B.Plan.tasks([1, 5], [0, 5], True, 4, 2, 128)) == B.EINVAL
    assert _status(lambda: B.Plan.tasks([0, 5], [2, 5], True, 4, 2, 128)) == B.EINVAL
    assert _status(lambda: B.Plan.tasks([0, 5, 3], [0, 5, 9], True, 4, 2, 128)) == B.EINVAL
    assert _status(lambda: B.Plan.tasks([0, 5, 9], [0, 5, 4], True, 4, 2, 128)) == B.EINVAL
    assert _status(lambda: B.Plan.tasks([0, 5], [0, 5, 7], True, 4, 2, 128)) == B.EINVAL
    assert _status(lambda: B.Plan.tasks([0, 5], [0, 5], True, 3, 2, 128)) == B.EINVAL
    assert _status(lambda: B.Plan.tasks([0, 5], [0, 5], True, 4, 2, 96)) == B.EUNSUPPORTED
    big = 1 << 30
    assert _status(lambda: B.Plan.tasks([0, 1], [0, big], True, 4, 2, 128)) == B.EINVAL


def test_task_plan_null_and_negative_counts():
    lib = B.lib()
    h = ctypes.c_void_p()
    cu = (ctypes.c_int32 * 2)(0, 4)
    assert lib.bdattn_plan_create_tasks(None, cu, 1, 1, 4, 2, 128, 0.0, ctypes.byref(h)) == B.EINVAL
    assert lib.bdattn_plan_create_tasks(cu, None, 1, 1, 4, 2, 128, 0.0, ctypes.byref(h)) == B.EINVAL
    assert lib.bdattn_plan_create_tasks(cu, cu, -1, 1, 4, 2, 128, 0.0, ctypes.byref(h)) == B.EINVAL
    assert lib.bdattn_plan_create_tasks(cu, cu, 1, 1, 4, 2, 128, 0.0, None) == B.EINVAL


def test_cad_split_rejects():
    lib = B.lib()
    cu = (ctypes.c_int32 * 3)(0, 4, 9)
    assert lib.bdattn_cad_split(None, 2, 10, None, None, None, 0) == B.EINVAL
    assert lib.bdattn_cad_split(cu, -1, 10, None, None, None, 0) == B.EINVAL
    assert lib.bdattn_cad_split(cu, 2, 0, None, None, None, 0) == B.EINVAL
    assert lib.bdattn_cad_split(cu, 2, 10, None, None, None, -1) == B.EINVAL
    assert lib.bdattn_cad_split(cu, 2, 10, None, None, None, 4) == B.EINVAL   # cap > 0, NULL outputs
    assert _status(lambda: B.cad_split([1, 4], 10)) == B.EINVAL
    assert _status(lambda: B.cad_split([0, 4, 2], 10)) == B.EINVAL
    # one 2^16-row document cut into single rows: contexts sum to ~2^31 rows
    assert _status(lambda: B.cad_split([0, 1 << 16], 1)) == B.EINVAL
    # counting call (cap = 0) writes nothing and returns the task count
    assert lib.bdattn_cad_split(cu, 2, 10, None, None, None, 0) == 3


def _addr(a):
    return ctypes.c_void_p(a)


def test_fwd_argument_errors_before_any_hip_call():
    """C-level validation of bdattn_fwd / bdattn_varlen_fwd (fake device addresses: every
    call below fails before the library touches them)."""
    lib = B.lib()
    plan = B.Plan.bdlm(**_problem())
    good = 1 << 20
    ws_n = plan.workspace_bytes
    args = dict(q=good, k_clean=good, v_clean=good, k_corr=good, v_corr=good, o=good, o_dtype=B.F32, lse=good,
                ws=good, ws_bytes=ws_n)

    def call(**kw):
        a = {**args, **kw}
        ptr = lambda x: None if x is None else _addr(x)
        return lib.bdattn_fwd(plan.handle, ptr(a["q"]), ptr(a["k_clean"]), ptr(a["v_clean"]), ptr(a["k_corr"]),
                              ptr(a["v_corr"]), ptr(a["o"]), a["o_dtype"], ptr(a["lse"]), ptr(a["ws"]),
                              a["ws_bytes"], None)

    assert call(q=None) == B.EINVAL
    assert call(k_corr=None) == B.EINVAL          # the plan has local corrupted keys
    assert call(q=good + 8) == B.EALIGN
    assert call(ws=good + 16) == B.EALIGN
    assert call(ws_bytes=16) == B.EWORKSPACE
    assert call(o_dtype=7) == B.EUNSUPPORTED
    # a varlen plan is refused by the BDLM entry point and vice versa
    vplan = B.Plan.varlen([0, 100], True, 4, 2, 128)
    p_ = _addr(good)
    assert lib.bdattn_fwd(vplan.handle, p_, p_, p_, p_, p_, p_, B.F32, p_, p_, vplan.workspace_bytes, None) == B.EINVAL
    assert lib.bdattn_varlen_fwd(plan.handle, p_, p_, p_, p_, B.F32, p_, p_, ws_n, None) == B.EINVAL


def test_bwd_and_prepare_argument_errors():
    lib = B.lib()
    plan = B.Plan.bdlm(**_problem())
    good = 1 << 20
    names = ["q", "k_clean", "v_clean", "k_corr", "v_corr", "dout", "lse", "delta", "dq_accum", "dk_clean",
             "dv_clean", "dk_corr", "dv_corr", "ws"]
    base = {n: good for n in names}

    def call(fn, skip=(), ws_bytes=None, **kw):
        a = {**base, **kw}
        ptrs = [None if a[n] is None else _addr(a[n]) for n in names if n not in skip]
        return fn(plan.handle, *ptrs, plan.workspace_bytes if ws_bytes is None else ws_bytes, None)

    assert call(lib.bdattn_bwd, dk_clean=None) == B.EINVAL
    assert call(lib.bdattn_bwd, dv_corr=None) == B.EINVAL
    assert call(lib.bdattn_bwd, ws_bytes=8) == B.EWORKSPACE
    assert call(lib.bdattn_bwd, lse=good + 4) == B.EALIGN
    dk_skip = ("dq_accum",)
    assert call(lib.bdattn_bwd_dkdv, skip=dk_skip, dk_corr=None) == B.EINVAL
    assert call(lib.bdattn_bwd_dkdv, skip=dk_skip, ws_bytes=8) == B.EWORKSPACE
    dq_skip = ("dk_clean", "dv_clean", "dk_corr", "dv_corr")
    assert call(lib.bdattn_bwd_dq, skip=dq_skip, dq_accum=None) == B.EINVAL
    assert call(lib.bdattn_bwd_dq, skip=dq_skip, delta=good + 4) == B.EALIGN
    vplan = B.Plan.varlen([0, 100], True, 4, 2, 128)
    p_ = _addr(good)
    assert lib.bdattn_bwd(vplan.handle, *([p_] * 14), vplan.workspace_bytes, None) == B.EINVAL
    # preparation: NULL output / input, unsupported O dtype
    assert lib.bdattn_bwd_prepare(plan.handle, None, B.BF16, p_, p_, p_, None) == B.EINVAL
    assert lib.bdattn_bwd_prepare(plan.handle, p_, B.BF16, p_, None, None, None) == B.EINVAL
    assert lib.bdattn_bwd_prepare(plan.handle, p_, 5, p_, p_, None, None) == B.EUNSUPPORTED
    assert lib.bdattn_bwd_prepare(None, p_, B.BF16, p_, p_, None, None) == B.EINVAL


def _cpu(shape, dtype=None):
    import torch
    return torch.zeros(shape, dtype=dtype or torch.bfloat16)


def test_binding_checks_every_tensor_before_the_call():
    """The ctypes binding checks dtype, shape (from the plan), contiguity and device
    of every tensor before calling into the library (CPU tensors: the device check
    is the last one, so each earlier rejection is reachable here)."""
    import torch
    plan = B.Plan.bdlm(**_problem())
    n_q, hq, d = plan.q_shape()
    assert (n_q, hq, d) == (128, 4, 128) and plan.heads == (4, 2, 128)
    kv0, kv1 = plan.kv_shape(0), plan.kv_shape(1)
    assert kv0 == (128, 2, 128) and kv1 == (64, 2, 128)
    f32 = torch.float32
    ok = dict(q=_cpu((n_q, hq, d)), k_clean=_cpu(kv0), v_clean=_cpu(kv0), k_corr=_cpu(kv1), v_corr=_cpu(kv1),
              o=_cpu((n_q, hq, d), f32), lse=_cpu((hq, n_q), f32), ws=_cpu((plan.workspace_bytes,), torch.uint8))
    fwd = lambda **kw: B.bdattn_fwd(plan, **{**ok, **kw})

    def err(fn, code, text):
        with pytest.raises(B.BdattnError) as e:
            fn()
        assert e.value.status == code, (e.value, code)
        assert text in str(e.value), (str(e.value), text)

    err(lambda: fwd(q=_cpu((n_q, hq, d), f32)), B.EUNSUPPORTED, "q has dtype")
    err(lambda: fwd(q=_cpu((n_q - 1, hq, d))), B.EINVAL, "q has shape")
    err(lambda: fwd(k_clean=_cpu((kv0[0] - 32,) + kv0[1:])), B.EINVAL, "k_clean has shape")
    err(lambda: fwd(v_corr=_cpu((kv1[0] + 32,) + kv1[1:])), B.EINVAL, "v_corr has shape")
    err(lambda: fwd(k_corr=None), B.EINVAL, "k_corr is None")
    err(lambda: fwd(o=_cpu((n_q, hq, d), torch.float16)), B.EUNSUPPORTED, "o has dtype")
    err(lambda: fwd(lse=_cpu((n_q, hq), f32)), B.EINVAL, "lse has shape")
    err(lambda: fwd(q=_cpu((n_q, d, hq)).transpose(1, 2)), B.EINVAL, "q must be contiguous")
    err(lambda: fwd(ws=_cpu((plan.workspace_bytes,), f32)), B.EUNSUPPORTED, "workspace has dtype")
    err(lambda: fwd(q="not a tensor"), B.EINVAL, "must be a torch.Tensor")
    err(lambda: fwd(), B.EINVAL, "must be a GPU tensor")
    # backward: the row side (dout, lse, delta, dq_accum) and the gradients follow the plan too
    bw = dict(q=ok["q"], k_clean=ok["k_clean"], v_clean=ok["v_clean"], k_corr=ok["k_corr"], v_corr=ok["v_corr"],
              dout=_cpu((n_q, hq, d)), lse=ok["lse"], delta=_cpu((hq, n_q), f32), dq_accum=_cpu((n_q, hq, d), f32),
              dk_clean=_cpu(kv0), dv_clean=_cpu(kv0), dk_corr=_cpu(kv1), dv_corr=_cpu(kv1), ws=ok["ws"])
    bwd = lambda **kw: B.bdattn_bwd(plan, **{**bw, **kw})
    err(lambda: bwd(dout=_cpu((n_q, hq, d), f32)), B.EUNSUPPORTED, "dout has dtype")
    err(lambda: bwd(delta=_cpu((hq, n_q + 1), f32)), B.EINVAL, "delta has shape")
    err(lambda: bwd(dq_accum=_cpu((n_q, hq, d))), B.EUNSUPPORTED, "dq_accum has dtype")
    err(lambda: bwd(dk_clean=_cpu((kv0[0], 1, d))), B.EINVAL, "dk_clean has shape")
    err(lambda: bwd(dv_corr=None), B.EINVAL, "dv_corr is None")
    err(lambda: bwd(), B.EINVAL, "must be a GPU tensor")
    err(lambda: B.bdattn_bwd_prepare(plan, ok["o"], bw["dout"], _cpu((hq, n_q))), B.EUNSUPPORTED, "delta has dtype")
    # merge: partial shapes follow o_parts
    S = 3
    op, lp = _cpu((S, n_q, hq, d), f32), _cpu((S, hq, n_q), f32)
    err(lambda: B.bdattn_lse_merge(op, _cpu((S, n_q, hq), f32), ok["o"], ok["lse"]), B.EINVAL, "lse_parts has shape")
    err(lambda: B.bdattn_lse_merge(op, lp, _cpu((n_q, hq, d - 1), f32), ok["lse"]), B.EINVAL, "o_out has shape")
    err(lambda: B.bdattn_lse_merge(op[:, :, :, :64], lp, ok["o"], ok["lse"]), B.EINVAL, "contiguous")
    err(lambda: B.bdattn_dq_finalize(ok["o"], _cpu((n_q, hq, d + 8))), B.EINVAL, "dq has shape")
    err(lambda: B.bdattn_cast_f32_bf16(ok["o"], _cpu((n_q, hq, d), f32)), B.EUNSUPPORTED, "dst has dtype")
    # varlen: K/V and gradients follow the packed key count
    vplan = B.Plan.varlen([0, 100, 164], True, 4, 2, 128)
    vq, vk = _cpu(vplan.q_shape()), _cpu(vplan.kv_shape(0))
    err(lambda: B.bdattn_varlen_fwd(vplan, vq, _cpu((100, 2, 128)), vk, _cpu(vplan.q_shape(), f32),
                                    _cpu(vplan.lse_shape(), f32), _cpu((vplan.workspace_bytes,), torch.uint8)),
        B.EINVAL, "k has shape")


def test_plans_beyond_the_size_limits_are_rejected():
    """Row and key counts of 2^30 or more, and grids beyond 2^32 work-items, never
    reach a kernel (the rejection happens before any table is built)."""
    lim = 1 << 30
    assert _status(lambda: B.Plan.varlen([0, lim], True, 4, 2, 128)) == B.EINVAL
    assert _status(lambda: B.Plan.tasks([0, lim], [0, 1], True, 4, 2, 128)) == B.EINVAL
    assert _status(lambda: B.Plan.bdlm(**_problem(clean_len=2 * lim, block_size=1 << 20, q_clean_offset=0,
                                                  q_clean_len=lim, owned_blocks=[], kv_clean_len=1 << 20))) == B.EINVAL
    assert _status(lambda: B.Plan.bdlm(**_problem(clean_len=2 * lim, block_size=1 << 20, q_clean_offset=0,
                                                  q_clean_len=1 << 20, owned_blocks=[], kv_clean_len=lim))) == B.EINVAL
    # 2^22 rows in 256-row shards x 4096 q-heads: the forward grid would hold
    # 2^22 / 256 * 4096 * 512 = 2^35 work-items
    cu = np.arange(0, (1 << 22) + 1, 256, dtype=np.int32)
    assert _status(lambda: B.Plan.varlen(cu, True, 4096, 1, 64)) == B.EUNSUPPORTED


def test_merge_and_finalize_argument_errors():
    lib = B.lib()
    p = ctypes.c_void_p(1 << 20)
    assert lib.bdattn_lse_merge(0, p, B.F32, p, 10, 2, 128, p, B.BF16, p, None) == B.EINVAL
    assert lib.bdattn_lse_merge(2, p, B.F32, p, 10, 2, 96, p, B.BF16, p, None) == B.EUNSUPPORTED
    assert lib.bdattn_lse_merge(2, p, 7, p, 10, 2, 128, p, B.BF16, p, None) == B.EUNSUPPORTED
    assert lib.bdattn_lse_merge(2, None, B.F32, p, 10, 2, 128, p, B.BF16, p, None) == B.EINVAL
    assert lib.bdattn_lse_merge(2, ctypes.c_void_p((1 << 20) + 4), B.F32, p, 10, 2, 128, p, B.BF16, p,
                                None) == B.EALIGN
    assert lib.bdattn_dq_finalize(None, p, 100, None) == B.EINVAL
    assert lib.bdattn_dq_finalize(p, p, -1, None) == B.EINVAL
    assert lib.bdattn_cast_f32_bf16(p, None, 100, None) == B.EINVAL
    assert lib.bdattn_cast_f32_bf16(ctypes.c_void_p((1 << 20) + 2), p, 100, None) == B.EALIGN
    # n_rows * h * d / 4 threads beyond 2^32 work-items
    assert lib.bdattn_lse_merge(2, p, B.F32, p, 1 << 28, 2, 128, p, B.BF16, p, None) == B.EUNSUPPORTED
    # nothing to do is not an error and touches no device
    assert lib.bdattn_lse_merge(2, None, B.F32, None, 0, 2, 128, None, B.BF16, None, None) == B.OK
    assert lib.bdattn_dq_finalize(None, None, 0, None) == B.OK


def test_plan_sizes_and_counts():
    plan = B.Plan.bdlm(**_problem())
    assert plan.n_q == 64 + 2 * 32
    assert plan.n_kv(0) == 128 and plan.n_kv(1) == 64
    assert plan.workspace_bytes > 0 and plan.workspace_bytes % 256 == 0
    # clean rows at positions 64..127 (blocks 2, 3) see keys [0, 96) and [0, 128) of the range;
    # block 3 sees [0, 96) plus its own 32; block 1 sees [0, 32) plus its own 32
    assert plan.useful_pairs == 32 * 96 + 32 * 128 + 32 * (96 + 32) + 32 * (32 + 32)


def test_dkdv_split_choice_and_override():
    """The automatic dK/dV split leaves a problem with many key tiles unsplit and
    splits a small one; an override is validated, resizes the workspace for the
    fp32 partials ([2][split][n_seg][h_kv][d] per segment), and 1 removes them."""
    # one clean K/V range of 16384 keys, 8 KV heads: 128 key tiles x 8 heads = 1024 workgroups
    big = B.Plan.bdlm(clean_len=262144, block_size=32, q_clean_offset=131072, q_clean_len=16384,
                      owned_blocks=list(range(2048, 2304)), kv_clean_offset=0, kv_clean_len=16384,
                      with_local_corrupt=False, h_q=32, h_kv=8, head_dim=128)
    assert big.dkdv_split == 1
    small = B.Plan.bdlm(**_problem())
    base = small.workspace_bytes
    for bad in (-1, 9, 100):
        with pytest.raises(B.BdattnError) as e:
            small.set_dkdv_split(bad)
        assert e.value.status == B.EINVAL
    small.set_dkdv_split(1)
    assert small.dkdv_split == 1
    unsplit = small.workspace_bytes
    small.set_dkdv_split(4)
    assert small.dkdv_split == 4
    keys = small.n_kv(0) + small.n_kv(1)
    assert small.workspace_bytes >= unsplit + 2 * 4 * keys * 2 * 128 * 4   # dK+dV, split 4, h_kv 2, d 128, fp32
    small.set_dkdv_split(1)
    assert small.workspace_bytes == unsplit
    small.set_dkdv_split(0)
    assert small.workspace_bytes == base


def _shard_plan():
    # 384 clean keys of the call: three buffers of 128
    return B.Plan.bdlm(**_problem(clean_len=512, kv_clean_len=384))


def _table(n=3, length=128, good=1 << 20, **set_):
    """A bdattn_kv_shards struct over fake device addresses; set_ maps 'k1' (array k,
    entry 1) and the like to a replacement address (0 = NULL)."""
    t = B.KvShards()
    t.n_shards, t.shard_len = n, length
    for i in range(B.MAX_SHARDS):
        t.k[i] = t.v[i] = t.dk[i] = t.dv[i] = good
    for key, val in set_.items():
        getattr(t, key[:-1])[int(key[-1])] = val or None
    return t


def test_shard_table_argument_errors_before_any_hip_call():
    """bdattn_fwd_shards and the bdattn_bwd*_shards calls check the buffer table against
    the plan's clean range (count, alignment, coverage, pointers) before any HIP call."""
    lib = B.lib()
    plan = _shard_plan()
    assert plan.n_kv(0) == 384
    good = 1 << 20
    p_ = _addr(good)
    ws_n = plan.workspace_bytes

    def fwd(t, ws_bytes=ws_n):
        kv = None if t is None else ctypes.byref(t)
        return lib.bdattn_fwd_shards(plan.handle, p_, kv, p_, p_, p_, B.F32, p_, p_, ws_bytes, None)

    assert fwd(None) == B.EINVAL
    assert fwd(_table(n=0)) == B.EINVAL
    assert fwd(_table(n=B.MAX_SHARDS + 1)) == B.EINVAL
    assert fwd(_table(length=100)) == B.EALIGN
    assert fwd(_table(length=0)) == B.EALIGN
    assert fwd(_table(length=-128)) == B.EALIGN
    assert fwd(_table(length=256)) == B.EINVAL          # the third buffer would hold nothing
    assert fwd(_table(n=2, length=128)) == B.EINVAL      # 256 positions cannot hold 384
    assert fwd(_table(n=2, length=1 << 40)) == B.EINVAL  # huge lengths do not wrap
    assert fwd(_table(k1=0)) == B.EINVAL
    assert fwd(_table(v2=good + 8)) == B.EALIGN
    # a valid table gets as far as the workspace check (shard_len is ignored for one buffer)
    assert fwd(_table(), ws_bytes=8) == B.EWORKSPACE
    assert fwd(_table(n=1, length=7), ws_bytes=8) == B.EWORKSPACE
    assert fwd(_table(n=2, length=256), ws_bytes=8) == B.EWORKSPACE   # last buffer holds 128

    def bwd(fn, t, n_ptrs, ws_bytes=ws_n):
        return fn(plan.handle, p_, ctypes.byref(t), *([p_] * n_ptrs), ws_bytes, None)

    # bdattn_bwd_shards: k_corr v_corr dout lse delta dq dk_corr dv_corr ws (9 pointers)
    assert bwd(lib.bdattn_bwd_shards, _table(dk1=0), 9) == B.EINVAL
    assert bwd(lib.bdattn_bwd_shards, _table(dv0=good + 4), 9) == B.EALIGN
    assert bwd(lib.bdattn_bwd_shards, _table(length=96), 9) == B.EALIGN
    assert bwd(lib.bdattn_bwd_shards, _table(), 9, ws_bytes=8) == B.EWORKSPACE
    # dK/dV only (8 pointers): gradient buffers needed
    assert bwd(lib.bdattn_bwd_dkdv_shards, _table(dv2=0), 8) == B.EINVAL
    assert bwd(lib.bdattn_bwd_dkdv_shards, _table(), 8, ws_bytes=8) == B.EWORKSPACE
    # dQ only (7 pointers): the gradient entries are not read, so NULL ones pass the table check
    t = _table()
    for i in range(B.MAX_SHARDS):
        t.dk[i] = t.dv[i] = None
    assert bwd(lib.bdattn_bwd_dq_shards, t, 7, ws_bytes=8) == B.EWORKSPACE
    assert bwd(lib.bdattn_bwd_dq_shards, _table(k0=0), 7) == B.EINVAL
    assert lib.bdattn_fwd_shards(None, p_, ctypes.byref(_table()), p_, p_, p_, B.F32, p_, p_, ws_n, None) == B.EINVAL


def test_shard_split_rules():
    assert B.shard_split(384, 3, 128) == [128, 128, 128]
    assert B.shard_split(300, 3, 128) == [128, 128, 44]
    assert B.shard_split(77, 1, 0) == [77]
    assert _status(lambda: B.shard_split(256, 3, 128)) == B.EINVAL
    assert _status(lambda: B.shard_split(384, 2, 128)) == B.EINVAL
    assert _status(lambda: B.shard_split(384, 3, 100)) == B.EALIGN
    assert _status(lambda: B.shard_split(384, 0, 128)) == B.EINVAL
    assert _status(lambda: B.shard_split(384, B.MAX_SHARDS + 1, 128)) == B.EINVAL


def test_binding_checks_shard_buffers():
    """bdattn_fwd_shards in the binding: each buffer's dtype, length (from the split),
    contiguity, then the device (CPU tensors reach only the last check)."""
    import torch
    plan = _shard_plan()
    n_q, hq, d = plan.q_shape()
    _, hkv, _ = plan.kv_shape(0)
    kv1 = plan.kv_shape(1)
    f32 = torch.float32
    ks = [_cpu((128, hkv, d)) for _ in range(3)]
    vs = [_cpu((128, hkv, d)) for _ in range(3)]
    ok = dict(q=_cpu((n_q, hq, d)), k_shards=ks, v_shards=vs, k_corr=_cpu(kv1), v_corr=_cpu(kv1),
              o=_cpu((n_q, hq, d), f32), lse=_cpu((hq, n_q), f32), ws=_cpu((plan.workspace_bytes,), torch.uint8))
    call = lambda **kw: B.bdattn_fwd_shards(plan, **{**ok, **kw})

    def err(code, text, **kw):
        with pytest.raises(B.BdattnError) as e:
            call(**kw)
        assert e.value.status == code and text in str(e.value), str(e.value)

    err(B.EINVAL, "must be a GPU tensor")
    err(B.EINVAL, "same length", v_shards=vs[:2])
    err(B.EINVAL, "k_shards[2] has shape", k_shards=ks[:2] + [_cpu((64, hkv, d))])
    err(B.EUNSUPPORTED, "v_shards[1] has dtype", v_shards=[vs[0], _cpu((128, hkv, d), f32), vs[2]])
    err(B.EINVAL, "v_shards[0] must be contiguous",
        v_shards=[_cpu((hkv, 128, d)).transpose(0, 1), vs[1], vs[2]])
    err(B.EALIGN, "multiple of 128", k_shards=[_cpu((96, hkv, d))] * 4, v_shards=[_cpu((96, hkv, d))] * 4)
    # the backward's gradient lists are checked the same way
    with pytest.raises(B.BdattnError) as e:
        B.bdattn_bwd_dkdv_shards(plan, ok["q"], ks, vs, ok["k_corr"], ok["v_corr"], _cpu((n_q, hq, d)),
                                 ok["lse"], _cpu((hq, n_q), f32), ks, vs[:1], _cpu(kv1), _cpu(kv1), ok["ws"])
    assert e.value.status == B.EINVAL and "one tensor per K/V buffer" in str(e.value)


def test_resident_shards_step_rejects_uneven_or_gapped_shards():
    from masked_long_context_amd import workloads as wl
    from masked_long_context_amd.rank_step import ResidentShardsStep
    cfg = wl.small_bdlm_config(512, 16, 4, 1, 4, 2, 128, 4)
    with pytest.raises(ValueError, match="consecutive"):
        ResidentShardsStep(cfg.problem, [(0, 128, False), (256, 128, True)])
    with pytest.raises(B.BdattnError):
        ResidentShardsStep(cfg.problem, [(0, 256, False), (256, 128, False), (384, 128, True)])
    with pytest.raises(B.BdattnError):
        ResidentShardsStep(cfg.problem, [(0, 96, False), (96, 96, False), (192, 320, True)])


def test_keep_tables_argument_errors_before_any_hip_call():
    lib = B.lib()
    plan = B.Plan.bdlm(**_problem())
    good = 1 << 20
    n = plan.workspace_bytes
    assert lib.bdattn_plan_keep_tables(None, _addr(good), n, None) == B.EINVAL
    assert lib.bdattn_plan_keep_tables(plan.handle, _addr(good + 16), n, None) == B.EALIGN
    assert lib.bdattn_plan_keep_tables(plan.handle, _addr(good), n - 1, None) == B.EWORKSPACE
    # NULL ends a claim (none held here): no HIP call
    assert lib.bdattn_plan_keep_tables(plan.handle, None, 0, None) == B.OK
    plan.keep_tables(None)
    with pytest.raises(B.BdattnError) as e:
        plan.keep_tables(_cpu((n,), __import__("torch").uint8))
    assert e.value.status == B.EINVAL and "GPU tensor" in str(e.value)
