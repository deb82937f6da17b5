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
              "bdattn_plan_create_tasks", "bdattn_cad_split"]:
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


class FakeTensor:
    """Stands in for a device tensor: only data_ptr/numel/dtype are read before validation fails."""

    def __init__(self, addr, numel=1 << 40, dtype=None):
        import torch
        self._a, self._n = addr, numel
        self.dtype = dtype or torch.bfloat16

    def data_ptr(self):
        return self._a

    def numel(self):
        return self._n


class FakeStream:
    cuda_stream = 0


def test_fwd_argument_errors_before_any_hip_call():
    import torch
    plan = B.Plan.bdlm(**_problem())
    good = FakeTensor(1 << 20)
    f32 = FakeTensor(1 << 20, dtype=torch.float32)
    ws_small = FakeTensor(1 << 20, numel=16)
    call = lambda **kw: B.bdattn_fwd(plan, **{**dict(q=good, k_clean=good, v_clean=good, k_corr=good,
                                                   v_corr=good, o=f32, lse=f32, ws=good,
                                                   stream=FakeStream()), **kw})
    assert _status(lambda: call(q=None)) == B.EINVAL
    assert _status(lambda: call(k_corr=None)) == B.EINVAL          # plan has local corrupted keys
    assert _status(lambda: call(q=FakeTensor((1 << 20) + 8))) == B.EALIGN
    assert _status(lambda: call(ws=FakeTensor((1 << 20) + 16))) == B.EALIGN
    assert _status(lambda: call(ws=ws_small)) == B.EWORKSPACE
    assert _status(lambda: call(o=FakeTensor(1 << 20, dtype=torch.float16))) == B.EUNSUPPORTED
    # a varlen plan is refused by the BDLM entry point and vice versa
    vplan = B.Plan.varlen([0, 100], True, 4, 2, 128)
    assert _status(lambda: B.bdattn_fwd(vplan, good, good, good, good, good, f32, f32, good,
                                        stream=FakeStream())) == B.EINVAL
    assert _status(lambda: B.bdattn_varlen_fwd(plan, good, good, good, f32, f32, good,
                                               stream=FakeStream())) == B.EINVAL


def test_bwd_and_prepare_argument_errors():
    import torch
    plan = B.Plan.bdlm(**_problem())
    good = FakeTensor(1 << 20)
    f32 = FakeTensor(1 << 20, dtype=torch.float32)
    st = FakeStream()
    args = dict(q=good, k_clean=good, v_clean=good, k_corr=good, v_corr=good, dout=good, lse=f32,
                delta=f32, dq_accum=f32, dk_clean=good, dv_clean=good, dk_corr=good,
                dv_corr=good, ws=good, stream=st)
    assert _status(lambda: B.bdattn_bwd(plan, **{**args, "dk_clean": None})) == B.EINVAL
    assert _status(lambda: B.bdattn_bwd(plan, **{**args, "dv_corr": None})) == B.EINVAL
    assert _status(lambda: B.bdattn_bwd(plan, **{**args, "ws": FakeTensor(1 << 20, numel=8)})) == B.EWORKSPACE
    assert _status(lambda: B.bdattn_bwd(plan, **{**args, "lse": FakeTensor((1 << 20) + 4)})) == B.EALIGN
    assert _status(lambda: B.bdattn_bwd_prepare(plan, None, good, f32, f32, st)) == B.EINVAL
    assert _status(lambda: B.bdattn_bwd_prepare(plan, good, good, None, None, st)) == B.EINVAL
    assert _status(lambda: B.bdattn_bwd_prepare(plan, FakeTensor(1 << 20, dtype=torch.float16), good, f32,
                                                None, st)) == B.EUNSUPPORTED
    vplan = B.Plan.varlen([0, 100], True, 4, 2, 128)
    assert _status(lambda: B.bdattn_bwd(vplan, **args)) == B.EINVAL
    dk_args = {k: v for k, v in args.items() if k != "dq_accum"}
    assert _status(lambda: B.bdattn_bwd_dkdv(plan, **{**dk_args, "dk_corr": None})) == B.EINVAL
    assert _status(lambda: B.bdattn_bwd_dkdv(plan, **{**dk_args, "ws": FakeTensor(1 << 20, numel=8)})) == B.EWORKSPACE
    dq_args = {k: v for k, v in args.items() if k not in ("dk_clean", "dv_clean", "dk_corr", "dv_corr")}
    assert _status(lambda: B.bdattn_bwd_dq(plan, **{**dq_args, "dq_accum": None})) == B.EINVAL
    assert _status(lambda: B.bdattn_bwd_dq(plan, **{**dq_args, "delta": FakeTensor((1 << 20) + 4)})) == B.EALIGN


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
