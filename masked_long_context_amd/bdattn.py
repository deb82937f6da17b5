"""ctypes binding of libbdattn.so: the C entry points under the same names.

Argument marshalling only: tensors become device pointers, the stream is
torch's current HIP stream, status codes become exceptions.  Every step of the
computation runs in the library's HIP kernels; there is no fallback.  PyTorch
supplies device memory and streams.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libbdattn.so")

OK, EINVAL, EALIGN, EUNSUPPORTED, EWORKSPACE, EHIP = 0, -1, -2, -3, -4, -5
BF16, F32 = 0, 1
STATUS_NAMES = {0: "OK", -1: "EINVAL", -2: "EALIGN", -3: "EUNSUPPORTED", -4: "EWORKSPACE", -5: "EHIP"}

c_int32, c_int64, c_float, c_void_p = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_void_p


class BdattnError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {msg}")
        self.status = status


class Problem(ctypes.Structure):
    """Mirror of bdattn_problem."""
    _fields_ = [("clean_len", c_int64), ("block_size", c_int32), ("q_clean_offset", c_int64),
                ("q_clean_len", c_int64), ("owned_blocks", ctypes.POINTER(c_int64)), ("n_owned", c_int64),
                ("kv_clean_offset", c_int64), ("kv_clean_len", c_int64), ("with_local_corrupt", c_int32),
                ("h_q", c_int32), ("h_kv", c_int32), ("head_dim", c_int32), ("softmax_scale", c_float)]


_LIB = None

_SIGS = {
    "bdattn_plan_create": (c_int32, [ctypes.POINTER(Problem), ctypes.POINTER(c_void_p)]),
    "bdattn_plan_create_varlen": (c_int32, [ctypes.POINTER(c_int32), c_int32, c_int32, c_int32, c_int32,
                                            c_int32, c_float, ctypes.POINTER(c_void_p)]),
    "bdattn_plan_create_tasks": (c_int32, [ctypes.POINTER(c_int32), ctypes.POINTER(c_int32), c_int32, c_int32,
                                           c_int32, c_int32, c_int32, c_float, ctypes.POINTER(c_void_p)]),
    "bdattn_cad_split": (c_int64, [ctypes.POINTER(c_int32), c_int32, c_int64, ctypes.POINTER(c_int32),
                                   ctypes.POINTER(c_int32), ctypes.POINTER(c_int32), c_int64]),
    "bdattn_plan_destroy": (None, [c_void_p]),
    "bdattn_plan_workspace_bytes": (c_int64, [c_void_p]),
    "bdattn_plan_useful_pairs": (c_int64, [c_void_p]),
    "bdattn_plan_set_dkdv_split": (c_int32, [c_void_p, c_int32]),
    "bdattn_plan_dkdv_split": (c_int32, [c_void_p]),
    "bdattn_plan_n_q": (c_int64, [c_void_p]),
    "bdattn_plan_n_kv": (c_int64, [c_void_p, c_int32]),
    "bdattn_plan_export": (c_int64, [c_void_p, c_int32, c_void_p, c_int64]),
    "bdattn_fwd": (c_int32, [c_void_p] * 7 + [c_int32, c_void_p, c_void_p, c_int64, c_void_p]),
    "bdattn_lse_merge": (c_int32, [c_int32, c_void_p, c_int32, c_void_p, c_int64, c_int32, c_int32, c_void_p,
                                   c_int32, c_void_p, c_void_p]),
    "bdattn_bwd_prepare": (c_int32, [c_void_p, c_void_p, c_int32, c_void_p, c_void_p, c_void_p, c_void_p]),
    "bdattn_bwd": (c_int32, [c_void_p] * 15 + [c_int64, c_void_p]),
    "bdattn_bwd_dkdv": (c_int32, [c_void_p] * 14 + [c_int64, c_void_p]),
    "bdattn_bwd_dq": (c_int32, [c_void_p] * 11 + [c_int64, c_void_p]),
    "bdattn_dq_finalize": (c_int32, [c_void_p, c_void_p, c_int64, c_void_p]),
    "bdattn_varlen_fwd": (c_int32, [c_void_p] * 5 + [c_int32, c_void_p, c_void_p, c_int64, c_void_p]),
    "bdattn_varlen_bwd": (c_int32, [c_void_p] * 11 + [c_int64, c_void_p]),
    "bdattn_last_error": (ctypes.c_char_p, []),
}


def lib():
    """Load libbdattn.so (after torch, so both share one HIP runtime)."""
    global _LIB
    if _LIB is None:
        import torch  # noqa: F401  (loads the HIP runtime the library binds to)
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built: run `python -m masked_long_context_amd.build`")
        h = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(h, name)
            f.restype = res
            f.argtypes = args
        _LIB = h
    return _LIB


def _check(rc: int):
    if rc != OK:
        raise BdattnError(rc, lib().bdattn_last_error().decode())


def _ptr(t):
    return None if t is None else c_void_p(t.data_ptr())


def _stream(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return c_void_p(stream.cuda_stream)


def _dtype_code(t):
    import torch
    if t is None:
        return BF16          # the library reports the NULL pointer
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise BdattnError(EUNSUPPORTED, f"dtype {t.dtype} not supported")


class Plan:
    """Owner of a bdattn_plan handle."""

    def __init__(self, handle: c_void_p, keep=None):
        self._h = handle
        self._keep = keep

    @classmethod
    def bdlm(cls, clean_len, block_size, q_clean_offset, q_clean_len, owned_blocks: Sequence[int],
             kv_clean_offset, kv_clean_len, with_local_corrupt, h_q, h_kv, head_dim, softmax_scale=0.0):
        owned = np.ascontiguousarray(np.asarray(owned_blocks, dtype=np.int64))
        pr = Problem(clean_len, block_size, q_clean_offset, q_clean_len,
                     owned.ctypes.data_as(ctypes.POINTER(c_int64)), owned.size, kv_clean_offset,
                     kv_clean_len, int(bool(with_local_corrupt)), h_q, h_kv, head_dim, softmax_scale)
        h = c_void_p()
        _check(lib().bdattn_plan_create(ctypes.byref(pr), ctypes.byref(h)))
        return cls(h)

    @classmethod
    def from_problem(cls, p):
        """From a workloads.BdlmProblem."""
        return cls.bdlm(p.clean_len, p.block_size, p.q_clean_offset, p.q_clean_len, p.owned_blocks,
                        p.kv_clean_offset, p.kv_clean_len, p.with_local_corrupt, p.h_q, p.h_kv,
                        p.head_dim, p.softmax_scale)

    @classmethod
    def varlen(cls, cu_seqlens, causal, h_q, h_kv, head_dim, softmax_scale=0.0):
        cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int32))
        h = c_void_p()
        _check(lib().bdattn_plan_create_varlen(cu.ctypes.data_as(ctypes.POINTER(c_int32)), cu.size - 1,
                                               int(bool(causal)), h_q, h_kv, head_dim, softmax_scale,
                                               ctypes.byref(h)))
        return cls(h)

    @classmethod
    def tasks(cls, q_cu, k_cu, causal, h_q, h_kv, head_dim, softmax_scale=0.0):
        """Core-attention tasks: task i owns query rows [q_cu[i], q_cu[i+1]) and key
        context [k_cu[i], k_cu[i+1]); causal masks align queries with the context end."""
        qc = np.ascontiguousarray(np.asarray(q_cu, dtype=np.int32))
        kc = np.ascontiguousarray(np.asarray(k_cu, dtype=np.int32))
        if qc.size != kc.size:
            raise BdattnError(EINVAL, "q_cu and k_cu must have the same length")
        h = c_void_p()
        p32 = ctypes.POINTER(c_int32)
        _check(lib().bdattn_plan_create_tasks(qc.ctypes.data_as(p32), kc.ctypes.data_as(p32), qc.size - 1,
                                              int(bool(causal)), h_q, h_kv, head_dim, softmax_scale,
                                              ctypes.byref(h)))
        return cls(h)

    @property
    def handle(self):
        return self._h

    @property
    def workspace_bytes(self) -> int:
        return lib().bdattn_plan_workspace_bytes(self._h)

    @property
    def useful_pairs(self) -> int:
        return lib().bdattn_plan_useful_pairs(self._h)

    @property
    def dkdv_split(self) -> int:
        return lib().bdattn_plan_dkdv_split(self._h)

    def set_dkdv_split(self, split: int):
        """0 = automatic, 1..8 = dK/dV workgroups per key tile (before first use)."""
        _check(lib().bdattn_plan_set_dkdv_split(self._h, split))

    @property
    def n_q(self) -> int:
        return lib().bdattn_plan_n_q(self._h)

    def n_kv(self, segment: int) -> int:
        return lib().bdattn_plan_n_kv(self._h, segment)

    def export(self, which: int) -> np.ndarray:
        width = {0: 4, 1: 12, 2: 12, 3: 4, 4: 1}[which]
        n = lib().bdattn_plan_export(self._h, which, None, 0)
        if n < 0:
            _check(int(n))
        out = np.zeros((max(n, 0), width), dtype=np.int32)
        if n:
            lib().bdattn_plan_export(self._h, which, out.ctypes.data_as(c_void_p), n)
        return out if width > 1 else out[:, 0]

    def close(self):
        if self._h is not None and self._h.value:
            lib().bdattn_plan_destroy(self._h)
        self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def workspace(nbytes: int, device="cuda"):
    """A caller-owned uint8 device buffer (torch allocations are 256-byte aligned)."""
    import torch
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


def bdattn_fwd(plan: Plan, q, k_clean, v_clean, k_corr, v_corr, o, lse, ws, stream=None):
    _check(lib().bdattn_fwd(plan.handle, _ptr(q), _ptr(k_clean), _ptr(v_clean), _ptr(k_corr), _ptr(v_corr),
                            _ptr(o), _dtype_code(o), _ptr(lse), _ptr(ws), ws.numel(), _stream(stream)))


def bdattn_varlen_fwd(plan: Plan, q, k, v, o, lse, ws, stream=None):
    _check(lib().bdattn_varlen_fwd(plan.handle, _ptr(q), _ptr(k), _ptr(v), _ptr(o), _dtype_code(o), _ptr(lse),
                                   _ptr(ws), ws.numel(), _stream(stream)))


def bdattn_lse_merge(o_parts, lse_parts, o_out, lse_out, stream=None):
    """o_parts [S, N, H, d], lse_parts [S, H, N] -> o_out [N, H, d], lse_out [H, N]."""
    S, N, H, D = o_parts.shape
    _check(lib().bdattn_lse_merge(S, _ptr(o_parts), _dtype_code(o_parts), _ptr(lse_parts), N, H, D,
                                  _ptr(o_out), _dtype_code(o_out), _ptr(lse_out), _stream(stream)))


def bdattn_bwd_prepare(plan: Plan, o, dout, delta, dq_accum=None, stream=None):
    _check(lib().bdattn_bwd_prepare(plan.handle, _ptr(o), _dtype_code(o), _ptr(dout), _ptr(delta),
                                    _ptr(dq_accum), _stream(stream)))


def bdattn_bwd(plan: Plan, q, k_clean, v_clean, k_corr, v_corr, dout, lse, delta, dq_accum,
               dk_clean, dv_clean, dk_corr, dv_corr, ws, stream=None):
    _check(lib().bdattn_bwd(plan.handle, _ptr(q), _ptr(k_clean), _ptr(v_clean), _ptr(k_corr), _ptr(v_corr),
                            _ptr(dout), _ptr(lse), _ptr(delta), _ptr(dq_accum), _ptr(dk_clean), _ptr(dv_clean),
                            _ptr(dk_corr), _ptr(dv_corr), _ptr(ws), ws.numel(), _stream(stream)))


def bdattn_bwd_dkdv(plan: Plan, q, k_clean, v_clean, k_corr, v_corr, dout, lse, delta,
                    dk_clean, dv_clean, dk_corr, dv_corr, ws, stream=None):
    _check(lib().bdattn_bwd_dkdv(plan.handle, _ptr(q), _ptr(k_clean), _ptr(v_clean), _ptr(k_corr), _ptr(v_corr),
                                 _ptr(dout), _ptr(lse), _ptr(delta), _ptr(dk_clean), _ptr(dv_clean), _ptr(dk_corr),
                                 _ptr(dv_corr), _ptr(ws), ws.numel(), _stream(stream)))


def bdattn_bwd_dq(plan: Plan, q, k_clean, v_clean, k_corr, v_corr, dout, lse, delta, dq_accum, ws, stream=None):
    _check(lib().bdattn_bwd_dq(plan.handle, _ptr(q), _ptr(k_clean), _ptr(v_clean), _ptr(k_corr), _ptr(v_corr),
                               _ptr(dout), _ptr(lse), _ptr(delta), _ptr(dq_accum), _ptr(ws), ws.numel(),
                               _stream(stream)))


def bdattn_varlen_bwd(plan: Plan, q, k, v, dout, lse, delta, dq_accum, dk, dv, ws, stream=None):
    _check(lib().bdattn_varlen_bwd(plan.handle, _ptr(q), _ptr(k), _ptr(v), _ptr(dout), _ptr(lse), _ptr(delta),
                                   _ptr(dq_accum), _ptr(dk), _ptr(dv), _ptr(ws), ws.numel(), _stream(stream)))


def bdattn_dq_finalize(dq_accum, dq, stream=None):
    _check(lib().bdattn_dq_finalize(_ptr(dq_accum), _ptr(dq), dq_accum.numel(), _stream(stream)))


def cad_split(cu_seqlens, max_pairs_per_task: int):
    """Split packed causal documents into bounded-work tasks with prefix context.

    Returns (q_cu, k_cu, kv_src) as int32 arrays: task t's queries are packed rows
    [q_cu[t], q_cu[t+1]) in document order, its context has k_cu[t+1] - k_cu[t]
    rows starting at packed row kv_src[t]."""
    cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int32))
    p32 = ctypes.POINTER(c_int32)
    n = lib().bdattn_cad_split(cu.ctypes.data_as(p32), cu.size - 1, int(max_pairs_per_task), None, None, None, 0)
    if n < 0:
        _check(int(n))
    q_cu = np.zeros(n + 1, np.int32)
    k_cu = np.zeros(n + 1, np.int32)
    kv_src = np.zeros(max(n, 1), np.int32)
    if n > 0:
        got = lib().bdattn_cad_split(cu.ctypes.data_as(p32), cu.size - 1, int(max_pairs_per_task),
                                     q_cu.ctypes.data_as(p32), k_cu.ctypes.data_as(p32),
                                     kv_src.ctypes.data_as(p32), n)
        if got != n:
            raise BdattnError(EINVAL, f"bdattn_cad_split returned {got}, expected {n}")
    return q_cu, k_cu, kv_src[:n]


def last_error() -> str:
    return lib().bdattn_last_error().decode()
