"""ctypes binding of libbdattn.so: the C entry points under the same names.

Argument marshalling only: tensors become device pointers, the stream is
torch's current HIP stream, status codes become exceptions.  Every step of the
computation runs in the library's HIP kernels; there is no fallback.  PyTorch
supplies device memory and streams.

The C ABI takes bare pointers, so before each call the binding checks every
tensor against what the kernels will read and write: a device tensor on the
stream's device, contiguous, of the documented dtype and of the exact shape
that the plan implies (rows, keys, heads, head dim).  A mismatch raises
BdattnError(EINVAL) (EUNSUPPORTED for a dtype) before any HIP call, so an
undersized, strided or wrongly typed tensor never reaches a kernel.
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


MAX_SHARDS, SHARD_ALIGN = 16, 128


class KvShards(ctypes.Structure):
    """Mirror of bdattn_kv_shards: the clean K/V range (and its gradients) split
    over several buffers."""
    _fields_ = [("n_shards", c_int32), ("shard_len", c_int64), ("k", c_void_p * MAX_SHARDS),
                ("v", c_void_p * MAX_SHARDS), ("dk", c_void_p * MAX_SHARDS), ("dv", c_void_p * MAX_SHARDS)]


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
    "bdattn_plan_keep_tables": (c_int32, [c_void_p, c_void_p, c_int64, c_void_p]),
    "bdattn_plan_useful_pairs": (c_int64, [c_void_p]),
    "bdattn_plan_set_dkdv_split": (c_int32, [c_void_p, c_int32]),
    "bdattn_plan_dkdv_split": (c_int32, [c_void_p]),
    "bdattn_plan_n_q": (c_int64, [c_void_p]),
    "bdattn_plan_n_kv": (c_int64, [c_void_p, c_int32]),
    "bdattn_plan_heads": (c_int32, [c_void_p, ctypes.POINTER(c_int32), ctypes.POINTER(c_int32),
                                    ctypes.POINTER(c_int32)]),
    "bdattn_plan_export": (c_int64, [c_void_p, c_int32, c_void_p, c_int64]),
    "bdattn_fwd": (c_int32, [c_void_p] * 7 + [c_int32, c_void_p, c_void_p, c_int64, c_void_p]),
    "bdattn_fwd_static": (c_int32, [c_void_p] * 7 + [c_int32, c_void_p, c_void_p]),
    "bdattn_lse_merge": (c_int32, [c_int32, c_void_p, c_int32, c_void_p, c_int64, c_int32, c_int32, c_void_p,
                                   c_int32, c_void_p, c_void_p]),
    "bdattn_bwd_prepare": (c_int32, [c_void_p, c_void_p, c_int32, c_void_p, c_void_p, c_void_p, c_void_p]),
    "bdattn_bwd": (c_int32, [c_void_p] * 15 + [c_int64, c_void_p]),
    "bdattn_bwd_dkdv": (c_int32, [c_void_p] * 14 + [c_int64, c_void_p]),
    "bdattn_bwd_dq": (c_int32, [c_void_p] * 11 + [c_int64, c_void_p]),
    "bdattn_dq_finalize": (c_int32, [c_void_p, c_void_p, c_int64, c_void_p]),
    "bdattn_cast_f32_bf16": (c_int32, [c_void_p, c_void_p, c_int64, c_void_p]),
    "bdattn_varlen_fwd": (c_int32, [c_void_p] * 5 + [c_int32, c_void_p, c_void_p, c_int64, c_void_p]),
    "bdattn_varlen_bwd": (c_int32, [c_void_p] * 11 + [c_int64, c_void_p]),
    "bdattn_fwd_shards": (c_int32, [c_void_p, c_void_p, ctypes.POINTER(KvShards), c_void_p, c_void_p, c_void_p,
                                    c_int32, c_void_p, c_void_p, c_int64, c_void_p]),
    "bdattn_bwd_shards": (c_int32, [c_void_p, c_void_p, ctypes.POINTER(KvShards)] + [c_void_p] * 9
                          + [c_int64, c_void_p]),
    "bdattn_bwd_dkdv_shards": (c_int32, [c_void_p, c_void_p, ctypes.POINTER(KvShards)] + [c_void_p] * 8
                               + [c_int64, c_void_p]),
    "bdattn_bwd_dq_shards": (c_int32, [c_void_p, c_void_p, ctypes.POINTER(KvShards)] + [c_void_p] * 7
                             + [c_int64, c_void_p]),
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


def _want(t, name, shape, dtypes, devs, optional=False):
    """Check one tensor argument: dtype among `dtypes`, exactly `shape`, contiguous.
    Its device is appended to `devs` (checked by _on_one_gpu once every tensor has
    passed these checks)."""
    import torch
    if t is None:
        if optional:
            return
        raise BdattnError(EINVAL, f"{name} is None")
    if not isinstance(t, torch.Tensor):
        raise BdattnError(EINVAL, f"{name} must be a torch.Tensor, got {type(t).__name__}")
    if t.dtype not in dtypes:
        raise BdattnError(EUNSUPPORTED, f"{name} has dtype {t.dtype}, expected {' or '.join(map(str, dtypes))}")
    if tuple(t.shape) != tuple(int(x) for x in shape):
        raise BdattnError(EINVAL, f"{name} has shape {tuple(t.shape)}, expected {tuple(int(x) for x in shape)}")
    if not t.is_contiguous():
        raise BdattnError(EINVAL, f"{name} must be contiguous")
    devs.append((name, t.device))


def _on_one_gpu(devs, stream):
    """Every tensor on one GPU, and the stream (if given) on that GPU too."""
    name0, dev0 = devs[0]
    for name, dev in devs:
        if dev.type != "cuda":
            raise BdattnError(EINVAL, f"{name} must be a GPU tensor (is on {dev})")
        if dev != dev0:
            raise BdattnError(EINVAL, f"{name} is on {dev}, {name0} on {dev0}")
    if stream is not None and stream.device != dev0:
        raise BdattnError(EINVAL, f"stream is on {stream.device}, the tensors on {dev0}")


def _bf16():
    import torch
    return (torch.bfloat16,)


def _f32():
    import torch
    return (torch.float32,)


def _bf16_or_f32():
    import torch
    return (torch.bfloat16, torch.float32)


def _want_ws(ws, plan, devs):
    import torch
    _want(ws, "workspace", (ws.numel() if isinstance(ws, torch.Tensor) else 0,), (torch.uint8,), devs)
    if ws.numel() < plan.workspace_bytes:
        raise BdattnError(EWORKSPACE, f"workspace has {ws.numel()} bytes, the plan needs {plan.workspace_bytes}")


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
        return lib().bdattn_plan_workspace_bytes(self._h)   # changes with set_dkdv_split

    @property
    def useful_pairs(self) -> int:
        return lib().bdattn_plan_useful_pairs(self._h)

    @property
    def dkdv_split(self) -> int:
        return lib().bdattn_plan_dkdv_split(self._h)

    def set_dkdv_split(self, split: int):
        """0 = automatic, 1..8 = dK/dV workgroups per key tile (before first use)."""
        _check(lib().bdattn_plan_set_dkdv_split(self._h, split))

    def keep_tables(self, ws, stream=None):
        """Upload the plan's tables into `ws` once; later calls with this plan and this
        workspace skip their per-call upload (bdattn_plan_keep_tables).  The workspace
        must stay untouched, and alive, while kept: ws None ends the claim."""
        if ws is None:
            _check(lib().bdattn_plan_keep_tables(self._h, None, 0, None))
            self._kept = None
            return
        dev = []
        _want_ws(ws, self, dev)
        _on_one_gpu(dev, stream)
        _check(lib().bdattn_plan_keep_tables(self._h, _ptr(ws), ws.numel(), _stream(stream)))
        self._kept = ws   # holds the buffer alive while the tables are kept in it

    @property
    def n_q(self) -> int:
        if getattr(self, "_n_q", None) is None:
            self._n_q = lib().bdattn_plan_n_q(self._h)
        return self._n_q

    @property
    def heads(self):
        """(h_q, h_kv, head_dim) of the plan."""
        if getattr(self, "_heads", None) is None:
            hq, hkv, d = c_int32(), c_int32(), c_int32()
            _check(lib().bdattn_plan_heads(self._h, ctypes.byref(hq), ctypes.byref(hkv), ctypes.byref(d)))
            self._heads = (hq.value, hkv.value, d.value)
        return self._heads

    def q_shape(self):
        """Shape of Q, O, dO and dQ: (n_q, h_q, head_dim)."""
        hq, _, d = self.heads
        return (self.n_q, hq, d)

    def kv_shape(self, segment: int):
        """Shape of K, V, dK and dV of a key segment: (n_kv(segment), h_kv, head_dim)."""
        _, hkv, d = self.heads
        return (self.n_kv(segment), hkv, d)

    def lse_shape(self):
        """Shape of LSE and delta: (h_q, n_q)."""
        return (self.heads[0], self.n_q)

    def n_kv(self, segment: int) -> int:
        """Key rows of segment 0 (clean range / packed keys) or 1 (local corrupted K/V).
        A plan is immutable, so its sizes are read from the library once."""
        if getattr(self, "_n_kv", None) is None:
            self._n_kv = (lib().bdattn_plan_n_kv(self._h, 0), lib().bdattn_plan_n_kv(self._h, 1))
        return self._n_kv[segment]

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


def _kv_args(plan, dev, k0, v0, k1, v1, g0="k_clean", g1="k_corr"):
    """Check the K/V of both key segments; segment 1 is passed only when the plan has keys there."""
    b = _bf16()
    for t, nm in ((k0, g0), (v0, g0.replace("k", "v", 1))):
        _want(t, nm, plan.kv_shape(0), b, dev)
    if plan.n_kv(1) > 0:
        for t, nm in ((k1, g1), (v1, g1.replace("k", "v", 1))):
            _want(t, nm, plan.kv_shape(1), b, dev)
        return k1, v1
    return None, None


def _grad_kv_args(plan, dev, dk0, dv0, dk1, dv1):
    b = _bf16()
    _want(dk0, "dk_clean", plan.kv_shape(0), b, dev)
    _want(dv0, "dv_clean", plan.kv_shape(0), b, dev)
    if plan.n_kv(1) > 0:
        _want(dk1, "dk_corr", plan.kv_shape(1), b, dev)
        _want(dv1, "dv_corr", plan.kv_shape(1), b, dev)
        return dk1, dv1
    return None, None


def shard_split(n_keys: int, n_shards: int, shard_len: int):
    """Lengths of the buffers of a range of n_keys positions split over n_shards
    buffers of shard_len positions (the last holds the rest), or an error."""
    if not 1 <= n_shards <= MAX_SHARDS:
        raise BdattnError(EINVAL, f"{n_shards} shard buffers; 1 .. {MAX_SHARDS} are allowed")
    if n_shards == 1:
        return [n_keys]
    if shard_len <= 0 or shard_len % SHARD_ALIGN:
        raise BdattnError(EALIGN, f"shard length {shard_len} is not a positive multiple of {SHARD_ALIGN}")
    if not (n_shards - 1) * shard_len < n_keys <= n_shards * shard_len:
        raise BdattnError(EINVAL, f"{n_shards} buffers of {shard_len} positions do not cover {n_keys} positions "
                                  "with at least one position in each")
    return [shard_len] * (n_shards - 1) + [n_keys - (n_shards - 1) * shard_len]


def make_shards(k_shards, v_shards, dk_shards=None, dv_shards=None) -> KvShards:
    """The bdattn_kv_shards struct of lists of per-buffer tensors (no checks)."""
    kv = KvShards()
    kv.n_shards = len(k_shards)
    kv.shard_len = int(k_shards[0].shape[0]) if len(k_shards) > 1 else 0
    for i in range(len(k_shards)):
        kv.k[i] = k_shards[i].data_ptr()
        kv.v[i] = v_shards[i].data_ptr()
        if dk_shards is not None:
            kv.dk[i] = dk_shards[i].data_ptr()
            kv.dv[i] = dv_shards[i].data_ptr()
    return kv


def _shard_args(plan, dev, k_shards, v_shards, dk_shards=None, dv_shards=None) -> KvShards:
    """Check per-buffer K/V (and dK/dV) lists against the plan's clean range."""
    k_shards, v_shards = list(k_shards), list(v_shards)
    if len(v_shards) != len(k_shards) or not k_shards:
        raise BdattnError(EINVAL, "k_shards and v_shards must be non-empty lists of the same length")
    lens = shard_split(plan.n_kv(0), len(k_shards), int(k_shards[0].shape[0]) if len(k_shards) > 1 else 0)
    _, h_kv, d = plan.kv_shape(0)
    b = _bf16()
    lists = [("k", k_shards), ("v", v_shards)]
    if dk_shards is not None or dv_shards is not None:
        dk_shards, dv_shards = list(dk_shards or []), list(dv_shards or [])
        if len(dk_shards) != len(k_shards) or len(dv_shards) != len(k_shards):
            raise BdattnError(EINVAL, "dk_shards and dv_shards must hold one tensor per K/V buffer")
        lists += [("dk", dk_shards), ("dv", dv_shards)]
    for nm, ts in lists:
        for i, t in enumerate(ts):
            _want(t, f"{nm}_shards[{i}]", (lens[i], h_kv, d), b, dev)
    return make_shards(k_shards, v_shards, dk_shards, dv_shards)


def _row_args(plan, dev, lse, delta=None, dout=None):
    _want(lse, "lse", plan.lse_shape(), _f32(), dev)
    if delta is not None:
        _want(delta, "delta", plan.lse_shape(), _f32(), dev)
    if dout is not None:
        _want(dout, "dout", plan.q_shape(), _bf16(), dev)


def bdattn_fwd(plan: Plan, q, k_clean, v_clean, k_corr, v_corr, o, lse, ws, stream=None):
    dev = []
    _want(q, "q", plan.q_shape(), _bf16(), dev)
    k_corr, v_corr = _kv_args(plan, dev, k_clean, v_clean, k_corr, v_corr)
    _want(o, "o", plan.q_shape(), _bf16_or_f32(), dev)
    _row_args(plan, dev, lse=lse)
    _want_ws(ws, plan, dev)
    _on_one_gpu(dev, stream)
    _check(lib().bdattn_fwd(plan.handle, _ptr(q), _ptr(k_clean), _ptr(v_clean), _ptr(k_corr), _ptr(v_corr),
                            _ptr(o), _dtype_code(o), _ptr(lse), _ptr(ws), ws.numel(), _stream(stream)))


def bdattn_fwd_static(plan: Plan, q, k_clean, v_clean, k_corr, v_corr, o, lse, stream=None):
    """bdattn_fwd without a workspace: the plan's forward tables go into the library's
    static per-GPU scratch array (no allocation anywhere in the call).  Calls that may
    overlap on one GPU race on that array."""
    dev = []
    _want(q, "q", plan.q_shape(), _bf16(), dev)
    k_corr, v_corr = _kv_args(plan, dev, k_clean, v_clean, k_corr, v_corr)
    _want(o, "o", plan.q_shape(), _bf16_or_f32(), dev)
    _row_args(plan, dev, lse=lse)
    _on_one_gpu(dev, stream)
    _check(lib().bdattn_fwd_static(plan.handle, _ptr(q), _ptr(k_clean), _ptr(v_clean), _ptr(k_corr), _ptr(v_corr),
                                   _ptr(o), _dtype_code(o), _ptr(lse), _stream(stream)))


def bdattn_varlen_fwd(plan: Plan, q, k, v, o, lse, ws, stream=None):
    dev = []
    _want(q, "q", plan.q_shape(), _bf16(), dev)
    _kv_args(plan, dev, k, v, None, None, g0="k")
    _want(o, "o", plan.q_shape(), _bf16_or_f32(), dev)
    _row_args(plan, dev, lse=lse)
    _want_ws(ws, plan, dev)
    _on_one_gpu(dev, stream)
    _check(lib().bdattn_varlen_fwd(plan.handle, _ptr(q), _ptr(k), _ptr(v), _ptr(o), _dtype_code(o), _ptr(lse),
                                   _ptr(ws), ws.numel(), _stream(stream)))


def bdattn_lse_merge(o_parts, lse_parts, o_out, lse_out, stream=None):
    """o_parts [S, N, H, d], lse_parts [S, H, N] -> o_out [N, H, d], lse_out [H, N]."""
    import torch
    if not isinstance(o_parts, torch.Tensor) or o_parts.dim() != 4:
        raise BdattnError(EINVAL, "o_parts must be a 4-d tensor [S, N, H, d]")
    S, N, H, D = o_parts.shape
    dev = []
    _want(o_parts, "o_parts", (S, N, H, D), _bf16_or_f32(), dev)
    _want(lse_parts, "lse_parts", (S, H, N), _f32(), dev)
    _want(o_out, "o_out", (N, H, D), _bf16_or_f32(), dev)
    _want(lse_out, "lse_out", (H, N), _f32(), dev)
    _on_one_gpu(dev, stream)
    _check(lib().bdattn_lse_merge(S, _ptr(o_parts), _dtype_code(o_parts), _ptr(lse_parts), N, H, D,
                                  _ptr(o_out), _dtype_code(o_out), _ptr(lse_out), _stream(stream)))


def bdattn_bwd_prepare(plan: Plan, o, dout, delta, dq_accum=None, stream=None):
    dev = []
    _want(o, "o", plan.q_shape(), _bf16_or_f32(), dev)
    _want(dout, "dout", plan.q_shape(), _bf16(), dev)
    _want(delta, "delta", plan.lse_shape(), _f32(), dev)
    _want(dq_accum, "dq_accum", plan.q_shape(), _f32(), dev, optional=True)
    _on_one_gpu(dev, stream)
    _check(lib().bdattn_bwd_prepare(plan.handle, _ptr(o), _dtype_code(o), _ptr(dout), _ptr(delta),
                                    _ptr(dq_accum), _stream(stream)))


def _bwd_common(plan, q, k_clean, v_clean, k_corr, v_corr, dout, lse, delta, ws):
    dev = []
    _want(q, "q", plan.q_shape(), _bf16(), dev)
    k_corr, v_corr = _kv_args(plan, dev, k_clean, v_clean, k_corr, v_corr)
    _row_args(plan, dev, lse=lse, delta=delta, dout=dout)
    _want_ws(ws, plan, dev)
    return dev, k_corr, v_corr


def bdattn_bwd(plan: Plan, q, k_clean, v_clean, k_corr, v_corr, dout, lse, delta, dq_accum,
               dk_clean, dv_clean, dk_corr, dv_corr, ws, stream=None):
    dev, k_corr, v_corr = _bwd_common(plan, q, k_clean, v_clean, k_corr, v_corr, dout, lse, delta, ws)
    _want(dq_accum, "dq_accum", plan.q_shape(), _f32(), dev)
    dk_corr, dv_corr = _grad_kv_args(plan, dev, dk_clean, dv_clean, dk_corr, dv_corr)
    _on_one_gpu(dev, stream)
    _check(lib().bdattn_bwd(plan.handle, _ptr(q), _ptr(k_clean), _ptr(v_clean), _ptr(k_corr), _ptr(v_corr),
                            _ptr(dout), _ptr(lse), _ptr(delta), _ptr(dq_accum), _ptr(dk_clean), _ptr(dv_clean),
                            _ptr(dk_corr), _ptr(dv_corr), _ptr(ws), ws.numel(), _stream(stream)))


def bdattn_bwd_dkdv(plan: Plan, q, k_clean, v_clean, k_corr, v_corr, dout, lse, delta,
                    dk_clean, dv_clean, dk_corr, dv_corr, ws, stream=None):
    dev, k_corr, v_corr = _bwd_common(plan, q, k_clean, v_clean, k_corr, v_corr, dout, lse, delta, ws)
    dk_corr, dv_corr = _grad_kv_args(plan, dev, dk_clean, dv_clean, dk_corr, dv_corr)
    _on_one_gpu(dev, stream)
    _check(lib().bdattn_bwd_dkdv(plan.handle, _ptr(q), _ptr(k_clean), _ptr(v_clean), _ptr(k_corr), _ptr(v_corr),
                                 _ptr(dout), _ptr(lse), _ptr(delta), _ptr(dk_clean), _ptr(dv_clean), _ptr(dk_corr),
                                 _ptr(dv_corr), _ptr(ws), ws.numel(), _stream(stream)))


def bdattn_bwd_dq(plan: Plan, q, k_clean, v_clean, k_corr, v_corr, dout, lse, delta, dq_accum, ws, stream=None):
    dev, k_corr, v_corr = _bwd_common(plan, q, k_clean, v_clean, k_corr, v_corr, dout, lse, delta, ws)
    _want(dq_accum, "dq_accum", plan.q_shape(), _f32(), dev)
    _on_one_gpu(dev, stream)
    _check(lib().bdattn_bwd_dq(plan.handle, _ptr(q), _ptr(k_clean), _ptr(v_clean), _ptr(k_corr), _ptr(v_corr),
                               _ptr(dout), _ptr(lse), _ptr(delta), _ptr(dq_accum), _ptr(ws), ws.numel(),
                               _stream(stream)))


def _corr_args(plan, dev, k_corr, v_corr, g="k_corr"):
    if plan.n_kv(1) > 0:
        for t, nm in ((k_corr, g), (v_corr, g.replace("k", "v", 1))):
            _want(t, nm, plan.kv_shape(1), _bf16(), dev)
        return k_corr, v_corr
    return None, None


def bdattn_fwd_shards(plan: Plan, q, k_shards, v_shards, k_corr, v_corr, o, lse, ws, stream=None):
    """bdattn_fwd over a clean range held in several buffers (lists of tensors)."""
    dev = []
    _want(q, "q", plan.q_shape(), _bf16(), dev)
    kv = _shard_args(plan, dev, k_shards, v_shards)
    k_corr, v_corr = _corr_args(plan, dev, k_corr, v_corr)
    _want(o, "o", plan.q_shape(), _bf16_or_f32(), dev)
    _row_args(plan, dev, lse=lse)
    _want_ws(ws, plan, dev)
    _on_one_gpu(dev, stream)
    _check(lib().bdattn_fwd_shards(plan.handle, _ptr(q), ctypes.byref(kv), _ptr(k_corr), _ptr(v_corr), _ptr(o),
                                   _dtype_code(o), _ptr(lse), _ptr(ws), ws.numel(), _stream(stream)))


def _bwd_shards_common(plan, q, k_shards, v_shards, k_corr, v_corr, dout, lse, delta, ws, dk_shards, dv_shards):
    dev = []
    _want(q, "q", plan.q_shape(), _bf16(), dev)
    kv = _shard_args(plan, dev, k_shards, v_shards, dk_shards, dv_shards)
    k_corr, v_corr = _corr_args(plan, dev, k_corr, v_corr)
    _row_args(plan, dev, lse=lse, delta=delta, dout=dout)
    _want_ws(ws, plan, dev)
    return dev, kv, k_corr, v_corr


def bdattn_bwd_shards(plan: Plan, q, k_shards, v_shards, k_corr, v_corr, dout, lse, delta, dq_accum,
                      dk_shards, dv_shards, dk_corr, dv_corr, ws, stream=None):
    dev, kv, k_corr, v_corr = _bwd_shards_common(plan, q, k_shards, v_shards, k_corr, v_corr, dout, lse, delta,
                                                 ws, dk_shards, dv_shards)
    _want(dq_accum, "dq_accum", plan.q_shape(), _f32(), dev)
    dk_corr, dv_corr = _corr_args(plan, dev, dk_corr, dv_corr, g="dk_corr")
    _on_one_gpu(dev, stream)
    _check(lib().bdattn_bwd_shards(plan.handle, _ptr(q), ctypes.byref(kv), _ptr(k_corr), _ptr(v_corr), _ptr(dout),
                                   _ptr(lse), _ptr(delta), _ptr(dq_accum), _ptr(dk_corr), _ptr(dv_corr), _ptr(ws),
                                   ws.numel(), _stream(stream)))


def bdattn_bwd_dkdv_shards(plan: Plan, q, k_shards, v_shards, k_corr, v_corr, dout, lse, delta,
                           dk_shards, dv_shards, dk_corr, dv_corr, ws, stream=None):
    dev, kv, k_corr, v_corr = _bwd_shards_common(plan, q, k_shards, v_shards, k_corr, v_corr, dout, lse, delta,
                                                 ws, dk_shards, dv_shards)
    dk_corr, dv_corr = _corr_args(plan, dev, dk_corr, dv_corr, g="dk_corr")
    _on_one_gpu(dev, stream)
    _check(lib().bdattn_bwd_dkdv_shards(plan.handle, _ptr(q), ctypes.byref(kv), _ptr(k_corr), _ptr(v_corr),
                                        _ptr(dout), _ptr(lse), _ptr(delta), _ptr(dk_corr), _ptr(dv_corr), _ptr(ws),
                                        ws.numel(), _stream(stream)))


def bdattn_bwd_dq_shards(plan: Plan, q, k_shards, v_shards, k_corr, v_corr, dout, lse, delta, dq_accum, ws,
                         stream=None):
    dev, kv, k_corr, v_corr = _bwd_shards_common(plan, q, k_shards, v_shards, k_corr, v_corr, dout, lse, delta,
                                                 ws, None, None)
    _want(dq_accum, "dq_accum", plan.q_shape(), _f32(), dev)
    _on_one_gpu(dev, stream)
    _check(lib().bdattn_bwd_dq_shards(plan.handle, _ptr(q), ctypes.byref(kv), _ptr(k_corr), _ptr(v_corr),
                                      _ptr(dout), _ptr(lse), _ptr(delta), _ptr(dq_accum), _ptr(ws), ws.numel(),
                                      _stream(stream)))


def bdattn_varlen_bwd(plan: Plan, q, k, v, dout, lse, delta, dq_accum, dk, dv, ws, stream=None):
    dev = []
    _want(q, "q", plan.q_shape(), _bf16(), dev)
    _kv_args(plan, dev, k, v, None, None, g0="k")
    _row_args(plan, dev, lse=lse, delta=delta, dout=dout)
    _want(dq_accum, "dq_accum", plan.q_shape(), _f32(), dev)
    _want(dk, "dk", plan.kv_shape(0), _bf16(), dev)
    _want(dv, "dv", plan.kv_shape(0), _bf16(), dev)
    _want_ws(ws, plan, dev)
    _on_one_gpu(dev, stream)
    _check(lib().bdattn_varlen_bwd(plan.handle, _ptr(q), _ptr(k), _ptr(v), _ptr(dout), _ptr(lse), _ptr(delta),
                                   _ptr(dq_accum), _ptr(dk), _ptr(dv), _ptr(ws), ws.numel(), _stream(stream)))


def bdattn_cast_f32_bf16(src, dst, stream=None):
    """dst (bf16) = src (fp32) rounded to nearest even; same shape."""
    import torch
    if not isinstance(src, torch.Tensor):
        raise BdattnError(EINVAL, "src must be a torch.Tensor")
    dev = []
    _want(src, "src", tuple(src.shape), _f32(), dev)
    _want(dst, "dst", tuple(src.shape), _bf16(), dev)
    _on_one_gpu(dev, stream)
    _check(lib().bdattn_cast_f32_bf16(_ptr(src), _ptr(dst), src.numel(), _stream(stream)))


def bdattn_dq_finalize(dq_accum, dq, stream=None):
    """dq (bf16) = dq_accum (fp32); same shape."""
    import torch
    if not isinstance(dq_accum, torch.Tensor):
        raise BdattnError(EINVAL, "dq_accum must be a torch.Tensor")
    dev = []
    _want(dq_accum, "dq_accum", tuple(dq_accum.shape), _f32(), dev)
    _want(dq, "dq", tuple(dq_accum.shape), _bf16(), dev)
    _on_one_gpu(dev, stream)
    _check(lib().bdattn_dq_finalize(_ptr(dq_accum), _ptr(dq), dq_accum.numel(), _stream(stream)))


# ----------------------------------------------------------------------------- unchecked calls
# The entry points above without the per-tensor checks, for a caller that owns
# its output buffers and checks its inputs against its plans once per step (the
# steps of rank_step.py): a Python check costs microseconds of host time per
# tensor, as long as a small kernel runs, and a small step is then bound by the
# host.  The library's own argument validation still runs on every call.
# Tensors are passed as torch tensors (or None); `stream` as a raw HIP stream.

def _p(t):
    return None if t is None else t.data_ptr()


def current_stream_handle():
    import torch
    return torch.cuda.current_stream().cuda_stream


def fwd_unchecked(plan, q, kc, vc, kx, vx, o, lse, ws, stream):
    _check(lib().bdattn_fwd(plan.handle, _p(q), _p(kc), _p(vc), _p(kx), _p(vx), _p(o), _dtype_code(o), _p(lse),
                            _p(ws), ws.numel(), stream))


def varlen_fwd_unchecked(plan, q, k, v, o, lse, ws, stream):
    _check(lib().bdattn_varlen_fwd(plan.handle, _p(q), _p(k), _p(v), _p(o), _dtype_code(o), _p(lse), _p(ws),
                                   ws.numel(), stream))


def lse_merge_unchecked(o_parts, lse_parts, o_out, lse_out, stream):
    S, N, H, D = o_parts.shape
    _check(lib().bdattn_lse_merge(S, _p(o_parts), _dtype_code(o_parts), _p(lse_parts), N, H, D, _p(o_out),
                                  _dtype_code(o_out), _p(lse_out), stream))


def bwd_prepare_unchecked(plan, o, dout, delta, dq_accum, stream):
    _check(lib().bdattn_bwd_prepare(plan.handle, _p(o), _dtype_code(o), _p(dout), _p(delta), _p(dq_accum), stream))


def bwd_dkdv_unchecked(plan, q, kc, vc, kx, vx, dout, lse, delta, dkc, dvc, dkx, dvx, ws, stream):
    _check(lib().bdattn_bwd_dkdv(plan.handle, _p(q), _p(kc), _p(vc), _p(kx), _p(vx), _p(dout), _p(lse), _p(delta),
                                 _p(dkc), _p(dvc), _p(dkx), _p(dvx), _p(ws), ws.numel(), stream))


def bwd_dq_unchecked(plan, q, kc, vc, kx, vx, dout, lse, delta, dq_accum, ws, stream):
    _check(lib().bdattn_bwd_dq(plan.handle, _p(q), _p(kc), _p(vc), _p(kx), _p(vx), _p(dout), _p(lse), _p(delta),
                               _p(dq_accum), _p(ws), ws.numel(), stream))


def fwd_shards_unchecked(plan, q, kv: KvShards, kx, vx, o, lse, ws, stream):
    _check(lib().bdattn_fwd_shards(plan.handle, _p(q), ctypes.byref(kv), _p(kx), _p(vx), _p(o), _dtype_code(o),
                                   _p(lse), _p(ws), ws.numel(), stream))


def bwd_dkdv_shards_unchecked(plan, q, kv: KvShards, kx, vx, dout, lse, delta, dkx, dvx, ws, stream):
    _check(lib().bdattn_bwd_dkdv_shards(plan.handle, _p(q), ctypes.byref(kv), _p(kx), _p(vx), _p(dout), _p(lse),
                                        _p(delta), _p(dkx), _p(dvx), _p(ws), ws.numel(), stream))


def bwd_dq_shards_unchecked(plan, q, kv: KvShards, kx, vx, dout, lse, delta, dq_accum, ws, stream):
    _check(lib().bdattn_bwd_dq_shards(plan.handle, _p(q), ctypes.byref(kv), _p(kx), _p(vx), _p(dout), _p(lse),
                                      _p(delta), _p(dq_accum), _p(ws), ws.numel(), stream))


def cast_unchecked(src, dst, stream):
    _check(lib().bdattn_cast_f32_bf16(_p(src), _p(dst), src.numel(), stream))


def dq_finalize_unchecked(dq_accum, dq, stream):
    _check(lib().bdattn_dq_finalize(_p(dq_accum), _p(dq), dq_accum.numel(), stream))


def check_inputs(named, devs=None):
    """Check (tensor, name, shape, dtypes) tuples as the public calls do, and that
    all of them sit on one GPU: used once per step by callers of the unchecked calls."""
    devs = [] if devs is None else devs
    for t, name, shape, dtypes in named:
        _want(t, name, shape, dtypes, devs)
    _on_one_gpu(devs, None)


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
