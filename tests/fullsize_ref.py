"""Oracle references at the workloads' full sizes (test infrastructure only).

The oracle (``oracle/``) is the plain definition: a dense masked softmax over
every key of a row chunk.  At full size that is too slow to run as written, so
this module composes the oracle's own calls in the way the method itself does:
the key axis is cut into pieces, each piece gives a partial (O, LSE) through
``oracle.attention_fwd`` with the oracle's mask evaluated at that piece's key
indices, and the partials are combined with ``oracle.lse_merge`` (exact: the
sharded-then-merged result equals the unsharded one, a pin of
tests/test_oracle.py).  A piece whose mask is empty for a row chunk contributes
LSE = -inf and O = 0 to the merge, so it is skipped; emptiness is decided from
the oracle's explicit mask, never from a formula.  The backward of a row chunk
is the sum over pieces of ``oracle.attention_bwd`` with the merged LSE and
delta (exact by linearity, pinned the same way).

Row chunks run on a thread pool (numpy releases the GIL inside its kernels),
with BLAS held to one thread per worker.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from typing import Callable, List, Optional, Sequence, Tuple

import numpy as np

import oracle

MaskFn = Callable[[np.ndarray, np.ndarray], np.ndarray]

PIECE = 16384       # keys per piece
ROW_CHUNK = 256     # query rows per work item


def n_threads() -> int:
    return max(1, min(16, len(os.sched_getaffinity(0))))


def _pool_map(fn, items, threads=None):
    from threadpoolctl import threadpool_limits
    with threadpool_limits(1):
        with ThreadPoolExecutor(threads or n_threads()) as ex:
            return list(ex.map(fn, items))


def shifted_mask(mask_fn: MaskFn, key0: int) -> MaskFn:
    """The mask of a piece whose local key j is key key0 + j of the whole key axis."""
    return lambda rows, keys: mask_fn(rows, np.asarray(keys, dtype=np.int64) + key0)


def _pieces(n_keys: int, piece: int) -> List[Tuple[int, int]]:
    return [(a, min(n_keys, a + piece)) for a in range(0, n_keys, piece)]


def _chunk_fwd(q, k, v, mask_fn, scale, rr, pieces):
    """Merged (O, LSE) of rows rr over every piece, and the pieces that hold a legal key."""
    o_parts, l_parts, used = [], [], []
    for (a, b) in pieces:
        mf = shifted_mask(mask_fn, a)
        if not mf(rr, np.arange(b - a)).any():
            continue
        o, l = oracle.attention_fwd(q, k[a:b], v[a:b], mf, scale, rows=rr)
        o_parts.append(o)
        l_parts.append(l)
        used.append((a, b))
    if not used:
        hq = q.shape[1]
        return np.zeros((rr.size, hq, q.shape[2])), np.full((hq, rr.size), -np.inf), used
    o, lse = oracle.lse_merge(np.stack(o_parts), np.stack(l_parts))
    return o, lse, used


def rows_reference(q, k, v, dout, mask_fn: MaskFn, scale: float, rows: Sequence[int], bwd: bool = True,
                   piece: int = PIECE, threads: Optional[int] = None):
    """O [R, H_q, d], LSE [H_q, R] and (bwd) dQ [R, H_q, d] of the given rows against every key.

    q, dout [N, H_q, d]; k, v [M, H_kv, d] (float64).  Each row's O, LSE and dQ
    depend on that row alone, so a sample of rows is exact."""
    rows = np.sort(np.asarray(rows, dtype=np.int64))
    pieces = _pieces(k.shape[0], piece)
    chunks = [rows[i:i + ROW_CHUNK] for i in range(0, rows.size, ROW_CHUNK)]

    def work(rr):
        o, lse, used = _chunk_fwd(q, k, v, mask_fn, scale, rr, pieces)
        dq = None
        if bwd:
            D = oracle.delta_rows(o, dout[rr])
            dq = np.zeros_like(o)
            for (a, b) in used:
                d_piece, _, _ = oracle.attention_bwd(q, k[a:b], v[a:b], dout, lse, D, shifted_mask(mask_fn, a),
                                                    scale, rows=rr)
                dq += d_piece
        return o, lse, dq

    res = _pool_map(work, chunks, threads)
    o = np.concatenate([r[0] for r in res])
    lse = np.concatenate([r[1] for r in res], axis=1)
    dq = np.concatenate([r[2] for r in res]) if bwd else None
    return rows, o, lse, dq


def group_reference(q, k, v, dout, mask_fn: MaskFn, scale: float, piece: int = PIECE,
                    threads: Optional[int] = None):
    """Every output of one KV-head group: O [N, H_q, d], LSE [H_q, N], dQ [N, H_q, d]
    and dK, dV [M, H_kv, d] over all N rows and M keys, in one pass over row chunks.
    Each (row chunk, key piece) pair with a legal key gives its dQ contribution and
    the piece's dK/dV contribution (``oracle.attention_bwd`` with the chunk's merged
    LSE and delta); the latter is added into the piece's rows under a per-piece lock."""
    import threading
    n, m = q.shape[0], k.shape[0]
    pieces = _pieces(m, piece)
    locks = [threading.Lock() for _ in pieces]
    dk = np.zeros((m, k.shape[1], k.shape[2]))
    dv = np.zeros_like(dk)
    starts = list(range(0, n, ROW_CHUNK))

    def work(r0):
        rr = np.arange(r0, min(n, r0 + ROW_CHUNK), dtype=np.int64)
        o, lse, used = _chunk_fwd(q, k, v, mask_fn, scale, rr, pieces)
        D = oracle.delta_rows(o, dout[rr])
        dq = np.zeros_like(o)
        for (a, b) in used:
            d_piece, dk_p, dv_p = oracle.attention_bwd(q, k[a:b], v[a:b], dout, lse, D, shifted_mask(mask_fn, a),
                                                       scale, rows=rr)
            dq += d_piece
            with locks[pieces.index((a, b))]:
                dk[a:b] += dk_p
                dv[a:b] += dv_p
        return o, lse, dq

    res = _pool_map(work, starts, threads)
    return (np.concatenate([r[0] for r in res]), np.concatenate([r[1] for r in res], axis=1),
            np.concatenate([r[2] for r in res]), dk, dv)


def lse_delta_all_rows(q, k, v, dout, mask_fn: MaskFn, scale: float, n_rows: int, piece: int = PIECE,
                       threads: Optional[int] = None):
    """LSE [H_q, N] and delta [H_q, N] (delta = <dO, O> of the oracle's O) of every row."""
    pieces = _pieces(k.shape[0], piece)
    starts = list(range(0, n_rows, ROW_CHUNK))

    def work(r0):
        rr = np.arange(r0, min(n_rows, r0 + ROW_CHUNK), dtype=np.int64)
        o, lse, _ = _chunk_fwd(q, k, v, mask_fn, scale, rr, pieces)
        return lse, oracle.delta_rows(o, dout[rr])

    res = _pool_map(work, starts, threads)
    return np.concatenate([r[0] for r in res], axis=1), np.concatenate([r[1] for r in res], axis=1)


def keys_reference(q, k, v, dout, lse, delta, mask_fn: MaskFn, scale: float, keys: Sequence[int],
                   threads: Optional[int] = None):
    """dK, dV [K, H_kv, d] of the selected keys from every row that attends them.

    lse and delta [H_q, N] must cover all N rows (the merged values of the full
    output).  Rows that attend none of the keys contribute nothing and are skipped."""
    keys = np.asarray(keys, dtype=np.int64)
    kk, vv = k[keys], v[keys]
    kmask = lambda rows, kj: mask_fn(rows, keys[np.asarray(kj, dtype=np.int64)])
    n = q.shape[0]
    starts = list(range(0, n, 4 * ROW_CHUNK))

    def work(r0):
        rr = np.arange(r0, min(n, r0 + 4 * ROW_CHUNK), dtype=np.int64)
        m = kmask(rr, np.arange(keys.size))
        rr = rr[m.any(axis=1)]
        if rr.size == 0:
            return None
        _, dk, dv = oracle.attention_bwd(q, kk, vv, dout, lse[:, rr], delta[:, rr], kmask, scale, rows=rr)
        return dk, dv

    res = [r for r in _pool_map(work, starts, threads) if r is not None]
    dk = np.zeros((keys.size, k.shape[1], k.shape[2]))
    dv = np.zeros_like(dk)
    for a, b in res:
        dk += a
        dv += b
    return dk, dv


# ----------------------------------------------------------------------------- workload views

def f64(t) -> np.ndarray:
    import torch
    return t.to(torch.float64).numpy()


def bdlm_group0(cfg, inp):
    """KV-head group 0 of a BDLM rank share as float64 arrays over the unsharded key axis
    (every clean key, then the local corrupted keys) with the oracle's mask."""
    p = cfg.problem
    G = p.h_q // p.h_kv
    q = f64(inp["q"][:, :G])
    do = f64(inp["dout"][:, :G])
    k = np.concatenate([f64(inp["k_clean"][:, :1]), f64(inp["k_corr"][:, :1])])
    v = np.concatenate([f64(inp["v_clean"][:, :1]), f64(inp["v_corr"][:, :1])])
    mask = oracle.bdlm_mask_fn(p.clean_len, p.block_size, p.q_clean_offset, p.q_clean_len, list(p.owned_blocks),
                               0, p.clean_len, True)
    return dict(q=q, dout=do, k=k, v=v, mask=mask, scale=p.scale, G=G)


def varlen_group0(cfg, inp):
    G = cfg.h_q // cfg.h_kv
    return dict(q=f64(inp["q"][:, :G]), dout=f64(inp["dout"][:, :G]), k=f64(inp["k"][:, :1]),
                v=f64(inp["v"][:, :1]), mask=oracle.varlen_mask_fn(cfg.cu_seqlens, cfg.causal), scale=cfg.scale, G=G)


def fingerprint(view) -> str:
    """SHA-256 of a strided sample of the float64 inputs (detects a change of the input recipe)."""
    import hashlib
    h = hashlib.sha256()
    for name in ("q", "dout", "k", "v"):
        a = np.ascontiguousarray(view[name][::997])
        h.update(name.encode() + str(view[name].shape).encode() + a.tobytes())
    return h.hexdigest()


def spread_keys(lo: int, hi: int, n: int, seed: int) -> np.ndarray:
    """n keys in [lo, hi): one seeded-random key in each of n equal strata (sorted, distinct)."""
    rng = np.random.default_rng(seed)
    edges = np.linspace(lo, hi, n + 1)
    out = []
    for i in range(n):
        a, b = int(np.ceil(edges[i])), int(np.ceil(edges[i + 1]))
        if b > a:
            out.append(int(rng.integers(a, b)))
    return np.unique(np.asarray(out, dtype=np.int64))
