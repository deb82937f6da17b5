"""Per-rank K/V exchange volume and attention work of two position shardings of
a BDLM training step over R ranks.

* CSBP ("Block Parallelism For Efficient Distributed Long-Context Diffusion
  Language Model Training", English abstract; rit.work explainer of CSBP,
  section on context-sharded block parallelism): rank r holds clean shard r and
  the zigzag pairs of corrupted blocks; only clean K/V cross devices, and a rank
  needs a remote clean shard only if one of its rows has a legal key in it.
* Conventional context parallelism (same explainer, section "why conventional
  context parallelism sends extra data"): rank r holds the positions of chunk r
  in both the clean and the corrupted copy, and the K/V exchange, blind to the
  mask, moves every remote chunk of both copies in the forward and returns their
  gradients in the backward, although no row attends another rank's corrupted
  keys.

Pair counts come from the library's tile planner (host code, no GPU needed).
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List

import numpy as np

from . import bdattn as B
from . import workloads as wl


@dataclasses.dataclass(frozen=True)
class RankExchange:
    scheme: str
    rank: int
    pairs: int                 # legal (row, key) pairs per q-head of the rank's rows
    remote_clean_needed: int   # remote clean shards holding a legal key for the rank
    kv_bytes_received: int     # forward K and V received; the backward returns as many gradient bytes
    kv_bytes_needed: int       # the part of kv_bytes_received that holds a legal key


def _owned(scheme: str, n_blocks: int, ranks: int, rank: int) -> np.ndarray:
    if scheme == "csbp":
        return wl.zigzag_owned_blocks(n_blocks, ranks, rank)
    if scheme == "cp":
        return wl.cp_owned_blocks(n_blocks, ranks, rank)
    raise ValueError(scheme)


def rank_exchange(clean_len: int, block_size: int, ranks: int, rank: int, h_kv: int, head_dim: int,
                  scheme: str, elem_bytes: int = 2) -> RankExchange:
    L, R = clean_len, ranks
    if L % R or (L // R) % block_size:
        raise ValueError("each rank's chunk must be whole blocks")
    n = L // R
    owned = tuple(int(b) for b in _owned(scheme, L // block_size, R, rank))
    chunk = n * h_kv * head_dim * 2 * elem_bytes          # K and V of one chunk of one copy
    pairs, needed = 0, 0
    for s in range(R):
        p = wl.BdlmProblem(L, block_size, rank * n, n, owned, s * n, n, s == rank, 1, 1, 64)
        u = B.Plan.from_problem(p).useful_pairs
        pairs += u
        if s != rank and u > 0:
            needed += 1
    copies = 1 if scheme == "csbp" else 2
    received = (needed if scheme == "csbp" else R - 1) * copies * chunk
    return RankExchange(scheme, rank, pairs, needed, received, needed * chunk)


def compare_schemes(clean_len: int, block_size: int, ranks: int, h_kv: int, head_dim: int) -> Dict:
    """Per-rank exchange and work of both schemes, with the balance of the work."""
    out: Dict[str, List[RankExchange]] = {}
    for scheme in ("csbp", "cp"):
        out[scheme] = [rank_exchange(clean_len, block_size, ranks, r, h_kv, head_dim, scheme)
                       for r in range(ranks)]
    summary = {}
    for scheme, rs in out.items():
        pr = np.array([x.pairs for x in rs], dtype=np.float64)
        summary[scheme] = {"pairs_max_over_mean": round(float(pr.max() / pr.mean()), 4),
                           "busiest_rank": int(pr.argmax()),
                           "kv_bytes_received_max": int(max(x.kv_bytes_received for x in rs)),
                           "kv_bytes_received_total": int(sum(x.kv_bytes_received for x in rs)),
                           "kv_bytes_needed_total": int(sum(x.kv_bytes_needed for x in rs))}
    return {"ranks": out, "summary": summary}
