"""Workload recipes for BDLM-masked core attention: problem sizes, the
corrupted-block ownership list of one rank, varlen shard lengths and seeded
synthetic tensors.

This module holds no attention arithmetic.  It is the only code shared by the
oracle tests and the GPU path: both receive the tensors it draws.

Sources (web pages on block-diffusion training):
  * "Block Parallelism For Efficient Distributed Long-Context Diffusion
    Language Model Training", English abstract: one rank owns each corrupted
    block (block parallelism); the clean sequence is sharded by position across
    the same ranks (context-sharded block parallelism, CSBP).
  * rit.work explainer of CSBP, section "why conventional context parallelism
    sends extra data": early and late blocks are assigned together to balance
    the load across devices.
  * "Efficient Long-context Language Model Training by Core Attention
    Disaggregation", English abstract: core attention over fused batches of
    token-level shards of arbitrary length.

Readings taken where the pages are silent:
  * ownership is a zigzag: rank r of R owns the block pairs (k, N_b-1-k) for
    k in [r*n, (r+1)*n) with n = N_b / (2R); rows list the early range
    ascending, then the late range ascending;
  * every tensor is drawn from its own torch CPU generator seeded with
    ``seed * 64 + index`` (index fixed per tensor name), as float32 N(0,1) times
    the config's scale, then rounded to bfloat16 (round to nearest even).
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

# Tensor names and their fixed generator index.
TENSOR_INDEX = {"q": 0, "k_clean": 1, "v_clean": 2, "k_corr": 3, "v_corr": 4,
                "dout": 5, "k": 6, "v": 7}


@dataclasses.dataclass(frozen=True)
class BdlmProblem:
    """One rank's BDLM attention problem against ONE clean K/V range.

    Query rows: the clean rows at global positions
    [q_clean_offset, q_clean_offset + q_clean_len), then B rows for each owned
    corrupted block, in ``owned_blocks`` order.
    Keys: clean positions [kv_clean_offset, kv_clean_offset + kv_clean_len),
    then (if with_local_corrupt) the local corrupted K/V rows, slot-major.
    """
    clean_len: int
    block_size: int
    q_clean_offset: int
    q_clean_len: int
    owned_blocks: Tuple[int, ...]
    kv_clean_offset: int
    kv_clean_len: int
    with_local_corrupt: bool
    h_q: int
    h_kv: int
    head_dim: int
    softmax_scale: float = 0.0   # <= 0 selects 1/sqrt(head_dim)

    @property
    def n_owned(self) -> int:
        return len(self.owned_blocks)

    @property
    def n_q(self) -> int:
        return self.q_clean_len + self.n_owned * self.block_size

    @property
    def n_corr(self) -> int:
        return self.n_owned * self.block_size

    @property
    def scale(self) -> float:
        return self.softmax_scale if self.softmax_scale > 0 else 1.0 / math.sqrt(self.head_dim)

    def with_kv(self, kv_offset: int, kv_len: int, local: bool) -> "BdlmProblem":
        return dataclasses.replace(self, kv_clean_offset=kv_offset, kv_clean_len=kv_len,
                                   with_local_corrupt=local)


@dataclasses.dataclass(frozen=True)
class BdlmConfig:
    """A BDLM workload: the rank's problem plus how its clean K/V is sharded."""
    name: str
    problem: BdlmProblem               # kv fields describe the UNSHARDED key set
    shards: Tuple[Tuple[int, int, bool], ...]   # (kv_offset, kv_len, with_local_corrupt)
    input_scale: float
    description: str

    def shard_problems(self) -> List[BdlmProblem]:
        return [self.problem.with_kv(o, n, loc) for (o, n, loc) in self.shards]


@dataclasses.dataclass(frozen=True)
class VarlenConfig:
    name: str
    seqlens: Tuple[int, ...]
    h_q: int
    h_kv: int
    head_dim: int
    causal: bool
    input_scale: float
    description: str
    softmax_scale: float = 0.0

    @property
    def total(self) -> int:
        return int(sum(self.seqlens))

    @property
    def cu_seqlens(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.seqlens)]).astype(np.int32)

    @property
    def scale(self) -> float:
        return self.softmax_scale if self.softmax_scale > 0 else 1.0 / math.sqrt(self.head_dim)


@dataclasses.dataclass(frozen=True)
class CadTaskConfig:
    """Packed causal documents cut into core-attention tasks with prefix context.

    The library's task splitter cuts every document of ``docs`` into runs of rows
    whose causal pairs stay within ``max_pairs`` ("Efficient Long-context Language
    Model Training by Core Attention Disaggregation", English abstract: token-level
    tasks rebatched to equalize compute); each task carries its document's prefix
    up to the run's end as key context, gathered into one packed K/V."""
    name: str
    docs: VarlenConfig
    max_pairs: int
    description: str

    @property
    def h_q(self) -> int:
        return self.docs.h_q

    @property
    def h_kv(self) -> int:
        return self.docs.h_kv

    @property
    def head_dim(self) -> int:
        return self.docs.head_dim

    @property
    def scale(self) -> float:
        return self.docs.scale


def task_context_rows(k_cu, kv_src) -> np.ndarray:
    """Packed document row of every context row of every task (int64): the gather index."""
    k_cu = np.asarray(k_cu, dtype=np.int64)
    src = np.asarray(kv_src, dtype=np.int64)
    lens = np.diff(k_cu)
    if lens.size == 0:
        return np.zeros(0, np.int64)
    return np.repeat(src - k_cu[:-1], lens) + np.arange(int(k_cu[-1]), dtype=np.int64)


def zigzag_owned_blocks(n_blocks: int, ranks: int, rank: int) -> np.ndarray:
    """Corrupted blocks owned by ``rank``: early range then mirrored late range."""
    if n_blocks % (2 * ranks) != 0:
        raise ValueError("n_blocks must be a multiple of 2*ranks")
    n = n_blocks // (2 * ranks)
    early = np.arange(rank * n, (rank + 1) * n, dtype=np.int64)
    late = np.arange(n_blocks - (rank + 1) * n, n_blocks - rank * n, dtype=np.int64)
    return np.concatenate([early, late])


def cp_owned_blocks(n_blocks: int, ranks: int, rank: int) -> np.ndarray:
    """Corrupted blocks of ``rank`` under conventional context parallelism: the
    position chunk [rank * n, (rank + 1) * n) of the corrupted copy, n = N_b / R,
    the same positions as the rank's clean chunk."""
    if n_blocks % ranks != 0:
        raise ValueError("n_blocks must be a multiple of ranks")
    n = n_blocks // ranks
    return np.arange(rank * n, (rank + 1) * n, dtype=np.int64)


def varlen_lengths(total: int = 262144, lo: int = 128, hi: int = 65536, seed: int = 0) -> List[int]:
    """Shard lengths log-uniform in [lo, hi] that sum exactly to ``total``.

    Draw floor(exp(U(ln lo, ln hi))) until a draw reaches the remainder; the last
    shard takes the remainder, and if that is below ``lo`` the deficit is moved
    from the previous shard.
    """
    rng = np.random.default_rng(seed)
    out: List[int] = []
    rem = total
    while rem > 0:
        ell = int(math.floor(math.exp(rng.uniform(math.log(lo), math.log(hi)))))
        if ell >= rem:
            ell = rem
        out.append(ell)
        rem -= ell
    if len(out) > 1 and out[-1] < lo:
        deficit = lo - out[-1]
        out[-2] -= deficit
        out[-1] += deficit
    return out


def _bdlm_config(name, L, B, R, rank, hq, hkv, d, scale, n_shards, local_shard, desc,
                 ownership=None) -> BdlmConfig:
    n_blocks = L // B
    owned = (ownership or zigzag_owned_blocks)(n_blocks, R, rank)
    q_off = rank * (L // R)
    q_len = L // R
    prob = BdlmProblem(clean_len=L, block_size=B, q_clean_offset=q_off, q_clean_len=q_len,
                       owned_blocks=tuple(int(b) for b in owned), kv_clean_offset=0,
                       kv_clean_len=L, with_local_corrupt=True, h_q=hq, h_kv=hkv, head_dim=d)
    sh = L // n_shards
    shards = tuple((i * sh, sh, i == local_shard) for i in range(n_shards))
    return BdlmConfig(name=name, problem=prob, shards=shards, input_scale=scale, description=desc)


def config(idx: int):
    """Workloads 1..7 (1: tiny, 2: 4K GQA, 3: 256K/16 rank share, 4: varlen, 5: 1M/8 rank share,
    6: workload 4 as core-attention tasks with prefix context, 7: conventional CP's share of the
    256K combined sequence, rank 8 of 16)."""
    if idx == 1:
        return _bdlm_config("tiny_L256_B32_h1_d64", 256, 32, 1, 0, 1, 1, 64, 1.0, 1, 0,
                            "L=256, B=32, 1/1 heads, d=64, unsharded, all 8 blocks")
    if idx == 2:
        return _bdlm_config("L4096_B64_h16x4_d128", 4096, 64, 1, 0, 16, 4, 128, 0.5, 4, 0,
                            "L=4096, B=64, 16/4 heads, d=128, inputs N(0,1)*0.5, 4 clean shards")
    if idx == 3:
        return _bdlm_config("csbp_256K_r8of16_B32_h32x8_d128", 262144, 32, 16, 8, 32, 8, 128, 1.0,
                            16, 8, "256K clean context split 16 ways, rank 8, B=32, 32/8 heads, d=128")
    if idx == 4:
        lens = tuple(varlen_lengths())
        return VarlenConfig(name="varlen_causal_262144_h32x8_d128", seqlens=lens, h_q=32, h_kv=8,
                            head_dim=128, causal=True, input_scale=1.0,
                            description="packed causal shards, log-uniform lengths in [128, 65536]")
    if idx == 5:
        return _bdlm_config("csbp_1M_r4of8_B16_h32x8_d128", 1048576, 16, 8, 4, 32, 8, 128, 1.0,
                            8, 4, "1M clean context split 8 ways, rank 4, B=16, 32/8 heads, d=128")
    if idx == 7:
        return _bdlm_config("cp_256K_r8of16_B32_h32x8_d128", 262144, 32, 16, 8, 32, 8, 128, 1.0, 16, 8,
                            "conventional context parallelism's share of the 256K combined sequence: "
                            "rank 8 of 16 holds positions [131072, 147456) of both copies",
                            ownership=cp_owned_blocks)
    if idx == 6:
        return CadTaskConfig(name="cad_tasks_262144_max2p26_h32x8_d128", docs=config(4), max_pairs=1 << 26,
                             description="workload 4's documents as core-attention tasks of at most 2^26 "
                                         "causal pairs, each with its prefix context")
    raise ValueError(idx)


def small_bdlm_config(L, B, R, rank, hq, hkv, d, n_shards, scale=1.0, name=None, cp=False) -> BdlmConfig:
    """A scaled-down rank share with the same structure as the large workloads (CSBP's
    zigzag ownership, or with cp=True conventional context parallelism's position chunk)."""
    local = min(rank * n_shards // R, n_shards - 1)
    return _bdlm_config(name or f"small_{'cp' if cp else 'csbp'}_L{L}_B{B}_R{R}_r{rank}", L, B, R, rank, hq,
                        hkv, d, scale, n_shards, local, "scaled-down rank share",
                        ownership=cp_owned_blocks if cp else None)


# ----------------------------------------------------------------------------- tensors

def _randn_bf16(shape, seed: int, index: int, scale: float, chunk_rows: int = 1 << 15):
    """float32 N(0,1)*scale drawn from one generator, rounded to bfloat16."""
    import torch
    g = torch.Generator(device="cpu")
    g.manual_seed(seed * 64 + index)
    out = torch.empty(shape, dtype=torch.bfloat16)
    n = shape[0]
    for s in range(0, n, chunk_rows):
        e = min(n, s + chunk_rows)
        x = torch.randn((e - s,) + tuple(shape[1:]), generator=g, dtype=torch.float32)
        if scale != 1.0:
            x.mul_(scale)
        out[s:e] = x.to(torch.bfloat16)
    return out


def bdlm_inputs(cfg: BdlmConfig, seed: int = 0, names: Optional[Sequence[str]] = None) -> Dict:
    """Seeded bf16 CPU tensors for a BDLM workload.

    q, dout: [n_q, h_q, d]; k_clean, v_clean: [clean_len, h_kv, d] (the whole clean
    sequence; a shard is a row range of it); k_corr, v_corr: [n_owned*B, h_kv, d].
    """
    p = cfg.problem
    shapes = {"q": (p.n_q, p.h_q, p.head_dim), "dout": (p.n_q, p.h_q, p.head_dim),
              "k_clean": (p.clean_len, p.h_kv, p.head_dim), "v_clean": (p.clean_len, p.h_kv, p.head_dim),
              "k_corr": (p.n_corr, p.h_kv, p.head_dim), "v_corr": (p.n_corr, p.h_kv, p.head_dim)}
    names = list(names) if names is not None else list(shapes)
    out = {}
    for nm in names:
        sc = 1.0 if nm == "dout" else cfg.input_scale
        out[nm] = _randn_bf16(shapes[nm], seed, TENSOR_INDEX[nm], sc)
    return out


def varlen_inputs(cfg: VarlenConfig, seed: int = 0, names: Optional[Sequence[str]] = None) -> Dict:
    """Seeded bf16 CPU tensors for packed shards: q, dout [T, h_q, d]; k, v [T, h_kv, d]."""
    T = cfg.total
    shapes = {"q": (T, cfg.h_q, cfg.head_dim), "dout": (T, cfg.h_q, cfg.head_dim),
              "k": (T, cfg.h_kv, cfg.head_dim), "v": (T, cfg.h_kv, cfg.head_dim)}
    names = list(names) if names is not None else list(shapes)
    out = {}
    for nm in names:
        sc = 1.0 if nm == "dout" else cfg.input_scale
        out[nm] = _randn_bf16(shapes[nm], seed, TENSOR_INDEX[nm], sc)
    return out


def task_inputs(n_q: int, n_keys: int, h_q: int, h_kv: int, head_dim: int, seed: int = 0,
                input_scale: float = 1.0) -> Dict:
    """Seeded bf16 CPU tensors for a fused batch of core-attention tasks with their
    own contexts: q, dout [n_q, h_q, d]; k, v [n_keys, h_kv, d]."""
    shapes = {"q": (n_q, h_q, head_dim), "dout": (n_q, h_q, head_dim),
              "k": (n_keys, h_kv, head_dim), "v": (n_keys, h_kv, head_dim)}
    return {nm: _randn_bf16(shp, seed, TENSOR_INDEX[nm], 1.0 if nm == "dout" else input_scale)
            for nm, shp in shapes.items()}


def merge_partials_inputs(n_parts: int, n_rows: int, h: int, d: int, seed: int = 0,
                          neg_inf_frac: float = 0.1):
    """Synthetic LSE-merge partials: O ~ N(0,1) fp32 [S,N,H,d]; LSE ~ U(0,15) fp32
    [S,H,N] with a fraction of entries set to -inf (rows with no legal key)."""
    import torch
    g = torch.Generator(device="cpu")
    g.manual_seed(seed * 64 + 40)
    o = torch.randn((n_parts, n_rows, h, d), generator=g, dtype=torch.float32)
    lse = torch.rand((n_parts, h, n_rows), generator=g, dtype=torch.float32) * 15.0
    drop = torch.rand((n_parts, h, n_rows), generator=g) < neg_inf_frac
    lse[drop] = float("-inf")
    return o, lse
