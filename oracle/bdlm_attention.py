"""Oracle for BDLM-masked core attention: plain, slow, obviously correct, CPU, fp64.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this module; only tests/, the smoke check of __graft_entry__ and the
cpu_baseline leg of bench.py use it.  It shares no code with the HIP path: it
builds the explicit boolean mask and does dense masked softmax attention and
its analytic gradients with numpy in float64.

What it follows (page titles; the pages print no formulas, so each function
states the definition it writes out):

* Mask -- rit.work explainer of CSBP, section "why conventional context
  parallelism sends extra data": every corrupted (noised) target block sees the
  clean prefix of the preceding blocks and its own noised version; corrupted
  K/V serve only the block that owns them.  "Block Parallelism For Efficient
  Distributed Long-Context Diffusion Language Model Training", English
  abstract: autoregressive dependencies across blocks, parallel denoising
  within a block -> clean tokens attend block-causally to clean tokens.
* Attention -- "Efficient Long-context Language Model Training by Core
  Attention Disaggregation", English abstract: core attention is
  softmax(QK^T)V, stateless and composable over token-level shards.
* Exactness of sharding -- the block-parallelism abstract: CSBP preserves the
  BDLM training semantics; the explainer: the loss and gradients do not change.
  Partials over clean K/V ranges therefore combine exactly through their
  log-sum-exp (LSE), and the backward of a range uses the merged LSE.

Conventions (readings where the pages are silent):
  scores S = scale * q.k with scale = 1/sqrt(d) unless given; natural-log LSE;
  q-head h uses KV head h // (H_q / H_kv); a row with no legal key has O = 0 and
  LSE = -inf; the backward is that of the scalar <dO, O>.
"""
from __future__ import annotations

import math
from typing import Callable, Optional, Sequence, Tuple

import numpy as np

NEG_INF = -np.inf

MaskFn = Callable[[np.ndarray, np.ndarray], np.ndarray]


# ----------------------------------------------------------------------------- masks

def bdlm_mask(clean_len: int, block_size: int, q_clean_offset: int, q_clean_len: int,
              owned_blocks: Sequence[int], kv_clean_offset: int, kv_clean_len: int,
              with_local_corrupt: bool, rows: Optional[np.ndarray] = None,
              keys: Optional[np.ndarray] = None) -> np.ndarray:
    """Explicit boolean BDLM mask M[row, key] for one rank against one clean K/V range.

    Rows: clean query rows (global clean positions q_clean_offset + i), then B rows
    per owned corrupted block in list order.  Keys: the clean positions
    kv_clean_offset + j, then (if with_local_corrupt) B local corrupted K/V rows
    per owned block in the same order.

      clean row p,      clean key t      : block(t) <= block(p)       (block-causal)
      clean row,        corrupted key    : never
      corrupted block b, clean key t     : block(t) <  b              (clean prefix only)
      corrupted slot m, corrupted slot m': m == m'                    (own noised block)
    """
    B = int(block_size)
    owned = np.asarray(owned_blocks, dtype=np.int64)
    n_q = q_clean_len + owned.size * B
    n_k = kv_clean_len + (owned.size * B if with_local_corrupt else 0)
    rows = np.arange(n_q, dtype=np.int64) if rows is None else np.asarray(rows, dtype=np.int64)
    keys = np.arange(n_k, dtype=np.int64) if keys is None else np.asarray(keys, dtype=np.int64)
    if rows.size and (rows.min() < 0 or rows.max() >= n_q):
        raise IndexError("row out of range")
    if keys.size and (keys.min() < 0 or keys.max() >= n_k):
        raise IndexError("key out of range")

    row_clean = rows < q_clean_len
    row_slot = np.where(row_clean, -1, (rows - q_clean_len) // B)
    # block of the row's token: its clean block, or the corrupted block it denoises
    row_block = np.where(row_clean, (q_clean_offset + rows) // B,
                         owned[np.clip(row_slot, 0, max(owned.size - 1, 0))] if owned.size else 0)

    key_clean = keys < kv_clean_len
    key_block = (kv_clean_offset + keys) // B          # meaningful for clean keys only
    key_slot = np.where(key_clean, -1, (keys - kv_clean_len) // B)

    rc = row_clean[:, None]
    kc = key_clean[None, :]
    clean_clean = rc & kc & (key_block[None, :] <= row_block[:, None])
    corr_clean = (~rc) & kc & (key_block[None, :] < row_block[:, None])
    corr_corr = (~rc) & (~kc) & (key_slot[None, :] == row_slot[:, None])
    return clean_clean | corr_clean | corr_corr


def bdlm_mask_fn(clean_len, block_size, q_clean_offset, q_clean_len, owned_blocks,
                 kv_clean_offset, kv_clean_len, with_local_corrupt) -> MaskFn:
    def fn(rows, keys):
        return bdlm_mask(clean_len, block_size, q_clean_offset, q_clean_len, owned_blocks,
                         kv_clean_offset, kv_clean_len, with_local_corrupt, rows, keys)
    return fn


def combined_mask(clean_len: int, block_size: int, rows: Optional[np.ndarray] = None,
                  keys: Optional[np.ndarray] = None) -> np.ndarray:
    """The BDLM mask over the whole combined sequence, before any sharding.

    Index i < L is the clean token at position i; index L + i is the corrupted
    (noised) token at position i, which belongs to target block i // B.  This is
    the sequence that conventional context parallelism shards by position
    ("Block Parallelism For Efficient Distributed Long-Context Diffusion Language
    Model Training", English abstract; rit.work explainer of CSBP, section "why
    conventional context parallelism sends extra data"):

      clean i      -> clean j      : block(j) <= block(i)
      clean i      -> corrupted    : never
      corrupted i  -> clean j      : block(j) <  block(i)
      corrupted i  -> corrupted j  : block(j) == block(i)
    """
    L, B = int(clean_len), int(block_size)
    rows = np.arange(2 * L, dtype=np.int64) if rows is None else np.asarray(rows, dtype=np.int64)
    keys = np.arange(2 * L, dtype=np.int64) if keys is None else np.asarray(keys, dtype=np.int64)
    rc, kc = rows < L, keys < L
    rb, kb = (rows % L) // B, (keys % L) // B
    cc = rc[:, None] & kc[None, :] & (kb[None, :] <= rb[:, None])
    xc = ~rc[:, None] & kc[None, :] & (kb[None, :] < rb[:, None])
    xx = ~rc[:, None] & ~kc[None, :] & (kb[None, :] == rb[:, None])
    return cc | xc | xx


def varlen_mask(cu_seqlens: Sequence[int], causal: bool, rows: Optional[np.ndarray] = None,
                keys: Optional[np.ndarray] = None) -> np.ndarray:
    """Packed independent shards: key j is legal for row i iff both lie in the same
    shard and (if causal) j <= i."""
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    total = int(cu[-1])
    rows = np.arange(total, dtype=np.int64) if rows is None else np.asarray(rows, dtype=np.int64)
    keys = np.arange(total, dtype=np.int64) if keys is None else np.asarray(keys, dtype=np.int64)
    rs = np.searchsorted(cu, rows, side="right") - 1
    ks = np.searchsorted(cu, keys, side="right") - 1
    m = rs[:, None] == ks[None, :]
    if causal:
        m &= keys[None, :] <= rows[:, None]
    return m


def varlen_mask_fn(cu_seqlens, causal) -> MaskFn:
    return lambda rows, keys: varlen_mask(cu_seqlens, causal, rows, keys)


def task_mask(q_cu: Sequence[int], k_cu: Sequence[int], causal: bool, rows: Optional[np.ndarray] = None,
              keys: Optional[np.ndarray] = None) -> np.ndarray:
    """Core-attention tasks that carry their own key context ("Efficient
    Long-context Language Model Training by Core Attention Disaggregation",
    English abstract: core attention as a stateless task over token-level shards).

    Task t owns query rows [q_cu[t], q_cu[t+1]) and key rows [k_cu[t], k_cu[t+1]).
    Key j is legal for row i iff both belong to the same task and, if causal, j is
    among the first k_len - q_len + i' + 1 keys of the task (i' = the row's index
    within its task): the queries are the last q_len positions of the task's
    context (bottom-right alignment), so a task whose keys are a document's
    prefix up to the end of a query chunk reproduces the document's causal
    attention for that chunk.
    """
    qc = np.asarray(q_cu, dtype=np.int64)
    kc = np.asarray(k_cu, dtype=np.int64)
    rows = np.arange(int(qc[-1]), dtype=np.int64) if rows is None else np.asarray(rows, dtype=np.int64)
    keys = np.arange(int(kc[-1]), dtype=np.int64) if keys is None else np.asarray(keys, dtype=np.int64)
    tr = np.searchsorted(qc, rows, side="right") - 1
    tk = np.searchsorted(kc, keys, side="right") - 1
    m = tr[:, None] == tk[None, :]
    if causal:
        q_len = qc[tr + 1] - qc[tr]
        k_len = kc[tr + 1] - kc[tr]
        limit = kc[tr] + k_len - q_len + (rows - qc[tr]) + 1    # legal keys lie below this index
        m &= keys[None, :] < limit[:, None]
    return m


def task_mask_fn(q_cu, k_cu, causal) -> MaskFn:
    return lambda rows, keys: task_mask(q_cu, k_cu, causal, rows, keys)


# ----------------------------------------------------------------------------- attention

def _heads(q, k):
    n, hq, d = q.shape
    hkv = k.shape[1]
    if hq % hkv:
        raise ValueError("h_q must be a multiple of h_kv")
    return hq, hkv, hq // hkv


def attention_fwd(q: np.ndarray, k: np.ndarray, v: np.ndarray, mask_fn: MaskFn, scale: float,
                  rows: Optional[np.ndarray] = None, row_block: int = 1024
                  ) -> Tuple[np.ndarray, np.ndarray]:
    """Masked softmax attention, fp64.

    q [N, H_q, d], k/v [M, H_kv, d].  Returns O [len(rows), H_q, d] and LSE
    [H_q, len(rows)] with LSE_i = ln sum_{j legal} exp(S_ij), O_i = sum_j P_ij v_j,
    P_ij = exp(S_ij - LSE_i); a row with no legal key gets O = 0, LSE = -inf.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    hq, hkv, G = _heads(q, k)
    rows = np.arange(q.shape[0]) if rows is None else np.asarray(rows, dtype=np.int64)
    keys = np.arange(k.shape[0])
    o = np.zeros((rows.size, hq, q.shape[2]))
    lse = np.full((hq, rows.size), NEG_INF)
    for r0 in range(0, rows.size, row_block):
        rr = rows[r0:r0 + row_block]
        m = mask_fn(rr, keys)
        for h in range(hq):
            g = h // G
            s = scale * (q[rr, h, :] @ k[:, g, :].T)
            s = np.where(m, s, NEG_INF)
            mx = s.max(axis=1, initial=NEG_INF)
            has = np.isfinite(mx)
            mx_safe = np.where(has, mx, 0.0)
            e = np.exp(s - mx_safe[:, None])          # exp(-inf) = 0 off the mask
            tot = e.sum(axis=1)
            l = np.where(has, mx_safe + np.log(np.where(has, tot, 1.0)), NEG_INF)
            p = np.where(has[:, None], e / np.where(has, tot, 1.0)[:, None], 0.0)
            o[r0:r0 + rr.size, h, :] = p @ v[:, g, :]
            lse[h, r0:r0 + rr.size] = l
    return o, lse


def softmax_probs(q, k, mask_fn, scale, h, rows=None):
    """P for one q-head (rows x all keys), used by the row-sum self-checks."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    hq, hkv, G = _heads(q, k)
    rows = np.arange(q.shape[0]) if rows is None else np.asarray(rows)
    m = mask_fn(rows, np.arange(k.shape[0]))
    s = np.where(m, scale * (q[rows, h, :] @ k[:, h // G, :].T), NEG_INF)
    mx = s.max(axis=1, initial=NEG_INF)
    has = np.isfinite(mx)
    e = np.exp(s - np.where(has, mx, 0.0)[:, None])
    tot = e.sum(axis=1)
    return np.where(has[:, None], e / np.where(has, tot, 1.0)[:, None], 0.0)


def delta_rows(o: np.ndarray, dout: np.ndarray) -> np.ndarray:
    """D[h, i] = <dO_i,h , O_i,h>: the row term of the softmax backward, [H_q, N]."""
    return np.einsum("nhd,nhd->hn", np.asarray(dout, np.float64), np.asarray(o, np.float64))


def attention_bwd(q, k, v, dout, lse, delta, mask_fn: MaskFn, scale: float,
                  rows: Optional[np.ndarray] = None, keys: Optional[np.ndarray] = None,
                  row_block: int = 1024):
    """Gradients of <dO, O> for masked softmax attention, fp64.

    ``lse`` [H_q, len(rows)] and ``delta`` [H_q, len(rows)] are those of the rows
    (for a sharded run: the MERGED LSE and D of the full output).  With
    P = exp(S - LSE) on the mask (0 elsewhere):
        dV_g += P^T dO_h,  dP = dO_h V_g^T,  dS = P o (dP - D),
        dQ_h  = scale dS K_g,  dK_g += scale dS^T Q_h.
    ``rows``/``keys`` restrict the computation to those rows and key columns (dQ
    is then only the part from the selected keys).  Returns dQ [len(rows), H_q, d],
    dK/dV [len(keys), H_kv, d].
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    dout = np.asarray(dout, dtype=np.float64)
    hq, hkv, G = _heads(q, k)
    rows = np.arange(q.shape[0]) if rows is None else np.asarray(rows, dtype=np.int64)
    keys = np.arange(k.shape[0]) if keys is None else np.asarray(keys, dtype=np.int64)
    lse = np.asarray(lse, dtype=np.float64)
    delta = np.asarray(delta, dtype=np.float64)
    dq = np.zeros((rows.size, hq, q.shape[2]))
    dk = np.zeros((keys.size, hkv, k.shape[2]))
    dv = np.zeros((keys.size, hkv, v.shape[2]))
    kk, vv = k[keys], v[keys]
    for r0 in range(0, rows.size, row_block):
        rr = rows[r0:r0 + row_block]
        sl = slice(r0, r0 + rr.size)
        m = mask_fn(rr, keys)
        for h in range(hq):
            g = h // G
            l = lse[h, sl]
            fin = np.isfinite(l)
            s = scale * (q[rr, h, :] @ kk[:, g, :].T)
            p = np.where(m & fin[:, None], np.exp(s - np.where(fin, l, 0.0)[:, None]), 0.0)
            dv[:, g, :] += p.T @ dout[rr, h, :]
            dp = dout[rr, h, :] @ vv[:, g, :].T
            ds = p * (dp - delta[h, sl][:, None])
            dq[sl, h, :] = scale * (ds @ kk[:, g, :])
            dk[:, g, :] += scale * (ds.T @ q[rr, h, :])
    return dq, dk, dv


# ----------------------------------------------------------------------------- merge

def lse_merge(o_parts: np.ndarray, lse_parts: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Exact merge of partials computed over disjoint key sets.

    o_parts [S, N, H, d], lse_parts [S, H, N]:
      m = max_s LSE_s,  LSE = m + ln sum_s exp(LSE_s - m),  O = sum_s exp(LSE_s - LSE) O_s;
    a row whose partials are all -inf gets O = 0 and LSE = -inf.
    """
    o_parts = np.asarray(o_parts, dtype=np.float64)
    lse_parts = np.asarray(lse_parts, dtype=np.float64)
    m = lse_parts.max(axis=0)
    has = np.isfinite(m)
    m_safe = np.where(has, m, 0.0)
    tot = np.exp(lse_parts - m_safe[None]).sum(axis=0)
    lse = np.where(has, m_safe + np.log(np.where(has, tot, 1.0)), NEG_INF)
    coef = np.where(has[None], np.exp(lse_parts - np.where(has, lse, 0.0)[None]), 0.0)
    o = np.zeros(o_parts.shape[1:])
    for s in range(o_parts.shape[0]):
        o += np.transpose(coef[s])[:, :, None] * o_parts[s]
    return o, lse


# ----------------------------------------------------------------------------- BDLM helpers

def bdlm_keys(k_clean_shard, k_corr, with_local_corrupt):
    """Key array of one call: the clean range rows, then the local corrupted rows."""
    if with_local_corrupt:
        return np.concatenate([np.asarray(k_clean_shard, np.float64), np.asarray(k_corr, np.float64)], axis=0)
    return np.asarray(k_clean_shard, np.float64)


def bdlm_fwd(prob: dict, q, k_clean_shard, v_clean_shard, k_corr, v_corr, rows=None):
    """Partial (O, LSE) of a rank's queries against one clean K/V range (+ local corrupted K/V).

    ``prob`` keys: clean_len, block_size, q_clean_offset, q_clean_len, owned_blocks,
    kv_clean_offset, kv_clean_len, with_local_corrupt, scale.
    """
    mf = bdlm_mask_fn(prob["clean_len"], prob["block_size"], prob["q_clean_offset"],
                      prob["q_clean_len"], prob["owned_blocks"], prob["kv_clean_offset"],
                      prob["kv_clean_len"], prob["with_local_corrupt"])
    k = bdlm_keys(k_clean_shard, k_corr, prob["with_local_corrupt"])
    v = bdlm_keys(v_clean_shard, v_corr, prob["with_local_corrupt"])
    return attention_fwd(q, k, v, mf, prob["scale"], rows=rows)


def bdlm_bwd(prob: dict, q, k_clean_shard, v_clean_shard, k_corr, v_corr, dout, lse, delta,
             rows=None, keys=None):
    """Gradients of one K/V range, given the merged LSE and D of the rows.

    Returns dQ (this range's contribution), and dK/dV of the range's keys: the clean
    rows first, then the local corrupted rows if the call has them.
    """
    mf = bdlm_mask_fn(prob["clean_len"], prob["block_size"], prob["q_clean_offset"],
                      prob["q_clean_len"], prob["owned_blocks"], prob["kv_clean_offset"],
                      prob["kv_clean_len"], prob["with_local_corrupt"])
    k = bdlm_keys(k_clean_shard, k_corr, prob["with_local_corrupt"])
    v = bdlm_keys(v_clean_shard, v_corr, prob["with_local_corrupt"])
    return attention_bwd(q, k, v, dout, lse, delta, mf, prob["scale"], rows=rows, keys=keys)


def varlen_fwd(q, k, v, cu_seqlens, causal, scale, rows=None):
    return attention_fwd(q, k, v, varlen_mask_fn(cu_seqlens, causal), scale, rows=rows)


def varlen_bwd(q, k, v, dout, lse, delta, cu_seqlens, causal, scale, rows=None, keys=None):
    return attention_bwd(q, k, v, dout, lse, delta, varlen_mask_fn(cu_seqlens, causal), scale,
                         rows=rows, keys=keys)


def task_fwd(q, k, v, q_cu, k_cu, causal, scale, rows=None):
    return attention_fwd(q, k, v, task_mask_fn(q_cu, k_cu, causal), scale, rows=rows)


def task_bwd(q, k, v, dout, lse, delta, q_cu, k_cu, causal, scale, rows=None, keys=None):
    return attention_bwd(q, k, v, dout, lse, delta, task_mask_fn(q_cu, k_cu, causal), scale,
                         rows=rows, keys=keys)


def count_pairs(mask_fn: MaskFn, n_rows: int, n_keys: int, row_block: int = 4096) -> int:
    """Number of legal (row, key) pairs, counted from the explicit mask."""
    keys = np.arange(n_keys)
    tot = 0
    for r0 in range(0, n_rows, row_block):
        tot += int(mask_fn(np.arange(r0, min(n_rows, r0 + row_block)), keys).sum())
    return tot
