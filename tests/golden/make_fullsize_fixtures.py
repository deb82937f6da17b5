"""Write the full-size dK/dV references of the GPU parity tests (calls only the
oracle, through tests/fullsize_ref.py, and the seeded input recipe).

    python tests/golden/make_fullsize_fixtures.py [--workloads 3 7 4 5] [--threads N]

A key's dK and dV depend on every row that attends it, and each of those rows
needs its LSE and delta (delta = <dO, O>), i.e. the whole forward of its
KV-head group over all keys: minutes of fp64 work per workload at full size
(about 1.5e11 legal pairs per head at the 1M rank share).  This script does
that work once, on the CPU, and stores, per workload, for KV head 0 (q-heads
0 .. G-1): the selected keys, their fp64 dK and dV, the fp64 LSE of every row
(rank shares of the 256K sequence only; 1 MiB each) and a fingerprint of the
inputs.  The GPU tests draw the same seeded inputs, check the fingerprint and
compare the GPU's dK/dV on those keys element by element.

Keys: one seeded-random key in each of equal strata of the attended key range
(so the bulk keys that almost every row attends are covered, not only the
rarely attended ones), a few keys past the last attended one (their gradients
are exactly zero), and whole corrupted self-blocks (rank shares); for the
varlen workload, strata over the whole packed axis plus strata inside the
longest document.
"""
from __future__ import annotations

import argparse
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
for p in (ROOT, os.path.dirname(HERE)):
    if p not in sys.path:
        sys.path.insert(0, p)

import fullsize_ref as fr  # noqa: E402
from masked_long_context_amd import workloads as wl  # noqa: E402

# workload -> (clean keys spread over the attended range, keys past it, corrupted self-blocks)
BDLM_KEYS = {3: (440, 8, 2), 7: (440, 8, 2), 5: (952, 8, 4)}
VARLEN_KEYS = (512, 256)     # spread over the packed axis, spread inside the longest document
STORE_LSE = {3, 7}


def fixture_path(idx: int) -> str:
    return os.path.join(HERE, f"fullsize_w{idx}.npz")


def bdlm_keys(cfg, n_clean: int, n_tail: int, n_blocks: int, seed: int) -> np.ndarray:
    p = cfg.problem
    B = p.block_size
    # the last clean key any row attends, + 1: a clean row's own block end, or a
    # corrupted block's start (its clean prefix)
    top = max(p.q_clean_offset + p.q_clean_len if p.q_clean_len else 0, max(p.owned_blocks) * B)
    clean = fr.spread_keys(0, top, n_clean, seed)
    tail = fr.spread_keys(top, p.clean_len, n_tail, seed + 1) if top < p.clean_len else np.zeros(0, np.int64)
    rng = np.random.default_rng(seed + 2)
    slots = np.sort(rng.choice(p.n_owned, n_blocks, replace=False))
    corr = np.concatenate([p.clean_len + np.arange(m * B, (m + 1) * B) for m in slots])
    return np.concatenate([clean, tail, corr]).astype(np.int64)


def varlen_keys(cfg, n_all: int, n_long: int, seed: int) -> np.ndarray:
    cu = cfg.cu_seqlens
    longest = int(np.argmax(cfg.seqlens))
    a = fr.spread_keys(0, cfg.total, n_all, seed)
    b = fr.spread_keys(int(cu[longest]), int(cu[longest + 1]), n_long, seed + 1)
    return np.unique(np.concatenate([a, b]))


def make(idx: int, threads: int):
    cfg = wl.config(idx)
    t0 = time.time()
    print(f"[w{idx}] {cfg.name}: drawing inputs", flush=True)
    if isinstance(cfg, wl.VarlenConfig):
        view = fr.varlen_group0(cfg, wl.varlen_inputs(cfg, seed=0))
        keys = varlen_keys(cfg, *VARLEN_KEYS, seed=100 + idx)
    else:
        view = fr.bdlm_group0(cfg, wl.bdlm_inputs(cfg, seed=0))
        keys = bdlm_keys(cfg, *BDLM_KEYS[idx], seed=100 + idx)
    n = view["q"].shape[0]
    print(f"[w{idx}] {n} rows x {view['G']} q-heads, {view['k'].shape[0]} keys; forward of every row "
          f"({time.time() - t0:.0f} s)", flush=True)
    lse, delta = fr.lse_delta_all_rows(view["q"], view["k"], view["v"], view["dout"], view["mask"], view["scale"],
                                       n, threads=threads)
    print(f"[w{idx}] dK/dV of {keys.size} keys ({time.time() - t0:.0f} s)", flush=True)
    dk, dv = fr.keys_reference(view["q"], view["k"], view["v"], view["dout"], lse, delta, view["mask"],
                               view["scale"], keys, threads=threads)
    out = dict(workload=np.array(cfg.name), fingerprint=np.array(fr.fingerprint(view)), keys=keys,
               dk=dk[:, 0], dv=dv[:, 0], group=np.array(view["G"]))
    if idx in STORE_LSE:
        out["lse"] = lse
    np.savez(fixture_path(idx), **out)
    print(f"[w{idx}] wrote {fixture_path(idx)} ({os.path.getsize(fixture_path(idx)) / 2**20:.1f} MiB, "
          f"{time.time() - t0:.0f} s)", flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--workloads", type=int, nargs="+", default=[3, 7, 4, 5])
    ap.add_argument("--threads", type=int, default=None)
    a = ap.parse_args()
    for idx in a.workloads:
        make(idx, a.threads)


if __name__ == "__main__":
    main()
