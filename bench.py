"""Benchmark: one CSBP rank's BDLM-masked attention step (forward + backward)
on one MI355X.

A step is the whole per-rank path over one batch of synthetic input: the
forward partial against every clean K/V shard, the LSE merge, the backward
preparation, the backward against every shard and the dQ finalize.  Inputs
are resident in HBM before the timed region.  Throughput counts useful
(unmasked) pairs only: 4d flops per pair and q-head in the forward (QK^T, PV)
and 10d in the backward (QK^T recompute, dO V^T, P^T dO, dS^T Q, dS K).

    python bench.py [--steps K] [--warmup W] [--config 3] [--no-cpu-baseline]

Prints one JSON line.  --gpus N with N > 1 is refused: this path runs on one GPU.
With the CPU baseline (the default), the line also carries "parity": the errors of
the step's outputs against the oracle's on the baseline's sample.

The roofline entry's "traffic" (HBM bytes per launch of the dK/dV kernel) comes
from rocprofv3 FETCH_SIZE and WRITE_SIZE passes recorded in profiles/; it is
reported only while the kernel sources still hash to the profiled ones.
"""
from __future__ import annotations

import argparse
import contextlib
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "BDLM attention fwd+bwd useful-pair TFLOP/s and % bf16 MFMA peak, 256K/rank"
PEAK_BF16_TFLOPS = 2500.0      # MI355X published dense bf16 MFMA peak
PEAK_HBM_GBS = 8000.0          # MI355X published HBM3E bandwidth
TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "dkdv_kernel_256K_rank_share_hbm_traffic.md")
KERNEL_SOURCES = ["masked_long_context_amd/csrc/tiling.h", "masked_long_context_amd/csrc/kernels/bwd.hip",
                  "masked_long_context_amd/csrc/kernels/common.h", "masked_long_context_amd/csrc/kernels/kernels.h",
                  "masked_long_context_amd/csrc/kernels/lds_layout.h", "masked_long_context_amd/csrc/kernels/tiles.h"]


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(rel.encode() + b"\0" + f.read())
    return h.hexdigest()


def profiled_traffic(workload: str):
    """HBM bytes per dK/dV launch from the committed counter summary, or None when
    the summary is missing, covers another workload, or the kernel changed since."""
    try:
        with open(TRAFFIC_PROFILE) as f:
            kv = dict(l.strip("` \n").split(" = ", 1) for l in f if l.startswith("`") and " = " in l)
    except OSError:
        return None
    if kv.get("kernel_source_sha256") != kernel_source_hash() or kv.get("workload") != workload:
        return None
    return int(kv["traffic_bytes_per_launch"])


def timed_steps(run_step, steps: int):
    """Run `steps` steps between two events on the current stream, with an event after
    each step: the mean step time over the whole span, and the median of the steps."""
    import torch
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    torch.cuda.synchronize()
    ev[0].record()
    for i in range(steps):
        run_step()
        ev[i + 1].record()
    torch.cuda.synchronize()
    per = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(steps))
    return ev[0].elapsed_time(ev[steps]) / steps, per[len(per) // 2]


def aux_bandwidth(tot, steps: int, rows: int, h: int, d: int) -> dict:
    """Achieved HBM rate of the step's bandwidth-bound calls, from their algorithmic
    bytes per (row, q-head): preprocess reads the fp32 O (4d) and dO (2d), writes
    delta (4) and clears the fp32 dQ accumulator (4d); the output cast and the dQ
    finalize each read 4d and write 2d."""
    out = {}
    for tag, per_rowhead in (("prepare", 10 * d + 4), ("cast", 6 * d), ("finalize", 6 * d)):
        t_ms = tot.get(tag, (0.0, 1))[0] / steps
        out[f"{tag}_ms"] = round(t_ms, 4)
        if t_ms > 0:
            gbs = rows * h * per_rowhead / (t_ms * 1e-3) / 1e9
            out[f"{tag}_gbs"] = round(gbs, 1)
            out[f"{tag}_frac_hbm"] = round(gbs / PEAK_HBM_GBS, 4)
    return out


class EventTimer:
    """HIP events on the current stream (the stream the library launches on) around each call."""

    def __init__(self):
        import torch
        self.torch = torch
        self.events = {}
        self.enabled = False

    @contextlib.contextmanager
    def __call__(self, tag):
        if not self.enabled:
            yield
            return
        t = self.torch
        a, b = t.cuda.Event(enable_timing=True), t.cuda.Event(enable_timing=True)
        a.record()
        yield
        b.record()
        self.events.setdefault(tag, []).append((a, b))

    def totals_ms(self):
        self.torch.cuda.synchronize()
        return {k: (sum(a.elapsed_time(b) for a, b in v), len(v)) for k, v in self.events.items()}


# Dense score elements (rows x keys x q-heads) the CPU baseline's sample aims at:
# about 10-30 s of the fp64 oracle on a GPU machine's host.
CPU_SAMPLE_ELEMS = 1.0e9


def _f64(t):
    import torch
    return t.to(dtype=torch.float64).numpy()


def cpu_baseline(cfg, inp_cpu, step_pairs: int, seed: int = 0, tasks=None):
    """The fp64 oracle, as it stands, timed on the host cores: forward + backward of a
    sample of the workload.  The tiny and the 4K workloads run whole (every row and
    head); the others run the q-heads of KV group 0 on seeded-random query rows
    against every key, sized to about CPU_SAMPLE_ELEMS dense score elements, and the
    step time is extrapolated linearly by useful pairs.  Returns the JSON object."""
    import numpy as np
    import oracle
    from masked_long_context_amd import workloads as wl
    rng = np.random.default_rng(seed)
    if isinstance(cfg, wl.BdlmConfig):
        p = cfg.problem
        whole = p.n_q * (p.clean_len + p.n_corr) * p.h_q <= CPU_SAMPLE_ELEMS * 2
        G = p.h_q if whole else p.h_q // p.h_kv
        hk = p.h_kv if whole else 1
        prob = dict(clean_len=p.clean_len, block_size=p.block_size, q_clean_offset=p.q_clean_offset,
                    q_clean_len=p.q_clean_len, owned_blocks=list(p.owned_blocks), kv_clean_offset=0,
                    kv_clean_len=p.clean_len, with_local_corrupt=True, scale=p.scale)
        n_q, n_keys, hq, d = p.n_q, p.clean_len + p.n_corr, p.h_q, p.head_dim
        q, do = _f64(inp_cpu["q"][:, :G]), _f64(inp_cpu["dout"][:, :G])
        kc, vc = _f64(inp_cpu["k_clean"][:, :hk]), _f64(inp_cpu["v_clean"][:, :hk])
        kx, vx = _f64(inp_cpu["k_corr"][:, :hk]), _f64(inp_cpu["v_corr"][:, :hk])
        mask = oracle.bdlm_mask_fn(p.clean_len, p.block_size, p.q_clean_offset, p.q_clean_len, list(p.owned_blocks),
                                   0, p.clean_len, True)
        fwd = lambda rows: oracle.bdlm_fwd(prob, q, kc, vc, kx, vx, rows=rows)
        bwd = lambda rows, lse, D: oracle.bdlm_bwd(prob, q, kc, vc, kx, vx, do, lse, D, rows=rows)
    else:
        docs = cfg.docs if tasks is not None else cfg
        hq, d = docs.h_q, docs.head_dim
        G, whole = hq // docs.h_kv, False
        q, do = _f64(inp_cpu["q"][:, :G]), _f64(inp_cpu["dout"][:, :G])
        k, v = _f64(inp_cpu["k"][:, :1]), _f64(inp_cpu["v"][:, :1])
        n_q = q.shape[0]
        if tasks is not None:
            q_cu, k_cu, rows_idx = tasks
            k, v = k[rows_idx], v[rows_idx]
            mask = oracle.task_mask_fn(q_cu, k_cu, True)
            fwd = lambda rows: oracle.task_fwd(q, k, v, q_cu, k_cu, True, docs.scale, rows=rows)
            bwd = lambda rows, lse, D: oracle.task_bwd(q, k, v, do, lse, D, q_cu, k_cu, True, docs.scale, rows=rows)
        else:
            cu = docs.cu_seqlens
            mask = oracle.varlen_mask_fn(cu, True)
            fwd = lambda rows: oracle.varlen_fwd(q, k, v, cu, True, docs.scale, rows=rows)
            bwd = lambda rows, lse, D: oracle.varlen_bwd(q, k, v, do, lse, D, cu, True, docs.scale, rows=rows)
        n_keys = k.shape[0]
    if whole:
        rows = np.arange(n_q)
    else:
        n = int(min(n_q, max(64, CPU_SAMPLE_ELEMS // (G * n_keys))))
        rows = np.sort(rng.choice(n_q, n, replace=False))
    t0 = time.perf_counter()
    o, lse = fwd(rows)
    D = oracle.delta_rows(o, do[rows])
    dq, dk, dv = bwd(rows, lse, D)
    dt = time.perf_counter() - t0
    ref = dict(rows=rows, G=G, o=o, lse=lse, dq=dq, dk=dk if whole else None, dv=dv if whole else None)
    pairs = sum(int(mask(rows[i:i + 4096], np.arange(n_keys)).sum()) for i in range(0, rows.size, 4096)) * G
    rate = pairs * 14 * d / dt
    out = {"value": round(rate / 1e12, 6), "unit": "TFLOP/s", "cores": blas_threads(), "kind": "oracle"}
    if whole:
        out["sample"] = f"the whole workload ({n_q} rows x {hq} q-heads, every key), fwd+bwd in fp64; {dt:.1f} s"
        out["extrapolated"] = False
        out["step_s"] = round(dt, 2)
    else:
        out["sample"] = (f"{rows.size} seeded-random query rows x {G} q-heads (KV group 0), every key, fwd+bwd in "
                         f"fp64: {pairs} useful pairs in {dt:.1f} s; whole-step time extrapolated by useful pairs")
        out["extrapolated"] = True
        out["step_s"] = round(step_pairs * hq * 14 * d / rate, 1)
    return out, ref


def parity_report(ref, o, lse, dq, dk=None, dv=None):
    """Errors of the GPU step's outputs against the oracle's on the CPU baseline's
    sample (its rows, q-heads of KV group 0; every output when the workload ran whole):
    max-abs and relative L2 of O, dQ (and dK, dV), max-abs of LSE over finite rows."""
    import numpy as np
    import torch
    rows, G = ref["rows"], ref["G"]
    idx = torch.from_numpy(rows)
    f64 = lambda t: t.detach().to("cpu", torch.float64).numpy()

    def err(got, want):
        diff = got - want
        n = float(np.linalg.norm(want))
        # every element within 2e-2 + 5e-3 |x| (the ratio must stay <= 1), and within
        # 2e-2 itself wherever |x| <= 4
        ratio = np.abs(diff) / (2e-2 + 5e-3 * np.abs(want))
        small = np.abs(want) <= 4.0
        return {"max_abs": float(f"{np.abs(diff).max():.3e}"),
                "max_abs_where_abs_ref_le_4": float(f"{np.abs(diff[small]).max():.3e}") if small.any() else 0.0,
                "element_bound_ratio": float(f"{ratio.max():.3e}"),
                "rel_l2": float(f"{(np.linalg.norm(diff) / n if n else np.linalg.norm(diff)):.3e}")}

    rep = {"rows": int(rows.size), "q_heads": int(G), "o": err(f64(o.index_select(0, idx.to(o.device))[:, :G]), ref["o"]),
           "dq": err(f64(dq.index_select(0, idx.to(dq.device))[:, :G]), ref["dq"])}
    gl = f64(lse[:G].index_select(1, idx.to(lse.device)))
    fin = np.isfinite(ref["lse"])
    rep["lse_max_abs"] = float(f"{np.abs(gl[fin] - ref['lse'][fin]).max():.3e}") if fin.any() else 0.0
    rep["lse_neginf_match"] = bool(np.array_equal(np.isneginf(gl), np.isneginf(ref["lse"])))
    if ref["dk"] is not None and dk is not None:
        hk = ref["dk"].shape[1]
        rep["dk"] = err(f64(dk[:, :hk]), ref["dk"])
        rep["dv"] = err(f64(dv[:, :hk]), ref["dv"])
    tol = lambda e: e["element_bound_ratio"] <= 1.0 and e["max_abs_where_abs_ref_le_4"] <= 2e-2 and e["rel_l2"] <= 5e-3
    rep["within_tolerance"] = bool(all(tol(rep[k]) for k in ("o", "dq", "dk", "dv") if k in rep)
                                   and rep["lse_max_abs"] <= 1e-5 and rep["lse_neginf_match"])
    return rep


def merge_microbench(p, n_parts: int = 16, reps: int = 5):
    """LSE merge of n_parts synthetic fp32 partials of the rank's shape: O ~ N(0, 1),
    LSE ~ U(0, 15), 10% of the (head, row) entries -inf; bf16 output."""
    import torch
    from masked_long_context_amd import bdattn
    gen = torch.Generator(device="cuda").manual_seed(7)
    o_parts = torch.randn((n_parts, p.n_q, p.h_q, p.head_dim), generator=gen, device="cuda", dtype=torch.float32)
    lse_parts = torch.rand((n_parts, p.h_q, p.n_q), generator=gen, device="cuda") * 15.0
    lse_parts[torch.rand((n_parts, p.h_q, p.n_q), generator=gen, device="cuda") < 0.1] = float("-inf")
    o = torch.empty((p.n_q, p.h_q, p.head_dim), device="cuda", dtype=torch.bfloat16)
    lse = torch.empty((p.h_q, p.n_q), device="cuda", dtype=torch.float32)
    bdattn.bdattn_lse_merge(o_parts, lse_parts, o, lse)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        bdattn.bdattn_lse_merge(o_parts, lse_parts, o, lse)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / reps
    nbytes = p.n_q * p.h_q * (n_parts * (4 * p.head_dim + 4) + (2 * p.head_dim + 4))
    del o_parts, lse_parts
    torch.cuda.empty_cache()
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"parts": n_parts, "ms": round(ms, 4), "bytes": nbytes, "gbs": round(gbs, 1),
            "frac_hbm": round(gbs / PEAK_HBM_GBS, 4)}


def gemm_ceiling(n: int = 8192, seconds: float = 1.0):
    """Sustained bf16 MFMA rate this GPU delivers on a plain dense contraction: the
    vendor GEMM (torch.matmul, which dispatches to hipBLASLt) on N(0, 1) operands,
    repeated for about `seconds` after a warm-up.  Under a long load the chip holds
    its clock to its power budget, and operand values set the MFMA power, so this
    rate (not the published peak) is what any bf16 MFMA kernel can sustain here."""
    import torch
    gen = torch.Generator(device="cuda").manual_seed(11)
    a = torch.randn((n, n), generator=gen, device="cuda", dtype=torch.bfloat16)
    b = torch.randn((n, n), generator=gen, device="cuda", dtype=torch.bfloat16)
    for _ in range(3):
        torch.matmul(a, b)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps, t0 = 0, time.perf_counter()
    e0.record()
    while time.perf_counter() - t0 < seconds:
        for _ in range(8):
            torch.matmul(a, b)
        reps += 8
        torch.cuda.synchronize()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1)
    del a, b
    torch.cuda.empty_cache()
    return {"kind": f"vendor bf16 GEMM (torch.matmul -> hipBLASLt), {n}^3, N(0,1) operands, {reps} reps",
            "ms": round(ms, 1), "tflops": round(2.0 * n ** 3 * reps / (ms * 1e-3) / 1e12, 1)}


def atomics_rate(n_q: int, h_q: int, d: int, src_rows: int = 1 << 22, reps: int = 5):
    """fp32 atomic-add rate of this GPU on the pattern a fused key-major backward
    would use for dQ: blocks of 64 (row, head) rows of d fp32 values, each added
    into a random 64-row block of an [n_q * h_q, d] accumulator (torch's
    index_add_, which adds with one fp32 atomic per element).  Returns the rate
    and what one atomic per useful pair and q-head (d / 128 per pair at 128 keys
    per workgroup) would cost."""
    import torch
    gen = torch.Generator(device="cuda").manual_seed(13)
    n_dst = n_q * h_q
    dst = torch.zeros((n_dst, d), device="cuda", dtype=torch.float32)
    src = torch.randn((src_rows, d), generator=gen, device="cuda", dtype=torch.float32)
    blocks = torch.randint(0, n_dst // 64, (src_rows // 64,), generator=gen, device="cuda")
    index = (blocks[:, None] * 64 + torch.arange(64, device="cuda")[None, :]).reshape(-1)
    dst.index_add_(0, index, src)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        dst.index_add_(0, index, src)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / reps
    n_atomics = src_rows * d
    del dst, src, index, blocks
    torch.cuda.empty_cache()
    return {"kind": "fp32 atomic add (torch index_add_), 64-row blocks into random 64-row blocks of a "
                    f"[{n_dst}, {d}] accumulator", "atomics": n_atomics, "ms": round(ms, 4),
            "g_atomics_per_s": round(n_atomics / (ms * 1e-3) / 1e9, 1)}


def bench_varlen(args, cfg):
    """The varlen workload (packed token-causal shards) or its core-attention task
    form (the same documents cut into tasks that carry their prefix context,
    gathered into one packed K/V before the timed region): one forward and one
    backward call per step (4d + 10d flops per useful pair and q-head)."""
    import numpy as np
    import torch
    from masked_long_context_amd import bdattn as B
    from masked_long_context_amd import workloads as wl
    from masked_long_context_amd.rank_step import TaskStep, VarlenStep
    tasks = isinstance(cfg, wl.CadTaskConfig)
    docs = cfg.docs if tasks else cfg
    print(f"# bench: generating inputs for {cfg.name}", file=sys.stderr, flush=True)
    inp = wl.varlen_inputs(docs, seed=0)
    g = {k: v.cuda() for k, v in inp.items()}
    extra = {}
    task_rows = None
    t_plan = time.perf_counter()
    if tasks:
        q_cu, k_cu, src = B.cad_split(docs.cu_seqlens, cfg.max_pairs)
        B.Plan.tasks(q_cu, k_cu, True, cfg.h_q, cfg.h_kv, cfg.head_dim)
    else:
        B.Plan.varlen(cfg.cu_seqlens, True, cfg.h_q, cfg.h_kv, cfg.head_dim)
    plan_ms = (time.perf_counter() - t_plan) * 1e3
    if tasks:
        task_rows = wl.task_context_rows(k_cu, src)
        idx = torch.from_numpy(task_rows).cuda()
        g["k"], g["v"] = g["k"].index_select(0, idx), g["v"].index_select(0, idx)
        del idx
        step = TaskStep(q_cu, k_cu, True, cfg.h_q, cfg.h_kv, cfg.head_dim)
        ql, kl = np.diff(q_cu), np.diff(k_cu)
        extra = {"tasks": int(src.size), "max_pairs_per_task": cfg.max_pairs, "context_rows": int(k_cu[-1]),
                 "task_q_len_min_med_max": [int(ql.min()), int(np.median(ql)), int(ql.max())],
                 "task_k_len_max": int(kl.max())}
    else:
        step = VarlenStep(cfg.cu_seqlens, True, cfg.h_q, cfg.h_kv, cfg.head_dim)
    timer = EventTimer()
    step.timer = timer
    pairs = step.useful_pairs
    flops = pairs * cfg.h_q * 14 * cfg.head_dim
    a = (g["q"], g["k"], g["v"], g["dout"])
    for _ in range(args.warmup):
        step.step(*a)
    torch.cuda.synchronize()
    timer.enabled = True
    ms, ms_median = timed_steps(lambda: step.step(*a), args.steps)
    tot = timer.totals_ms()
    tflops = flops / (ms * 1e-3) / 1e12
    graph = None
    if args.graph:
        from masked_long_context_amd.rank_step import StepGraph
        sg = StepGraph(step, *a)
        for _ in range(args.warmup):
            sg.replay()
        torch.cuda.synchronize()
        graph = {"eager_value": round(tflops, 2), "eager_ms_per_step": round(ms, 4)}
        ms, ms_median = timed_steps(sg.replay, args.steps)
        tflops = flops / (ms * 1e-3) / 1e12
        del sg
    fwd_ms = tot["fwd"][0] / args.steps
    dkdv_ms = tot["dkdv"][0] / args.steps
    dq_ms = tot["dq"][0] / args.steps
    d = cfg.head_dim
    dk_flops = pairs * cfg.h_q * 8 * d
    dk_achieved = dk_flops / (dkdv_ms * 1e-3) / 1e12
    n_keys = step.n_keys
    dk_alg_bytes = int(2 * step.T * cfg.h_q * d * 2 + 4 * n_keys * cfg.h_kv * d * 2 + 2 * cfg.h_q * step.T * 4)
    out = {
        "metric": ("core-attention task batch (prefix contexts) fwd+bwd useful-pair TFLOP/s" if tasks else
                   "varlen packed causal attention fwd+bwd useful-pair TFLOP/s"), "value": round(tflops, 2),
        "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 3),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": cfg.name, "shards": len(docs.seqlens), "tokens": docs.total, "h_q": cfg.h_q,
                   "h_kv": cfg.h_kv, "head_dim": cfg.head_dim, "useful_pairs_per_head": pairs,
                   "flops_per_step": flops, **extra},
        "pct_of_bf16_peak": round(100 * tflops / PEAK_BF16_TFLOPS, 2),
        "plan_ms": round(plan_ms, 2),
        "roofline": {"kernel": f"dkdv_kernel<{d}, false>", "bound": "mfma", "achieved": round(dk_achieved, 2),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(dk_achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": profiled_traffic(cfg.name), "algorithmic_bytes": dk_alg_bytes,
                     "ms_per_launch": round(dkdv_ms, 4), "flops_per_launch": dk_flops},
        "executed_tflops": round(pairs * cfg.h_q * 18 * d / (ms * 1e-3) / 1e12, 2),
        "kernels": {"fwd": {"ms": round(fwd_ms, 4), "tflops": round(pairs * cfg.h_q * 4 * d / (fwd_ms * 1e-3) / 1e12, 2)},
                    "dkdv": {"ms": round(dkdv_ms, 4), "tflops": round(dk_achieved, 2)},
                    "dq": {"ms": round(dq_ms, 4), "tflops": round(pairs * cfg.h_q * 6 * d / (dq_ms * 1e-3) / 1e12, 2)},
                    **aux_bandwidth(tot, args.steps, step.T, cfg.h_q, d)},
        # the same work counted without the backward's recompute of S (12d per pair)
        "value_12d": round(pairs * cfg.h_q * 12 * d / (ms * 1e-3) / 1e12, 2),
        "ms_per_step_median": round(ms_median, 3),
    }
    if graph is not None:
        out["metric"] += " (step replayed from a HIP graph)"
        out["config"]["hip_graph"] = True
        out["graph"] = graph
    if not args.no_cpu_baseline:
        print("# bench: cpu baseline (oracle)", file=sys.stderr, flush=True)
        out["cpu_baseline"], ref = cpu_baseline(cfg, inp, pairs, tasks=(q_cu, k_cu, task_rows) if tasks else None)
        out["parity"] = parity_report(ref, step.o, step.lse, step.dq)
    print(json.dumps(out), flush=True)


def exchange_report(p, scheme: str, ranks: int):
    """K/V bytes this rank receives per step (its gradients go back in the backward) and the
    balance of attention work over all ranks, for this rank's scheme and the other one."""
    from masked_long_context_amd import exchange
    rank = p.q_clean_offset // (p.clean_len // ranks)
    c = exchange.compare_schemes(p.clean_len, p.block_size, ranks, p.h_kv, p.head_dim)
    mine = c["ranks"][scheme][rank]
    return {"scheme": scheme, "rank": rank, "ranks": ranks,
            "kv_bytes_received": mine.kv_bytes_received, "kv_bytes_needed": mine.kv_bytes_needed,
            "remote_clean_shards_needed": mine.remote_clean_needed,
            "per_scheme": c["summary"]}


def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        n = [i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"]
        return max(n) if n else 1
    except Exception:
        return len(os.sched_getaffinity(0))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", type=int, default=3, choices=[1, 2, 3, 4, 5, 6, 7],
                    help="workload: 3 = the 256K rank share (default); 4 = varlen packed causal shards; "
                         "6 = workload 4's documents as core-attention tasks with prefix contexts; "
                         "7 = conventional context parallelism's share of the same 256K sequence")
    ap.add_argument("--fused", action="store_true",
                    help="workloads 1-3, 5, 7: every clean shard resident, each in a buffer of its own, and "
                         "one launch per kernel over all of them (no partials, no merge)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--streams", type=int, default=1,
                    help="spread the independent per-shard calls over this many streams (workloads 1-3, 5, 7)")
    ap.add_argument("--graph", action="store_true",
                    help="also capture one step as a HIP graph and time its replays (launch-bound small "
                         "workloads); value is then the replay rate, the eager figures stay beside it")
    ap.add_argument("--no-ceiling", action="store_true",
                    help="skip the sustained-MFMA ceiling measurement (vendor bf16 GEMM, about 1 s)")
    ap.add_argument("--atomics", action="store_true",
                    help="also measure the fp32 atomic-add rate on a dQ-shaped accumulator (what a fused backward "
                         "with atomic dQ would pay instead of the dQ kernel's recompute)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="after the timed steps, run one plain 1 GiB device copy (HBM counter scale)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: --gpus {args.gpus} refused: this BDLM attention path runs on one GPU "
              "(one CSBP rank's share); multi-GPU runs are not supported.", file=sys.stderr)
        sys.exit(2)

    import torch
    from masked_long_context_amd import workloads as wl
    from masked_long_context_amd.rank_step import BdlmRankStep, ResidentShardsStep

    cfg = wl.config(args.config)
    if args.config in (4, 6):
        bench_varlen(args, cfg)
        return
    p = cfg.problem
    print(f"# bench: generating inputs for {cfg.name}", file=sys.stderr, flush=True)
    inp = wl.bdlm_inputs(cfg, seed=0)
    g = {k: v.cuda() for k, v in inp.items()}
    # --fused: every clean K/V shard resident at once, each in a buffer of its own
    # (as received), and one launch per kernel over all of them: the forward
    # writes O and LSE directly (no fp32 partials, no merge)
    shards = list(cfg.shards)
    workload = cfg.name + ("_resident_shards_one_launch" if args.fused else "")
    # plan building (host only, once per problem; outside the timed step)
    from masked_long_context_amd import bdattn as B
    t_plan = time.perf_counter()
    if args.fused:
        B.Plan.from_problem(p.with_kv(0, p.clean_len, True))
    else:
        for (o_, n_, loc) in shards:
            B.Plan.from_problem(p.with_kv(o_, n_, loc))
    plan_ms = (time.perf_counter() - t_plan) * 1e3
    if args.fused:
        step = ResidentShardsStep(p, shards)
        k_sh = [g["k_clean"][o_:o_ + n_].clone() for (o_, n_, _) in shards]
        v_sh = [g["v_clean"][o_:o_ + n_].clone() for (o_, n_, _) in shards]
        args_ = (g["q"], k_sh, v_sh, g["k_corr"], g["v_corr"], g["dout"])
        n_launch, n_act = 1, 0
    else:
        step = BdlmRankStep(p, shards, streams=args.streams)
        args_ = (g["q"], g["k_clean"], g["v_clean"], g["k_corr"], g["v_corr"], g["dout"])
        n_launch, n_act = len(shards), len(step.active)
    timer = EventTimer()
    step.timer = timer
    pairs = step.useful_pairs
    flops = pairs * p.h_q * 14 * p.head_dim
    print(f"# bench: warmup {args.warmup}", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step.step(*args_)
    torch.cuda.synchronize()
    timer.enabled = True
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ms, ms_median = timed_steps(lambda: step.step(*args_), args.steps)
    wall = time.perf_counter() - t0
    tot = timer.totals_ms()
    tflops = flops / (ms * 1e-3) / 1e12

    # per-kernel rates from the events around each library call (one kernel per call)
    n_sh = len(shards)
    per = {}
    for tag, dflops in (("fwd", 4), ("dkdv", 8), ("dq", 6)):
        tms, tn = tot.get(tag, (0.0, 1))
        per[tag] = dict(ms_per_step=tms / args.steps, launches_per_step=tn // args.steps,
                        ms_per_launch=tms / tn,
                        tflops=pairs * p.h_q * dflops * p.head_dim * args.steps / (tms * 1e-3) / 1e12 if tms else 0.0)
    # dominant kernel: the key-major dK/dV kernel (8d flops per useful pair and q-head)
    dk = per["dkdv"]
    dk_flops_per_launch = pairs * p.h_q * 8 * p.head_dim / n_launch
    dk_achieved = dk_flops_per_launch / (dk["ms_per_launch"] * 1e-3) / 1e12
    # algorithmic HBM bytes of one dK/dV launch, averaged over the launches: Q and dO
    # of every query row, the range's K and V read and dK and dV written, LSE and delta
    kv_rows = sum(n + (p.n_corr if loc else 0) for (_, n, loc) in shards) / n_launch
    dk_alg_bytes = int(2 * p.n_q * p.h_q * p.head_dim * 2 + 4 * kv_rows * p.h_kv * p.head_dim * 2
                       + 2 * p.h_q * p.n_q * 4)
    merge_ms, merge_n = tot.get("merge", (0.0, 1))
    merge_bytes = p.n_q * p.h_q * (n_act * (4 * p.head_dim + 4) + (2 * p.head_dim + 4))
    merge_gbs = merge_bytes / (merge_ms / merge_n * 1e-3) / 1e9 if merge_ms else 0.0
    merge_micro = merge_microbench(p)
    if args.copy_calibration:
        # a plain copy of known size, for scaling HBM counters read by rocprofv3
        src = torch.empty(1 << 28, dtype=torch.float32, device="cuda").fill_(1.0)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        print(f"# bench: copy calibration moved {src.numel() * 4} bytes each way", file=sys.stderr, flush=True)

    graph = None
    if args.graph:
        from masked_long_context_amd.rank_step import StepGraph
        sg = StepGraph(step, *args_)
        for _ in range(args.warmup):
            sg.replay()
        torch.cuda.synchronize()
        graph = {"eager_value": round(tflops, 2), "eager_ms_per_step": round(ms, 4)}
        ms, ms_median = timed_steps(sg.replay, args.steps)
        tflops = flops / (ms * 1e-3) / 1e12
        del sg

    ceiling = None
    if not args.no_ceiling:
        try:
            ceiling = gemm_ceiling()
        except RuntimeError as e:   # a missing or failing vendor GEMM leaves the rest of the line intact
            print(f"# bench: sustained-ceiling GEMM failed: {e}", file=sys.stderr, flush=True)

    metric = METRIC if args.config == 3 else f"BDLM attention fwd+bwd useful-pair TFLOP/s and % bf16 MFMA peak, {cfg.name}"
    if args.fused:
        metric += " (all clean shards resident, one launch per kernel)"
    if args.graph:
        metric += " (step replayed from a HIP graph)"
    out = {
        "metric": metric, "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 3), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": workload, "clean_len": p.clean_len, "block_size": p.block_size,
                   "q_rows": p.n_q, "h_q": p.h_q, "h_kv": p.h_kv, "head_dim": p.head_dim,
                   "clean_shards": n_sh, "useful_pairs_per_head": pairs,
                   "flops_per_step": flops},
        "pct_of_bf16_peak": round(100 * tflops / PEAK_BF16_TFLOPS, 2),
        "plan_ms": round(plan_ms, 2),
        "roofline": {"kernel": f"dkdv_kernel<{p.head_dim}, {'true' if args.fused and n_sh > 1 else 'false'}>",
                     "bound": "mfma", "achieved": round(dk_achieved, 2),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(dk_achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": profiled_traffic(workload), "algorithmic_bytes": dk_alg_bytes,
                     "ms_per_launch": round(dk["ms_per_launch"], 4),
                     "flops_per_launch": dk_flops_per_launch},
        # MFMA work the kernels execute per useful pair and q-head: 4d forward, 8d dK/dV,
        # 6d dQ (S and dP recomputed); 14d of it is counted in `value`
        "executed_tflops": round(pairs * p.h_q * 18 * p.head_dim / (ms * 1e-3) / 1e12, 2),
        "kernels": {
            **{k: {kk: round(vv, 4) for kk, vv in v.items()} for k, v in per.items()},
            "merge": {"ms": round(merge_ms / max(merge_n, 1), 4), "parts": n_act, "gbs": round(merge_gbs, 1),
                      "frac_hbm": round(merge_gbs / PEAK_HBM_GBS, 4)},
            "merge_micro": merge_micro,
            **aux_bandwidth(tot, args.steps, p.n_q, p.h_q, p.head_dim),
        },
        # the same work counted without the backward's recompute of S (12d per pair)
        "value_12d": round(pairs * p.h_q * 12 * p.head_dim / (ms * 1e-3) / 1e12, 2),
        "ms_per_step_median": round(ms_median, 3),
        "wall_s": round(wall, 3),
    }
    if args.streams > 1:
        out["config"]["streams"] = args.streams
    if graph is not None:
        out["config"]["hip_graph"] = True
        out["graph"] = graph
    if ceiling is not None:
        ceiling["dominant_kernel_frac"] = round(dk_achieved / ceiling["tflops"], 4)
        ceiling["kernel_fracs"] = {k: round(v["tflops"] / ceiling["tflops"], 4) for k, v in per.items()}
        ceiling["step_executed_frac"] = round(out["executed_tflops"] / ceiling["tflops"], 4)
        out["roofline"]["sustained_ceiling"] = ceiling
    if args.atomics:
        at = atomics_rate(p.n_q, p.h_q, p.head_dim)
        # a fused key-major backward adds dQ with d / 128 atomics per useful pair and
        # q-head (one 64 x d block per 64 x 128 tile of pairs)
        need = pairs * p.h_q * p.head_dim / 128
        at["fused_dq_atomics_per_step"] = int(need)
        at["fused_dq_atomics_ms_per_step"] = round(need / (at["g_atomics_per_s"] * 1e9) * 1e3, 1)
        at["dq_kernel_ms_per_step"] = round(per["dq"]["ms_per_step"], 2)
        out["atomics"] = at
    if args.config in (3, 7):
        out["exchange"] = exchange_report(p, "cp" if args.config == 7 else "csbp", len(cfg.shards))
    if not args.no_cpu_baseline:
        print("# bench: cpu baseline (oracle)", file=sys.stderr, flush=True)
        out["cpu_baseline"], ref = cpu_baseline(cfg, inp, pairs)
        dk_c = torch.cat(step.dk_shards) if args.fused else step.dk_clean
        dv_c = torch.cat(step.dv_shards) if args.fused else step.dv_clean
        corr = [step.dk_corr] if step.dk_corr is not None else []
        corv = [step.dv_corr] if step.dv_corr is not None else []
        out["parity"] = parity_report(ref, step.o, step.lse, step.dq, torch.cat([dk_c] + corr),
                                      torch.cat([dv_c] + corv))
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
