"""One rank's attention step under context-sharded block parallelism (CSBP).

The rank holds its clean query rows, the corrupted blocks it owns and their
local corrupted K/V, and sees the clean K/V as position shards ("Block
Parallelism For Efficient Distributed Long-Context Diffusion Language Model
Training", English abstract).  The step runs, on the caller's HIP stream (or,
optionally, with its independent per-shard calls spread over several streams):

    for each clean K/V shard s:  bdattn_fwd  -> partial (O_s, LSE_s)
    bdattn_lse_merge             -> O (fp32), LSE
    bdattn_cast_f32_bf16         -> O (bf16, the layer output)
    bdattn_bwd_prepare           -> delta = rowsum(dO o O) from the fp32 O, cleared dQ accumulator
    for each clean K/V shard s:  bdattn_bwd_dkdv -> dK_s, dV_s; bdattn_bwd_dq -> dQ (accumulated)
    bdattn_dq_finalize           -> dQ (bf16)

The merged output is kept in fp32 until the backward: delta is a row sum of
dO o O, and dS = P o (dP - delta) is a small difference wherever one key
dominates a row, so rounding O to bf16 before that sum would cost dK accuracy
on peaked softmax rows (exact_delta=False takes delta from the bf16 O instead
and keeps no fp32 copy).  The local corrupted K/V join the call of one chosen shard.  Shards whose plan
has no legal pair are left out of the forward and the merge (their partial
would carry LSE = -inf everywhere); their backward still runs and writes zero
gradients.  When a single shard has legal pairs -- in particular when the whole
clean K/V is resident and passed as one range -- its forward writes the bf16
output and the LSE directly: no fp32 partial and no merge.  A whole step can
also be captured once as a HIP graph and replayed (StepGraph), which removes
the per-call launch cost of small, launch-bound problems.  ResidentShardsStep
runs the same step with every shard resident in its own buffer as one launch
per kernel over all of them (online merge in registers, no partials).  This module only
sequences calls and owns buffers; every arithmetic step runs in libbdattn.so.
"""
from __future__ import annotations

from typing import List, Optional, Sequence, Tuple

import torch

from . import bdattn as B


def keep_workspaces(plans, device):
    """One workspace per plan, holding that plan's tables (bdattn_plan_keep_tables):
    uploaded once here, on the current stream, which is then synchronized so that
    the step may run on any stream."""
    wss = [B.workspace(pl.workspace_bytes, device) for pl in plans]
    for pl, ws in zip(plans, wss):
        pl.keep_tables(ws)
    torch.cuda.current_stream(device).synchronize()
    return wss


class BdlmRankStep:
    def __init__(self, problem, shards: Sequence[Tuple[int, int, bool]], device="cuda",
                 part_dtype=torch.float32, dkdv_split: int = 0, streams: int = 1, exact_delta: bool = True,
                 keep_tables: bool = True):
        self.problem = problem
        self.shards = list(shards)
        self.device = device
        self.plans: List[B.Plan] = [B.Plan.from_problem(problem.with_kv(o, n, loc)) for (o, n, loc) in shards]
        if dkdv_split:   # 0 keeps each plan's automatic choice
            for pl in self.plans:
                pl.set_dkdv_split(dkdv_split)
        self.active = [i for i, pl in enumerate(self.plans) if pl.useful_pairs > 0]
        p = problem
        self.n_q, self.h_q, self.h_kv, self.d = p.n_q, p.h_q, p.h_kv, p.head_dim
        # streams > 1: the per-shard forward and dK/dV calls, which are independent,
        # alternate over the caller's stream and streams - 1 side streams (default
        # priority), each with its own workspace; the dQ calls, which add into one
        # accumulator, stay on the caller's stream in shard order
        self.side = [torch.cuda.Stream(device=device) for _ in range(max(1, int(streams)) - 1)]
        # keep_tables: every plan keeps its tables in a workspace of its own, uploaded
        # once here, so no call of a step waits for a table upload; otherwise one
        # workspace per stream, into which every call uploads its plan's tables
        self.ws_plan = keep_workspaces(self.plans, device) if keep_tables else None
        ws_bytes = max(pl.workspace_bytes for pl in self.plans)
        self.ws = None if keep_tables else B.workspace(ws_bytes, device)
        self.ws_side = [] if keep_tables else [B.workspace(ws_bytes, device) for _ in self.side]
        # one active shard: its forward writes O and LSE itself (no partials)
        self.direct = len(self.active) == 1
        n_parts = 0 if self.direct else max(1, len(self.active))
        self.o_parts = torch.empty((n_parts, self.n_q, self.h_q, self.d), dtype=part_dtype, device=device)
        self.lse_parts = torch.empty((n_parts, self.h_q, self.n_q), dtype=torch.float32, device=device)
        self.o = torch.empty((self.n_q, self.h_q, self.d), dtype=torch.bfloat16, device=device)
        # fp32 merged output kept for the backward's delta (None: delta from the bf16 O)
        self.o32 = torch.empty((self.n_q, self.h_q, self.d), dtype=torch.float32, device=device) \
            if exact_delta else None
        self.lse = torch.empty((self.h_q, self.n_q), dtype=torch.float32, device=device)
        self.delta = torch.empty((self.h_q, self.n_q), dtype=torch.float32, device=device)
        self.dq_acc = torch.empty((self.n_q, self.h_q, self.d), dtype=torch.float32, device=device)
        self.dq = torch.empty((self.n_q, self.h_q, self.d), dtype=torch.bfloat16, device=device)
        self.dk_clean = torch.empty((p.clean_len, self.h_kv, self.d), dtype=torch.bfloat16, device=device)
        self.dv_clean = torch.empty_like(self.dk_clean)
        self.dk_corr = torch.empty((p.n_corr, self.h_kv, self.d), dtype=torch.bfloat16, device=device)
        self.dv_corr = torch.empty_like(self.dk_corr)
        self.timer = None      # optional callable(tag) -> context manager around each library call
        self._main = None      # raw handle of the caller's stream during a forward or backward

    @property
    def useful_pairs(self) -> int:
        """Legal pairs per q-head over the whole step (all shards)."""
        return sum(pl.useful_pairs for pl in self.plans)

    def _t(self, tag):
        import contextlib
        return self.timer(tag) if self.timer is not None else contextlib.nullcontext()

    def _lane(self, j, i):
        """Stream context, workspace and stream handle of the j-th independent call,
        of plan i (lane 0: the caller's stream)."""
        import contextlib
        k = j % (len(self.side) + 1)
        ws = self.ws_plan[i] if self.ws_plan is not None else (self.ws if k == 0 else self.ws_side[k - 1])
        if k == 0:
            return contextlib.nullcontext(), ws, self._main
        return torch.cuda.stream(self.side[k - 1]), ws, self.side[k - 1].cuda_stream

    def _fork(self):
        main = torch.cuda.current_stream()
        for s in self.side:
            s.wait_stream(main)

    def _join(self):
        main = torch.cuda.current_stream()
        for s in self.side:
            main.wait_stream(s)

    def _to_bf16(self):
        if self.o32 is not None:
            with self._t("cast"):
                B.cast_unchecked(self.o32, self.o, self._main)

    def check_inputs(self, q, k_clean, v_clean, k_corr, v_corr, dout=None):
        """The caller's tensors against the problem (once per call of forward or
        backward; the library calls of the step then go unchecked)."""
        p = self.problem
        bf = (torch.bfloat16,)
        kv = (p.clean_len, self.h_kv, self.d)
        named = [(q, "q", (self.n_q, self.h_q, self.d), bf), (k_clean, "k_clean", kv, bf), (v_clean, "v_clean", kv, bf)]
        if p.n_corr:
            cr = (p.n_corr, self.h_kv, self.d)
            named += [(k_corr, "k_corr", cr, bf), (v_corr, "v_corr", cr, bf)]
        if dout is not None:
            named.append((dout, "dout", (self.n_q, self.h_q, self.d), bf))
        B.check_inputs(named, [("o", self.o.device)])

    def forward(self, q, k_clean, v_clean, k_corr, v_corr):
        self.check_inputs(q, k_clean, v_clean, k_corr, v_corr)
        return self._forward(q, k_clean, v_clean, k_corr, v_corr)

    def _forward(self, q, k_clean, v_clean, k_corr, v_corr):
        self._main = B.current_stream_handle()
        out = self.o32 if self.o32 is not None else self.o
        if not self.active:
            out.zero_()
            self.lse.fill_(float("-inf"))
            self._to_bf16()
            return self.o, self.lse
        if self.direct:
            i = self.active[0]
            off, n, local = self.shards[i]
            with self._t("fwd"):
                B.fwd_unchecked(self.plans[i], q, k_clean[off:off + n], v_clean[off:off + n],
                                k_corr if local else None, v_corr if local else None, out, self.lse,
                                self.ws_plan[i] if self.ws_plan is not None else self.ws, self._main)
            self._to_bf16()
            return self.o, self.lse
        self._fork()
        for slot, i in enumerate(self.active):
            off, n, local = self.shards[i]
            lane, ws, st = self._lane(slot, i)
            with lane, self._t("fwd"):
                B.fwd_unchecked(self.plans[i], q, k_clean[off:off + n], v_clean[off:off + n],
                                k_corr if local else None, v_corr if local else None,
                                self.o_parts[slot], self.lse_parts[slot], ws, st)
        self._join()
        with self._t("merge"):
            B.lse_merge_unchecked(self.o_parts[:len(self.active)], self.lse_parts[:len(self.active)], out, self.lse,
                                  self._main)
        self._to_bf16()
        return self.o, self.lse

    def backward(self, q, k_clean, v_clean, k_corr, v_corr, dout):
        self.check_inputs(q, k_clean, v_clean, k_corr, v_corr, dout)
        return self._backward(q, k_clean, v_clean, k_corr, v_corr, dout)

    def _backward(self, q, k_clean, v_clean, k_corr, v_corr, dout):
        self._main = B.current_stream_handle()
        with self._t("prepare"):
            B.bwd_prepare_unchecked(self.plans[0], self.o32 if self.o32 is not None else self.o, dout, self.delta,
                                    self.dq_acc, self._main)
        # the two steps of bdattn_bwd, called apart so that each can be timed
        self._fork()
        for i, (off, n, local) in enumerate(self.shards):
            kc, vc = k_clean[off:off + n], v_clean[off:off + n]
            kx, vx = (k_corr, v_corr) if local else (None, None)
            lane, ws, st = self._lane(i, i)
            with lane, self._t("dkdv"):
                B.bwd_dkdv_unchecked(self.plans[i], q, kc, vc, kx, vx, dout, self.lse, self.delta,
                                     self.dk_clean[off:off + n], self.dv_clean[off:off + n],
                                     self.dk_corr if local else None, self.dv_corr if local else None, ws, st)
            with self._t("dq"):
                B.bwd_dq_unchecked(self.plans[i], q, kc, vc, kx, vx, dout, self.lse, self.delta, self.dq_acc,
                                   self.ws_plan[i] if self.ws_plan is not None else self.ws, self._main)
        self._join()
        with self._t("finalize"):
            B.dq_finalize_unchecked(self.dq_acc, self.dq, self._main)
        return self.dq, self.dk_clean, self.dv_clean, self.dk_corr, self.dv_corr

    def step(self, q, k_clean, v_clean, k_corr, v_corr, dout):
        self.check_inputs(q, k_clean, v_clean, k_corr, v_corr, dout)
        self._forward(q, k_clean, v_clean, k_corr, v_corr)
        return self._backward(q, k_clean, v_clean, k_corr, v_corr, dout)


class ResidentShardsStep:
    """One rank step with every clean shard it attends resident, each in the buffer
    it arrived in (the fused multi-shard form).  One plan covers the span of the
    shards, and each kernel runs once over all of them, reading the clean K/V
    through a table of buffers.  The online softmax then merges the shards in
    registers: no fp32 partials, no merge call, one launch per kernel however many
    shards there are:

        bdattn_fwd_shards       -> O (fp32), LSE
        bdattn_cast_f32_bf16    -> O (bf16, the layer output)
        bdattn_bwd_prepare      -> delta from the fp32 O, cleared dQ accumulator
        bdattn_bwd_dkdv_shards  -> dK, dV into one buffer per shard (and the local corrupted ones)
        bdattn_bwd_dq_shards    -> dQ accumulated
        bdattn_dq_finalize      -> dQ (bf16)

    shards: (offset, length, local) of consecutive clean ranges, as for
    BdlmRankStep; every shard but the last holds the same number of positions, a
    multiple of 128 (the library's shard alignment)."""

    def __init__(self, problem, shards: Sequence[Tuple[int, int, bool]], device="cuda", exact_delta: bool = True,
                 keep_tables: bool = True, dkdv_split: int = 0):
        shards = list(shards)
        if not shards:
            raise ValueError("no shards")
        off0, pos = shards[0][0], shards[0][0]
        for (off, n, _) in shards:
            if off != pos:
                raise ValueError("the shards must be consecutive clean ranges")
            pos += n
        total = pos - off0
        self.shard_lens = [n for (_, n, _) in shards]
        if B.shard_split(total, len(shards), self.shard_lens[0] if len(shards) > 1 else 0) != self.shard_lens:
            raise ValueError(f"shard lengths {self.shard_lens}: every shard but the last must hold the same "
                             f"number of positions")
        self.problem, self.shards, self.device = problem, shards, device
        self.plan = B.Plan.from_problem(problem.with_kv(off0, total, any(loc for (_, _, loc) in shards)))
        if dkdv_split:   # 0 keeps the plan's automatic choice
            self.plan.set_dkdv_split(dkdv_split)
        p = problem
        self.n_q, self.h_q, self.h_kv, self.d = p.n_q, p.h_q, p.h_kv, p.head_dim
        self.has_corr = self.plan.n_kv(1) > 0
        self.ws = keep_workspaces([self.plan], device)[0] if keep_tables else \
            B.workspace(self.plan.workspace_bytes, device)
        q_shape = (self.n_q, self.h_q, self.d)
        self.o = torch.empty(q_shape, dtype=torch.bfloat16, device=device)
        self.o32 = torch.empty(q_shape, dtype=torch.float32, device=device) if exact_delta else None
        self.lse = torch.empty((self.h_q, self.n_q), dtype=torch.float32, device=device)
        self.delta = torch.empty((self.h_q, self.n_q), dtype=torch.float32, device=device)
        self.dq_acc = torch.empty(q_shape, dtype=torch.float32, device=device)
        self.dq = torch.empty(q_shape, dtype=torch.bfloat16, device=device)
        kv = lambda n: torch.empty((n, self.h_kv, self.d), dtype=torch.bfloat16, device=device)
        self.dk_shards = [kv(n) for n in self.shard_lens]
        self.dv_shards = [kv(n) for n in self.shard_lens]
        self.dk_corr = kv(p.n_corr) if self.has_corr else None
        self.dv_corr = kv(p.n_corr) if self.has_corr else None
        self.timer = None      # optional callable(tag) -> context manager around each library call
        self._kv = None        # the bdattn_kv_shards struct of the current call's buffers

    @property
    def useful_pairs(self) -> int:
        return self.plan.useful_pairs

    def _t(self, tag):
        import contextlib
        return self.timer(tag) if self.timer is not None else contextlib.nullcontext()

    def check_inputs(self, q, k_shards, v_shards, k_corr, v_corr, dout=None):
        """The caller's tensors against the plan (once per call of forward or
        backward; the library calls of the step then go unchecked)."""
        bf = (torch.bfloat16,)
        if len(k_shards) != len(self.shard_lens) or len(v_shards) != len(self.shard_lens):
            raise B.BdattnError(B.EINVAL, f"expected {len(self.shard_lens)} K and V shard buffers")
        named = [(q, "q", (self.n_q, self.h_q, self.d), bf)]
        for i, n in enumerate(self.shard_lens):
            named += [(k_shards[i], f"k_shards[{i}]", (n, self.h_kv, self.d), bf),
                      (v_shards[i], f"v_shards[{i}]", (n, self.h_kv, self.d), bf)]
        if self.has_corr:
            cr = (self.problem.n_corr, self.h_kv, self.d)
            named += [(k_corr, "k_corr", cr, bf), (v_corr, "v_corr", cr, bf)]
        if dout is not None:
            named.append((dout, "dout", (self.n_q, self.h_q, self.d), bf))
        B.check_inputs(named, [("o", self.o.device)])
        self._kv = B.make_shards(k_shards, v_shards, self.dk_shards, self.dv_shards)

    def forward(self, q, k_shards, v_shards, k_corr, v_corr):
        self.check_inputs(q, k_shards, v_shards, k_corr, v_corr)
        return self._forward(q, k_corr, v_corr)

    def _forward(self, q, k_corr, v_corr):
        st = B.current_stream_handle()
        kx, vx = (k_corr, v_corr) if self.has_corr else (None, None)
        out = self.o32 if self.o32 is not None else self.o
        with self._t("fwd"):
            B.fwd_shards_unchecked(self.plan, q, self._kv, kx, vx, out, self.lse, self.ws, st)
        if self.o32 is not None:
            with self._t("cast"):
                B.cast_unchecked(self.o32, self.o, st)
        return self.o, self.lse

    def backward(self, q, k_shards, v_shards, k_corr, v_corr, dout):
        self.check_inputs(q, k_shards, v_shards, k_corr, v_corr, dout)
        return self._backward(q, k_corr, v_corr, dout)

    def _backward(self, q, k_corr, v_corr, dout):
        st = B.current_stream_handle()
        kx, vx = (k_corr, v_corr) if self.has_corr else (None, None)
        with self._t("prepare"):
            B.bwd_prepare_unchecked(self.plan, self.o32 if self.o32 is not None else self.o, dout, self.delta,
                                    self.dq_acc, st)
        with self._t("dkdv"):
            B.bwd_dkdv_shards_unchecked(self.plan, q, self._kv, kx, vx, dout, self.lse, self.delta, self.dk_corr,
                                        self.dv_corr, self.ws, st)
        with self._t("dq"):
            B.bwd_dq_shards_unchecked(self.plan, q, self._kv, kx, vx, dout, self.lse, self.delta, self.dq_acc,
                                      self.ws, st)
        with self._t("finalize"):
            B.dq_finalize_unchecked(self.dq_acc, self.dq, st)
        return self.dq, self.dk_shards, self.dv_shards, self.dk_corr, self.dv_corr

    def step(self, q, k_shards, v_shards, k_corr, v_corr, dout):
        self.check_inputs(q, k_shards, v_shards, k_corr, v_corr, dout)
        self._forward(q, k_corr, v_corr)
        return self._backward(q, k_corr, v_corr, dout)


class StepGraph:
    """A step (BdlmRankStep, VarlenStep or TaskStep) captured once as a HIP graph
    (torch.cuda.CUDAGraph over torch's current stream, which the library launches
    on) and replayed.  The graph holds every table upload and kernel launch of one
    step, so a replay costs one graph launch where the eager step issues one call
    per kernel; this matters when the step is launch-bound (small problems).  The
    input and output tensors are fixed at capture: refill the inputs in place.
    The step runs once eagerly first, so that the plans' pinned table copies exist
    before capture (no host allocation happens during it)."""

    def __init__(self, step, *inputs):
        import torch
        self.step, self.inputs = step, inputs
        timer, step.timer = step.timer, None
        step.step(*inputs)
        torch.cuda.synchronize()
        self.graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.graph):
            self.outputs = step.step(*inputs)
        torch.cuda.synchronize()
        step.timer = timer

    def replay(self):
        self.graph.replay()
        return self.outputs


class VarlenStep:
    """Forward + backward of packed independent shards (one call each)."""

    def __init__(self, cu_seqlens, causal, h_q, h_kv, head_dim, device="cuda", softmax_scale=0.0, plan=None,
                 exact_delta: bool = True, keep_tables: bool = True):
        self.plan = plan if plan is not None else B.Plan.varlen(cu_seqlens, causal, h_q, h_kv, head_dim,
                                                                softmax_scale)
        T, n_keys = self.plan.n_q, self.plan.n_kv(0)
        self.T, self.n_keys, self.h_q, self.h_kv, self.d = T, n_keys, h_q, h_kv, head_dim
        self.ws = keep_workspaces([self.plan], device)[0] if keep_tables else \
            B.workspace(self.plan.workspace_bytes, device)
        self.o = torch.empty((T, h_q, head_dim), dtype=torch.bfloat16, device=device)
        # fp32 output kept for the backward's delta (see BdlmRankStep)
        self.o32 = torch.empty((T, h_q, head_dim), dtype=torch.float32, device=device) if exact_delta else None
        self.lse = torch.empty((h_q, T), dtype=torch.float32, device=device)
        self.delta = torch.empty((h_q, T), dtype=torch.float32, device=device)
        self.dq_acc = torch.empty((T, h_q, head_dim), dtype=torch.float32, device=device)
        self.dq = torch.empty((T, h_q, head_dim), dtype=torch.bfloat16, device=device)
        self.dk = torch.empty((n_keys, h_kv, head_dim), dtype=torch.bfloat16, device=device)
        self.dv = torch.empty_like(self.dk)
        self.timer = None      # optional callable(tag) -> context manager around each library call

    @property
    def useful_pairs(self) -> int:
        return self.plan.useful_pairs

    def _t(self, tag):
        import contextlib
        return self.timer(tag) if self.timer is not None else contextlib.nullcontext()

    def check_inputs(self, q, k, v, dout=None):
        bf = (torch.bfloat16,)
        kv = (self.n_keys, self.h_kv, self.d)
        named = [(q, "q", (self.T, self.h_q, self.d), bf), (k, "k", kv, bf), (v, "v", kv, bf)]
        if dout is not None:
            named.append((dout, "dout", (self.T, self.h_q, self.d), bf))
        B.check_inputs(named, [("o", self.o.device)])

    def forward(self, q, k, v):
        self.check_inputs(q, k, v)
        return self._forward(q, k, v)

    def _forward(self, q, k, v):
        st = B.current_stream_handle()
        with self._t("fwd"):
            B.varlen_fwd_unchecked(self.plan, q, k, v, self.o32 if self.o32 is not None else self.o, self.lse,
                                   self.ws, st)
        if self.o32 is not None:
            with self._t("cast"):
                B.cast_unchecked(self.o32, self.o, st)
        return self.o, self.lse

    def backward(self, q, k, v, dout):
        self.check_inputs(q, k, v, dout)
        return self._backward(q, k, v, dout)

    def _backward(self, q, k, v, dout):
        st = B.current_stream_handle()
        with self._t("prepare"):
            B.bwd_prepare_unchecked(self.plan, self.o32 if self.o32 is not None else self.o, dout, self.delta,
                                    self.dq_acc, st)
        # the two kernels of bdattn_varlen_bwd, called apart so that each can be timed
        with self._t("dkdv"):
            B.bwd_dkdv_unchecked(self.plan, q, k, v, None, None, dout, self.lse, self.delta, self.dk, self.dv,
                                 None, None, self.ws, st)
        with self._t("dq"):
            B.bwd_dq_unchecked(self.plan, q, k, v, None, None, dout, self.lse, self.delta, self.dq_acc, self.ws, st)
        with self._t("finalize"):
            B.dq_finalize_unchecked(self.dq_acc, self.dq, st)
        return self.dq, self.dk, self.dv

    def step(self, q, k, v, dout):
        self.check_inputs(q, k, v, dout)
        self._forward(q, k, v)
        return self._backward(q, k, v, dout)


class TaskStep(VarlenStep):
    """Forward + backward of a fused batch of core-attention tasks, each with its own
    key context (packed task queries [q_cu[-1], h_q, d], packed contexts
    [k_cu[-1], h_kv, d]); dk/dv hold one gradient per context row."""

    def __init__(self, q_cu, k_cu, causal, h_q, h_kv, head_dim, device="cuda", softmax_scale=0.0,
                 exact_delta: bool = True, keep_tables: bool = True):
        plan = B.Plan.tasks(q_cu, k_cu, causal, h_q, h_kv, head_dim, softmax_scale)
        super().__init__(None, causal, h_q, h_kv, head_dim, device, softmax_scale, plan=plan,
                         exact_delta=exact_delta, keep_tables=keep_tables)
