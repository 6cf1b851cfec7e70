"""One focused block-diffusion step on the GPU: score -> select -> compact (hidden) -> attend.

`FocusStep` preallocates every output and workspace once for a fixed batch shape, then `run()`
issues the C-ABI calls back to back on the current stream with no host synchronisation: ragged
sizes stay on the device, and the attention is sized by the host-known bound max_kept.  With
per-request budgets the front end (score, select, compact) is one call of two launches; with the
adaptive rule it is two calls (score + select, then compaction).  The attention reads the kept
tokens' queries in place, at their kept positions (focus_ragged_paged_attn_pos), so the
compaction gathers only the hidden states; gather_q=True gathers the queries too and runs the
attention on the compacted copy (focus_ragged_paged_attn), with the same results.
`capture()` records one step into a HIP graph (no allocation, no memset node: the kernels reset
their own arrival counters), and `replay()` launches it, for callers that replay a fixed step.
With the host ahead of the device the eager launches leave no gap between the kernels; on
ROCm 7 a replay measured a few microseconds slower than the same kernels launched eagerly (the
kernel durations are the same).
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import torch

from . import binding as F


@dataclass
class StepInputs:
    """Device tensors of one step (layouts as in include/focus.h)."""
    q0: torch.Tensor
    k0: torch.Tensor
    q1: torch.Tensor
    k1: torch.Tensor
    masked: torch.Tensor          # [B, blk] u8
    budget: Optional[torch.Tensor]  # [B] i32, or None with `adaptive`
    adaptive: Optional[tuple]     # (beta, lo, hi) or None
    max_kept: int
    q_att: torch.Tensor           # [B, blk, Hq, d] bf16
    k_cache: torch.Tensor
    v_cache: torch.Tensor
    page_table: torch.Tensor
    prefix_len: torch.Tensor
    k_blk: torch.Tensor
    v_blk: torch.Tensor
    sm_scale: float
    hidden: Optional[torch.Tensor] = None  # [B, blk, W] bf16


class FocusStep:
    def __init__(self, inp: StepInputs, cap: Optional[int] = None, want_lse: bool = True,
                 gather_q: bool = False):
        B, blk, Hq, d = inp.q_att.shape
        Hkv = inp.k_blk.shape[1]
        dev = inp.q_att.device
        self.inp = inp
        self.B, self.blk, self.Hq, self.Hkv, self.d = B, blk, Hq, Hkv, d
        self.cap = B * blk if cap is None else cap
        self.delta = torch.empty((B, blk), dtype=torch.float32, device=dev)
        self.keep = torch.empty((B, blk), dtype=torch.uint8, device=dev)
        self.kept_count = torch.empty(B, dtype=torch.int32, device=dev)
        self.offsets = torch.empty(B + 1, dtype=torch.int32, device=dev)
        self.kept_pos = torch.empty(max(self.cap, 1), dtype=torch.int32, device=dev)
        self.gather_q = gather_q
        self.q_rows = torch.empty((max(self.cap, 1), Hq, d), dtype=torch.bfloat16, device=dev) \
            if gather_q else None
        self.hidden_rows = None
        if inp.hidden is not None:
            self.hidden_rows = torch.empty((max(self.cap, 1), inp.hidden.shape[2]),
                                           dtype=inp.hidden.dtype, device=dev)
        self.out = torch.empty((max(self.cap, 1), Hq, d), dtype=torch.bfloat16, device=dev)
        self.lse = torch.empty((max(self.cap, 1), Hq), dtype=torch.float32, device=dev) \
            if want_lse else None
        nsc = F.lib().focus_score_l01_workspace_size(B, blk, Hq, Hkv, d)
        self.ws_score = torch.zeros(max(nsc, 1), dtype=torch.uint8, device=dev)
        S = inp.k_cache.shape[3]
        nat = F.attn_workspace_bytes(B, blk, Hq, Hkv, d, S, inp.page_table.shape[1], inp.max_kept)
        self.ws_attn = torch.zeros(max(nat, 1), dtype=torch.uint8, device=dev)  # zeros once

    def score(self):
        i = self.inp
        F.score_l01(i.q0, i.k0, i.q1, i.k1, i.sm_scale, delta=self.delta, workspace=self.ws_score)

    def select(self):
        i = self.inp
        F.select_budget(self.delta, i.masked, i.budget, i.adaptive, keep=self.keep,
                        kept_count=self.kept_count)

    def compact_hidden(self):
        """Offsets, kept positions and (if the step has them) the gathered hidden states."""
        F.compact(self.keep, self.inp.hidden, self.cap, offsets=self.offsets,
                  kept_pos=self.kept_pos, gathered=self.hidden_rows)

    def compact_q(self):
        F.compact(self.keep, self.inp.q_att, self.cap, offsets=self.offsets,
                  kept_pos=self.kept_pos, gathered=self.q_rows)

    def attend(self):
        i = self.inp
        if self.gather_q:
            F.ragged_paged_attn(self.q_rows, self.offsets, i.k_cache, i.v_cache, i.page_table,
                                i.prefix_len, i.k_blk, i.v_blk, i.max_kept, i.sm_scale,
                                out=self.out, lse=self.lse, want_lse=self.lse is not None,
                                workspace=self.ws_attn)
        else:
            F.ragged_paged_attn_pos(i.q_att, self.kept_pos, self.offsets, i.k_cache, i.v_cache,
                                    i.page_table, i.prefix_len, i.k_blk, i.v_blk, i.max_kept,
                                    i.sm_scale, out=self.out, lse=self.lse,
                                    want_lse=self.lse is not None, workspace=self.ws_attn)

    def score_select(self):
        i = self.inp
        F.score_select(i.q0, i.k0, i.q1, i.k1, i.sm_scale, i.masked, i.budget, i.adaptive,
                       delta=self.delta, keep=self.keep, kept_count=self.kept_count,
                       workspace=self.ws_score)

    def compact(self):
        sets, outs = self._row_sets()
        F.compact_multi(self.keep, sets, self.cap, offsets=self.offsets, kept_pos=self.kept_pos,
                        gathered=outs)

    def _row_sets(self):
        sets, outs = [], []
        if self.inp.hidden is not None:
            sets.append(self.inp.hidden)
            outs.append(self.hidden_rows)
        if self.gather_q:
            sets.append(self.inp.q_att)
            outs.append(self.q_rows)
        return sets, outs

    def score_select_compact(self):
        """Score partials, then reduction + selection + compaction (hidden states, and the
        queries with gather_q) in one launch (per-request budgets only)."""
        i = self.inp
        sets, outs = self._row_sets()
        F.score_select_compact(i.q0, i.k0, i.q1, i.k1, i.sm_scale, i.masked, i.budget, sets,
                               self.cap, max_kept=i.max_kept, delta=self.delta, keep=self.keep,
                               kept_count=self.kept_count, offsets=self.offsets,
                               kept_pos=self.kept_pos, gathered=outs, workspace=self.ws_score)

    @property
    def front_stages(self):
        """The calls of the step before the attention."""
        if self.inp.adaptive is None:
            return ("score_select_compact",)
        return ("score_select", "compact")

    def run(self):
        """The front end (two launches with per-request budgets: score partials, then
        reduction + selection + compaction; three with the adaptive rule: score + select,
        compaction), then the attention."""
        for name in self.front_stages:
            getattr(self, name)()
        self.attend()

    def run_unfused(self):
        """The same step as separate calls, one per entry point of the path (the queries'
        compaction only with gather_q)."""
        self.score()
        self.select()
        self.compact_hidden()
        if self.gather_q:
            self.compact_q()
        self.attend()

    def capture(self):
        """Record one step into a HIP graph; the buffers above are its fixed inputs/outputs."""
        side = torch.cuda.Stream(device=self.inp.q_att.device)  # default priority
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            self.run()  # the library's one-time queries happen outside the capture
        torch.cuda.current_stream().wait_stream(side)
        self.graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.graph):
            self.run()
        return self.graph

    def replay(self):
        self.graph.replay()


class FullBlockStep:
    """The unfocused baseline on the same kernels: every block token is a query (k_r = blk), so
    no scoring, selection or gather is needed -- the block queries [B, blk, Hq, d] already are
    the ragged row list with offsets r * blk -- and the ragged paged attention runs on all of
    them.  Project page "FOCUS: DLLMs Know How to Tame Their Compute Bound", card "Motivation"
    (block diffusion recomputes the full block at every step)."""

    def __init__(self, inp: StepInputs, want_lse: bool = True):
        B, blk, Hq, d = inp.q_att.shape
        dev = inp.q_att.device
        self.inp = inp
        self.B, self.blk = B, blk
        self.q = inp.q_att.view(B * blk, Hq, d)
        self.offsets = torch.arange(0, (B + 1) * blk, blk, dtype=torch.int32, device=dev)
        self.out = torch.empty((B * blk, Hq, d), dtype=torch.bfloat16, device=dev)
        self.lse = torch.empty((B * blk, Hq), dtype=torch.float32, device=dev) \
            if want_lse else None
        S = inp.k_cache.shape[3]
        Hkv = inp.k_blk.shape[1]
        nat = F.attn_workspace_bytes(B, blk, Hq, Hkv, d, S, inp.page_table.shape[1], blk)
        self.ws_attn = torch.zeros(max(nat, 1), dtype=torch.uint8, device=dev)  # zeros once

    def attend(self):
        i = self.inp
        F.ragged_paged_attn(self.q, self.offsets, i.k_cache, i.v_cache, i.page_table,
                            i.prefix_len, i.k_blk, i.v_blk, self.blk, i.sm_scale, out=self.out,
                            lse=self.lse, want_lse=self.lse is not None, workspace=self.ws_attn)

    run = attend


class FullDomainScore:
    """Importance over the full attention domain (prefix + block keys) of layers 0 and 1: each
    layer's ragged paged attention runs on every block query (rows r*blk + i) over that layer's
    prefix cache and block keys, and its log-sum-exp output normalises the block keys' weights in
    focus_score_l01_lse.  Project page "FOCUS: DLLMs Know How to Tame Their Compute Bound", card
    "Design" (importance from the early layers' attention).  In a model the two LSEs come with
    the layers' own attention; here they are computed by the attention kernel's log-sum-exp-only
    mode, which reads no values."""

    def __init__(self, inp: StepInputs, k_cache0: torch.Tensor, k_blk0: torch.Tensor):
        B, blk, Hq, d = inp.q_att.shape
        dev = inp.q_att.device
        self.inp, self.k_cache0, self.k_blk0 = inp, k_cache0, k_blk0
        self.B, self.blk, self.Hq, self.d = B, blk, Hq, d
        self.offsets = torch.arange(0, (B + 1) * blk, blk, dtype=torch.int32, device=dev)
        self.lse0 = torch.empty((B * blk, Hq), dtype=torch.float32, device=dev)
        self.lse1 = torch.empty((B * blk, Hq), dtype=torch.float32, device=dev)
        self.delta = torch.empty((B, blk), dtype=torch.float32, device=dev)
        S = inp.k_cache.shape[3]
        Hkv = inp.k_blk.shape[1]
        nat = F.attn_workspace_bytes(B, blk, Hq, Hkv, d, S, inp.page_table.shape[1], blk)
        self.ws_attn = torch.zeros(max(nat, 1), dtype=torch.uint8, device=dev)
        nsc = F.lib().focus_score_l01_workspace_size(B, blk, Hq, Hkv, d)
        self.ws_score = torch.zeros(max(nsc, 1), dtype=torch.uint8, device=dev)

    def layer_lse(self):
        i = self.inp
        for q, kc, kb, lse in ((i.q0, self.k_cache0, self.k_blk0, self.lse0),
                               (i.q1, i.k_cache, i.k_blk, self.lse1)):
            F.ragged_paged_attn(q.reshape(self.B * self.blk, self.Hq, self.d), self.offsets, kc,
                                None, i.page_table, i.prefix_len, kb, None, self.blk,
                                i.sm_scale, lse=lse, workspace=self.ws_attn, want_out=False)

    def score(self):
        i = self.inp
        F.score_l01_lse(i.q0, i.k0, i.q1, i.k1, self.lse0.view(self.B, self.blk, self.Hq),
                        self.lse1.view(self.B, self.blk, self.Hq), i.sm_scale, delta=self.delta,
                        workspace=self.ws_score)

    def run(self):
        self.layer_lse()
        self.score()
        return self.delta
