"""Host-side decode loop over moe_verify_step (argument marshalling and
bookkeeping only; every step of the verify path runs in the HIP library).

Each of B0 sequences runs until it has committed its target number of tokens.  A step
takes the sequences still running, B of them, with K drafts each, and
verifies their T = B (K + 1) rows in one moe_verify_step call; the host then
reads the commit counts (the one device-to-host copy of a step) and decides
who goes on.  The output hidden rows are the next step's input rows, row for
row; finished sequences drop out and the rows of the others are compacted.
When K changes from one step to the next, a sequence's input rows are its
first K + 1 output rows, the last one repeated if there are fewer.  (The
verify path has no attention, so these rows stand in for the hidden states
a full decoder would produce; the feedback keeps every step's input new.)

The draft length of a step is chosen per step by `k_policy(B)`: a fixed K,
or `AdaptiveK`, which calls mv_choose_k with the step costs measured at the
current batch.  The accept rule (FastMTP paragraph of "Jina AI Releases
jina-ocr-v1, a 3.4B MoE Document Parser With Built-In Speculative Decoding")
commits 1 + (accepted drafts) tokens per sequence and step; with drafts that
match independently with probability q that is 1 + q + ... + q^K on average,
and the best K depends on what a step costs at the batch size at hand.

Drafts are synthetic: a rehearsal of the loop runs each step once with
placeholder drafts to learn the verifier's argmax (which does not depend on
the drafts), draws drafts equal to it with probability p, and records them
with the step's K; a replay then runs exactly those steps.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Callable, Dict, List, Optional, Sequence

import numpy as np


@dataclass
class StepRecord:
    """One step of a loop: what ran, for replay and for spot checks."""
    index: int
    seqs: np.ndarray            # original ids of the sequences in the step, in row order
    K: int
    drafts: object              # device int32 [B, K]
    compacted: bool             # the step's input rows were regathered (finish or K change)
    h_in: object = None         # device copy of the input rows, when recorded
    outputs: Dict[str, np.ndarray] = field(default_factory=dict)


@dataclass
class LoopResult:
    steps: List[StepRecord]
    rows: int                   # token rows verified
    committed: int              # tokens committed, capped at target per sequence
    per_seq_step: float         # mean tokens committed per sequence and step
    k_hist: Dict[int, int]      # steps per draft length


class FixedK:
    def __init__(self, K: int):
        self.K = int(K)

    def __call__(self, B: int) -> int:
        return self.K


class AdaptiveK:
    """Draft length per step from measured step costs: cost[B][K] is the
    time of one step with B sequences and K drafts (measured at a few batch
    sizes; between them linear in B, beyond them the nearest).  Each step
    calls mv_choose_k(q, cost at the current B)."""

    def __init__(self, bd, q: float, cost: Dict[int, Sequence[float]]):
        self.bd, self.q = bd, float(q)
        self.bs = sorted(cost)
        self.cost = {b: [float(c) for c in cost[b]] for b in self.bs}
        self.k_max = len(self.cost[self.bs[0]]) - 1

    def costs_at(self, B: int) -> List[float]:
        bs = self.bs
        if B <= bs[0]:
            return self.cost[bs[0]]
        if B >= bs[-1]:
            return self.cost[bs[-1]]
        hi = next(i for i, b in enumerate(bs) if b >= B)
        b0, b1 = bs[hi - 1], bs[hi]
        f = (B - b0) / (b1 - b0)
        return [(1 - f) * c0 + f * c1 for c0, c1 in zip(self.cost[b0], self.cost[b1])]

    def __call__(self, B: int) -> int:
        return self.bd.mv_choose_k(self.q, self.costs_at(B))[0]


def run_loop(bd, model, h_start, B0: int, target, k_policy: Callable[[int], int], k_max: int,
             draw_drafts: Optional[Callable] = None, plan: Optional[List[StepRecord]] = None,
             before_verify: Optional[Callable] = None, record: Optional[Callable[[int, bool], bool]] = None,
             stream=None) -> LoopResult:
    """Run the loop once.

    h_start: device [B0 * (k_max + 1), d], each sequence's first input rows.
    target: tokens each sequence commits before it stops (one int, or one
      per sequence).
    plan None (rehearsal): each step is run with placeholder drafts, then
      draw_drafts(step, argmax [B, K+1] numpy, seqs) gives its drafts (numpy
      int32 [B, K]) and it is run again with them.
    plan given (replay): the recorded K and drafts of each step.
    before_verify(B, K, h_in): called before each verify call (e.g. to run
      the draft block's work for the step).
    record(step, compacted) True: keep a copy of that step's input rows and
      its outputs (compacted: its input rows were regathered).
    """
    import torch

    dev = h_start.device
    dims = model.dims
    d = dims.d_model
    per = k_max + 1
    T_max = B0 * per
    outs = dict(argmax=torch.empty(T_max, dtype=torch.int32, device=dev),
                n_accepted=torch.empty(B0, dtype=torch.int32, device=dev),
                committed=torch.empty((B0, per), dtype=torch.int32, device=dev),
                n_committed=torch.empty(B0, dtype=torch.int32, device=dev))
    bufs = [torch.empty((T_max, d), dtype=h_start.dtype, device=dev) for _ in range(2)]
    zero = torch.zeros((B0, max(k_max, 1)), dtype=torch.int32, device=dev)

    targets = np.broadcast_to(np.asarray(target, np.int64), (B0,))
    done = np.zeros(B0, np.int64)
    alive = np.arange(B0)
    cur, cur_K = h_start, k_max           # current input rows and their rows per sequence - 1
    steps: List[StepRecord] = []
    rows = seq_steps = raw = 0
    k_hist: Dict[int, int] = {}
    finished_last = False

    def verify(h_in, h_out, drafts, B, K):
        if before_verify is not None:
            before_verify(B, K, h_in)
        bd.moe_verify_step(model.cfg, model.weights, B, K, h_in, drafts, h_out, outs["argmax"],
                           outs["n_accepted"], outs["committed"], outs["n_committed"], None,
                           model.ws, model.ws_bytes, stream)

    s = 0
    while alive.size:
        B = alive.size
        K = plan[s].K if plan is not None else int(k_policy(B))
        T = B * (K + 1)
        # input rows: the first K + 1 of each sequence's current rows (last repeated)
        compacted = finished_last or K != cur_K
        if K != cur_K:
            idx = (np.arange(B)[:, None] * (cur_K + 1) + np.minimum(np.arange(K + 1), cur_K)[None, :]).reshape(-1)
            cur = cur.index_select(0, torch.from_numpy(idx).to(dev))
        h_in = cur[:T]
        h_out = bufs[s % 2][:T]
        if plan is None:
            verify(h_in, h_out, zero.view(-1)[:B * K], B, K)
            g = bd.to_host(outs["argmax"][:T]).reshape(B, K + 1)
            drafts = bd.to_device(np.ascontiguousarray(draw_drafts(s, g, alive), np.int32).reshape(B, K))
        else:
            drafts = plan[s].drafts
        rec = StepRecord(s, alive.copy(), K, drafts, compacted)
        if record is not None and record(s, compacted):
            rec.h_in = h_in.clone()
        verify(h_in, h_out, drafts, B, K)
        n_com = bd.to_host(outs["n_committed"][:B])      # the host decides who goes on
        if rec.h_in is not None:
            rec.outputs = {k: bd.to_host(outs[k][:n]) for k, n in
                           (("argmax", T), ("n_accepted", B), ("n_committed", B))}
            rec.outputs["committed"] = bd.to_host(outs["committed"].view(-1)[:T]).reshape(B, K + 1)
            rec.outputs["h_out"] = bd.to_host(h_out)
        steps.append(rec)
        k_hist[K] = k_hist.get(K, 0) + 1
        done[alive] += n_com
        seq_steps += B
        raw += int(n_com.sum())
        rows += T
        keep = done[alive] < targets[alive]
        finished_last = not keep.all()
        if finished_last:
            idx = (np.nonzero(keep)[0][:, None] * (K + 1) + np.arange(K + 1)[None, :]).reshape(-1)
            h_out = h_out.index_select(0, torch.from_numpy(idx).to(dev)) if idx.size else h_out[:0]
            alive = alive[keep]
        cur, cur_K = h_out, K
        s += 1
    return LoopResult(steps, rows, int(np.minimum(done, targets).sum()), raw / max(seq_steps, 1), k_hist)
