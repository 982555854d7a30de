"""Comparison rules between the GPU path and the CPU oracle.

Exactness: routing (the set of selected experts per token and layer),
argmax and accept/commit must match exactly, except where the oracle's own
fp32 decision margin is below a near-tie threshold (top-k cut: 6th minus 7th
logit; argmax: largest minus second-largest logit).  A token with such a
near-tie is counted and dropped from every later exact check (and its
sequence from the accept/commit check).  Floating point rows must agree to
max|gpu - ref| / max|ref| <= tol per token row (bf16: 2e-2; fp32: 1e-4).

Threshold: 1e-3 for one layer fed the same input on both sides.  Through a
stack of layers, bf16 storage turns last-bit differences of fp32 sums into
whole-ulp differences of the stored hidden state, which grow from layer to
layer; the threshold there is max(1e-3, 4 * delta), where delta is the gap
between the oracle's float64 run and its float32-working-precision run of the
same algorithm on the same inputs (per token and layer: max over the logits).
Where those two oracle runs already route a token differently, that token's
decision is ill-conditioned at fp32 noise and it is treated as a near-tie.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

MARGIN = 1e-3
TOL = {"bf16": 2e-2, "f32": 1e-4}


def row_rel_err(gpu: np.ndarray, ref: np.ndarray) -> np.ndarray:
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    scale = np.maximum(np.abs(ref).max(axis=1), 1e-30)
    return np.abs(gpu - ref).max(axis=1) / scale


@dataclass
class Tally:
    """forced=False (a stack run end to end on both sides): a token with a
    near-tie anywhere is dropped from every later check, since from there
    the two sides may compute on different inputs.  forced=True (teacher
    forcing: every layer and the LM head of the oracle are fed the GPU's own
    input): the inputs agree by construction, so a near-tie drops a token
    only where the two sides actually decided differently, and only from the
    checks that difference invalidates: a routing difference skips that
    layer's row check, an argmax difference the sequence's commit check.  In
    both modes `excluded` marks the tokens not checked to the end."""
    T: int
    forced: bool = False
    excluded: np.ndarray = None
    near_ties: int = 0
    tolerated: int = 0
    failures: list = field(default_factory=list)

    def __post_init__(self):
        if self.excluded is None:
            self.excluded = np.zeros(self.T, bool)
        self._skip_rows = np.zeros(self.T, bool)     # forced: this layer's routing differed
        self._argmax_off = np.zeros(self.T, bool)    # forced: the argmax differed (near-tie)

    def _live(self):
        return np.ones(self.T, bool) if self.forced else ~self.excluded

    def routing(self, layer, gpu_ids, ref_ids, ref_margin, threshold=MARGIN, ill=None):
        gpu_sets = np.sort(np.asarray(gpu_ids), axis=1)
        ref_sets = np.sort(np.asarray(ref_ids), axis=1)
        differ = np.any(gpu_sets != ref_sets, axis=1)
        near = np.asarray(ref_margin) < threshold
        if ill is not None:
            near = near | ill
        live = self._live()
        self.near_ties += int(np.sum(near & live))
        self.tolerated += int(np.sum(differ & near & live))
        bad = np.flatnonzero(differ & ~near & live)
        for t in bad:
            self.failures.append(f"layer {layer} token {t}: gpu {gpu_sets[t]} oracle {ref_sets[t]} "
                                 f"(margin {ref_margin[t]:.3g})")
        if self.forced:
            self._skip_rows = differ
            self.excluded |= differ
        else:
            self.excluded |= near | differ

    def rows(self, what, gpu, ref, tol):
        err = row_rel_err(gpu, ref)
        live = ~self._skip_rows if self.forced else ~self.excluded
        bad = np.flatnonzero(live & (err > tol))
        for t in bad:
            self.failures.append(f"{what} token {t}: rel err {err[t]:.3g} > {tol}")
        return float(err[live].max()) if live.any() else 0.0

    def argmax(self, gpu_g, ref_g, ref_margin, threshold=MARGIN, ill=None):
        near = np.asarray(ref_margin) < threshold
        if ill is not None:
            near = near | ill
        differ = np.asarray(gpu_g) != np.asarray(ref_g)
        live = self._live()
        self.near_ties += int(np.sum(near & live))
        self.tolerated += int(np.sum(differ & near & live))
        for t in np.flatnonzero(differ & ~near & live):
            self.failures.append(f"argmax token {t}: gpu {gpu_g[t]} oracle {ref_g[t]} "
                                 f"(margin {ref_margin[t]:.3g})")
        if self.forced:
            self._argmax_off |= differ
            self.excluded |= differ
        else:
            self.excluded |= near | differ

    def commits(self, B, K, gpu, ref):
        """gpu/ref: dicts with n_accepted [B], committed [B,K+1], n_committed [B]."""
        off = self._argmax_off if self.forced else self.excluded
        seq_ok = ~off.reshape(B, K + 1).any(axis=1)
        for key in ("n_accepted", "committed", "n_committed"):
            g = np.asarray(gpu[key]).reshape(B, -1)
            r = np.asarray(ref[key]).reshape(B, -1)
            for b in np.flatnonzero(seq_ok & np.any(g != r, axis=1)):
                self.failures.append(f"{key} seq {b}: gpu {g[b]} oracle {r[b]}")
        return int(seq_ok.sum())

    @property
    def checked(self) -> int:
        return int(self.T - self.excluded.sum())

    def assert_ok(self, label="", min_checked=None):
        """No failures, and (so that a comparison cannot pass by excluding
        everything) at least a fraction min_checked of the tokens checked to
        the end: by default 3/4 of the tokens (end to end through 12 layers
        about 15% of tokens meet a near-tie; teacher-forced only the far
        fewer where the two sides then decide differently are dropped)."""
        if min_checked is None:
            min_checked = 0.75
        msg = f"{label}: {len(self.failures)} failures, near-ties {self.near_ties}, " \
              f"tolerated mismatches {self.tolerated}, checked tokens {self.checked}/{self.T}"
        print(msg)
        assert not self.failures, msg + "\n" + "\n".join(self.failures[:20])
        assert self.checked >= min_checked * self.T, f"{msg}: fewer than {min_checked:.0%} checked"


def stack_conditioning(ref64, ref32):
    """Per-layer (threshold, ill) for routing and (threshold, ill) for the
    argmax, from an oracle float64 run and a float32-working-precision run of
    the same stack on the same rows."""
    layers = []
    for a, b in zip(ref64["layers"], ref32["layers"]):
        delta = np.abs(a["logits"] - b["logits"]).max(axis=1)
        ill = np.any(np.sort(a["ids"], axis=1) != np.sort(b["ids"], axis=1), axis=1)
        layers.append((np.maximum(MARGIN, 4 * delta), ill))
    final = None
    if "logits" in ref64 and "logits" in ref32:
        dz = np.abs(ref64["logits"] - ref32["logits"]).max(axis=1)
        final = (np.maximum(MARGIN, 4 * dz), np.asarray(ref64["argmax"]) != np.asarray(ref32["argmax"]))
    return layers, final


def forced_stack(bd, torch, dims, W, model, h_dev, rows, label, tally=None, ids_expect=None):
    """Teacher-forced walk of the layer stack on the device rows h_dev [T, d]:
    moe_layer_forward layer by layer on the GPU, and at every layer the
    oracle's layer fed the GPU's own input rows `rows` must route like the GPU
    (single-layer near-tie rule) and agree on the output rows.  Then the
    oracle's LM head on the GPU's final rows.  ids_expect [L, T, k]: routing
    the chain must reproduce bit for bit (a verify step's).  Returns the
    tally, the GPU's final rows (host) and the oracle's LM-head result."""
    from oracle import moe_oracle as O

    rows = np.asarray(rows)
    tally = tally if tally is not None else Tally(len(rows), forced=True)
    cur = h_dev
    for layer in range(dims.n_layers):
        lo = bd.run_layer_forward(model, layer, cur)
        torch.cuda.synchronize()
        gid = bd.to_host(lo["topk_ids"])
        if ids_expect is not None:
            assert np.array_equal(gid, ids_expect[layer]), f"{label}: layer {layer}: chain and step route differently"
        ref = O.moe_layer(O.widen(bd.to_host(cur), dims.dtype)[rows], W, layer, dims)
        tally.routing(layer, gid[rows], ref["ids"], ref["margin"])
        tally.rows(f"{label} layer {layer} h_out", O.widen(bd.to_host(lo["h_out"]), dims.dtype)[rows],
                   ref["h_out"], TOL[dims.dtype])
        cur = lo["h_out"]
    h_fin = bd.to_host(cur)
    lm = O.lm_head_argmax(O.widen(h_fin, dims.dtype)[rows], W["final_norm"], W["lm_head"], dims)
    return tally, h_fin, lm
