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
    T: int
    excluded: np.ndarray = None
    near_ties: int = 0
    tolerated: int = 0
    failures: list = field(default_factory=list)

    def __post_init__(self):
        if self.excluded is None:
            self.excluded = np.zeros(self.T, bool)

    def routing(self, layer, gpu_ids, ref_ids, ref_margin, threshold=MARGIN, ill=None):
        gpu_sets = np.sort(np.asarray(gpu_ids), axis=1)
        ref_sets = np.sort(np.asarray(ref_ids), axis=1)
        differ = np.any(gpu_sets != ref_sets, axis=1)
        near = np.asarray(ref_margin) < threshold
        if ill is not None:
            near = near | ill
        live = ~self.excluded
        self.near_ties += int(np.sum(near & live))
        self.tolerated += int(np.sum(differ & near & live))
        bad = np.flatnonzero(differ & ~near & live)
        for t in bad:
            self.failures.append(f"layer {layer} token {t}: gpu {gpu_sets[t]} oracle {ref_sets[t]} "
                                 f"(margin {ref_margin[t]:.3g})")
        self.excluded |= near | differ

    def rows(self, what, gpu, ref, tol):
        err = row_rel_err(gpu, ref)
        live = ~self.excluded
        bad = np.flatnonzero(live & (err > tol))
        for t in bad:
            self.failures.append(f"{what} token {t}: rel err {err[t]:.3g} > {tol}")
        return float(err[live].max()) if live.any() else 0.0

    def argmax(self, gpu_g, ref_g, ref_margin, threshold=MARGIN, ill=None):
        near = np.asarray(ref_margin) < threshold
        if ill is not None:
            near = near | ill
        differ = np.asarray(gpu_g) != np.asarray(ref_g)
        live = ~self.excluded
        self.near_ties += int(np.sum(near & live))
        self.tolerated += int(np.sum(differ & near & live))
        for t in np.flatnonzero(differ & ~near & live):
            self.failures.append(f"argmax token {t}: gpu {gpu_g[t]} oracle {ref_g[t]} "
                                 f"(margin {ref_margin[t]:.3g})")
        self.excluded |= near | differ

    def commits(self, B, K, gpu, ref):
        """gpu/ref: dicts with n_accepted [B], committed [B,K+1], n_committed [B]."""
        seq_ok = ~self.excluded.reshape(B, K + 1).any(axis=1)
        for key in ("n_accepted", "committed", "n_committed"):
            g = np.asarray(gpu[key]).reshape(B, -1)
            r = np.asarray(ref[key]).reshape(B, -1)
            for b in np.flatnonzero(seq_ok & np.any(g != r, axis=1)):
                self.failures.append(f"{key} seq {b}: gpu {g[b]} oracle {r[b]}")
        return int(seq_ok.sum())

    def assert_ok(self, label=""):
        msg = f"{label}: {len(self.failures)} failures, near-ties {self.near_ties}, " \
              f"tolerated mismatches {self.tolerated}, excluded tokens {int(self.excluded.sum())}/{self.T}"
        print(msg)
        assert not self.failures, msg + "\n" + "\n".join(self.failures[:20])


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
