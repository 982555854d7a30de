"""bench.py's host-side arithmetic and its one-GPU contract.  No GPU needed.

The algorithmic byte and flop counts that bench.py divides by the measured
time are pinned to closed forms: every expert weight, router row, norm vector
and LM-head row counted once per use, plus the hidden rows in and out."""
import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from oracle import moe_oracle as O  # noqa: E402
from speculative_decode_verification_router_amd import synth  # noqa: E402

D = synth.DS3B_BF16


def _ids_hitting(n_per_layer, T, k, E, seed=0):
    """Top-k ids [L, T, k] whose layer l uses exactly n_per_layer[l] experts."""
    rng = np.random.default_rng(seed)
    out = []
    for n in n_per_layer:
        experts = rng.permutation(E)[:n]
        rows = []
        for t in range(T):
            # every expert of the set appears somewhere; rows stay duplicate-free
            first = [experts[(t * k + j) % n] for j in range(k)]
            if len(set(first)) < k:
                first = list(rng.permutation(experts)[:k])
            rows.append(first)
        ids = np.array(rows, np.int32)
        assert len(np.unique(ids)) == n
        out.append(ids)
    return np.stack(out)


def test_step_bytes_closed_form():
    T, k = 16, D.top_k
    n = [8, 13, 21, 30, 40, 50, 64, 9, 17, 33, 44, 60]
    ids = _ids_hitting(n, T, k, D.n_routed)
    got, distinct = bench.step_bytes(D, ids, T)
    assert distinct == n
    es, d, F = 2, D.d_model, D.d_ff
    want = sum(x + D.n_shared for x in n) * 3 * F * d * es
    want += D.n_layers * (D.n_routed * d + d) * es + D.vocab * d * es + d * es + 2 * T * d * es
    assert got == want


def test_step_bytes_equals_the_byte_model_when_every_expert_is_hit():
    T = 128
    ids = _ids_hitting([D.n_routed] * D.n_layers, T, D.top_k, D.n_routed)
    got, _ = bench.step_bytes(D, ids, T)
    # the model's verify step (no draft positions) at 128 rows expects
    # 64 (1 - (58/64)^128) distinct experts per layer, short of 64 by 2.2e-4
    short = D.n_routed - O.expected_distinct_experts(T, D.n_routed, D.top_k)
    assert 0 < short < 3e-4
    expert = 3 * D.d_ff * D.d_model * 2
    assert got - O.step_bytes(D, T, 0, 0) == pytest.approx(D.n_layers * short * expert, rel=1e-6)


def test_stack_flops():
    # 10,048 rows: router 2 d E plus 8 experts of 6 d F multiply-adds x 2 per row and layer
    assert bench.stack_flops(D, 10048) == 10048 * 12 * (2 * 1280 * 64 + 8 * 6 * 1280 * 896)
    assert bench.stack_flops(D, 10048) == 6657492910080


def test_draft_bytes_matches_the_byte_model():
    Fm = synth.mtp_d_ff(D)
    es, d = 2, D.d_model
    for B, K in ((1, 1), (1, 3), (32, 3)):
        # the model's step minus its verify step over T = B (K + 1) rows
        want = O.step_bytes(D, B, K, Fm) - O.step_bytes(D, B * (K + 1), 0, 0)
        assert bench.draft_bytes(D, Fm, B, K) == pytest.approx(want, rel=1e-9)
        assert bench.draft_bytes(D, Fm, B, K) == K * ((2 * d * d + 3 * Fm * d + D.vocab * d + 4 * d) * es
                                                      + B * 3 * d * es)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""
