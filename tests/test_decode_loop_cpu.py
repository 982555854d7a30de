"""Host bookkeeping of the decode loop (decode_loop.run_loop) without a GPU.

A stand-in for the library's verify step (a host function on CPU tensors)
lets the loop run on the CPU: each step's output rows are its input rows
plus one, its argmax is read off the rows, and its commits are the oracle's
accept rule.  The tests check the loop's own logic against an independent
simulation: feedback of output rows, compaction of finished sequences, the
input rows after a change of K (the first K + 1 output rows, the last one
repeated), the per-sequence stop, and that a replay of the recorded plan
repeats the rehearsal.  AdaptiveK is checked against the oracle's choose_k.
"""
import types

import numpy as np
import pytest
import torch

from oracle import moe_oracle as O
from speculative_decode_verification_router_amd import decode_loop as DL
from speculative_decode_verification_router_amd import synth

V = 97


class FakeBinding:
    """The entry points run_loop calls, on CPU tensors."""

    def __init__(self):
        self.calls = 0

    def moe_verify_step(self, cfg, weights, B, K, h_in, drafts, h_out, argmax, n_accepted, committed,
                        n_committed, dbg, ws, ws_bytes, stream):
        self.calls += 1
        T = B * (K + 1)
        h_out[:T] = h_in[:T] + 1.0
        g = (h_in[:T, 0].to(torch.int64) * 31 + h_in[:T, 1].to(torch.int64)) % V
        argmax[:T] = g.to(torch.int32)
        d = drafts.reshape(-1)[:B * K].reshape(B, K).numpy() if K else np.zeros((B, 0), np.int32)
        n_acc, com, n_com = O.spec_accept(g.numpy().reshape(B, K + 1), d)
        n_accepted[:B] = torch.from_numpy(n_acc.astype(np.int32))
        committed.view(-1)[:T] = torch.from_numpy(com.astype(np.int32).reshape(-1))
        n_committed[:B] = torch.from_numpy(n_com.astype(np.int32))

    def to_host(self, t):  # a copy, as a device-to-host copy is
        return t.detach().cpu().numpy().copy()

    def to_device(self, a):
        return torch.from_numpy(np.ascontiguousarray(a))

    def mv_choose_k(self, q, cost):
        return O.choose_k(q, cost)


def _model(d=8):
    dims = types.SimpleNamespace(d_model=d)
    return types.SimpleNamespace(dims=dims, cfg=None, weights=None, ws=None, ws_bytes=0)


def _start(B0, k_max, d=8):
    h = np.zeros((B0 * (k_max + 1), d), np.float32)
    for b in range(B0):
        for j in range(k_max + 1):
            h[b * (k_max + 1) + j, 0] = 100 * b + j
            h[b * (k_max + 1) + j, 1] = b
    return torch.from_numpy(h)


def _simulate(h0, B0, k_max, target, ks_per_step, n_com_per_step):
    """Independent bookkeeping: the input rows every step should see."""
    rows = {b: [h0[b * (k_max + 1) + j].copy() for j in range(k_max + 1)] for b in range(B0)}
    Kc = {b: k_max for b in range(B0)}
    done = np.zeros(B0, np.int64)
    alive = list(range(B0))
    expect = []
    for K, ncom in zip(ks_per_step, n_com_per_step):
        inp = []
        for b in alive:
            inp += [rows[b][min(j, Kc[b])] for j in range(K + 1)]
        expect.append((list(alive), np.stack(inp)))
        for i, b in enumerate(alive):
            rows[b] = [r + 1.0 for r in inp[i * (K + 1):(i + 1) * (K + 1)]]
            Kc[b] = K
            done[b] += ncom[i]
        alive = [b for b in alive if done[b] < target[b]]
    return expect, done


def _draw(p):
    return lambda step, g, seqs: synth.make_drafts(g, p, V, seed=1, step=step)


@pytest.mark.parametrize("policy", ["fixed", "changing"])
def test_loop_feeds_back_compacts_and_stops(policy):
    bd = FakeBinding()
    B0, k_max = 5, 3
    target = np.array([9, 3, 17, 1, 12])
    h0 = _start(B0, k_max)
    pol = DL.FixedK(2) if policy == "fixed" else (lambda B: 3 if B >= 4 else (1 if B >= 2 else 2))
    res = DL.run_loop(bd, _model(), h0, B0, target, pol, k_max, draw_drafts=_draw(0.7),
                      record=lambda s, c: True)
    steps = res.steps
    expect, done = _simulate(h0.numpy(), B0, k_max, target, [st.K for st in steps],
                             [st.outputs["n_committed"] for st in steps])
    assert len(expect) == len(steps)
    for st, (alive, rows) in zip(steps, expect):
        assert st.seqs.tolist() == alive, st.index
        assert np.array_equal(st.h_in.numpy(), rows), st.index
        assert st.K == pol(len(alive))
    assert np.all(done >= target) and res.committed == int(target.sum())
    assert res.rows == sum(len(st.seqs) * (st.K + 1) for st in steps)
    assert sum(res.k_hist.values()) == len(steps)
    # compaction flags: set when a sequence finished in the previous step or K changed
    for prev, cur in zip(steps, steps[1:]):
        assert cur.compacted == (len(cur.seqs) < len(prev.seqs) or cur.K != prev.K)


def test_replay_repeats_the_rehearsal():
    bd = FakeBinding()
    B0, k_max = 4, 3
    target = np.array([10, 10, 10, 10])
    h0 = _start(B0, k_max)
    pol = lambda B: 3 if B > 2 else 1  # noqa: E731
    reh = DL.run_loop(bd, _model(), h0, B0, target, pol, k_max, draw_drafts=_draw(0.5))
    calls = bd.calls
    rep = DL.run_loop(bd, _model(), h0, B0, target, pol, k_max, plan=reh.steps)
    assert bd.calls - calls == len(reh.steps)          # one verify call per replayed step
    assert calls == 2 * len(reh.steps)                 # the rehearsal verifies twice per step
    assert [s.K for s in rep.steps] == [s.K for s in reh.steps]
    assert [s.seqs.tolist() for s in rep.steps] == [s.seqs.tolist() for s in reh.steps]
    assert rep.committed == reh.committed == 40


def test_adaptive_k_matches_the_oracle_policy():
    bd = FakeBinding()
    cost = {1: [0.40, 0.44, 0.47, 0.50], 4: [0.49, 0.58, 0.59, 0.64], 32: [0.78, 1.05, 1.26, 1.48]}
    pol = DL.AdaptiveK(bd, 0.6, cost)
    assert pol.costs_at(1) == cost[1] and pol.costs_at(32) == cost[32] and pol.costs_at(64) == cost[32]
    mid = pol.costs_at(18)                              # linear between B = 4 and B = 32
    f = (18 - 4) / 28
    assert np.allclose(mid, [(1 - f) * a + f * b for a, b in zip(cost[4], cost[32])])
    for B in (1, 2, 4, 10, 18, 32):
        assert pol(B) == O.choose_k(0.6, pol.costs_at(B))[0]
    # at this acceptance the best draft length shrinks as the batch grows
    assert pol(1) > pol(32)
