"""Draft length: the oracle's expected commits, distinct-expert count and
policy pinned against simulation, limits and a hand computation, and the C
ABI's mv_choose_k / mv_step_bytes against the oracle.  No GPU needed."""
import numpy as np
import pytest

from oracle import moe_oracle as O
from speculative_decode_verification_router_amd import binding as bd
from speculative_decode_verification_router_amd import synth


@pytest.fixture(scope="module")
def lib():
    import os

    if not os.path.exists(bd.LIB_PATH):
        from speculative_decode_verification_router_amd import build

        build.build()
    return bd.load()


# ---------------------------------------------------------------- oracle pins


@pytest.mark.parametrize("q,K", [(0.3, 1), (0.6, 3), (0.9, 5)])
def test_expected_committed_matches_the_accept_rule(q, K):
    """Drafts right independently with probability q through the oracle's
    accept rule: the mean commit count agrees with 1 + q + ... + q^K."""
    rng = np.random.default_rng(7)
    B = 40000
    g = np.zeros((B, K + 1), np.int64)
    drafts = np.where(rng.random((B, K)) < q, 0, 1)
    _, _, n_com = O.spec_accept(g, drafts)
    mean, sd = n_com.mean(), n_com.std() / np.sqrt(B)
    assert abs(mean - O.expected_committed(q, K)) < 4 * sd


@pytest.mark.parametrize("T", [1, 2, 4, 16, 128])
def test_expected_distinct_experts_matches_sampling(T):
    rng = np.random.default_rng(T)
    E, k, n = 64, 6, 4000
    counts = np.array([len(np.unique(np.concatenate([rng.choice(E, k, replace=False) for _ in range(T)])))
                       for _ in range(n)])
    assert abs(counts.mean() - O.expected_distinct_experts(T, E, k)) < 4 * counts.std() / np.sqrt(n) + 1e-9
    if T == 1:
        assert O.expected_distinct_experts(1, E, k) == pytest.approx(k)


def test_choose_k_limits_and_a_hand_computation():
    cost = [0.421, 0.624, 0.78, 0.925]
    # no draft is ever right: every K commits one token, the cheapest step wins
    assert O.choose_k(0.0, cost)[0] == 0
    assert O.choose_k(0.0, [2.0, 1.0, 1.0])[0] == 1           # ties go to the smaller K
    # every draft is right: K + 1 tokens per step
    assert O.choose_k(1.0, cost)[0] == int(np.argmax(np.arange(1, 5) / np.array(cost)))
    # q = 0.576 with these step times: 1/0.421 = 2.375, 1.576/0.624 = 2.526,
    # 1.908/0.78 = 2.446, 2.099/0.925 = 2.269 tokens per ms
    k, r = O.choose_k(0.576, cost)
    assert k == 1 and r == pytest.approx(1.576 / 0.624)


def test_step_bytes_closed_form_when_every_expert_is_hit():
    d = synth.DS3B_BF16
    es, E, S, L = 2, d.n_routed, d.n_shared, d.n_layers
    expert = 3 * d.d_ff * d.d_model * es
    T = 1024
    want = (L * (E + S) * expert + L * (E * d.d_model + d.d_model) * es + d.vocab * d.d_model * es
            + d.d_model * es + 2 * T * d.d_model * es)
    assert O.step_bytes(d, T, 0, 0) == pytest.approx(want, rel=1e-9)
    # the draft FFN is streamed once per draft position
    Fm = 1792
    for K in (1, 3):
        dff = O.step_bytes(d, 1, K, Fm) - O.step_bytes(d, 1, K, 0)
        assert dff == pytest.approx(K * 3 * Fm * d.d_model * es, rel=1e-12)
    # the LM head is read once per draft position and once by the verify step
    import dataclasses

    small = dataclasses.replace(d, vocab=d.vocab - 1000)
    for K in (0, 1, 3):
        dv = O.step_bytes(d, 2, K, Fm) - O.step_bytes(small, 2, K, Fm)
        assert dv == pytest.approx((K + 1) * 1000 * d.d_model * es, rel=1e-9)


# ---------------------------------------------------------------- C ABI


def test_choose_k_matches_the_oracle(lib):
    rng = np.random.default_rng(3)
    for _ in range(300):
        k_max = int(rng.integers(0, 16))
        cost = rng.uniform(0.1, 3.0, k_max + 1).astype(np.float32)
        q = np.float32(rng.uniform(0, 1))
        want_k, want_r = O.choose_k(float(q), [float(c) for c in cost])
        rates = sorted(O.expected_committed(float(q), K) / float(c) for K, c in enumerate(cost))
        if len(rates) > 1 and rates[-1] - rates[-2] < 1e-6 * rates[-1]:
            continue  # a near-tie: either K is right
        k, r = bd.mv_choose_k(float(q), cost)
        assert k == want_k
        assert r == pytest.approx(want_r, rel=1e-6)


def test_choose_k_rejects_bad_arguments(lib):
    import ctypes

    c = (ctypes.c_float * 2)(1.0, 1.0)
    k = ctypes.c_int32()
    assert lib.mv_choose_k(1, 0.5, None, ctypes.byref(k), None) == bd.MV_ERR_NULL
    assert lib.mv_choose_k(1, 0.5, c, None, None) == bd.MV_ERR_NULL
    assert lib.mv_choose_k(16, 0.5, c, ctypes.byref(k), None) == bd.MV_ERR_SHAPE
    assert lib.mv_choose_k(1, 1.5, c, ctypes.byref(k), None) == bd.MV_ERR_SHAPE
    assert lib.mv_choose_k(1, float("nan"), c, ctypes.byref(k), None) == bd.MV_ERR_SHAPE
    bad = (ctypes.c_float * 2)(1.0, 0.0)
    assert lib.mv_choose_k(1, 0.5, bad, ctypes.byref(k), None) == bd.MV_ERR_SHAPE
    assert lib.mv_choose_k(0, 0.5, c, ctypes.byref(k), None) == bd.MV_OK and k.value == 0


@pytest.mark.parametrize("dims,Fm", [(synth.DS3B_BF16, 1792), (synth.TINY_F32, 256)])
def test_step_bytes_matches_the_oracle(lib, dims, Fm):
    cfg = bd.make_config(dims)
    for B in (1, 4, 32):
        for K in (0, 1, 3, 15):
            assert bd.mv_step_bytes(cfg, B, K, Fm) == pytest.approx(O.step_bytes(dims, B, K, Fm), rel=1e-12)
    with pytest.raises(bd.MvError):
        bd.mv_step_bytes(cfg, 1, 16, Fm)
