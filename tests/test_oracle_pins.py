"""Pins of the CPU oracle against things other than itself: library routines,
closed forms, invariants, brute force and the pages' printed statistics.
No GPU needed."""
import itertools
import math
import os

import numpy as np
import pytest
import torch

from oracle import moe_oracle as O
from speculative_decode_verification_router_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def golden(name):
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if line:
                k, v = line.split()
                out[k] = float(v)
    return out


# ---------------------------------------------------------------- storage


def test_bf16_rounding_matches_torch_rne():
    rng = np.random.default_rng(1)
    v = rng.standard_normal(200000).astype(np.float32) * np.float32(3.0)
    # exact halfway cases: low 16 bits = 0x8000, both parities of the kept lsb
    hi = rng.integers(0x3F00, 0x4100, 1000).astype(np.uint32)
    half = ((hi << 16) | 0x8000).view(np.float32)
    v = np.concatenate([v, half, -half, np.float32([0.0, -0.0, np.inf, -np.inf,
                                                     3.3895314e38, 1e-40])])
    ours = O.fp32_to_bf16_rne(v)
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    assert np.isnan(O.widen(O.fp32_to_bf16_rne(np.float32([np.nan])), "bf16")[0])


def test_store_is_idempotent_and_lands_on_bf16_grid():
    v = np.random.default_rng(2).standard_normal(5000) * 10
    s = O.store(v, "bf16")
    assert np.array_equal(O.store(s, "bf16"), s)
    assert np.all(np.abs(s - v) <= np.abs(v) * 2.0 ** -8 + 1e-300)
    assert np.array_equal(O.store(v, "f32"), v.astype(np.float32).astype(np.float64))


# ---------------------------------------------------------------- RMSNorm


def test_rms_norm_matches_torch():
    rng = np.random.default_rng(3)
    h = rng.standard_normal((7, 96)) * 3
    g = rng.uniform(0.5, 1.5, 96)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(h), (96,), torch.from_numpy(g),
                                       eps=1e-6).numpy()
    np.testing.assert_allclose(O.rms_norm(h, g, 1e-6), ref, rtol=1e-13, atol=1e-15)


def test_rms_norm_constant_row_closed_form():
    for c in [1e-4, 0.3, -2.0, 50.0]:
        h = np.full((1, 64), c)
        g = np.linspace(0.5, 1.5, 64)
        expect = c / math.sqrt(c * c + 1e-6) * g
        np.testing.assert_allclose(O.rms_norm(h, g, 1e-6)[0], expect, rtol=1e-14)


# ---------------------------------------------------------------- router


def test_router_logits_one_hot_rows_pick_coordinates():
    # W_r row e = unit vector on coordinate perm[e] -> logit e = x[perm[e]].
    rng = np.random.default_rng(4)
    d, E = 48, 20
    perm = rng.permutation(d)[:E]
    W = np.zeros((E, d))
    W[np.arange(E), perm] = 1.0
    x = rng.standard_normal((3, d))
    b = rng.standard_normal(E)
    l = O.router_logits(x, W, b)
    np.testing.assert_array_equal(l, (x[:, perm] + b).astype(np.float32).astype(np.float64))


def _brute_top_k(l, k):
    order = np.argsort(-l, kind="stable")   # stable: equal values keep id order
    return list(order[:k]), float(l[order[k - 1]] - l[order[k]])


def test_top_k_matches_stable_sort_including_exact_ties():
    rng = np.random.default_rng(5)
    for trial in range(300):
        l = rng.standard_normal(64).astype(np.float32).astype(np.float64)
        if trial % 3 == 0:   # heavy exact ties: a few distinct values
            l = rng.integers(0, 4, 64).astype(np.float64)
        if trial % 3 == 1:   # tie straddling the cut
            l[rng.permutation(64)[:10]] = l.max() - 0.5
        sel, margin = O.select_top_k(l, 6)
        bsel, bmargin = _brute_top_k(l, 6)
        assert sel == bsel
        assert margin == bmargin


def test_top_k_all_equal_takes_lowest_ids():
    sel, margin = O.select_top_k(np.zeros(64), 6)
    assert sel == [0, 1, 2, 3, 4, 5] and margin == 0.0


def test_gates_sum_to_one_and_equal_renormalised_full_softmax():
    from scipy.special import softmax

    rng = np.random.default_rng(6)
    for _ in range(100):
        l = rng.standard_normal(64) * 4
        sel, _ = O.select_top_k(l, 6)
        w = O.gate_weights(l[sel])
        assert abs(w.sum() - 1.0) < 1e-12
        p = softmax(l)
        np.testing.assert_allclose(w, p[sel] / p[sel].sum(), rtol=1e-12)
        assert np.all(np.diff(w) <= 0)     # selection order is descending logit


def test_silu_matches_torch():
    z = np.linspace(-50, 50, 1001)
    np.testing.assert_allclose(O.silu(z), torch.nn.functional.silu(torch.from_numpy(z)).numpy(),
                               rtol=1e-14, atol=1e-300)
    assert O.silu(np.array([-1000.0]))[0] == 0.0


# ---------------------------------------------------------------- experts


def _tiny_weights(dtype="f32", gamma="uniform", seed=0):
    dims = synth.ModelDims(64, 32, 64, 2, 6, 2, 97, 1e-6, dtype)
    W = synth.make_weights(dims, seed=seed, gamma=gamma)
    return dims, W


def _torch_ffn(x, wgu, wd):
    x, wgu, wd = (torch.from_numpy(np.asarray(a, np.float64)) for a in (x, wgu, wd))
    F = wgu.shape[0] // 2
    a = torch.nn.functional.silu(x @ wgu[:F].T) * (x @ wgu[F:].T)
    return (a @ wd.T).numpy()


def test_swiglu_expert_matches_torch_dense_ffn():
    rng = np.random.default_rng(7)
    x = rng.standard_normal((5, 64))
    wgu = rng.standard_normal((64, 64)) * 0.2
    wd = rng.standard_normal((64, 32)) * 0.2
    # f32 storage of a: within fp32 rounding of the float64 reference
    np.testing.assert_allclose(O.swiglu_expert(x, wgu, wd, "f32"), _torch_ffn(x, wgu, wd),
                               rtol=2e-6, atol=2e-6)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_one_hot_gate_equals_dense_ffn_plus_shared(dtype):
    """Router bias +1e4 on expert e*, -1e4 elsewhere: the other selected gates
    are exactly 0, so the layer is h + FFN_e*(x) + shared FFNs."""
    dims, W = _tiny_weights(dtype)
    e_star = 37
    b = np.full((dims.n_layers, 64), -1e4, np.float32)
    b[:, e_star] = 1e4
    W["router_b"] = b
    h = O.widen(synth.make_hidden(dims, 9, seed=1), dtype)
    r = O.moe_layer(h, W, 0, dims)
    assert np.all(r["ids"][:, 0] == e_star)
    assert np.all(r["gates"][:, 0] == 1.0) and np.all(r["gates"][:, 1:] == 0.0)
    wid = lambda a: O.widen(a, dtype)
    x = r["x"]
    ref = _torch_ffn(x, wid(W["w_gate_up"][0, e_star]), wid(W["w_down"][0, e_star]))
    for s in range(2):
        ref = ref + _torch_ffn(x, wid(W["ws_gate_up"][0, s]), wid(W["ws_down"][0, s]))
    tol = 2e-6 if dtype == "f32" else 2e-2   # oracle rounds a to storage, torch does not
    scale = np.abs(ref).max(axis=1, keepdims=True)
    assert np.all(np.abs(r["y"] - ref) <= tol * scale)


def test_two_shared_experts_equal_one_double_width_ffn():
    dims, W = _tiny_weights("f32")
    F = dims.d_ff
    x = np.random.default_rng(8).standard_normal((6, dims.d_model))
    g0, g1 = W["ws_gate_up"][0, 0].astype(np.float64), W["ws_gate_up"][0, 1].astype(np.float64)
    wide_gu = np.concatenate([g0[:F], g1[:F], g0[F:], g1[F:]])
    wide_d = np.concatenate([W["ws_down"][0, 0], W["ws_down"][0, 1]], axis=1).astype(np.float64)
    two = (O.swiglu_expert(x, g0, W["ws_down"][0, 0].astype(np.float64), "f32")
           + O.swiglu_expert(x, g1, W["ws_down"][0, 1].astype(np.float64), "f32"))
    np.testing.assert_allclose(two, O.swiglu_expert(x, wide_gu, wide_d, "f32"),
                               rtol=1e-12, atol=1e-12)


def test_zero_router_selects_first_six_with_equal_gates():
    dims, W = _tiny_weights("f32")
    W["router_w"][...] = 0.0
    h = O.widen(synth.make_hidden(dims, 4, seed=2), "f32")
    r = O.moe_layer(h, W, 1, dims)
    assert np.all(r["ids"] == np.arange(6))
    np.testing.assert_allclose(r["gates"], 1.0 / 6.0, rtol=1e-15)
    x = r["x"]
    ref = sum(_torch_ffn(x, W["w_gate_up"][1, e], W["w_down"][1, e]) for e in range(6)) / 6.0
    ref = ref + sum(_torch_ffn(x, W["ws_gate_up"][1, s], W["ws_down"][1, s]) for s in range(2))
    np.testing.assert_allclose(r["y"], ref, rtol=1e-5, atol=1e-6)


def test_zero_down_projection_leaves_residual_only():
    dims, W = _tiny_weights("bf16")
    W["w_down"][...] = 0
    W["ws_down"][...] = 0
    h = O.widen(synth.make_hidden(dims, 5, seed=3), "bf16")
    r = O.moe_layer(h, W, 0, dims)
    assert np.array_equal(r["h_out"], h)


def test_layer_rows_are_independent():
    dims, W = _tiny_weights("bf16")
    h = O.widen(synth.make_hidden(dims, 12, seed=4), "bf16")
    full = O.moe_layer(h, W, 0, dims)
    perm = np.random.default_rng(9).permutation(12)
    part = O.moe_layer(h[perm[:5]], W, 0, dims)
    assert np.array_equal(part["h_out"], full["h_out"][perm[:5]])
    assert np.array_equal(part["ids"], full["ids"][perm[:5]])


def test_bf16_layer_stores_on_bf16_grid():
    dims, W = _tiny_weights("bf16")
    h = O.widen(synth.make_hidden(dims, 3, seed=5), "bf16")
    r = O.moe_layer(h, W, 0, dims)
    for key in ("h_out", "x"):
        assert np.array_equal(O.store(r[key], "bf16"), r[key])


# ---------------------------------------------------------------- LM head


def test_lm_head_argmax_matches_numpy_and_ties_take_lowest_id():
    dims, W = _tiny_weights("f32")
    rng = np.random.default_rng(10)
    h = rng.standard_normal((8, dims.d_model))
    r = O.lm_head_argmax(h, W["final_norm"], W["lm_head"], dims)
    xf = O.rms_norm(h, W["final_norm"].astype(np.float64), 1e-6)
    z = xf @ W["lm_head"].astype(np.float64).T
    assert np.array_equal(r["argmax"], np.argmax(z, axis=1))
    # duplicate the winning row at a lower and a higher id: lowest id wins
    lm = W["lm_head"].copy()
    win = int(r["argmax"][0])
    lo, hi = (win - 3) % dims.vocab, (win + 5) % dims.vocab
    lm[lo] = lm[win]
    lm[hi] = lm[win]
    r2 = O.lm_head_argmax(h[:1], W["final_norm"], lm, dims)
    assert r2["argmax"][0] == min(lo, win, hi)
    assert r2["margin"][0] == 0.0


# ---------------------------------------------------------------- accept


def _accept_by_prefix(g, d):
    n = len(list(itertools.takewhile(lambda p: p[0] == p[1], zip(d, g[:len(d)]))))
    return n, list(g[:n + 1]) + [-1] * (len(d) - n)


@pytest.mark.parametrize("K", [1, 2, 3])
def test_spec_accept_exhaustive_v3(K):
    gs = np.array(list(itertools.product(range(3), repeat=K + 1)))
    ds = np.array(list(itertools.product(range(3), repeat=K)))
    G = np.repeat(gs, len(ds), axis=0)
    D = np.tile(ds, (len(gs), 1))
    n_acc, committed, n_com = O.spec_accept(G, D)
    for i in range(len(G)):
        n, c = _accept_by_prefix(list(G[i]), list(D[i]))
        assert n_acc[i] == n and list(committed[i]) == c and n_com[i] == n + 1
        assert 1 <= n_com[i] <= K + 1
        # every accepted draft is a token the decoder itself chose
        assert list(D[i][:n]) == list(G[i][:n])


def test_spec_accept_zero_drafts_commits_one():
    n_acc, committed, n_com = O.spec_accept(np.array([[7], [3]]), np.zeros((2, 0), np.int64))
    assert list(n_acc) == [0, 0] and list(n_com) == [1, 1]
    assert committed.tolist() == [[7], [3]]


def test_committed_per_step_matches_closed_form():
    V, K, B = 1024, 3, 40000
    rng = np.random.default_rng(11)
    for p in (0.4, 0.6, 0.8):
        g = rng.integers(0, V, (B, K + 1))
        d = synth.make_drafts(g, p, V, seed=12, step=int(p * 10))
        _, _, n_com = O.spec_accept(g, d)
        q = p + (1 - p) / V
        expect = 1 + sum(q ** i for i in range(1, K + 1))
        sigma = n_com.std() / math.sqrt(B)
        assert abs(n_com.mean() - expect) < 4 * sigma


def test_page_statistics_are_consistent_with_accept_rule():
    """2.73 committed tokens per step at K=3 and a 57.6% acceptance rate are
    both printed; committed = accepted + 1 with acceptance = accepted / K
    ties them together: 1 + 3 * 0.576 = 2.728."""
    g = golden("page_statistics.txt")
    K = int(g["k_draft"])
    assert round(1 + K * g["acceptance_rate"], 2) == g["committed_per_step"]
    # per-position match probability q giving the same mean with independent
    # positions: 1 + q + q^2 + q^3 = 2.728  ->  q ~ 0.7485
    from scipy.optimize import brentq

    q = brentq(lambda q: sum(q ** i for i in range(K + 1)) - (1 + K * g["acceptance_rate"]),
               0.0, 1.0)
    assert abs(q - 0.7485) < 5e-4
    assert round(g["l4_eager_fastmtp_tok_s"] / g["l4_eager_greedy_tok_s"], 2) == g["l4_eager_speedup"]
    assert round(g["l4_graph_fastmtp_k1_tok_s"] / g["l4_graph_greedy_tok_s"], 2) == g["l4_graph_speedup"]
    assert (synth.DS3B_BF16.n_layers, synth.DS3B_BF16.n_routed, synth.DS3B_BF16.n_shared,
            synth.DS3B_BF16.top_k) == (g["n_layers"], g["n_routed"], g["n_shared"], g["top_k"])


# ---------------------------------------------------------------- lossless


def _greedy_table(dims, W, emb):
    """f(tok) for every token id: the decoder's greedy next token when the
    verified row carries that token (rows are independent on this path)."""
    out = O.forward_tokens(emb, W, dims)
    return np.asarray(out["argmax"])


def _spec_decode(dims, W, emb, start, n_tokens, K, p, seed, accept=O.spec_accept):
    table = _greedy_table(dims, W, emb)
    seq, c, step = [], start, 0
    while len(seq) < n_tokens:
        # drafts: the true continuation with probability p, else uniform
        truth = [c]
        for _ in range(K):
            truth.append(int(table[truth[-1]]))
        drafts = synth.make_drafts(np.array([truth[1:] + [0]]), p, dims.vocab, seed=seed,
                                   step=step)
        h = np.stack([emb[c]] + [emb[int(t)] for t in drafts[0]])
        out = O.forward_tokens(h, W, dims)
        g = np.asarray(out["argmax"]).reshape(1, K + 1)
        n_acc, committed, n_com = accept(g, drafts)
        seq.extend(int(t) for t in committed[0, :n_com[0]])
        c = seq[-1]
        step += 1
    return seq[:n_tokens], step


def test_lossless_spec_decode_equals_plain_greedy():
    dims = synth.TINY_F32
    W = synth.make_weights(dims, seed=0)
    emb = synth.make_embedding(dims, seed=0)
    table = _greedy_table(dims, W, emb)
    start, n = 17, 200
    greedy = [start]
    for _ in range(n):
        greedy.append(int(table[greedy[-1]]))
    spec, steps = _spec_decode(dims, W, emb, start, n, K=3, p=0.6, seed=3)
    assert spec == greedy[1:]
    assert steps < n          # drafts were actually accepted


def test_lossless_pin_catches_commit_past_first_mismatch():
    """Planted mistake (in the oracle's accept rule, on the CPU): committing
    the decoder's token one position past the first rejected draft uses a
    choice made on a wrong input, which breaks equality with greedy decoding."""
    def one_too_many(g, d):
        B, K = d.shape
        n_acc, _, _ = O.spec_accept(g, d)
        n_acc = np.minimum(n_acc + (n_acc < K), K)
        committed = np.full((B, K + 1), -1)
        for b in range(B):
            committed[b, :n_acc[b] + 1] = g[b, :n_acc[b] + 1]
        return n_acc, committed, n_acc + 1

    dims = synth.TINY_F32
    W = synth.make_weights(dims, seed=0)
    emb = synth.make_embedding(dims, seed=0)
    table = _greedy_table(dims, W, emb)
    greedy = [17]
    for _ in range(60):
        greedy.append(int(table[greedy[-1]]))
    spec, _ = _spec_decode(dims, W, emb, 17, 60, K=3, p=0.6, seed=3, accept=one_too_many)
    assert spec != greedy[1:]


# ---------------------------------------------------------------- the layer stack


def _stack_weights(dtype="f32", layers=3, seed=11):
    import dataclasses

    dims = dataclasses.replace(synth.TINY_F32, n_layers=layers, dtype=dtype)
    return dims, synth.make_weights(dims, seed=seed, gamma="uniform")


def test_stack_with_zero_down_projections_is_the_identity():
    """Every expert's down projection zero in every layer: each layer adds an
    exact zero, so the stack returns its input bit for bit (a loop that
    carried x, or anything but h, from layer to layer would not)."""
    for dtype in ("f32", "bf16"):
        dims, W = _stack_weights(dtype)
        W["w_down"][...] = 0
        W["ws_down"][...] = 0
        h = synth.make_hidden(dims, 7, seed=12)
        out = O.forward_tokens(h, W, dims, lm_head=False)
        assert np.array_equal(out["h_out"], O.widen(h, dtype))
        assert len(out["layers"]) == dims.n_layers


def _one_hot_chain(dims, W, e_star):
    """Router bias +1e4 on expert e_star[l] and -1e4 elsewhere in layer l."""
    b = np.full((dims.n_layers, dims.n_routed), -1e4, np.float32)
    for layer, e in enumerate(e_star):
        b[layer, e] = 1e4
    W = dict(W)
    W["router_b"] = b
    return W


def _torch_chain(dims, W, h, e_star):
    """h <- h + FFN_{e*_l}(x) + FFN_shared0(x) + FFN_shared1(x), x = RMSNorm(h) * gamma_l,
    layer by layer, in float64 torch with no intermediate rounding."""
    wid = lambda a: O.widen(a, dims.dtype)
    ht = torch.from_numpy(O.widen(h, dims.dtype))
    for layer, e in enumerate(e_star):
        g = torch.from_numpy(wid(W["ffn_norm"][layer]))
        x = torch.nn.functional.rms_norm(ht, (dims.d_model,), g, eps=dims.rms_eps).numpy()
        y = _torch_ffn(x, wid(W["w_gate_up"][layer, e]), wid(W["w_down"][layer, e]))
        for s in range(dims.n_shared):
            y = y + _torch_ffn(x, wid(W["ws_gate_up"][layer, s]), wid(W["ws_down"][layer, s]))
        ht = ht + torch.from_numpy(y)
    return ht.numpy()


E_STAR = (37, 5, 62)


def _chain_agrees(forward=O.forward_tokens):
    dims, W = _stack_weights("f32")
    W = _one_hot_chain(dims, W, E_STAR)
    h = synth.make_hidden(dims, 6, seed=13)
    out = forward(h, W, dims, lm_head=False)
    ids_ok = all(np.all(out["layers"][layer]["ids"][:, 0] == e) for layer, e in enumerate(E_STAR))
    ref = _torch_chain(dims, W, h, E_STAR)
    err = np.abs(out["h_out"] - ref).max(axis=1) / np.abs(ref).max(axis=1)
    # fp32 storage of x, a and h in three layers against float64 without rounding
    return ids_ok and bool(np.all(err < 1e-5)), float(err.max())


def test_stack_with_one_hot_routers_chains_the_dense_ffns():
    """Per-layer one-hot router biases with a different expert in every layer:
    the stack is the chain of those experts' dense SwiGLU FFNs plus the shared
    ones, each behind its own layer's RMSNorm, compared with torch."""
    ok, err = _chain_agrees()
    assert ok, err


def test_chain_pin_catches_a_wrong_layer_index(monkeypatch):
    """Planted mistake (in the oracle, on the CPU): every layer of the stack
    reads layer 0's weights.  The chain pin fails."""
    real = O.moe_layer
    monkeypatch.setattr(O, "moe_layer", lambda h, W, layer, dims, ftype=np.float64: real(h, W, 0, dims, ftype))
    ok, _ = _chain_agrees()
    assert not ok


def test_chain_pin_catches_x_carried_forward(monkeypatch):
    """Planted mistake: the loop carries the normalised input x to the next
    layer instead of h_out.  The chain and identity pins both fail."""
    real = O.moe_layer

    def carries_x(h, W, layer, dims, ftype=np.float64):
        r = dict(real(h, W, layer, dims, ftype))
        r["h_out"] = r["x"]
        return r

    monkeypatch.setattr(O, "moe_layer", carries_x)
    ok, _ = _chain_agrees()
    assert not ok
    dims, W = _stack_weights("f32")
    W["w_down"][...] = 0
    W["ws_down"][...] = 0
    h = synth.make_hidden(dims, 3, seed=12)
    assert not np.array_equal(O.forward_tokens(h, W, dims, lm_head=False)["h_out"], O.widen(h, "f32"))


def test_float32_working_precision_tracks_float64_on_one_layer():
    """The same algorithm at float32 working precision (the precision of a
    plain fp32 CPU implementation) stays within fp32 accumulation error of the
    float64 run: the two differ only in rounding, not in arithmetic."""
    dims, W = _stack_weights("f32", layers=1)
    h = O.widen(synth.make_hidden(dims, 16, seed=14), "f32")
    r64 = O.moe_layer(h, W, 0, dims)
    r32 = O.moe_layer(h, W, 0, dims, ftype=np.float32)
    same = np.all(np.sort(r64["ids"], 1) == np.sort(r32["ids"], 1), axis=1)
    assert same.mean() >= 0.9
    err = np.abs(r32["y"] - r64["y"]).max(axis=1) / np.abs(r64["y"]).max(axis=1)
    assert np.all(err[same] < 1e-5), err[same].max()


def test_lossless_on_a_three_layer_model():
    """Losslessness (the accept rule commits exactly the greedy tokens) on a
    stack of three layers, so the loop over layers is part of both sides."""
    dims, W = _stack_weights("f32", layers=3, seed=0)
    emb = synth.make_embedding(dims, seed=0)
    table = _greedy_table(dims, W, emb)
    start, n = 29, 120
    greedy = [start]
    for _ in range(n):
        greedy.append(int(table[greedy[-1]]))
    spec, steps = _spec_decode(dims, W, emb, start, n, K=3, p=0.6, seed=5)
    assert spec == greedy[1:]
    assert steps < n
