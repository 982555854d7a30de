"""GPU path (through the C ABI) against the CPU oracle on the same seeded
inputs.  Rules in tests/parity.py."""
import itertools

import numpy as np
import pytest

from oracle import moe_oracle as O
from parity import TOL, Tally, forced_stack, stack_conditioning
from speculative_decode_verification_router_amd import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_cuda(gpu_lib):
    import torch

    return torch


@pytest.fixture(scope="module")
def bd(gpu_lib):
    from speculative_decode_verification_router_amd import binding

    return binding


_MODELS = []  # every DeviceModel of this module, for the status check after each test


def _model(bd, dims, W, max_tokens):
    m = bd.DeviceModel(dims, W, max_tokens=max_tokens)
    m.ws[:256].zero_()  # a status word no call has written yet reads 0
    _MODELS.append(m)
    return m


@pytest.fixture(autouse=True)
def _calls_completed(request):
    """After every test: the last call on each workspace ended every bounded
    wait of its fused launches as it should (mv_step_status = 0)."""
    yield
    if "bd" not in request.fixturenames:
        return
    from speculative_decode_verification_router_amd import binding

    for m in _MODELS:
        assert binding.step_status(m) == 0, "a fused launch's wait gave up"


@pytest.fixture(scope="module")
def tiny(bd):
    dims = synth.TINY_F32
    W = synth.make_weights(dims, seed=0, gamma="uniform")
    return dims, W, _model(bd, dims, W, 512)


@pytest.fixture(scope="module")
def big(bd):
    dims = synth.DS3B_BF16
    W = synth.make_weights(dims, seed=0, sigma=0.02)
    return dims, W, _model(bd, dims, W, 10048)


@pytest.fixture(scope="module")
def tiny3(bd):
    """The tiny fp32 model with three layers: an odd layer count, so the first
    combine of a verify step with h_out aliasing h_in would land on h_in."""
    import dataclasses

    dims = dataclasses.replace(synth.TINY_F32, n_layers=3)
    W = synth.make_weights(dims, seed=4, gamma="uniform")
    return dims, W, _model(bd, dims, W, 64)


# Other model shapes the library takes: fewer routed experts (the routing's
# expert groups, the top-k lanes and the tile search past E), no shared
# expert and one to four of them, top-k from 1 (a gate of exactly 1) to 8,
# several layers.  odd16g fits the large-batch GEMM path (d % 256 == 0,
# d_ff % 128 == 0, at most 2 shared).
ODD_F32 = synth.ModelDims(128, 64, 20, 1, 4, 3, 300, 1e-6, "f32")
ODD_BF16 = synth.ModelDims(256, 192, 40, 3, 8, 2, 5000, 1e-6, "bf16")
ODD_BF16_GEMM = synth.ModelDims(256, 256, 24, 2, 5, 2, 3000, 1e-6, "bf16")
ODD_NO_SHARED = synth.ModelDims(128, 128, 16, 0, 1, 2, 400, 1e-6, "f32")
ODD_FOUR_SHARED = synth.ModelDims(256, 128, 32, 4, 2, 2, 2000, 1e-6, "bf16")


@pytest.fixture(scope="module")
def odd(bd):
    out = {}
    for name, dims, sigma in (("odd32", ODD_F32, None), ("odd16", ODD_BF16, 0.05), ("odd16g", ODD_BF16_GEMM, 0.05),
                              ("s0k1", ODD_NO_SHARED, None), ("s4k2", ODD_FOUR_SHARED, 0.05)):
        W = synth.make_weights(dims, seed=11, sigma=sigma, gamma="uniform")
        out[name] = (dims, W, _model(bd, dims, W, 700))
    return out


def _dev(bd, a):
    return bd.to_device(a)


def _host(bd, t):
    return bd.to_host(t)


def _sync(torch):
    torch.cuda.synchronize()


# ---------------------------------------------------------------- accept


@pytest.mark.parametrize("K", [0, 1, 2, 3])
def test_spec_accept_exhaustive(bd, torch_cuda, K):
    gs = np.array(list(itertools.product(range(3), repeat=K + 1)), np.int32)
    if K:
        ds = np.array(list(itertools.product(range(3), repeat=K)), np.int32)
        G, D = np.repeat(gs, len(ds), axis=0), np.tile(ds, (len(gs), 1))
    else:
        G, D = gs, np.zeros((len(gs), 0), np.int32)
    B = len(G)
    g_t, d_t = _dev(bd, G), (_dev(bd, D) if K else None)
    n_acc = torch_cuda.empty(B, dtype=torch_cuda.int32, device="cuda")
    com = torch_cuda.empty((B, K + 1), dtype=torch_cuda.int32, device="cuda")
    n_com = torch_cuda.empty(B, dtype=torch_cuda.int32, device="cuda")
    bd.spec_accept(B, K, g_t, d_t, n_acc, com, n_com)
    _sync(torch_cuda)
    r_acc, r_com, r_ncom = O.spec_accept(G, D)
    assert np.array_equal(_host(bd, n_acc), r_acc)
    assert np.array_equal(_host(bd, com), r_com)
    assert np.array_equal(_host(bd, n_com), r_ncom)


def test_spec_accept_out_of_range_drafts_never_match(bd, torch_cuda):
    G = np.array([[5, 6, 7, 8]], np.int32)
    D = np.array([[5, -1, 7]], np.int32)
    n_acc = torch_cuda.empty(1, dtype=torch_cuda.int32, device="cuda")
    com = torch_cuda.empty((1, 4), dtype=torch_cuda.int32, device="cuda")
    n_com = torch_cuda.empty(1, dtype=torch_cuda.int32, device="cuda")
    bd.spec_accept(1, 3, _dev(bd, G), _dev(bd, D), n_acc, com, n_com)
    _sync(torch_cuda)
    assert _host(bd, n_acc).tolist() == [1]
    assert _host(bd, com).tolist() == [[5, 6, -1, -1]]


# ---------------------------------------------------------------- one layer


def _layer_check(bd, torch, dims, W, model, layer, h, label):
    out = bd.run_layer_forward(model, layer, _dev(bd, h))
    _sync(torch)
    ref = O.moe_layer(O.widen(h, dims.dtype), W, layer, dims)
    tally = Tally(h.shape[0], forced=True)  # one layer: both sides take the same input
    tally.routing(layer, _host(bd, out["topk_ids"]), ref["ids"], ref["margin"])
    # gates of tokens whose routing matched: same experts in the same order
    live = ~tally.excluded
    gw = _host(bd, out["topk_w"]).astype(np.float64)
    gid = _host(bd, out["topk_ids"])
    same_order = np.all(gid == ref["ids"], axis=1) & live
    if same_order.any():
        # x is rounded to bf16 from fp32 on the GPU and from fp64 in the
        # oracle; an element within fp32 noise of a rounding boundary lands
        # one ulp apart (up to 2^-5 for |x| < 8), moving a logit by at most
        # ulp * max|W_r| and a gate by at most twice that, relatively.  Such
        # tokens are rare; every other gate must agree to 1e-4.
        rel = np.abs(gw[same_order] - ref["gates"][same_order]) / ref["gates"][same_order]
        flip_tol = 2 * 2.0 ** -5 * float(np.abs(O.widen(W["router_w"][layer], dims.dtype)).max())
        loose = np.any(rel > 1e-4, axis=1)
        assert loose.sum() <= max(2, 0.01 * same_order.sum()), (label, int(loose.sum()))
        assert rel.max() <= max(1e-4, flip_tol), (label, float(rel.max()), flip_tol)
    tol = TOL[dims.dtype]
    e_y = tally.rows(f"{label} y_moe", _host(bd, out["y_moe"]), ref["y"], tol)
    e_h = tally.rows(f"{label} h_out", O.widen(_host(bd, out["h_out"]), dims.dtype),
                     ref["h_out"], tol)
    print(f"{label}: max rel err y {e_y:.3g} h {e_h:.3g}")
    tally.assert_ok(label)
    return out


@pytest.mark.parametrize("T", [1, 5, 16, 37, 64, 65, 130])
def test_layer_forward_tiny_fp32(bd, torch_cuda, tiny, T):
    dims, W, model = tiny
    h = synth.make_hidden(dims, T, seed=100 + T)
    _layer_check(bd, torch_cuda, dims, W, model, 0, h, f"tiny T={T}")


@pytest.mark.timeout(600)
@pytest.mark.parametrize("model_name,layer", [("tiny", 0), ("big", 6)])
def test_layer_forward_maximum_batch(bd, torch_cuda, tiny, big, model_name, layer):
    """The largest batch the library takes, 65,535 rows, through one layer:
    at full width the GEMM path with a ragged last tile (65,535 = 255 x 256 +
    255) after the large-batch routing and counting-sort grouping; in fp32 the
    64-row tiles.  256 sampled rows (the first and the last among them)
    against the oracle, single-layer near-tie rule."""
    torch = torch_cuda
    dims, W, model = {"tiny": tiny, "big": big}[model_name]
    T = 65535
    ws_bytes = bd.mv_workspace_bytes(model.cfg, T)
    ws = torch.zeros(ws_bytes, dtype=torch.uint8, device="cuda")
    h = synth.make_hidden(dims, T, seed=65535)
    ht = _dev(bd, h)
    out = {"h_out": torch.empty_like(ht),
           "topk_ids": torch.empty((T, dims.top_k), dtype=torch.int32, device="cuda"),
           "topk_w": torch.empty((T, dims.top_k), dtype=torch.float32, device="cuda"),
           "y_moe": torch.empty((T, dims.d_model), dtype=torch.float32, device="cuda")}
    bd.moe_layer_forward(model.cfg, model.weights, layer, T, ht, out["h_out"], out["topk_ids"], out["topk_w"],
                         out["y_moe"], ws, ws_bytes)
    _sync(torch)
    sample = np.sort(np.random.default_rng(7).choice(np.arange(1, T - 1), 254, replace=False))
    sample = np.concatenate([[0], sample, [T - 1]])
    ref = O.moe_layer(O.widen(h[sample], dims.dtype), W, layer, dims)
    tally = Tally(len(sample), forced=True)
    tally.routing(layer, _host(bd, out["topk_ids"])[sample], ref["ids"], ref["margin"])
    tol = TOL[dims.dtype]
    tally.rows(f"max batch {model_name} y_moe", _host(bd, out["y_moe"])[sample], ref["y"], tol)
    tally.rows(f"max batch {model_name} h_out", O.widen(_host(bd, out["h_out"]), dims.dtype)[sample],
               ref["h_out"], tol)
    tally.assert_ok(f"{model_name}: 65,535 rows, 256 sampled")
    del ws


# 128 / 129 and 512 / 513 sit on either side of a batch-path switch (16-row
# tiles, 64-row tiles, 256-row GEMM tiles); 513 leaves the GEMM a one-row tile.
@pytest.mark.parametrize("T,layer", [(4, 0), (37, 11), (128, 5), (129, 2), (200, 3), (512, 4), (513, 9),
                                     (600, 7)])
def test_layer_forward_bf16_full_width(bd, torch_cuda, big, T, layer):
    dims, W, model = big
    h = synth.make_hidden(dims, T, seed=200 + T)
    _layer_check(bd, torch_cuda, dims, W, model, layer, h, f"bf16 T={T} layer={layer}")


def test_layer_forward_in_place(bd, torch_cuda, tiny):
    dims, W, model = tiny
    h = synth.make_hidden(dims, 21, seed=7)
    ref = bd.run_layer_forward(model, 0, _dev(bd, h))
    ht = _dev(bd, h)
    bd.moe_layer_forward(model.cfg, model.weights, 0, 21, ht, ht, None, None, None, model.ws,
                         model.ws_bytes)
    _sync(torch_cuda)
    assert np.array_equal(_host(bd, ht), _host(bd, ref["h_out"]))


# ---------------------------------------------------------------- verify step


def _verify_check(bd, torch, dims, W, model, h, B, K, match_p, seed, label, rows=None):
    """GPU verify on all B sequences; oracle on the sequences in `rows`
    (default all), drafts built from the oracle's argmax."""
    seqs = np.arange(B) if rows is None else np.asarray(rows)
    T = B * (K + 1)
    tok = (seqs[:, None] * (K + 1) + np.arange(K + 1)[None, :]).reshape(-1)
    ref = O.forward_tokens(h[tok], W, dims, keep_logits=True)
    ref32 = O.forward_tokens(h[tok], W, dims, ftype=np.float32, keep_logits=True)
    cond_layers, cond_final = stack_conditioning(ref, ref32)
    g_ref_sub = np.asarray(ref["argmax"]).reshape(len(seqs), K + 1)
    # drafts for every sequence: oracle argmax where computed, else a draw
    g_full = np.zeros((B, K + 1), np.int64)
    g_full[seqs] = g_ref_sub
    drafts = synth.make_drafts(g_full, match_p, dims.vocab, seed=seed)
    out = bd.run_verify_step(model, _dev(bd, h), _dev(bd, drafts), B, K, routing=True)
    _sync(torch)
    r_acc, r_com, r_ncom = O.spec_accept(g_ref_sub, drafts[seqs])

    tally = Tally(len(tok))
    ids = _host(bd, out["topk_ids"])
    for layer in range(dims.n_layers):
        lr = ref["layers"][layer]
        thr, ill = cond_layers[layer]
        tally.routing(layer, ids[layer][tok], lr["ids"], lr["margin"], thr, ill)
    tol = TOL[dims.dtype]
    e_h = tally.rows(f"{label} h_out", O.widen(_host(bd, out["h_out"]), dims.dtype)[tok],
                     ref["h_out"], tol)
    tally.argmax(_host(bd, out["argmax"])[tok], ref["argmax"], ref["margin"], *cond_final)
    gpu_c = {k: _host(bd, out[k])[seqs] for k in ("n_accepted", "committed", "n_committed")}
    n_seq_checked = tally.commits(len(seqs), K, gpu_c,
                                  dict(n_accepted=r_acc, committed=r_com, n_committed=r_ncom))
    print(f"{label}: h rel err {e_h:.3g}; sequences checked {n_seq_checked}/{len(seqs)}; "
          f"committed/step {np.mean(_host(bd, out['n_committed'])):.3f}")
    tally.assert_ok(label)
    return out, tally


def test_verify_tiny_fp32(bd, torch_cuda, tiny):
    dims, W, model = tiny
    wl = synth.WORKLOADS["tiny_f32_b4_k3"]
    h = synth.workload_hidden(wl)
    _verify_check(bd, torch_cuda, dims, W, model, h, wl.batch, wl.k_draft, wl.match_p, 0,
                  "tiny verify")


@pytest.mark.parametrize("B", [1, 2, 4])
def test_verify_three_layers_in_place(bd, torch_cuda, tiny3, B):
    """Three layers against the oracle; then the same step with h_out aliasing
    h_in (the combines keep reading a buffer other than the one they write)
    gives bit-identical results.  B = 1, 2 route to logits with the fused
    expert launch, B = 4 the separate launches."""
    dims, W, model = tiny3
    K = 3
    T = B * (K + 1)
    h = synth.make_hidden(dims, T, seed=13)
    _verify_check(bd, torch_cuda, dims, W, model, h, B, K, 0.6, 5, f"3-layer B={B}")
    drafts = _dev(bd, np.random.default_rng(3).integers(0, dims.vocab, (B, K)).astype(np.int32))
    ref = bd.run_verify_step(model, _dev(bd, h), drafts, B, K, routing=True)
    torch = torch_cuda
    ht = _dev(bd, h)
    out = {key: torch.empty_like(ref[key])
           for key in ("argmax", "n_accepted", "committed", "n_committed", "topk_ids")}
    bd.moe_verify_step(model.cfg, model.weights, B, K, ht, drafts, ht, out["argmax"], out["n_accepted"],
                       out["committed"], out["n_committed"], out["topk_ids"], model.ws, model.ws_bytes)
    _sync(torch)
    assert np.array_equal(_host(bd, ht), _host(bd, ref["h_out"]))
    for key in out:
        assert np.array_equal(_host(bd, out[key]), _host(bd, ref[key])), key


@pytest.mark.parametrize("B,K", [(1, 0), (3, 1), (7, 3), (5, 15)])
def test_verify_tiny_shapes(bd, torch_cuda, tiny, B, K):
    dims, W, model = tiny
    h = synth.make_hidden(dims, B * (K + 1), seed=300 + B * 17 + K)
    _verify_check(bd, torch_cuda, dims, W, model, h, B, K, 0.7, 5, f"tiny verify B={B} K={K}")


def _forced_check(bd, torch, dims, W, model, h, B, K, match_p, seed, label, seqs=None, min_checked=None):
    """Teacher-forced parity of a full-width verify step on the sequences in
    `seqs` (default all).  The step runs once with placeholder drafts (its
    routing, hidden state and argmax do not depend on the drafts), and the
    chain of moe_layer_forward calls must reproduce its routing and final
    hidden state bit for bit.  Every layer is then checked on the GPU's own
    input to it: the oracle's layer fed that input must route like the GPU
    (single-layer near-tie rule, margin 1e-3) and agree on the output rows
    (2e-2), and the oracle's LM head on the GPU's final hidden state must give
    the GPU's argmax.  Drafts for the checked sequences come from that oracle
    argmax with probability match_p (the others are random); the step is run
    again with them, and its commits must be the oracle's accept rule on the
    oracle's argmax.  A token with a near-tie is dropped from later checks,
    and at least a fraction min_checked of the tokens must be checked to the
    end (Tally.assert_ok)."""
    seqs = np.arange(B) if seqs is None else np.asarray(seqs)
    rows = (seqs[:, None] * (K + 1) + np.arange(K + 1)[None, :]).reshape(-1)
    hd = _dev(bd, h)
    pre = bd.run_verify_step(model, hd, _dev(bd, np.zeros((B, K), np.int32)), B, K, routing=True)
    _sync(torch)
    assert bd.step_status(model) == 0
    g_gpu, h_step = _host(bd, pre["argmax"]), _host(bd, pre["h_out"])
    tally, h_fin, lm = forced_stack(bd, torch, dims, W, model, hd, rows, label, ids_expect=_host(bd, pre["topk_ids"]))
    assert np.array_equal(h_fin, h_step), f"{label}: chain and step end in different states"
    tally.argmax(g_gpu[rows], lm["argmax"], lm["margin"])
    g_ref = np.asarray(lm["argmax"]).reshape(len(seqs), K + 1)
    g_full = np.zeros((B, K + 1), np.int64)
    g_full[seqs] = g_ref
    drafts = synth.make_drafts(g_full, match_p, dims.vocab, seed=seed)
    out = bd.run_verify_step(model, hd, _dev(bd, drafts), B, K)
    _sync(torch)
    assert np.array_equal(_host(bd, out["argmax"]), g_gpu) and np.array_equal(_host(bd, out["h_out"]), h_step)
    r_acc, r_com, r_ncom = O.spec_accept(g_ref, drafts[seqs])
    gpu_c = {k: _host(bd, out[k])[seqs] for k in ("n_accepted", "committed", "n_committed")}
    n_seq = tally.commits(len(seqs), K, gpu_c, dict(n_accepted=r_acc, committed=r_com, n_committed=r_ncom))
    print(f"{label}: sequences with commits checked {n_seq}/{len(seqs)}; "
          f"committed/step {np.mean(_host(bd, out['n_committed'])):.3f}")
    tally.assert_ok(label, min_checked)
    assert n_seq >= 0.75 * len(seqs), f"{label}: commits checked on only {n_seq}/{len(seqs)} sequences"
    return tally


@pytest.mark.timeout(600)
def test_verify_b1_k3_full_size(bd, torch_cuda, big):
    """The headline workload (one sequence, three drafts, full width), and the
    same shape on three more hidden states: 16 rows in all."""
    dims, W, model = big
    wl = synth.WORKLOADS["b1_k3"]
    hs = [synth.workload_hidden(wl)] + [synth.make_hidden(dims, 4, seed=s) for s in (101, 102, 103)]
    tallies = [_forced_check(bd, torch_cuda, dims, W, model, h, 1, 3, wl.match_p, i, f"b1_k3 #{i}", min_checked=0.5)
               for i, h in enumerate(hs)]
    checked = sum(t.checked for t in tallies)
    assert checked >= 0.75 * 16, f"b1_k3: {checked}/16 tokens checked"


@pytest.mark.timeout(600)
def test_verify_c32_k3_sampled(bd, torch_cuda, big):
    """32 sequences x 4 rows (16-row tiles); the oracle checks 16 sequences."""
    dims, W, model = big
    wl = synth.WORKLOADS["c32_k3"]
    _forced_check(bd, torch_cuda, dims, W, model, synth.workload_hidden(wl), wl.batch, wl.k_draft, wl.match_p, 0,
                  "c32_k3", seqs=np.arange(0, 32, 2))


@pytest.mark.timeout(600)
@pytest.mark.parametrize("B,K,seqs", [(2, 1, None), (4, 1, None), (64, 1, [0, 1, 31, 32, 62, 63]),
                                      (8, 3, [0, 3, 7])])
def test_verify_teacher_forced(bd, torch_cuda, big, B, K, seqs):
    """Full width at one or three drafts per sequence: up to 8 rows (the fused
    expert launch), 128 rows (16-row tiles), 32 rows (two 16-row tiles)."""
    dims, W, model = big
    T = B * (K + 1)
    h0 = synth.make_hidden(dims, T, seed=700 + B + 10 * K)
    _forced_check(bd, torch_cuda, dims, W, model, h0, B, K, 0.6, 4, f"verify B={B} K={K}", seqs=seqs)


@pytest.mark.timeout(600)
def test_verify_large_batch_sampled(bd, torch_cuda, big):
    """150 sequences x 4 rows: the LDS-tiled GEMM path with the combine in
    the shared experts' down projection; the oracle checks 10 sequences."""
    dims, W, model = big
    B, K = 150, 3
    h = synth.make_hidden(dims, B * (K + 1), seed=600)
    _forced_check(bd, torch_cuda, dims, W, model, h, B, K, 0.6, 3, "verify B=150 K=3",
                  seqs=[0, 1, 37, 74, 75, 111, 112, 140, 148, 149])


@pytest.mark.timeout(900)
def test_prefill_stack_sampled(bd, torch_cuda, big):
    """10,048 tokens through the 12 layers (moe_layer_forward chained on the
    GPU, the GEMM path); each layer is checked on the GPU's own input to it
    on 512 sampled rows (single-layer near-tie rule)."""
    dims, W, model = big
    wl = synth.WORKLOADS["prefill_10048"]
    h = synth.workload_hidden(wl)
    T = h.shape[0]
    sample = np.sort(np.random.default_rng(0).choice(np.arange(1, T - 1), 510, replace=False))
    sample = np.concatenate([[0], sample, [T - 1]])
    ht = _dev(bd, h)
    forced = Tally(len(sample), forced=True)
    for layer in range(dims.n_layers):
        h_in = O.widen(_host(bd, ht), "bf16")[sample]
        out = bd.run_layer_forward(model, layer, ht)
        _sync(torch_cuda)
        ht = out["h_out"]
        ref_l = O.moe_layer(h_in, W, layer, dims)
        forced.routing(layer, _host(bd, out["topk_ids"])[sample], ref_l["ids"], ref_l["margin"])
        forced.rows(f"prefill layer {layer}", O.widen(_host(bd, ht), "bf16")[sample], ref_l["h_out"], TOL["bf16"])
    forced.assert_ok("prefill 10,048 rows, 512 sampled, teacher-forced")


@pytest.mark.timeout(600)
def test_router_bias_zipf(bd, torch_cuda, big):
    """Zipf-skewed routing (the decode-loop workload's router bias): 8 sequences."""
    dims, W, model = big
    wl = synth.WORKLOADS["zipf_loop_c32"]
    Wz = dict(W)
    Wz["router_b"] = synth.make_router_bias(dims.n_layers, dims.n_routed, wl.zipf_s)
    modelz = model.with_router_bias(Wz["router_b"])
    h = synth.make_hidden(dims, 8 * 4, seed=55)
    _forced_check(bd, torch_cuda, dims, Wz, modelz, h, 8, 3, 0.6, 9, "zipf bias verify")


# ---------------------------------------------------------------- other shapes


@pytest.mark.parametrize("name,T", [("odd32", 4), ("odd32", 100), ("odd32", 300), ("odd16", 4), ("odd16", 100),
                                    ("odd16", 300), ("odd16g", 600), ("s0k1", 4), ("s0k1", 100), ("s0k1", 600),
                                    ("s4k2", 4), ("s4k2", 100), ("s4k2", 600)])
def test_layer_forward_other_shapes(bd, torch_cuda, odd, name, T):
    """One layer of each odd shape on the 16-row, 64-row and (odd16g, 600
    rows) GEMM paths against the oracle."""
    dims, W, model = odd[name]
    h = synth.make_hidden(dims, T, seed=500 + T)
    _layer_check(bd, torch_cuda, dims, W, model, dims.n_layers - 1, h, f"{name} T={T}")


@pytest.mark.parametrize("name,B", [("odd32", 1), ("odd32", 2), ("odd32", 8), ("odd32", 40), ("odd16", 1),
                                    ("odd16", 2), ("odd16", 8), ("odd16", 40), ("s0k1", 1), ("s0k1", 2),
                                    ("s0k1", 8), ("s0k1", 40), ("s4k2", 1), ("s4k2", 2), ("s4k2", 8), ("s4k2", 40)])
def test_verify_other_shapes(bd, torch_cuda, odd, name, B):
    """Verify steps of the odd shapes (B = 1, 2: routing inside the fused
    launch; 8: 16-row tiles; 40: 64-row tiles) against the oracle."""
    dims, W, model = odd[name]
    K = 3
    h = synth.make_hidden(dims, B * (K + 1), seed=600 + B)
    _verify_check(bd, torch_cuda, dims, W, model, h, B, K, 0.6, 7, f"{name} verify B={B}")


@pytest.mark.parametrize("name", ["odd32", "odd16", "s0k1", "s4k2"])
def test_other_shapes_same_results_on_every_batch_path(bd, torch_cuda, odd, name):
    """The batch-path invariance on the odd shapes, and the one-launch step
    bit-identical to the launches at B = 1, 2."""
    dims, W, model = odd[name]
    K = 3
    n_seq = 34
    h = synth.make_hidden(dims, n_seq * (K + 1), seed=92)
    drafts = np.random.default_rng(5).integers(0, dims.vocab, (n_seq, K)).astype(np.int32)
    batches = (1, 2, 4, 16, 34)
    runs = {B: bd.run_verify_step(model, _dev(bd, h[:B * (K + 1)]), _dev(bd, drafts[:B]), B, K, routing=True)
            for B in batches}
    ones = {B: bd.run_verify_step(model, _dev(bd, h[:B * (K + 1)]), _dev(bd, drafts[:B]), B, K, routing=True,
                                  one_launch=True)
            for B in (1, 2)}
    _sync(torch_cuda)
    ref = runs[batches[-1]]
    for B in batches[:-1]:
        run, T = runs[B], B * (K + 1)
        for key in ("h_out", "argmax", "committed", "n_committed"):
            n = B if key in ("committed", "n_committed") else T
            assert np.array_equal(_host(bd, run[key])[:n], _host(bd, ref[key])[:n]), (B, key)
        assert np.array_equal(_host(bd, run["topk_ids"]), _host(bd, ref["topk_ids"])[:, :T]), B
    for B, one in ones.items():
        for key in ("h_out", "argmax", "committed", "n_committed", "topk_ids"):
            assert np.array_equal(_host(bd, one[key]), _host(bd, runs[B][key])), ("one launch", B, key)


# ---------------------------------------------------------------- invariants


def test_deterministic_and_batch_invariant(bd, torch_cuda, big):
    dims, W, model = big
    B, K = 6, 3
    h = synth.make_hidden(dims, B * (K + 1), seed=77)
    drafts = np.random.default_rng(1).integers(0, dims.vocab, (B, K)).astype(np.int32)
    a = bd.run_verify_step(model, _dev(bd, h), _dev(bd, drafts), B, K, routing=True)
    b = bd.run_verify_step(model, _dev(bd, h), _dev(bd, drafts), B, K, routing=True)
    sub = [4, 1]
    rows = np.concatenate([np.arange(s * (K + 1), (s + 1) * (K + 1)) for s in sub])
    c = bd.run_verify_step(model, _dev(bd, h[rows]), _dev(bd, drafts[sub]), len(sub), K, routing=True)
    _sync(torch_cuda)
    for key in ("h_out", "argmax", "committed", "n_committed", "topk_ids"):
        assert np.array_equal(_host(bd, a[key]), _host(bd, b[key])), key
    assert np.array_equal(_host(bd, a["h_out"])[rows], _host(bd, c["h_out"]))
    assert np.array_equal(_host(bd, a["argmax"])[rows], _host(bd, c["argmax"]))
    assert np.array_equal(_host(bd, a["topk_ids"])[:, rows], _host(bd, c["topk_ids"]))


@pytest.mark.parametrize("model_name", ["tiny", "big"])
def test_same_results_on_every_batch_path(bd, torch_cuda, tiny, big, model_name):
    """Batches of up to 8 rows route in expert groups and take the top-k in
    the fused expert launch, up to 128 rows group the pairs inside the gate/up
    blocks, and larger batches use 64-row expert tiles after a grouping
    kernel.  All paths do the same per-row arithmetic in the same order, so a
    sequence's results are bit-identical whichever path its batch takes."""
    dims, W, model = tiny if model_name == "tiny" else big
    K = 3
    n_seq = 33
    h = synth.make_hidden(dims, n_seq * (K + 1), seed=91)
    drafts = np.random.default_rng(2).integers(0, dims.vocab, (n_seq, K)).astype(np.int32)
    batches = (1, 2, 4, 16, 17, 33)
    runs = {B: bd.run_verify_step(model, _dev(bd, h[:B * (K + 1)]), _dev(bd, drafts[:B]), B, K,
                                  routing=True)
            for B in batches}
    _sync(torch_cuda)
    ref = runs[batches[-1]]
    for B in batches[:-1]:
        run, T = runs[B], B * (K + 1)
        for key in ("h_out", "argmax", "committed", "n_committed"):
            n = B if key in ("committed", "n_committed") else T
            assert np.array_equal(_host(bd, run[key])[:n], _host(bd, ref[key])[:n]), (B, key)
        assert np.array_equal(_host(bd, run["topk_ids"]), _host(bd, ref["topk_ids"])[:, :T]), B


def test_lossless_gpu_decode_loop(bd, torch_cuda, tiny):
    """Spec-decode loop on the GPU (drafts right with p = 0.6) commits exactly
    the oracle's plain greedy continuation."""
    dims, W, model = tiny
    emb = synth.make_embedding(dims, seed=0)
    table_ref = O.forward_tokens(emb, W, dims)
    table, margin = np.asarray(table_ref["argmax"]), np.asarray(table_ref["margin"])
    start, n, K = 17, 120, 3
    greedy = [start]
    for _ in range(n):
        greedy.append(int(table[greedy[-1]]))
    if np.any(margin[greedy] < 1e-3):
        pytest.skip("near-tie on the greedy path; exact comparison not defined")
    seq, c, step = [], start, 0
    while len(seq) < n:
        truth = [c]
        for _ in range(K):
            truth.append(int(table[truth[-1]]))
        drafts = synth.make_drafts(np.array([truth[1:] + [0]]), 0.6, dims.vocab, seed=4, step=step)
        h = np.stack([emb[c]] + [emb[int(t)] for t in drafts[0]])
        out = bd.run_verify_step(model, _dev(bd, h), _dev(bd, drafts), 1, K)
        _sync(torch_cuda)
        k = int(_host(bd, out["n_committed"])[0])
        seq.extend(int(t) for t in _host(bd, out["committed"])[0, :k])
        c = seq[-1]
        step += 1
    assert seq[:n] == greedy[1:]
    assert step < n


@pytest.mark.parametrize("B,K", [(1, 3), (8, 3)])
def test_verify_step_in_a_graph(bd, torch_cuda, big, B, K):
    """The verify step captured in a HIP graph: every replay, with eager
    work on the stream between replays, equals the eager step bit for bit."""
    torch = torch_cuda
    dims, W, model = big
    h = _dev(bd, synth.make_hidden(dims, B * (K + 1), seed=810 + B))
    drafts = _dev(bd, np.random.default_rng(B).integers(0, dims.vocab, (B, K)).astype(np.int32))
    ref = bd.run_verify_step(model, h, drafts, B, K)
    _sync(torch)
    ref = {k: _host(bd, v) for k, v in ref.items() if v is not None}
    out = bd.run_verify_step(model, h, drafts, B, K)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        bd.moe_verify_step(model.cfg, model.weights, B, K, h, drafts, out["h_out"], out["argmax"],
                           out["n_accepted"], out["committed"], out["n_committed"], None, model.ws,
                           model.ws_bytes, side)
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        bd.moe_verify_step(model.cfg, model.weights, B, K, h, drafts, out["h_out"], out["argmax"],
                           out["n_accepted"], out["committed"], out["n_committed"], None, model.ws,
                           model.ws_bytes, torch.cuda.current_stream())
    for rep in range(3):
        for v in out.values():
            if v is not None:
                v.fill_(-7)            # eager work between replays
        graph.replay()
        _sync(torch)
        for key, want in ref.items():
            assert np.array_equal(_host(bd, out[key]), want), (rep, key)


# ---------------------------------------------------------------- bounded waits


@pytest.mark.parametrize("B", [1, 2])
def test_wait_timeout_is_reported(bd, torch_cuda, big, B):
    """The fused launch's waits are bounded.  With the bound set to zero polls
    from the host, waits that find their counters short give up at once, the
    kernels still run to their end, and the call's status word reads 1; the
    next call with the default bound clears it and reads 0 again, with the
    same results as before the forced timeout."""
    torch = torch_cuda
    dims, W, model = big
    K = 3
    h = _dev(bd, synth.make_hidden(dims, B * (K + 1), seed=830 + B))
    drafts = _dev(bd, np.zeros((B, K), np.int32))
    ref = bd.run_verify_step(model, h, drafts, B, K, routing=True)
    _sync(torch)
    assert bd.step_status(model) == 0
    prev = bd.mv_set_spin_limit(0)
    try:
        bd.run_verify_step(model, h, drafts, B, K, routing=True)
        _sync(torch)
        forced = bd.step_status(model)
    finally:
        bd.mv_set_spin_limit(prev)
    assert forced == 1
    again = bd.run_verify_step(model, h, drafts, B, K, routing=True)
    _sync(torch)
    assert bd.step_status(model) == 0
    for key in ("h_out", "argmax", "topk_ids"):
        assert np.array_equal(_host(bd, again[key]), _host(bd, ref[key])), key


# ---------------------------------------------------------------- one launch


def _one_launch_case(bd, torch, dims, model, B, K, seed):
    """Inputs of a one-launch comparison: drafts that accept fully in sequence 0
    (its argmax) and random ones elsewhere, and the launches' outputs on them."""
    T = B * (K + 1)
    h = _dev(bd, synth.make_hidden(dims, T, seed=seed))
    rnd = np.random.default_rng(seed).integers(0, dims.vocab, (B, K)).astype(np.int32)
    first = bd.run_verify_step(model, h, _dev(bd, rnd), B, K)
    _sync(torch)
    g = _host(bd, first["argmax"]).reshape(B, K + 1)
    rnd[0] = g[0, :K]
    drafts = _dev(bd, rnd)
    ref = bd.run_verify_step(model, h, drafts, B, K, routing=True)
    _sync(torch)
    return h, drafts, {k: _host(bd, v) for k, v in ref.items() if v is not None}


@pytest.mark.parametrize("model_name,B,K", [("big", 1, 0), ("big", 1, 3), ("big", 2, 1), ("big", 2, 3),
                                            ("big", 8, 0), ("big", 4, 1), ("tiny", 1, 3), ("tiny", 2, 3),
                                            ("tiny", 4, 1), ("tiny3", 1, 1), ("tiny3", 2, 3)])
def test_one_launch_step_equals_the_launches(bd, torch_cuda, tiny, tiny3, big, model_name, B, K):
    """moe_verify_step_one_launch runs the launches' blocks as virtual blocks
    of one launch with the same arithmetic: every output equals
    moe_verify_step's bit for bit, twice in a row on one workspace (the setup
    kernel clears what the first call left), and no wait gave up."""
    torch = torch_cuda
    dims, W, model = {"tiny": tiny, "tiny3": tiny3, "big": big}[model_name]
    h, drafts, ref = _one_launch_case(bd, torch, dims, model, B, K, seed=900 + 10 * B + K)
    if K:
        assert ref["n_committed"][0] == K + 1  # sequence 0 takes the bonus token
    for rep in range(2):
        out = bd.run_verify_step(model, h, drafts, B, K, routing=True, one_launch=True)
        _sync(torch)
        assert bd.step_status(model) == 0
        for key, want in ref.items():
            assert np.array_equal(_host(bd, out[key]), want), (rep, key)


@pytest.mark.parametrize("model_name", ["tiny3", "big"])
def test_one_launch_step_in_place_and_shrinking(bd, torch_cuda, tiny3, big, model_name):
    """h_out aliasing h_in (the combines keep reading buffers other than the
    one they write), then a smaller batch on the same workspace: both equal
    the launches bit for bit."""
    torch = torch_cuda
    dims, W, model = {"tiny3": tiny3, "big": big}[model_name]
    for B, K in ((2, 3), (1, 1)):
        h, drafts, ref = _one_launch_case(bd, torch, dims, model, B, K, seed=950 + B)
        ht = h.clone()
        T = B * (K + 1)
        out = {"argmax": torch.empty(T, dtype=torch.int32, device="cuda"),
               "n_accepted": torch.empty(B, dtype=torch.int32, device="cuda"),
               "committed": torch.empty((B, K + 1), dtype=torch.int32, device="cuda"),
               "n_committed": torch.empty(B, dtype=torch.int32, device="cuda"),
               "topk_ids": torch.empty((dims.n_layers, T, dims.top_k), dtype=torch.int32, device="cuda")}
        bd.moe_verify_step_one_launch(model.cfg, model.weights, B, K, ht, drafts, ht, out["argmax"],
                                      out["n_accepted"], out["committed"], out["n_committed"], out["topk_ids"],
                                      model.ws, model.ws_bytes)
        _sync(torch)
        assert bd.step_status(model) == 0
        assert np.array_equal(_host(bd, ht), ref["h_out"]), (B, K)
        for key, v in out.items():
            assert np.array_equal(_host(bd, v), ref[key]), (B, K, key)


def test_one_launch_wait_timeout_is_reported(bd, torch_cuda, big):
    """The one-launch step's waits are bounded like the fused launch's: with
    the bound set to zero polls from the host the kernel still runs to its end
    and the status word reads 1; the next call with the default bound reads 0
    and gives the launches' results again."""
    torch = torch_cuda
    dims, W, model = big
    B, K = 1, 3
    h, drafts, ref = _one_launch_case(bd, torch, dims, model, B, K, seed=970)
    prev = bd.mv_set_spin_limit(0)
    try:
        bd.run_verify_step(model, h, drafts, B, K, routing=True, one_launch=True)
        _sync(torch)
        forced = bd.step_status(model)
    finally:
        bd.mv_set_spin_limit(prev)
    assert forced == 1
    again = bd.run_verify_step(model, h, drafts, B, K, routing=True, one_launch=True)
    _sync(torch)
    assert bd.step_status(model) == 0
    for key, want in ref.items():
        assert np.array_equal(_host(bd, again[key]), want), key
