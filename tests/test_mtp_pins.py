"""Pins of the oracle's FastMTP draft block against things other than itself:
special weights that reduce the block to the decoder's own greedy choice or to
a plain LM-head argmax of an embedding, the dense FFN against torch, the
recursion, and row independence.  No GPU needed."""
import numpy as np
import pytest
import torch

from oracle import moe_oracle as O
from speculative_decode_verification_router_amd import synth

DIMS = synth.TINY_F32


@pytest.fixture(scope="module")
def model():
    return synth.make_weights(DIMS, gamma="uniform"), synth.make_mtp_weights(DIMS, gamma="uniform")


def _with(M, **kw):
    out = dict(M)
    out.update(kw)
    return out


def _proj(half):
    """[d, 2d] projection taking the h half (0) or the embedding half (1)."""
    d = DIMS.d_model
    p = np.zeros((d, 2 * d), np.float32)
    p[:, half * d:(half + 1) * d] = np.eye(d, dtype=np.float32)
    return p


def test_identity_projection_drafts_the_decoders_own_choice(model):
    """W_proj = [I | 0], unit scales on the h side and a zero FFN down
    projection: the block's output is RMSNorm(h) and its draft is the
    decoder's greedy token for h (RMSNorm is idempotent up to eps)."""
    W, M = model
    d = DIMS.d_model
    ones = np.ones(d, np.float32)
    M1 = _with(M, w_proj=_proj(0), norm_h=ones, w_down=np.zeros_like(M["w_down"]),
               norm_out=W["final_norm"])
    h = synth.make_hidden(DIMS, 64, code=21)
    tokens = np.arange(64) * 7 % DIMS.vocab
    r = O.mtp_draft(h, tokens, M1, W, DIMS, 1)
    ref = O.lm_head_argmax(O.widen(h, "f32"), W["final_norm"], W["lm_head"], DIMS)
    ok = ref["margin"] > 1e-3
    assert ok.sum() > 50
    assert np.array_equal(r["drafts"][ok, 0], ref["argmax"][ok])
    # the tokens play no part on this side of the projection
    r2 = O.mtp_draft(h, tokens[::-1].copy(), M1, W, DIMS, 1)
    assert np.array_equal(r2["drafts"], r["drafts"])


def test_embedding_projection_drafts_the_argmax_of_the_embedding(model):
    """W_proj = [0 | I], unit scales and a zero FFN: the draft is the LM-head
    argmax of the normalised embedding of the token, computed here with a
    direct matrix product."""
    W, M = model
    d = DIMS.d_model
    ones = np.ones(d, np.float32)
    M1 = _with(M, w_proj=_proj(1), norm_e=ones, norm_out=ones, w_down=np.zeros_like(M["w_down"]))
    tokens = np.arange(48) * 13 % DIMS.vocab
    h = synth.make_hidden(DIMS, 48, code=22)
    r = O.mtp_draft(h, tokens, M1, W, DIMS, 1)
    e = M["embed"][tokens].astype(np.float64)
    x = e / np.sqrt(np.mean(e * e, axis=1, keepdims=True) + DIMS.rms_eps)
    z = x @ W["lm_head"].astype(np.float64).T
    top2 = np.sort(z, axis=1)[:, -2:]
    ok = top2[:, 1] - top2[:, 0] > 1e-3
    assert ok.sum() > 40
    assert np.array_equal(r["drafts"][ok, 0], np.argmax(z, axis=1)[ok])


def test_dense_ffn_residual_matches_torch(model):
    """With W_proj = [I | 0] the block's output minus its projection is the
    dense SwiGLU FFN of the normalised projection (torch, float64)."""
    W, M = model
    M1 = _with(M, w_proj=_proj(0))
    h = O.widen(synth.make_hidden(DIMS, 9, code=23), "f32")
    tokens = np.arange(9)
    h1, h2 = O.mtp_block(h, tokens, M1, DIMS)
    x = O.store(O.rms_norm(h1, O.widen(M["norm_ffn"], "f32"), DIMS.rms_eps), "f32")
    F = synth.mtp_d_ff(DIMS)
    gu = torch.from_numpy(M["w_gate_up"].astype(np.float64))
    xt = torch.from_numpy(x)
    a = torch.nn.functional.silu(xt @ gu[:F].T) * (xt @ gu[F:].T)
    a = a.to(torch.float32).to(torch.float64)
    y = (a @ torch.from_numpy(M["w_down"].astype(np.float64)).T).numpy()
    ref = (h1 + y).astype(np.float32).astype(np.float64)
    assert np.allclose(h2, ref, rtol=1e-6, atol=1e-6)
    # and the projection itself: h1 = round(RMSNorm(h) * g_h)
    uh = O.rms_norm(h, O.widen(M["norm_h"], "f32"), DIMS.rms_eps)
    assert np.allclose(h1, uh.astype(np.float32), rtol=1e-6, atol=1e-7)


def test_recursion_is_the_block_applied_to_its_own_output(model):
    W, M = model
    h = synth.make_hidden(DIMS, 5, code=24)
    tokens = np.array([3, 1, 4, 1, 5])
    r3 = O.mtp_draft(h, tokens, M, W, DIMS, 3)
    hh, tt = O.widen(h, "f32"), tokens
    for j in range(3):
        r1 = O.mtp_draft(hh, tt, M, W, DIMS, 1)
        assert np.array_equal(r1["drafts"][:, 0], r3["drafts"][:, j])
        hh, tt = r1["h_out"], r1["drafts"][:, 0]
    assert np.array_equal(hh, r3["h_out"])


def test_rows_are_independent(model):
    W, M = model
    h = synth.make_hidden(DIMS, 6, code=25)
    tokens = np.array([10, 20, 30, 40, 50, 60])
    r = O.mtp_draft(h, tokens, M, W, DIMS, 2)
    for b in range(6):
        rb = O.mtp_draft(h[b:b + 1], tokens[b:b + 1], M, W, DIMS, 2)
        assert np.array_equal(rb["drafts"][0], r["drafts"][b])
        assert np.array_equal(rb["h_out"][0], r["h_out"][b])


def test_zero_drafts():
    W = synth.make_weights(DIMS)
    M = synth.make_mtp_weights(DIMS)
    h = synth.make_hidden(DIMS, 2, code=26)
    r = O.mtp_draft(h, np.array([0, 1]), M, W, DIMS, 0)
    assert r["drafts"].shape == (2, 0)
    assert np.array_equal(r["h_out"], O.widen(h, "f32"))
