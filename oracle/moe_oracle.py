"""CPU oracle of the MoE verify step.  TEST INFRASTRUCTURE ONLY.

Only the test suite, the package smoke check and the benchmark's CPU-baseline
leg may import this module.  The GPU library never calls it and it imports
nothing from the GPU library; the two share only the seeded input arrays.

What it computes, and from where
--------------------------------
The decoder is the one on "Jina AI Releases jina-ocr-v1, a 3.4B MoE Document
Parser With Built-In Speculative Decoding" (ainewsfeed.tech), architecture
paragraph: a stack of MoE layers with 64 routed experts, two always-on shared
experts and top-6 routing.  Its FastMTP paragraph fixes the verify rule: the
decoder's own greedy choice at every position, acceptance of the longest
draft prefix that matches those choices, and one more token committed by the
decoder itself (a bonus token when every draft matched), so that the
committed text is exactly what plain greedy decoding would produce.  The
modelscope.ai paper page ("Jina-OCR-v1: Efficient Document Parsing with
Speculative Decoding and Dense Verifiable Rewards", Abstract) gives K = 3 and
that greedy verification is lossless.

Readings where the pages are silent (each listed with its reason in the
design notes): SwiGLU experts, a = SiLU(gate) * up; RMSNorm with eps 1e-6 and
order (h * inv) * gamma; the router is a linear map to 64 logits, selection is
on logits, ties go to the lower expert id, gates are the softmax over the 6
chosen logits; shared experts have weight 1; each layer is h <- h + MoE(RMSNorm(h));
a final RMSNorm precedes the LM head; argmax ties go to the lowest token id.

Precision
---------
All arithmetic is float64 (``ftype=np.float64``, the reference).  The same
algorithm can also run with float32 working precision (``ftype=np.float32``);
the tests use the gap between the two runs to measure how far rounding noise
alone can move each routing and argmax decision after many layers.  Values the kernel *stores* in the model's dtype
are rounded to it, through fp32, exactly where the kernel rounds: the hidden
state between layers, the normalised input x of each layer, the SwiGLU
product a, and the final normalised x_f.  Router logits and LM-head logits
are rounded to fp32 (the precision the kernel holds them in) before the
integer decisions taken on them (top-6, argmax), and the decision margins are
measured on those fp32 values.  Everything else stays float64.

The FastMTP draft block (mtp_block, mtp_draft) follows the same pages'
FastMTP paragraph: one dense block whose parameters are shared by every
draft position, fed by the decoder's last hidden state and the token that
follows it, drafting through the decoder's own LM head.  Its inner layers are
not on the pages; the plainest reading is used: RMSNorm of the hidden state
and of the token's embedding, a linear projection of the two laid end to end
back to d, a residual dense SwiGLU FFN behind an RMSNorm, and an RMSNorm
before the LM head.

Parity status: every function here is pinned by tests/test_oracle_pins.py
and tests/test_mtp_pins.py (library special cases, closed forms, invariants,
brute force, and the lossless greedy-equivalence property).  The loop over
layers (forward_tokens) is pinned on a three-layer model: zero down
projections give the identity, and per-layer one-hot router biases give the
chain of the chosen experts' dense FFNs computed with torch.
"""
from __future__ import annotations

from typing import Dict, List, Optional

import numpy as np

# ---------------------------------------------------------------------------
# storage formats
# ---------------------------------------------------------------------------


def widen(a: np.ndarray, dtype: str) -> np.ndarray:
    """Stored tensor -> float64.  bf16 tensors arrive as uint16 bit patterns."""
    if dtype == "bf16":
        bits = np.asarray(a, dtype=np.uint16).astype(np.uint32) << 16
        return bits.view(np.float32).astype(np.float64)
    if dtype == "f32":
        return np.asarray(a, dtype=np.float32).astype(np.float64)
    raise ValueError(dtype)


def fp32_to_bf16_rne(v32: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round to nearest, ties to even.

    bf16 keeps the top 16 bits of the fp32 pattern.  Adding 0x7FFF plus the
    lowest kept bit to the pattern before truncating rounds to nearest with
    ties going to the even kept value.  NaNs stay NaN (quiet bit forced).
    """
    u = np.ascontiguousarray(v32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)).astype(np.uint32)
    nan = np.isnan(np.asarray(v32, dtype=np.float32))
    r = np.where(nan, (u >> np.uint64(16)).astype(np.uint32) | np.uint32(0x40), r)
    return r.astype(np.uint16)


def store(v: np.ndarray, dtype: str) -> np.ndarray:
    """Round a float64 value to the model's storage dtype (via fp32), returned
    as float64 so the next step computes on exactly the stored value."""
    v32 = np.asarray(v, dtype=np.float64).astype(np.float32)
    if dtype == "f32":
        return v32.astype(np.float64)
    if dtype == "bf16":
        return widen(fp32_to_bf16_rne(v32), "bf16")
    raise ValueError(dtype)


def as_fp32(v: np.ndarray) -> np.ndarray:
    """Round to fp32 and return as float64 (decision precision of the kernel)."""
    return np.asarray(v, dtype=np.float64).astype(np.float32).astype(np.float64)


# ---------------------------------------------------------------------------
# the per-layer steps
# ---------------------------------------------------------------------------


def rms_norm(h: np.ndarray, gamma: np.ndarray, eps: float, ftype=np.float64) -> np.ndarray:
    """RMSNorm of each row: (h * (mean(h^2) + eps)^(-1/2)) * gamma."""
    h = np.asarray(h, dtype=ftype)
    inv = ftype(1.0) / np.sqrt(np.mean(h * h, axis=-1, keepdims=True) + ftype(eps))
    return (h * inv) * np.asarray(gamma, ftype)


def router_logits(x: np.ndarray, w_router: np.ndarray,
                  bias: Optional[np.ndarray], ftype=np.float64) -> np.ndarray:
    """Router logits l = x W_r^T (+ b), returned rounded to fp32."""
    l = np.asarray(x, ftype) @ np.asarray(w_router, ftype).T
    if bias is not None:
        l = l + np.asarray(bias, dtype=ftype)
    return as_fp32(l)


def select_top_k(l32: np.ndarray, k: int):
    """Top-k of one token's logits.

    Experts are ordered by (logit descending, expert id ascending) and the
    first k are kept, in that order.  The margin is the gap between the k-th
    and (k+1)-th logit of that order (0 for an exact tie across the cut).
    """
    order = sorted(range(len(l32)), key=lambda e: (-l32[e], e))
    sel = order[:k]
    margin = float(l32[order[k - 1]] - l32[order[k]]) if len(order) > k else np.inf
    return sel, margin


def gate_weights(l_sel: np.ndarray, ftype=np.float64) -> np.ndarray:
    """Softmax over the selected logits (equal to the softmax over all experts
    renormalised to the selected ones)."""
    l_sel = np.asarray(l_sel, dtype=ftype)
    z = np.exp(l_sel - np.max(l_sel))
    return z / np.sum(z)


def silu(z: np.ndarray) -> np.ndarray:
    """SiLU(z) = z / (1 + e^-z)."""
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def swiglu_expert(x: np.ndarray, w_gate_up: np.ndarray, w_down: np.ndarray,
                  dtype: str, ftype=np.float64) -> np.ndarray:
    """One SwiGLU expert on rows x [m, d]: gate rows [0, F) and up rows [F, 2F)
    of w_gate_up [2F, d]; a = SiLU(gate) * up is stored in the model dtype;
    y = a W_down^T with w_down [d, F]."""
    F = w_gate_up.shape[0] // 2
    x = np.asarray(x, ftype)
    w_gate_up = np.asarray(w_gate_up, ftype)
    g = x @ w_gate_up[:F].T
    u = x @ w_gate_up[F:].T
    a = np.asarray(store(silu(g) * u, dtype), ftype)
    return a @ np.asarray(w_down, ftype).T


def moe_layer(h: np.ndarray, W: Dict[str, Optional[np.ndarray]], layer: int,
              dims, ftype=np.float64) -> Dict[str, np.ndarray]:
    """One layer h_out = h + MoE(RMSNorm(h)) for every row of h [T, d]
    (float64 holding stored values).  Rows are independent.

    Returns h_out (stored values), x, logits (fp32), ids [T,k] in selection
    order, gates [T,k], y (float64 MoE output before the residual) and the
    per-token top-k margin.
    """
    dt, k, S = dims.dtype, dims.top_k, dims.n_shared
    E, eps = dims.n_routed, dims.rms_eps
    T, d = h.shape
    gamma = widen(W["ffn_norm"][layer], dt)
    x = store(rms_norm(h, gamma, eps, ftype), dt)
    bias = None if W.get("router_b") is None else W["router_b"][layer]
    l32 = router_logits(x, widen(W["router_w"][layer], dt), bias, ftype)

    ids = np.zeros((T, k), np.int64)
    gates = np.zeros((T, k))
    margin = np.zeros(T)
    for t in range(T):
        sel, margin[t] = select_top_k(l32[t], k)
        ids[t] = sel
        gates[t] = gate_weights(l32[t, sel], ftype)

    # slot[t, s] = contribution of the s-th selected expert (gate applied);
    # slots k.. are the shared experts.  Each expert runs on the rows that
    # selected it; each row is computed exactly as for a token alone.
    slot = np.zeros((T, k + S, d), ftype)
    for e in range(E):
        rows, pos = np.nonzero(ids == e)
        if rows.size == 0:
            continue
        y_e = swiglu_expert(x[rows], widen(W["w_gate_up"][layer, e], dt),
                            widen(W["w_down"][layer, e], dt), dt, ftype)
        slot[rows, pos] = np.asarray(gates[rows, pos], ftype)[:, None] * y_e
    for s in range(S):
        slot[:, k + s] = swiglu_expert(x, widen(W["ws_gate_up"][layer, s], dt),
                                       widen(W["ws_down"][layer, s], dt), dt, ftype)

    y = np.zeros((T, d), ftype)
    for s in range(k + S):          # fixed order: routed slots, then shared
        y = y + slot[:, s]
    h_out = store(np.asarray(h, ftype) + y, dt)
    return dict(h_out=h_out, x=x, logits=l32, ids=ids, gates=gates,
                y=y.astype(np.float64), margin=margin)


def lm_head_argmax(h: np.ndarray, final_norm: np.ndarray, lm_head: np.ndarray,
                   dims, chunk: int = 16384, ftype=np.float64,
                   keep_logits: bool = False) -> Dict[str, np.ndarray]:
    """Final RMSNorm, LM-head logits z = x_f W_lm^T (fp32 for the decision),
    greedy choice g = lowest id among the maximal logits, and the margin
    between the largest and second-largest logit."""
    dt = dims.dtype
    xf = store(rms_norm(h, widen(final_norm, dt), dims.rms_eps, ftype), dt)
    V = lm_head.shape[0]
    z = np.empty((h.shape[0], V), ftype)
    xq = np.asarray(xf, ftype)
    for v0 in range(0, V, chunk):       # the matrix is widened piecewise
        z[:, v0:v0 + chunk] = xq @ np.asarray(widen(lm_head[v0:v0 + chunk], dt), ftype).T
    z32 = as_fp32(z)
    zmax = z32.max(axis=1)
    g = np.array([int(np.flatnonzero(z32[t] == zmax[t])[0]) for t in range(len(zmax))],
                 dtype=np.int64)
    top2 = np.sort(z32, axis=1)[:, -2:] if V > 1 else np.repeat(z32, 2, axis=1)
    out = dict(xf=xf, argmax=g, margin=top2[:, 1] - top2[:, 0])
    if keep_logits:
        out["logits"] = z32
    return out


def spec_accept(argmax: np.ndarray, drafts: np.ndarray):
    """Greedy verification of K drafts per sequence.

    argmax [B, K+1]: the decoder's choice after the committed token (position
    0) and after each draft (positions 1..K).  Draft j is accepted when it and
    every earlier draft equal the decoder's choice at the same position.  With
    n accepted drafts the committed tokens are argmax[b, 0..n] (the n accepted
    drafts themselves, then the decoder's own token: a correction, or a bonus
    when n = K), padded with -1.
    """
    argmax = np.asarray(argmax)
    drafts = np.asarray(drafts)
    B, K = drafts.shape
    n_acc = np.zeros(B, np.int64)
    committed = np.full((B, K + 1), -1, np.int64)
    for b in range(B):
        n = 0
        while n < K and drafts[b, n] == argmax[b, n]:
            n += 1
        n_acc[b] = n
        committed[b, :n + 1] = argmax[b, :n + 1]
    return n_acc, committed, n_acc + 1


def forward_tokens(h_in: np.ndarray, W, dims, n_layers: Optional[int] = None,
                   lm_head: bool = True, ftype=np.float64,
                   keep_logits: bool = False) -> Dict[str, object]:
    """The verify step's forward for any set of token rows (rows are
    independent): the MoE stack, then optionally the final norm + LM argmax."""
    L = dims.n_layers if n_layers is None else n_layers
    h = widen(h_in, dims.dtype)
    layers: List[Dict[str, np.ndarray]] = []
    for layer in range(L):
        r = moe_layer(h, W, layer, dims, ftype)
        layers.append(r)
        h = r["h_out"]
    out: Dict[str, object] = dict(h_out=h, layers=layers)
    if lm_head:
        out.update(lm_head_argmax(h, W["final_norm"], W["lm_head"], dims, ftype=ftype,
                                  keep_logits=keep_logits))
    return out


def verify_step(h_in: np.ndarray, drafts: np.ndarray, W, dims) -> Dict[str, object]:
    """One verify step: h_in [B*(K+1), d] (row b*(K+1) is sequence b's
    committed token, rows +1..K its drafts), drafts [B, K]."""
    drafts = np.asarray(drafts)
    B, K = drafts.shape
    out = forward_tokens(h_in, W, dims)
    g = np.asarray(out["argmax"]).reshape(B, K + 1)
    n_acc, committed, n_committed = spec_accept(g, drafts)
    out.update(n_accepted=n_acc, committed=committed, n_committed=n_committed)
    return out


# ---------------------------------------------------------------------------
# FastMTP draft block
# ---------------------------------------------------------------------------


def mtp_block(h: np.ndarray, tokens: np.ndarray, M: Dict[str, np.ndarray], dims,
              ftype=np.float64):
    """One application of the draft block to rows h [B, d] (stored values)
    with the tokens [B] that follow them.

    u  = [ R(RMSNorm(h) * g_h) ; R(RMSNorm(E[t]) * g_e) ]      (2d values)
    h1 = R(u W_proj^T)
    h2 = R(h1 + SwiGLU(R(RMSNorm(h1) * g_ffn)))
    R() is the storage rounding.  Returns (h1, h2).
    """
    dt, eps = dims.dtype, dims.rms_eps
    e = widen(np.asarray(M["embed"])[np.asarray(tokens, np.int64)], dt)
    uh = store(rms_norm(h, widen(M["norm_h"], dt), eps, ftype), dt)
    ue = store(rms_norm(e, widen(M["norm_e"], dt), eps, ftype), dt)
    u = np.concatenate([uh, ue], axis=1)
    h1 = store(np.asarray(u, ftype) @ np.asarray(widen(M["w_proj"], dt), ftype).T, dt)
    x = store(rms_norm(h1, widen(M["norm_ffn"], dt), eps, ftype), dt)
    y = swiglu_expert(x, widen(M["w_gate_up"], dt), widen(M["w_down"], dt), dt, ftype)
    h2 = store(np.asarray(h1, ftype) + y, dt)
    return h1, h2


def mtp_draft(h_in: np.ndarray, tokens: np.ndarray, M: Dict[str, np.ndarray], W, dims,
              K: int, ftype=np.float64) -> Dict[str, np.ndarray]:
    """K draft tokens per sequence.  h_in [B, d]: the decoder's last hidden
    state of each sequence (its stored values); tokens [B]: the token that
    follows it (the last committed one).  Draft j is the greedy choice of the
    decoder's LM head on the block's output after RMSNorm (scale norm_out);
    the block is then applied again to its own output and that draft.
    Returns drafts [B, K], the block's last hidden state h_out, and each
    draft's argmax margin [B, K]."""
    h = widen(h_in, dims.dtype)
    t = np.asarray(tokens, np.int64)
    drafts, margins = [], []
    for _ in range(K):
        _, h = mtp_block(h, t, M, dims, ftype)
        r = lm_head_argmax(h, M["norm_out"], W["lm_head"], dims, ftype=ftype)
        t = np.asarray(r["argmax"], np.int64)
        drafts.append(t)
        margins.append(r["margin"])
    B = h.shape[0]
    return dict(drafts=np.stack(drafts, 1) if K else np.zeros((B, 0), np.int64), h_out=h,
                margin=np.stack(margins, 1) if K else np.zeros((B, 0)))


# ---------------------------------------------------------------------------
# draft length
# ---------------------------------------------------------------------------


def expected_committed(q: float, K: int) -> float:
    """Expected tokens committed per sequence and step with K drafts, each
    accepted independently with probability q: the accept rule commits the
    accepted prefix n plus one token, and P(n >= i) = q^i, so
    E[n + 1] = 1 + q + ... + q^K."""
    return float(sum(q ** i for i in range(K + 1)))


def choose_k(q: float, cost) -> tuple:
    """Draft length K in [0, len(cost)) with the most expected committed
    tokens per unit of cost (cost[K]: time or bytes of a step with K drafts);
    the smallest K on ties.  Returns (K, rate)."""
    rates = [expected_committed(q, K) / float(c) for K, c in enumerate(cost)]
    best = max(range(len(rates)), key=lambda K: (rates[K], -K))
    return best, rates[best]


def expected_distinct_experts(T: int, E: int, k: int) -> float:
    """Expected number of distinct experts chosen by T tokens that each pick
    k of E experts uniformly without replacement: an expert is missed by one
    token with probability 1 - k/E, by all T with (1 - k/E)^T."""
    return E * (1.0 - (1.0 - k / E) ** T)


def step_bytes(dims, B: int, K: int, d_ff_mtp: int) -> float:
    """Expected HBM bytes of one speculative step: K positions of the draft
    block (its matrices, the LM head, four norm vectors, and per sequence the
    embedding row and hidden rows in and out), then the verify step over
    T = B (K + 1) rows (the routed experts the tokens choose under uniform
    routing, the shared experts, router and norm vectors, the LM head and
    the hidden rows in and out)."""
    es = 2 if dims.dtype == "bf16" else 4
    d, F, E, S, L, V = dims.d_model, dims.d_ff, dims.n_routed, dims.n_shared, dims.n_layers, dims.vocab
    T = B * (K + 1)
    expert = 3 * F * d * es
    verify = L * (expected_distinct_experts(T, E, dims.top_k) + S) * expert
    verify += L * (E * d + d) * es + V * d * es + d * es + 2 * T * d * es
    draft = K * ((2 * d * d + 3 * d_ff_mtp * d + V * d + 4 * d) * es + B * 3 * d * es)
    return float(verify + draft)
