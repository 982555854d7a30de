"""Seeded synthetic inputs for the MoE verify step.

This module only draws numbers: model weights, hidden states, draft tokens
and router biases, each from its own keyed Philox stream so that any tensor
can be regenerated alone.  It contains none of the verify step's arithmetic;
both the CPU oracle (through the tests) and the GPU library consume what it
produces.

Shapes follow the decoder described on "Jina AI Releases jina-ocr-v1, a 3.4B
MoE Document Parser With Built-In Speculative Decoding" (ainewsfeed.tech),
architecture paragraph: 12 layers, 64 routed experts, two shared experts,
top-6 routing, weights released in BF16 (weights/licence paragraph).  The
widths (d_model 1280, expert FFN 896, vocab 129,280) and the value
distributions are the workload definitions this library is measured on.

bf16 tensors are returned as ``np.uint16`` arrays holding the raw bf16 bit
patterns; fp32 tensors as ``np.float32``.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field, replace
from typing import Dict, Optional

import numpy as np

# ---------------------------------------------------------------------------
# model shapes and workloads
# ---------------------------------------------------------------------------


@dataclass(frozen=True)
class ModelDims:
    d_model: int
    d_ff: int
    n_routed: int
    n_shared: int
    top_k: int
    n_layers: int
    vocab: int
    rms_eps: float
    dtype: str  # "f32" or "bf16"

    @property
    def n_slots(self) -> int:
        return self.top_k + self.n_shared


# Tiny single-layer model held in fp32 (parity and lossless tests).
TINY_F32 = ModelDims(256, 128, 64, 2, 6, 1, 1024, 1e-6, "f32")
# DeepSeek-3B-MoE-shaped FFN stack: 12 layers, 64 routed top-6 + 2 shared.
DS3B_BF16 = ModelDims(1280, 896, 64, 2, 6, 12, 129280, 1e-6, "bf16")


@dataclass(frozen=True)
class Workload:
    name: str
    dims: ModelDims
    batch: int          # sequences (0 for a plain token batch)
    k_draft: int        # draft tokens per sequence
    match_p: float      # probability a draft equals the verifier's argmax
    tokens: int         # tokens pushed through the stack per call
    lm_head: bool
    weight_sigma: Optional[float]  # None: 1/sqrt(fan_in)
    zipf_s: Optional[float] = None  # router bias giving Zipf popularity
    code: int = 0       # stream key for this workload's activations


WORKLOADS: Dict[str, Workload] = {
    w.name: w
    for w in [
        Workload("tiny_f32_b4_k3", TINY_F32, 4, 3, 0.6, 16, True, None, code=1),
        Workload("b1_k3", DS3B_BF16, 1, 3, 0.576, 4, True, 0.02, code=2),
        Workload("c32_k3", DS3B_BF16, 32, 3, 0.6, 128, True, 0.02, code=3),
        Workload("prefill_10048", DS3B_BF16, 0, 0, 0.0, 10048, False, 0.02, code=4),
        Workload("zipf_loop_c32", DS3B_BF16, 32, 3, 0.6, 128, True, 0.02,
                 zipf_s=1.1, code=5),
    ]
}

# stream keys, one per tensor kind
_K_NORM, _K_ROUTER, _K_RBIAS, _K_GU, _K_DOWN = 1, 2, 3, 4, 5
_K_SGU, _K_SDOWN, _K_FNORM, _K_LM, _K_HIDDEN = 6, 7, 8, 9, 10
_K_DRAFT, _K_EMB, _K_PERM, _K_MTP = 11, 12, 13, 14

_THREADS = max(1, min(16, os.cpu_count() or 1))


def _rng(*key: int) -> np.random.Generator:
    return np.random.Generator(np.random.Philox(np.random.SeedSequence(list(key))))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round to nearest even (torch's conversion)."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def bf16_bits_to_f32(u: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to fp32 (for host-side inspection)."""
    return (np.asarray(u, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _store(a32: np.ndarray, dtype: str) -> np.ndarray:
    return f32_to_bf16_bits(a32) if dtype == "bf16" else a32.astype(np.float32)


def _normal_block(out: np.ndarray, idx, sigma: float, dtype: str, key) -> None:
    shape = out[idx].shape
    v = _rng(*key).standard_normal(int(np.prod(shape)), dtype=np.float32)
    v *= np.float32(sigma)
    out[idx] = _store(v, dtype).reshape(shape)


def _alloc(shape, dtype: str) -> np.ndarray:
    return np.empty(shape, dtype=np.uint16 if dtype == "bf16" else np.float32)


# ---------------------------------------------------------------------------
# weights
# ---------------------------------------------------------------------------


def make_weights(dims: ModelDims, seed: int = 0, sigma: Optional[float] = None,
                 gamma: str = "ones", zipf_s: Optional[float] = None,
                 layers: Optional[int] = None) -> Dict[str, Optional[np.ndarray]]:
    """All weights of the MoE FFN stack.

    sigma: standard deviation of every matrix; None means 1/sqrt(fan_in).
    gamma: "ones" (RMSNorm scales = 1) or "uniform" (U[0.5, 1.5], tests only).
    zipf_s: if set, a per-layer router bias b_e = -s * ln(rank_e) over a seeded
      random ranking of the experts; otherwise no bias (None).
    layers: generate only this many layers (tests that need a prefix).

    Layout (row-major, [out, in] per matrix as in a torch Linear):
      ffn_norm   [L, d]          router_w  [L, E, d]     router_b [L, E] f32
      w_gate_up  [L, E, 2F, d]   rows [0, F) gate, [F, 2F) up
      w_down     [L, E, d, F]
      ws_gate_up [L, S, 2F, d]   ws_down   [L, S, d, F]
      final_norm [d]             lm_head   [V, d]
    """
    d, F, E, S, V = dims.d_model, dims.d_ff, dims.n_routed, dims.n_shared, dims.vocab
    L = dims.n_layers if layers is None else layers
    dt = dims.dtype

    def sd(fan_in):
        return sigma if sigma is not None else 1.0 / np.sqrt(fan_in)

    w: Dict[str, Optional[np.ndarray]] = {}
    w["ffn_norm"] = _alloc((L, d), dt)
    w["router_w"] = _alloc((L, E, d), dt)
    w["w_gate_up"] = _alloc((L, E, 2 * F, d), dt)
    w["w_down"] = _alloc((L, E, d, F), dt)
    w["ws_gate_up"] = _alloc((L, S, 2 * F, d), dt)
    w["ws_down"] = _alloc((L, S, d, F), dt)
    w["final_norm"] = _alloc((d,), dt)
    w["lm_head"] = _alloc((V, d), dt)

    jobs = []
    for layer in range(L):
        jobs.append((w["router_w"], (layer,), sd(d), (seed, _K_ROUTER, layer)))
        for e in range(E):
            jobs.append((w["w_gate_up"], (layer, e), sd(d), (seed, _K_GU, layer, e)))
            jobs.append((w["w_down"], (layer, e), sd(F), (seed, _K_DOWN, layer, e)))
        for s in range(S):
            jobs.append((w["ws_gate_up"], (layer, s), sd(d), (seed, _K_SGU, layer, s)))
            jobs.append((w["ws_down"], (layer, s), sd(F), (seed, _K_SDOWN, layer, s)))
    rows_per_job = 8192
    for r0 in range(0, V, rows_per_job):
        jobs.append((w["lm_head"], (slice(r0, min(V, r0 + rows_per_job)),), sd(d),
                     (seed, _K_LM, r0)))

    with ThreadPoolExecutor(_THREADS) as ex:
        list(ex.map(lambda j: _normal_block(j[0], j[1], j[2], dt, j[3]), jobs))

    if gamma == "ones":
        w["ffn_norm"][...] = _store(np.ones((L, d), np.float32), dt)
        w["final_norm"][...] = _store(np.ones((d,), np.float32), dt)
    elif gamma == "uniform":
        w["ffn_norm"][...] = _store(
            _rng(seed, _K_NORM).uniform(0.5, 1.5, (L, d)).astype(np.float32), dt)
        w["final_norm"][...] = _store(
            _rng(seed, _K_FNORM).uniform(0.5, 1.5, (d,)).astype(np.float32), dt)
    else:
        raise ValueError(gamma)

    w["router_b"] = None if zipf_s is None else make_router_bias(L, E, zipf_s, seed)
    return w


def make_router_bias(n_layers: int, n_routed: int, zipf_s: float, seed: int = 0) -> np.ndarray:
    """Router bias [L, E] fp32 skewing expert popularity: b_e = -s * ln(rank_e)
    over a seeded random ranking of the experts in each layer."""
    b = np.empty((n_layers, n_routed), np.float32)
    for layer in range(n_layers):
        rank = _rng(seed, _K_PERM, layer).permutation(n_routed) + 1
        b[layer] = (-zipf_s * np.log(rank.astype(np.float64))).astype(np.float32)
    return b


def workload_weights(wl: Workload, seed: int = 0, **kw):
    return make_weights(wl.dims, seed=seed, sigma=wl.weight_sigma, zipf_s=wl.zipf_s, **kw)


# ---------------------------------------------------------------------------
# activations and drafts
# ---------------------------------------------------------------------------


def make_hidden(dims: ModelDims, tokens: int, seed: int = 0, code: int = 0) -> np.ndarray:
    """Hidden states h ~ N(0, 1), [tokens, d], in the model's storage dtype."""
    v = _rng(seed, _K_HIDDEN, code).standard_normal((tokens, dims.d_model), dtype=np.float32)
    return _store(v, dims.dtype)


def workload_hidden(wl: Workload, seed: int = 0) -> np.ndarray:
    return make_hidden(wl.dims, wl.tokens, seed, wl.code)


def make_drafts(target: np.ndarray, match_p: float, vocab: int, seed: int = 0,
                step: int = 0, code: int = 0) -> np.ndarray:
    """Draft tokens [B, K]: each position independently equals target[b, j]
    with probability match_p, otherwise a uniform draw from [0, vocab) (which
    may coincide with the target).  ``target`` is [B, K+1] or [B, K] argmax ids.
    """
    target = np.asarray(target)
    B = target.shape[0]
    K = target.shape[1] - 1 if target.shape[1] > 0 else 0
    if target.ndim != 2:
        raise ValueError("target must be [B, K+1]")
    g = _rng(seed, _K_DRAFT, code, step)
    hit = g.random((B, K)) < match_p
    rnd = g.integers(0, vocab, (B, K), dtype=np.int64)
    return np.where(hit, target[:, :K], rnd).astype(np.int32)


def make_embedding(dims: ModelDims, seed: int = 0) -> np.ndarray:
    """Test-only token embedding table [V, d] ~ N(0, 1) in the storage dtype
    (the decoder's real embedding is outside the verified path)."""
    v = _rng(seed, _K_EMB).standard_normal((dims.vocab, dims.d_model), dtype=np.float32)
    return _store(v, dims.dtype)


# ---------------------------------------------------------------------------
# FastMTP draft block
# ---------------------------------------------------------------------------


def mtp_d_ff(dims: ModelDims) -> int:
    """Width of the draft block's dense SwiGLU FFN: 2F, the width of the two
    always-on shared experts together (the pages give no width)."""
    return 2 * dims.d_ff


def make_mtp_weights(dims: ModelDims, seed: int = 0, sigma: Optional[float] = None,
                     gamma: str = "ones") -> Dict[str, np.ndarray]:
    """Weights of the FastMTP draft block (one dense block whose parameters
    are shared by every draft position; its LM head is the decoder's own).

    Layout (row-major, [out, in] per matrix):
      embed     [V, d]        token embeddings ~ N(0, 1)
      norm_h    [d]           RMSNorm scale of the incoming hidden state
      norm_e    [d]           RMSNorm scale of the token's embedding
      w_proj    [d, 2d]       projection of [norm(h) ; norm(e)]
      norm_ffn  [d]           RMSNorm scale before the dense FFN
      w_gate_up [2Fm, d]      rows [0, Fm) gate, [Fm, 2Fm) up
      w_down    [d, Fm]
      norm_out  [d]           RMSNorm scale before the LM head
    sigma: standard deviation of the matrices; None means 1/sqrt(fan_in).
    """
    d, dt, Fm = dims.d_model, dims.dtype, mtp_d_ff(dims)

    def sd(fan_in):
        return sigma if sigma is not None else 1.0 / np.sqrt(fan_in)

    m: Dict[str, np.ndarray] = {"embed": make_embedding(dims, seed)}
    for i, (name, shape, fan) in enumerate([("w_proj", (d, 2 * d), 2 * d),
                                            ("w_gate_up", (2 * Fm, d), d),
                                            ("w_down", (d, Fm), Fm)]):
        m[name] = _alloc(shape, dt)
        _normal_block(m[name], (), sd(fan), dt, (seed, _K_MTP, i))
    for i, name in enumerate(["norm_h", "norm_e", "norm_ffn", "norm_out"]):
        if gamma == "ones":
            v = np.ones(d, np.float32)
        elif gamma == "uniform":
            v = _rng(seed, _K_MTP, 10 + i).uniform(0.5, 1.5, d).astype(np.float32)
        else:
            raise ValueError(gamma)
        m[name] = _store(v, dt)
    return m
