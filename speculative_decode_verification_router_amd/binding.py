"""ctypes binding of libmoeverify.so.

Argument marshalling only: every step of the verify path runs in the HIP
kernels behind the C ABI declared in include/moe_verify.h.  PyTorch supplies
device memory (tensor ``data_ptr()``) and the stream
(``torch.cuda.current_stream().cuda_stream``).  If the shared library is not
built, ``load()`` raises: there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, Optional

import numpy as np

from .build import LIB_PATH

MV_F32, MV_BF16 = 0, 1
MV_OK, MV_ERR_NULL, MV_ERR_SHAPE, MV_ERR_UNSUPPORTED, MV_ERR_WORKSPACE, MV_ERR_HIP = 0, -1, -2, -3, -4, -5

EXPORTED = ("mv_workspace_bytes", "moe_layer_forward", "moe_verify_step", "moe_verify_step_noalloc",
            "moe_verify_step_one_launch", "spec_accept",
            "mtp_workspace_bytes", "mtp_draft", "mv_choose_k", "mv_step_bytes", "mv_step_status",
            "mv_set_spin_limit", "mv_last_error")


class MvConfig(ctypes.Structure):
    _fields_ = [("d_model", ctypes.c_int32), ("d_ff", ctypes.c_int32),
                ("n_routed", ctypes.c_int32), ("n_shared", ctypes.c_int32),
                ("top_k", ctypes.c_int32), ("n_layers", ctypes.c_int32),
                ("vocab", ctypes.c_int32), ("rms_eps", ctypes.c_float),
                ("dtype", ctypes.c_int32)]


class MvWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "ffn_norm", "router_w", "router_b", "w_gate_up", "w_down", "ws_gate_up", "ws_down",
        "final_norm", "lm_head")]


class MtpWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "embed", "norm_h", "norm_e", "w_proj", "norm_ffn", "w_gate_up", "w_down", "norm_out")] + [
        ("d_ff", ctypes.c_int32)]


_lib: Optional[ctypes.CDLL] = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the library (after torch, so that one HIP runtime serves both)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run __graft_entry__.build() first")
    try:
        import torch  # noqa: F401  (HIP runtime loaded by torch first)
    except ImportError:
        pass
    lib = ctypes.CDLL(path)
    P, I, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    cfgp, wp = ctypes.POINTER(MvConfig), ctypes.POINTER(MvWeights)
    lib.mv_workspace_bytes.argtypes = [cfgp, I]
    lib.mv_workspace_bytes.restype = SZ
    lib.moe_layer_forward.argtypes = [cfgp, wp, I, I, P, P, P, P, P, P, SZ, P]
    lib.moe_layer_forward.restype = ctypes.c_int
    lib.moe_verify_step.argtypes = [cfgp, wp, I, I, P, P, P, P, P, P, P, P, P, SZ, P]
    lib.moe_verify_step.restype = ctypes.c_int
    lib.moe_verify_step_noalloc.argtypes = [cfgp, wp, I, I, P, P, P, P, P, P, P, P, P]
    lib.moe_verify_step_noalloc.restype = ctypes.c_int
    lib.moe_verify_step_one_launch.argtypes = [cfgp, wp, I, I, P, P, P, P, P, P, P, P, P, SZ, P]
    lib.moe_verify_step_one_launch.restype = ctypes.c_int
    lib.spec_accept.argtypes = [I, I, P, P, P, P, P, P]
    lib.spec_accept.restype = ctypes.c_int
    mwp = ctypes.POINTER(MtpWeights)
    lib.mtp_workspace_bytes.argtypes = [cfgp, I, I]
    lib.mtp_workspace_bytes.restype = SZ
    lib.mtp_draft.argtypes = [cfgp, wp, mwp, I, I, P, P, P, P, P, SZ, P]
    lib.mtp_draft.restype = ctypes.c_int
    lib.mv_choose_k.argtypes = [I, ctypes.c_float, ctypes.POINTER(ctypes.c_float), ctypes.POINTER(I),
                                ctypes.POINTER(ctypes.c_float)]
    lib.mv_choose_k.restype = ctypes.c_int
    lib.mv_step_bytes.argtypes = [cfgp, I, I, I]
    lib.mv_step_bytes.restype = ctypes.c_double
    lib.mv_step_status.argtypes = [P, P, P]
    lib.mv_step_status.restype = ctypes.c_int
    lib.mv_set_spin_limit.argtypes = [I]
    lib.mv_set_spin_limit.restype = I
    lib.mv_last_error.argtypes = []
    lib.mv_last_error.restype = ctypes.c_char_p
    _lib = lib
    return lib


class MvError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"[{code}] {msg}")
        self.code = code


def _check(rc: int) -> None:
    if rc != MV_OK:
        raise MvError(rc, load().mv_last_error().decode())


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch

        return torch.cuda.current_stream().cuda_stream
    return stream if isinstance(stream, int) else stream.cuda_stream


def make_config(dims) -> MvConfig:
    return MvConfig(dims.d_model, dims.d_ff, dims.n_routed, dims.n_shared, dims.top_k,
                    dims.n_layers, dims.vocab, dims.rms_eps,
                    MV_BF16 if dims.dtype == "bf16" else MV_F32)


# ---------------------------------------------------------------- entry points


def mv_last_error() -> str:
    return load().mv_last_error().decode()


def mv_workspace_bytes(cfg: MvConfig, max_tokens: int) -> int:
    return int(load().mv_workspace_bytes(ctypes.byref(cfg), int(max_tokens)))


def moe_layer_forward(cfg: MvConfig, weights: MvWeights, layer: int, T: int, h_in, h_out,
                      topk_ids=None, topk_w=None, y_moe=None, ws=None, ws_bytes: int = 0,
                      stream=None) -> None:
    _check(load().moe_layer_forward(ctypes.byref(cfg), ctypes.byref(weights), layer, T,
                                    _ptr(h_in), _ptr(h_out), _ptr(topk_ids), _ptr(topk_w),
                                    _ptr(y_moe), _ptr(ws), ws_bytes, _stream(stream)))


def moe_verify_step(cfg: MvConfig, weights: MvWeights, B: int, K: int, h_in, drafts, h_out,
                    argmax, n_accepted, committed, n_committed, dbg_topk_ids=None, ws=None,
                    ws_bytes: int = 0, stream=None) -> None:
    _check(load().moe_verify_step(ctypes.byref(cfg), ctypes.byref(weights), B, K, _ptr(h_in),
                                  _ptr(drafts), _ptr(h_out), _ptr(argmax), _ptr(n_accepted),
                                  _ptr(committed), _ptr(n_committed), _ptr(dbg_topk_ids),
                                  _ptr(ws), ws_bytes, _stream(stream)))


def moe_verify_step_one_launch(cfg: MvConfig, weights: MvWeights, B: int, K: int, h_in, drafts, h_out,
                               argmax, n_accepted, committed, n_committed, dbg_topk_ids=None, ws=None,
                               ws_bytes: int = 0, stream=None) -> None:
    _check(load().moe_verify_step_one_launch(ctypes.byref(cfg), ctypes.byref(weights), B, K, _ptr(h_in),
                                             _ptr(drafts), _ptr(h_out), _ptr(argmax), _ptr(n_accepted),
                                             _ptr(committed), _ptr(n_committed), _ptr(dbg_topk_ids),
                                             _ptr(ws), ws_bytes, _stream(stream)))


def moe_verify_step_noalloc(cfg: MvConfig, weights: MvWeights, B: int, K: int, h_in, drafts, h_out,
                            argmax, n_accepted, committed, n_committed, dbg_topk_ids=None,
                            stream=None) -> None:
    _check(load().moe_verify_step_noalloc(ctypes.byref(cfg), ctypes.byref(weights), B, K, _ptr(h_in),
                                          _ptr(drafts), _ptr(h_out), _ptr(argmax), _ptr(n_accepted),
                                          _ptr(committed), _ptr(n_committed), _ptr(dbg_topk_ids),
                                          _stream(stream)))


def spec_accept(B: int, K: int, argmax, drafts, n_accepted, committed, n_committed,
                stream=None) -> None:
    _check(load().spec_accept(B, K, _ptr(argmax), _ptr(drafts), _ptr(n_accepted),
                              _ptr(committed), _ptr(n_committed), _stream(stream)))


def mtp_workspace_bytes(cfg: MvConfig, d_ff: int, max_rows: int) -> int:
    return int(load().mtp_workspace_bytes(ctypes.byref(cfg), int(d_ff), int(max_rows)))


def mtp_draft(cfg: MvConfig, weights: MvWeights, mtp: MtpWeights, B: int, K: int, h_in, tokens,
              drafts, h_out=None, ws=None, ws_bytes: int = 0, stream=None) -> None:
    _check(load().mtp_draft(ctypes.byref(cfg), ctypes.byref(weights), ctypes.byref(mtp), B, K,
                            _ptr(h_in), _ptr(tokens), _ptr(drafts), _ptr(h_out), _ptr(ws),
                            ws_bytes, _stream(stream)))


def mv_choose_k(q: float, cost) -> tuple:
    """(K, rate): the draft length with the most expected committed tokens
    per unit of cost, cost[K] for K = 0 .. len(cost) - 1."""
    c = (ctypes.c_float * len(cost))(*[float(x) for x in cost])
    k = ctypes.c_int32(-1)
    r = ctypes.c_float(0.0)
    _check(load().mv_choose_k(len(cost) - 1, float(q), c, ctypes.byref(k), ctypes.byref(r)))
    return int(k.value), float(r.value)


def mv_step_bytes(cfg: MvConfig, B: int, K: int, d_ff_mtp: int) -> float:
    v = float(load().mv_step_bytes(ctypes.byref(cfg), int(B), int(K), int(d_ff_mtp)))
    if v < 0:
        raise MvError(MV_ERR_SHAPE, mv_last_error())
    return v


def mv_step_status(ws, status, stream=None) -> None:
    """Enqueue the copy of workspace ws's status word into status[0] (int32)."""
    _check(load().mv_step_status(_ptr(ws), _ptr(status), _stream(stream)))


def mv_set_spin_limit(polls: int) -> int:
    """Bound of the fused launch's waits for later calls (< 0: the default);
    returns the previous bound."""
    return int(load().mv_set_spin_limit(int(polls)))


# ---------------------------------------------------------------- device memory


class DeviceModel:
    """Weights resident in device memory (torch tensors) plus the C structs
    that point at them, and a workspace sized for ``max_tokens`` rows."""

    def __init__(self, dims, weights: Dict[str, Optional[np.ndarray]], max_tokens: int,
                 device: str = "cuda"):
        import torch

        self.dims = dims
        self.cfg = make_config(dims)
        self.tensors: Dict[str, Optional["torch.Tensor"]] = {}
        for name, arr in weights.items():
            self.tensors[name] = None if arr is None else to_device(arr, device)
        self.weights = MvWeights(*[_ptr(self.tensors.get(n)) for n, _ in MvWeights._fields_])
        self.ws_bytes = mv_workspace_bytes(self.cfg, max_tokens)
        if self.ws_bytes == 0 and max_tokens > 0:
            raise MvError(MV_ERR_UNSUPPORTED, mv_last_error())
        self.ws = torch.empty(max(self.ws_bytes, 256), dtype=torch.uint8, device=device)
        self.max_tokens = max_tokens

    def with_router_bias(self, bias: Optional[np.ndarray]) -> "DeviceModel":
        """Same weights and workspace, another router bias [L, E] (or none)."""
        import copy

        m = copy.copy(self)
        m.tensors = dict(self.tensors)
        m.tensors["router_b"] = None if bias is None else to_device(
            np.asarray(bias, np.float32), self.ws.device)
        m.weights = MvWeights(*[_ptr(m.tensors.get(n)) for n, _ in MvWeights._fields_])
        return m


class DeviceMtp:
    """FastMTP draft-block weights in device memory, the C struct pointing at
    them, and a workspace for up to ``max_rows`` sequences."""

    def __init__(self, dims, mtp: Dict[str, np.ndarray], max_rows: int, device: str = "cuda"):
        import torch

        names = [n for n, _ in MtpWeights._fields_ if n != "d_ff"]
        self.tensors = {n: to_device(mtp[n], device) for n in names}
        self.d_ff = int(mtp["w_down"].shape[1])
        self.weights = MtpWeights(*[_ptr(self.tensors[n]) for n in names], self.d_ff)
        cfg = make_config(dims)
        self.ws_bytes = mtp_workspace_bytes(cfg, self.d_ff, max_rows)
        if self.ws_bytes == 0 and max_rows > 0:
            raise MvError(MV_ERR_UNSUPPORTED, mv_last_error())
        self.ws = torch.empty(max(self.ws_bytes, 256), dtype=torch.uint8, device=device)


def run_mtp_draft(model: DeviceModel, mtp: DeviceMtp, h_in, tokens, K: int, stream=None):
    """Allocate drafts [B, K] and h_out [B, d], enqueue one mtp_draft (no sync)."""
    import torch

    B = h_in.shape[0]
    out = dict(drafts=torch.empty((B, K), dtype=torch.int32, device=h_in.device),
               h_out=torch.empty_like(h_in))
    mtp_draft(model.cfg, model.weights, mtp.weights, B, K, h_in, tokens, out["drafts"],
              out["h_out"], mtp.ws, mtp.ws_bytes, stream)
    return out


def step_status(model: "DeviceModel", stream=None) -> int:
    """Status word of the last call on the model's workspace (0: every wait
    of that call ended as it should); synchronises the stream."""
    import torch

    out = torch.empty(1, dtype=torch.int32, device=model.ws.device)
    mv_step_status(model.ws, out, stream)
    return int(out.cpu()[0])


def to_device(arr: np.ndarray, device: str = "cuda"):
    """numpy (float32, int32 or uint16 bf16 bits) -> torch device tensor."""
    import torch

    arr = np.ascontiguousarray(arr)
    if arr.dtype == np.uint16:
        return torch.from_numpy(arr.view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(arr).to(device)


def to_host(t) -> np.ndarray:
    """torch tensor -> numpy; bf16 comes back as uint16 bit patterns."""
    import torch

    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


# ---------------------------------------------------------------- convenience


def run_verify_step(model: DeviceModel, h_in, drafts, B: int, K: int, h_out: bool = True,
                    routing: bool = False, stream=None, one_launch: bool = False) -> Dict[str, object]:
    """Allocate the outputs and enqueue one moe_verify_step, or with
    one_launch moe_verify_step_one_launch (no sync)."""
    import torch

    dev = h_in.device
    T = B * (K + 1)
    out = dict(
        argmax=torch.empty(T, dtype=torch.int32, device=dev),
        n_accepted=torch.empty(B, dtype=torch.int32, device=dev),
        committed=torch.empty((B, K + 1), dtype=torch.int32, device=dev),
        n_committed=torch.empty(B, dtype=torch.int32, device=dev),
        h_out=torch.empty_like(h_in) if h_out else None,
        topk_ids=(torch.empty((model.dims.n_layers, T, model.dims.top_k), dtype=torch.int32,
                              device=dev) if routing else None),
    )
    step = moe_verify_step_one_launch if one_launch else moe_verify_step
    step(model.cfg, model.weights, B, K, h_in, drafts, out["h_out"], out["argmax"],
         out["n_accepted"], out["committed"], out["n_committed"], out["topk_ids"],
         model.ws, model.ws_bytes, stream)
    return out


def run_layer_forward(model: DeviceModel, layer: int, h_in, stream=None) -> Dict[str, object]:
    """Allocate the outputs and enqueue one moe_layer_forward (no sync)."""
    import torch

    dev = h_in.device
    T = h_in.shape[0]
    out = dict(
        h_out=torch.empty_like(h_in),
        topk_ids=torch.empty((T, model.dims.top_k), dtype=torch.int32, device=dev),
        topk_w=torch.empty((T, model.dims.top_k), dtype=torch.float32, device=dev),
        y_moe=torch.empty((T, model.dims.d_model), dtype=torch.float32, device=dev),
    )
    moe_layer_forward(model.cfg, model.weights, layer, T, h_in, out["h_out"], out["topk_ids"],
                      out["topk_w"], out["y_moe"], model.ws, model.ws_bytes, stream)
    return out
