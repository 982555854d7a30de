"""The C ABI without a GPU: the library loads, exports every function the
header declares, sizes workspaces, and rejects bad arguments before it
enqueues anything."""
import ctypes
import os
import re

import pytest

from speculative_decode_verification_router_amd import binding as bd
from speculative_decode_verification_router_amd import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_verify.h")


def header_functions():
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_]\w*\s*\**\s*([A-Za-z_]\w*)\s*\(", text, re.M)
    return sorted(set(names) - {"if", "while", "for", "return"})


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(bd.LIB_PATH):
        from speculative_decode_verification_router_amd import build

        build.build()
    return bd.load()


def test_header_declares_the_boundary():
    assert header_functions() == sorted(bd.EXPORTED)


def test_library_exports_every_declared_function(lib):
    for name in header_functions():
        assert hasattr(lib, name), name


def _cfg(dims=synth.DS3B_BF16, **kw):
    c = bd.make_config(dims)
    for k, v in kw.items():
        setattr(c, k, v)
    return c


def test_workspace_bytes(lib):
    c = _cfg()
    w4, w128 = bd.mv_workspace_bytes(c, 4), bd.mv_workspace_bytes(c, 128)
    assert 0 < w4 < w128
    assert w4 % 256 == 0
    # dominant terms: fp32 slot buffer and bf16 SwiGLU rows, 8 slots per token
    assert w128 >= 128 * 8 * (1280 * 4 + 896 * 2)
    assert bd.mv_workspace_bytes(c, 0) > 0
    assert bd.mv_workspace_bytes(c, -1) == 0
    assert bd.mv_workspace_bytes(c, 65536) == 0
    assert bd.mv_workspace_bytes(_cfg(d_model=1000), 4) == 0
    assert bd.mv_workspace_bytes(_cfg(dtype=7), 4) == 0


FAKE = 0x1000  # never dereferenced: every call below fails validation or is a no-op


def _weights(**kw):
    w = bd.MvWeights(*([FAKE] * 9))
    w.router_b = None
    for k, v in kw.items():
        setattr(w, k, v)
    return w


def _verify(lib, cfg, w, B=1, K=3, h_in=FAKE, drafts=FAKE, argmax=FAKE, ws=FAKE, ws_bytes=1 << 40):
    return lib.moe_verify_step(ctypes.byref(cfg) if cfg is not None else None,
                               ctypes.byref(w) if w is not None else None, B, K, h_in, drafts,
                               None, argmax, FAKE, FAKE, FAKE, None, ws, ws_bytes, None)


@pytest.mark.parametrize("case,code", [
    (dict(cfg=None), bd.MV_ERR_NULL),
    (dict(w=None), bd.MV_ERR_NULL),
    (dict(h_in=None), bd.MV_ERR_NULL),
    (dict(argmax=None), bd.MV_ERR_NULL),
    (dict(drafts=None), bd.MV_ERR_NULL),
    (dict(ws=None), bd.MV_ERR_NULL),
    (dict(B=-1), bd.MV_ERR_SHAPE),
    (dict(K=-1), bd.MV_ERR_SHAPE),
    (dict(K=16), bd.MV_ERR_SHAPE),
    (dict(B=20000, K=3), bd.MV_ERR_SHAPE),
    (dict(ws_bytes=1024), bd.MV_ERR_WORKSPACE),
    (dict(ws=FAKE + 8), bd.MV_ERR_WORKSPACE),
    (dict(cfg_kw=dict(dtype=3)), bd.MV_ERR_UNSUPPORTED),
    (dict(cfg_kw=dict(top_k=9)), bd.MV_ERR_UNSUPPORTED),
    (dict(cfg_kw=dict(n_routed=65)), bd.MV_ERR_UNSUPPORTED),
    (dict(cfg_kw=dict(d_model=1300)), bd.MV_ERR_UNSUPPORTED),
    (dict(cfg_kw=dict(d_ff=100)), bd.MV_ERR_UNSUPPORTED),
    (dict(cfg_kw=dict(rms_eps=0.0)), bd.MV_ERR_UNSUPPORTED),
    (dict(w_kw=dict(lm_head=None)), bd.MV_ERR_NULL),
    (dict(w_kw=dict(ws_down=None)), bd.MV_ERR_NULL),
])
def test_verify_step_rejects_bad_arguments(lib, case, code):
    case = dict(case)
    cfg = _cfg(**case.pop("cfg_kw", {})) if "cfg" not in case else case.pop("cfg")
    w = _weights(**case.pop("w_kw", {})) if "w" not in case else case.pop("w")
    assert _verify(lib, cfg, w, **case) == code
    assert bd.mv_last_error() != ""


def test_zero_sequences_is_a_no_op(lib):
    assert _verify(lib, _cfg(), _weights(), B=0, h_in=None, argmax=None, ws=None) == bd.MV_OK
    assert bd.mv_last_error() == ""


def test_layer_forward_rejects_bad_arguments(lib):
    cfg, w = _cfg(), _weights()
    call = lambda layer, T, h_in=FAKE, ws=FAKE, ws_bytes=1 << 40: lib.moe_layer_forward(
        ctypes.byref(cfg), ctypes.byref(w), layer, T, h_in, FAKE, None, None, None, ws, ws_bytes, None)
    assert call(12, 4) == bd.MV_ERR_SHAPE
    assert call(-1, 4) == bd.MV_ERR_SHAPE
    assert call(0, -1) == bd.MV_ERR_SHAPE
    assert call(0, 4, h_in=None) == bd.MV_ERR_NULL
    assert call(0, 4, ws_bytes=10) == bd.MV_ERR_WORKSPACE
    assert call(0, 0, h_in=None, ws=None) == bd.MV_OK


def test_spec_accept_rejects_bad_arguments(lib):
    assert lib.spec_accept(-1, 3, FAKE, FAKE, FAKE, FAKE, FAKE, None) == bd.MV_ERR_SHAPE
    assert lib.spec_accept(1, 16, FAKE, FAKE, FAKE, FAKE, FAKE, None) == bd.MV_ERR_SHAPE
    assert lib.spec_accept(1, 3, None, FAKE, FAKE, FAKE, FAKE, None) == bd.MV_ERR_NULL
    assert lib.spec_accept(1, 3, FAKE, None, FAKE, FAKE, FAKE, None) == bd.MV_ERR_NULL
    assert lib.spec_accept(0, 3, None, None, None, None, None, None) == bd.MV_OK


# ---------------------------------------------------------------- draft block


def test_mtp_workspace_bytes(lib):
    c = _cfg()
    w1, w16 = bd.mtp_workspace_bytes(c, 1792, 1), bd.mtp_workspace_bytes(c, 1792, 16)
    assert 0 < w1 < w16 and w16 % 256 == 0
    # projection input [B, 2d], fp32 accumulator [B, d], FFN products [B, Fm]
    assert w16 >= 16 * (2 * 1280 * 2 + 1280 * 4 + 1792 * 2)
    assert bd.mtp_workspace_bytes(c, 1800, 4) == 0           # not a multiple of 64
    assert bd.mtp_workspace_bytes(c, 8192, 4) == 0           # FFN tile too wide for LDS
    assert bd.mtp_workspace_bytes(_cfg(d_model=4096), 1792, 4) == 0  # projection tile too wide
    assert bd.mtp_workspace_bytes(c, 1792, -1) == 0
    assert bd.mtp_workspace_bytes(_cfg(dims=synth.TINY_F32), 256, 4) > 0


def _mtp(**kw):
    m = bd.MtpWeights(*([FAKE] * 8), 1792)
    for k, v in kw.items():
        setattr(m, k, v)
    return m


def _draft(lib, cfg, w, m, B=1, K=3, h_in=FAKE, tokens=FAKE, drafts=FAKE, ws=FAKE, ws_bytes=1 << 40):
    return lib.mtp_draft(ctypes.byref(cfg), ctypes.byref(w) if w is not None else None,
                         ctypes.byref(m) if m is not None else None, B, K, h_in, tokens, drafts,
                         None, ws, ws_bytes, None)


@pytest.mark.parametrize("case,code", [
    (dict(w=None), bd.MV_ERR_NULL),
    (dict(m=None), bd.MV_ERR_NULL),
    (dict(h_in=None), bd.MV_ERR_NULL),
    (dict(tokens=None), bd.MV_ERR_NULL),
    (dict(drafts=None), bd.MV_ERR_NULL),
    (dict(ws=None), bd.MV_ERR_NULL),
    (dict(B=-1), bd.MV_ERR_SHAPE),
    (dict(K=16), bd.MV_ERR_SHAPE),
    (dict(B=70000), bd.MV_ERR_SHAPE),
    (dict(ws_bytes=1024), bd.MV_ERR_WORKSPACE),
    (dict(ws=FAKE + 8), bd.MV_ERR_WORKSPACE),
    (dict(m_kw=dict(d_ff=100)), bd.MV_ERR_UNSUPPORTED),
    (dict(m_kw=dict(w_proj=None)), bd.MV_ERR_NULL),
    (dict(w_kw=dict(lm_head=None)), bd.MV_ERR_NULL),
])
def test_mtp_draft_rejects_bad_arguments(lib, case, code):
    case = dict(case)
    w = _weights(**case.pop("w_kw", {})) if "w" not in case else case.pop("w")
    m = _mtp(**case.pop("m_kw", {})) if "m" not in case else case.pop("m")
    assert _draft(lib, _cfg(), w, m, **case) == code
    assert bd.mv_last_error() != ""


def test_mtp_draft_zero_work_is_a_no_op(lib):
    assert _draft(lib, _cfg(), _weights(), _mtp(), B=0, h_in=None, tokens=None, drafts=None,
                  ws=None) == bd.MV_OK
    assert _draft(lib, _cfg(), _weights(), _mtp(), K=0, h_in=None, tokens=None, drafts=None,
                  ws=None) == bd.MV_OK


# ---------------------------------------------------------------- call status


def test_step_status_rejects_bad_arguments(lib):
    assert lib.mv_step_status(FAKE, None, None) == bd.MV_ERR_NULL
    assert lib.mv_step_status(FAKE + 8, FAKE, None) == bd.MV_ERR_WORKSPACE
    assert bd.mv_last_error() != ""


def test_spin_limit_hook_round_trip(lib):
    default = 1 << 18
    assert bd.mv_set_spin_limit(5) == default
    assert bd.mv_set_spin_limit(0) == 5
    assert bd.mv_set_spin_limit(-1) == 0
    assert bd.mv_set_spin_limit(-1) == default


def test_status_word_sits_before_every_region(lib):
    """The status word is at offset 0 whatever the call's T: a workspace
    sized for T rows is larger than one sized for fewer rows by whole
    regions, never by a shift of the status word (it is the first region)."""
    c = _cfg()
    assert bd.mv_workspace_bytes(c, 0) >= 256


def test_noalloc_verify_step_rejects_bad_arguments(lib):
    """Validation happens before the static scratch is looked up: none of
    these touches a device."""
    cfg, w = _cfg(), _weights()

    def call(B=1, K=3, h_in=FAKE, argmax=FAKE, c=cfg, ww=w):
        return lib.moe_verify_step_noalloc(ctypes.byref(c), ctypes.byref(ww), B, K, h_in, FAKE, None, argmax,
                                           FAKE, FAKE, FAKE, None, None)
    assert call(h_in=None) == bd.MV_ERR_NULL
    assert call(argmax=None) == bd.MV_ERR_NULL
    assert call(K=16) == bd.MV_ERR_SHAPE
    assert call(c=_cfg(dtype=3)) == bd.MV_ERR_UNSUPPORTED
    # 64 sequences x 4 rows need 16.2 MiB of workspace, above the 16 MiB array
    assert bd.mv_workspace_bytes(cfg, 256) > 16 << 20 >= bd.mv_workspace_bytes(cfg, 128)
    assert call(B=64) == bd.MV_ERR_WORKSPACE
    assert "16 MiB" in bd.mv_last_error()
    assert call(B=0, h_in=None, argmax=None) == bd.MV_OK


def test_one_launch_verify_step_rejects_bad_arguments(lib):
    """The one-launch step takes batches of at most 8 rows and 16 layers; it
    validates like moe_verify_step before anything is enqueued."""
    cfg, w = _cfg(), _weights()

    def call(B=1, K=3, h_in=FAKE, argmax=FAKE, c=cfg, ws_bytes=1 << 40):
        return lib.moe_verify_step_one_launch(ctypes.byref(c), ctypes.byref(w), B, K, h_in, FAKE, None, argmax,
                                              FAKE, FAKE, FAKE, None, FAKE, ws_bytes, None)
    assert call(h_in=None) == bd.MV_ERR_NULL
    assert call(K=16) == bd.MV_ERR_SHAPE
    assert call(ws_bytes=1024) == bd.MV_ERR_WORKSPACE
    assert call(B=3, K=3) == bd.MV_ERR_UNSUPPORTED  # 12 rows
    assert "8 rows" in bd.mv_last_error()
    assert call(c=_cfg(n_layers=17)) == bd.MV_ERR_UNSUPPORTED
    assert call(B=0, h_in=None, argmax=None) == bd.MV_OK


def test_one_launch_workspace_holds_its_counters(lib):
    """Batches of up to 8 rows reserve the one-launch step's counter lines
    (one set per layer) and argument block; larger batches do not."""
    c = _cfg()
    per_row = bd.mv_workspace_bytes(c, 9) - bd.mv_workspace_bytes(c, 8)
    assert per_row < 0  # the 8-row workspace carries the one-launch regions
    assert bd.mv_workspace_bytes(c, 8) - bd.mv_workspace_bytes(c, 4) > 0
