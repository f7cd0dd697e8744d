"""The C-ABI library loads, exports every entry point include/dflash.h declares,
and rejects invalid arguments on the host before touching the GPU (CPU only:
every call here returns from argument checks, none launches a kernel)."""
import ctypes
import os
import re

import pytest

from block_diffusion_drafter_injection_amd import binding as B
from block_diffusion_drafter_injection_amd import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dflash.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(dflash_[a-z_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(B.LIB_PATH):
        from block_diffusion_drafter_injection_amd import build
        build.build()
    return B.lib()


def test_every_declared_symbol_is_exported(L):
    names = declared_functions()
    assert len(names) >= 8
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(B.EXPORTS)


def test_status_strings(L):
    for code in range(0, -7, -1):
        assert B.dflash_status_string(code) != "unknown status"


def _cfg(**kw):
    c = B.make_config(synth.small_dims())
    for k, v in kw.items():
        setattr(c, k, v)
    return c


def test_workspace_size_rejects_bad_configs(L):
    assert B.dflash_workspace_size(_cfg(), 4, 8, 64, 512) > 0
    assert B.dflash_workspace_size(_cfg(head_dim=96), 4, 8, 64, 512) == 0
    assert B.dflash_workspace_size(_cfg(n_kv_heads=3), 4, 8, 64, 512) == 0
    assert B.dflash_workspace_size(_cfg(page_size=32), 4, 8, 64, 512) == 0
    assert B.dflash_workspace_size(_cfg(dtype=7), 4, 8, 64, 512) == 0
    assert B.dflash_workspace_size(_cfg(), 4, 17, 64, 512) > 0    # a target forward of 17 tokens
    assert B.dflash_workspace_size(_cfg(), 4, 33, 64, 512) == 0
    assert B.dflash_workspace_size(_cfg(hidden=500), 4, 8, 64, 512) == 0
    assert B.dflash_workspace_size(_cfg(hidden=8256), 4, 8, 64, 512) == 0   # rows wider than 8192
    assert B.dflash_workspace_size(_cfg(denoise_schedule=1), 4, 8, 64, 512) > 0
    assert B.dflash_workspace_size(_cfg(denoise_schedule=3), 4, 8, 64, 512) == 0


def test_workspace_grows_with_batch_and_context(L):
    c = B.make_config(synth.QWEN3_8B_SHAPE)
    a = B.dflash_workspace_size(c, 1, 16, 0, 4096)
    b = B.dflash_workspace_size(c, 32, 16, 0, 4096)
    assert b > a > 0
    assert B.dflash_workspace_size(c, 32, 16, 8192, 0) >= B.dflash_workspace_size(c, 32, 16, 1024, 0)


def _weights_stub(n_layers):
    arr = (ctypes.c_void_p * n_layers)(*([8] * n_layers))
    pp = ctypes.cast(arr, ctypes.POINTER(ctypes.c_void_p))
    w = B.dflash_weights(8, 8, 8, 8, 8, pp, pp, pp, pp, pp, pp, pp)
    return w, arr


def _draft(L, cfg, w, **kw):
    args = dict(pool=8, n_pages=4, table=8, max_pages=4, ctx=8, max_ctx=16, batch=2, B=8, S=2, T=0.0,
                anchor=None, tok=8, ws=256, ws_bytes=1 << 40)
    args.update(kw)
    return L.dflash_draft_block(ctypes.byref(cfg), ctypes.byref(w), args["pool"], args["n_pages"], args["table"],
                                args["max_pages"], args["ctx"], args["max_ctx"], args["batch"], args["B"],
                                args["S"], args["T"], 0, args["anchor"], args["tok"], None, None, args["ws"],
                                args["ws_bytes"], None)


def test_draft_argument_errors_return_before_launch(L):
    cfg = _cfg()
    w, keep = _weights_stub(cfg.n_layers)
    assert _draft(L, cfg, w, B=17) == -4
    assert _draft(L, cfg, w, B=0) == -4
    assert _draft(L, cfg, w, S=9) == -1
    assert _draft(L, cfg, w, S=0) == -1
    assert _draft(L, cfg, w, T=-1.0) == -1
    assert _draft(L, cfg, w, T=float("nan")) == -1
    assert _draft(L, cfg, w, tok=None) == -1
    assert _draft(L, cfg, w, ws=None) == -5
    assert _draft(L, cfg, w, ws=300) == -5                      # not 256-byte aligned
    assert _draft(L, cfg, w, ws_bytes=1024) == -5               # too small
    assert _draft(L, _cfg(dtype=5), w) == -3
    assert _draft(L, _cfg(mask_token_id=-1), w) == -1
    assert _draft(L, _cfg(denoise_schedule=2), w) == -1         # unknown schedule
    assert _draft(L, _cfg(denoise_schedule=-1), w) == -1
    assert _draft(L, cfg, w, batch=0) == 0                      # nothing to do
    assert _draft(L, cfg, w, S=8, anchor=8) == -1               # an anchor leaves B - 1 positions to denoise
    assert _draft(L, cfg, w, B=1, S=1, anchor=8) == -1          # nothing left to draft
    w2, keep2 = _weights_stub(cfg.n_layers)
    keep2[1] = None
    assert _draft(L, cfg, w2) == -1                             # a missing per-layer weight


def _target(L, cfg, w, **kw):
    args = dict(pool=8, n_pages=4, table=8, max_pages=4, ctx=8, max_ctx=16, batch=2, n=17, tokens=8, caps=[0],
                logits=8, hidden=8, ws=256, ws_bytes=1 << 40)
    args.update(kw)
    caps = (ctypes.c_int32 * max(len(args["caps"]), 1))(*args["caps"])
    return L.dflash_target_forward(ctypes.byref(cfg), ctypes.byref(w), args["pool"], args["n_pages"], args["table"],
                                   args["max_pages"], args["ctx"], args["max_ctx"], args["batch"], args["n"],
                                   args["tokens"], caps, len(args["caps"]), args["logits"], args["hidden"],
                                   args["ws"], args["ws_bytes"], None)


def test_target_forward_argument_errors_return_before_launch(L):
    cfg = _cfg()
    w, keep = _weights_stub(cfg.n_layers)
    assert _target(L, cfg, w, n=0) == -4
    assert _target(L, cfg, w, n=33) == -4
    assert _target(L, _cfg(dtype=0), w) == -2                   # fp32 target: not supported
    assert _target(L, _cfg(head_dim=64), w) == -2               # head_dim 64: not supported
    assert _target(L, cfg, w, caps=[cfg.n_layers]) == -1       # capture layer out of range
    assert _target(L, cfg, w, caps=[0, 0]) == -1               # repeated capture layer
    assert _target(L, cfg, w, hidden=None) == -1               # captures without an output
    assert _target(L, cfg, w, tokens=None) == -1
    assert _target(L, cfg, w, logits=None) == -1
    assert _target(L, cfg, w, ws=300) == -5
    assert _target(L, cfg, w, ws_bytes=1024) == -5
    assert _target(L, cfg, w, batch=0) == 0                     # nothing to do
    assert _target(L, cfg, w, batch=0, caps=[]) == 0
    # QK-norm targets are not limited to 16 layers (only injection is)
    qk = _cfg(qk_norm=1, n_layers=36)
    w36, keep36 = _weights_stub(36)
    w36.q_norm = w36.w_q
    w36.k_norm = w36.w_q
    assert _target(L, qk, w36, batch=0) == 0
    assert L.dflash_inject_kv(ctypes.byref(qk), ctypes.byref(w36), 8, 8, 8, 1, 8, 4, 8, 1, 4, 256, 1 << 40,
                              None) == -4


def test_verify_and_inject_argument_errors(L):
    f = L.dflash_verify_block
    assert f(2, 17, 100, 8, 8, 0.0, None, None, 8, 8, 256, 1 << 30, None) == -4
    assert f(2, 8, 100, 8, 8, 1.0, None, None, 8, 8, 256, 1 << 30, None) == -1   # T > 0 needs draft logits
    assert f(2, 8, 100, None, 8, 0.0, None, None, 8, 8, 256, 1 << 30, None) == -1
    assert f(2, 8, 100, 8, 8, 0.0, None, None, 8, 8, 256, 8, None) == -5
    # one byte short of the documented size is refused before any launch (sampled path too)
    need = L.dflash_verify_workspace_size(32, 16, 151936)
    assert need > 32 * 33 * 19 * 16                 # chunk pairs alone are not enough
    assert f(32, 16, 151936, 8, 8, 1.0, 8, 8, 8, 8, 256, need - 1, None) == -5
    assert f(32, 16, 151936, 8, 8, 0.0, None, None, 8, 8, 256, need - 1, None) == -5
    assert f(0, 8, 100, None, None, 0.0, None, None, None, None, None, 0, None) == 0
    cfg = _cfg()
    w, keep = _weights_stub(cfg.n_layers)
    g = L.dflash_inject_kv
    assert g(ctypes.byref(cfg), ctypes.byref(w), 8, 8, 8, -1, 8, 4, 8, 1, 4, 256, 1 << 30, None) == -1
    assert g(ctypes.byref(cfg), ctypes.byref(w), 8, 8, 8, 0, 8, 4, 8, 1, 4, 256, 1 << 30, None) == 0
    assert g(ctypes.byref(cfg), ctypes.byref(w), None, 8, 8, 5, 8, 4, 8, 1, 4, 256, 1 << 30, None) == -1
    assert g(ctypes.byref(cfg), ctypes.byref(w), 8, 8, 8, 5, 8, 4, 8, 1, 4, 256, 16, None) == -5


def test_advance_context_argument_errors(L):
    f = L.dflash_advance_context
    assert f(-1, 8, 8, 8, 8, 8, None) == -1
    assert f(2, 0, 8, 8, 8, 8, None) == -4
    assert f(2, 17, 8, 8, 8, 8, None) == -4
    assert f(2, 8, None, 8, 8, 8, None) == -1
    assert f(2, 8, 8, 8, None, 8, None) == -1
    assert f(0, 8, None, None, None, None, None) == 0


def test_profiler_select_validates_class(L):
    assert L.dflash_prof_select(99) == -1
    assert L.dflash_prof_select(0) == 0


def test_debug_variant_exports_the_same_symbols():
    if not os.path.exists(B.DEBUG_LIB_PATH):
        from block_diffusion_drafter_injection_amd import build
        build.build()
    D = B.debug_lib()
    for n in declared_functions():
        assert hasattr(D, n), n
