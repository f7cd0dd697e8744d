"""ctypes binding of libdflash (include/dflash.h): argument marshalling only.

Every function here converts torch tensors to device pointers and calls the
C entry point of the same name; all computation happens in the HIP library.
If the library has not been built this module raises on first use — there
is no fallback path.
"""
import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("DFLASH_LIB") or os.path.join(_PKG, "libdflash.so")
# the same kernels behind a host layer that checks device-resident indices first
DEBUG_LIB_PATH = os.path.join(_PKG, "libdflash_debug.so")

DFLASH_F32, DFLASH_BF16 = 0, 1
SCHEDULES = {"progressive": 0, "repredict": 1}   # dflash_schedule
PROF = dict(none=0, attn=1, gemm_qkv=2, gemm_o=3, gemm_gateup=4, gemm_down=5, lmhead=6, inject_fc=7,
            inject_kv=8, verify=9)
STATUS = {0: "ok", -1: "invalid argument", -2: "unsupported or inconsistent shape", -3: "unknown dtype",
          -4: "capacity exceeded", -5: "workspace missing, misaligned or too small", -6: "HIP error"}


class DflashError(RuntimeError):
    def __init__(self, fn, code):
        super().__init__(f"{fn} returned {code} ({STATUS.get(code, '?')})")
        self.code = code


class dflash_config(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "hidden", "n_layers", "n_q_heads", "n_kv_heads", "head_dim", "intermediate", "vocab", "n_fuse",
        "target_hidden", "page_size", "mask_token_id")] + [
        ("rope_base", ctypes.c_float), ("rms_eps", ctypes.c_float), ("dtype", ctypes.c_int32),
        ("denoise_schedule", ctypes.c_int32), ("qk_norm", ctypes.c_int32)]


_PP = ctypes.POINTER(ctypes.c_void_p)


class dflash_weights(ctypes.Structure):
    _fields_ = [("w_fc", ctypes.c_void_p), ("w_kv", ctypes.c_void_p), ("embed", ctypes.c_void_p),
                ("final_norm", ctypes.c_void_p), ("lm_head", ctypes.c_void_p),
                ("attn_norm", _PP), ("w_q", _PP), ("w_o", _PP), ("mlp_norm", _PP),
                ("w_gate", _PP), ("w_up", _PP), ("w_down", _PP), ("q_norm", _PP), ("k_norm", _PP)]


_libs = {}
EXPORTS = ["dflash_workspace_size", "dflash_inject_kv", "dflash_draft_block", "dflash_verify_workspace_size",
           "dflash_verify_block", "dflash_verify_block_static", "dflash_advance_context",
           "dflash_adaptive_block_size", "dflash_target_forward",
           "dflash_status_string",
           "dflash_prof_select", "dflash_prof_collect"]


def lib():
    """Load libdflash.so (raises if it is missing)."""
    return _load(LIB_PATH)


def debug_lib():
    """Load libdflash_debug.so, the variant that checks device indices on the host."""
    return _load(DEBUG_LIB_PATH)


def _load(path):
    if path in _libs:
        return _libs[path]
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run python -m block_diffusion_drafter_injection_amd.build")
    L = ctypes.CDLL(path)
    vp, i32, sz, f32, u64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t, ctypes.c_float, ctypes.c_uint64
    cfgp, wp = ctypes.POINTER(dflash_config), ctypes.POINTER(dflash_weights)
    L.dflash_workspace_size.argtypes = [cfgp, i32, i32, i32, i32]
    L.dflash_workspace_size.restype = sz
    L.dflash_inject_kv.argtypes = [cfgp, wp, vp, vp, vp, i32, vp, i32, vp, i32, i32, vp, sz, vp]
    L.dflash_inject_kv.restype = i32
    L.dflash_draft_block.argtypes = [cfgp, wp, vp, i32, vp, i32, vp, i32, i32, i32, i32, f32, u64, vp, vp, vp,
                                     vp, vp, sz, vp]
    L.dflash_draft_block.restype = i32
    L.dflash_verify_workspace_size.argtypes = [i32, i32, i32]
    L.dflash_verify_workspace_size.restype = sz
    L.dflash_verify_block.argtypes = [i32, i32, i32, vp, vp, f32, vp, vp, vp, vp, vp, sz, vp]
    L.dflash_verify_block.restype = i32
    L.dflash_verify_block_static.argtypes = [i32, i32, i32, vp, vp, f32, vp, vp, vp, vp, vp]
    L.dflash_verify_block_static.restype = i32
    L.dflash_advance_context.argtypes = [i32, i32, vp, vp, vp, vp, vp]
    L.dflash_advance_context.restype = i32
    L.dflash_target_forward.argtypes = [cfgp, wp, vp, i32, vp, i32, vp, i32, i32, i32, vp,
                                        ctypes.POINTER(i32), i32, vp, vp, vp, sz, vp]
    L.dflash_target_forward.restype = i32
    ip, fp = ctypes.POINTER(i32), ctypes.POINTER(f32)
    L.dflash_adaptive_block_size.argtypes = [ip, ip, i32, ip, fp, i32, f32, f32, fp]
    L.dflash_adaptive_block_size.restype = i32
    L.dflash_status_string.argtypes = [i32]
    L.dflash_status_string.restype = ctypes.c_char_p
    L.dflash_prof_select.argtypes = [i32]
    L.dflash_prof_select.restype = i32
    L.dflash_prof_collect.argtypes = [ctypes.POINTER(f32), ctypes.POINTER(i32)]
    L.dflash_prof_collect.restype = i32
    _libs[path] = L
    return L


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _check(fn, code):
    if code != 0:
        raise DflashError(fn, code)


def make_config(dims, schedule="progressive"):
    """dflash_config from a ModelDims-like object; schedule is 'progressive' or 'repredict'."""
    return dflash_config(dims.hidden, dims.n_layers, dims.n_q_heads, dims.n_kv_heads, dims.head_dim,
                         dims.intermediate, dims.vocab, dims.n_fuse, dims.target_hidden, dims.page_size,
                         dims.mask_token_id, float(dims.rope_base), float(dims.rms_eps),
                         DFLASH_BF16 if dims.dtype == "bf16" else DFLASH_F32, SCHEDULES[schedule],
                         1 if getattr(dims, "qk_norm", False) else 0)


class Weights:
    """dflash_weights over a dict of device tensors (keeps the pointer arrays alive)."""

    def __init__(self, W):
        self.tensors = W
        L = len(W["w_q"])
        arr = ctypes.c_void_p * L
        self._arrays = {k: arr(*[t.data_ptr() for t in W[k]]) for k in
                        ("attn_norm", "w_q", "w_o", "mlp_norm", "w_gate", "w_up", "w_down", "q_norm", "k_norm")
                        if k in W}
        a = self._arrays
        qk = {k: ctypes.cast(a[k], _PP) if k in a else None for k in ("q_norm", "k_norm")}
        self.c = dflash_weights(W["w_fc"].data_ptr(), W["w_kv"].data_ptr(), W["embed"].data_ptr(),
                                W["final_norm"].data_ptr(), W["lm_head"].data_ptr(),
                                ctypes.cast(a["attn_norm"], _PP), ctypes.cast(a["w_q"], _PP),
                                ctypes.cast(a["w_o"], _PP), ctypes.cast(a["mlp_norm"], _PP),
                                ctypes.cast(a["w_gate"], _PP), ctypes.cast(a["w_up"], _PP),
                                ctypes.cast(a["w_down"], _PP), qk["q_norm"], qk["k_norm"])


def dflash_workspace_size(cfg, max_batch, block_size, max_inject_tokens, max_ctx_len):
    return lib().dflash_workspace_size(ctypes.byref(cfg), max_batch, block_size, max_inject_tokens, max_ctx_len)


def dflash_verify_workspace_size(batch, block_size, vocab):
    return lib().dflash_verify_workspace_size(batch, block_size, vocab)


def dflash_inject_kv(cfg, weights, target_hidden, tok_seq, tok_pos, n_tok, kv_pool, n_pages, block_table, n_seqs,
                     max_pages, workspace, ws_bytes, stream=None):
    code = lib().dflash_inject_kv(ctypes.byref(cfg), ctypes.byref(weights.c), _ptr(target_hidden), _ptr(tok_seq),
                                  _ptr(tok_pos), n_tok, _ptr(kv_pool), n_pages, _ptr(block_table), n_seqs,
                                  max_pages, _ptr(workspace), ws_bytes, _stream(stream))
    _check("dflash_inject_kv", code)


def dflash_draft_block(cfg, weights, kv_pool, n_pages, block_table, max_pages, ctx_len, max_ctx_len, batch,
                       block_size, n_steps, temperature, seed, out_tokens, out_logits, out_conf, workspace,
                       ws_bytes, stream=None, anchor=None):
    """anchor: optional device int32 [batch], the token block position 0 starts from."""
    code = lib().dflash_draft_block(ctypes.byref(cfg), ctypes.byref(weights.c), _ptr(kv_pool), n_pages,
                                    _ptr(block_table), max_pages, _ptr(ctx_len), max_ctx_len, batch, block_size,
                                    n_steps, float(temperature), int(seed), _ptr(anchor), _ptr(out_tokens),
                                    _ptr(out_logits), _ptr(out_conf), _ptr(workspace), ws_bytes, _stream(stream))
    _check("dflash_draft_block", code)


def dflash_verify_block(batch, block_size, vocab, target_logits, draft_tokens, temperature, draft_logits, uniforms,
                        accept_len, out_tokens, workspace, ws_bytes, stream=None):
    code = lib().dflash_verify_block(batch, block_size, vocab, _ptr(target_logits), _ptr(draft_tokens),
                                     float(temperature), _ptr(draft_logits), _ptr(uniforms), _ptr(accept_len),
                                     _ptr(out_tokens), _ptr(workspace), ws_bytes, _stream(stream))
    _check("dflash_verify_block", code)


def dflash_verify_block_static(batch, block_size, vocab, target_logits, draft_tokens, temperature, draft_logits,
                               uniforms, accept_len, out_tokens, stream=None):
    code = lib().dflash_verify_block_static(batch, block_size, vocab, _ptr(target_logits), _ptr(draft_tokens),
                                            float(temperature), _ptr(draft_logits), _ptr(uniforms), _ptr(accept_len),
                                            _ptr(out_tokens), _stream(stream))
    _check("dflash_verify_block_static", code)


def dflash_advance_context(batch, block_size, accept_len, ctx_len, tok_seq, tok_pos, stream=None):
    code = lib().dflash_advance_context(batch, block_size, _ptr(accept_len), _ptr(ctx_len), _ptr(tok_seq),
                                        _ptr(tok_pos), _stream(stream))
    _check("dflash_advance_context", code)


def dflash_target_forward(cfg, weights, kv_pool, n_pages, block_table, max_pages, ctx_len, max_ctx_len, batch,
                          n_tok, tokens, capture_layers, out_logits, out_hidden, workspace, ws_bytes, stream=None):
    caps = (ctypes.c_int32 * max(len(capture_layers), 1))(*[int(x) for x in capture_layers])
    code = lib().dflash_target_forward(ctypes.byref(cfg), ctypes.byref(weights.c), _ptr(kv_pool), n_pages,
                                       _ptr(block_table), max_pages, _ptr(ctx_len), max_ctx_len, batch, n_tok,
                                       _ptr(tokens), caps, len(capture_layers), _ptr(out_logits), _ptr(out_hidden),
                                       _ptr(workspace), ws_bytes, _stream(stream))
    _check("dflash_target_forward", code)


def dflash_adaptive_block_size(accept_len, block_of, cand_block, step_time, prior_a=1.0, prior_b=1.0):
    """Host lists in, (chosen block size, estimated match probability) out."""
    n, m = len(accept_len), len(cand_block)
    if len(block_of) != n or len(step_time) != m:
        raise ValueError("accept_len/block_of and cand_block/step_time must pair up")
    i32a, f32a = ctypes.c_int32, ctypes.c_float
    a = (i32a * max(n, 1))(*[int(x) for x in accept_len])
    b = (i32a * max(n, 1))(*[int(x) for x in block_of])
    c = (i32a * m)(*[int(x) for x in cand_block])
    t = (f32a * m)(*[float(x) for x in step_time])
    p = f32a(0.0)
    code = lib().dflash_adaptive_block_size(a, b, n, c, t, m, float(prior_a), float(prior_b), ctypes.byref(p))
    if code < 0:
        raise DflashError("dflash_adaptive_block_size", code)
    return int(code), float(p.value)


def dflash_status_string(code):
    return lib().dflash_status_string(code).decode()


def dflash_prof_select(kernel_class):
    k = PROF[kernel_class] if isinstance(kernel_class, str) else int(kernel_class)
    _check("dflash_prof_select", lib().dflash_prof_select(k))


def dflash_prof_collect():
    ms, n = ctypes.c_float(), ctypes.c_int32()
    _check("dflash_prof_collect", lib().dflash_prof_collect(ctypes.byref(ms), ctypes.byref(n)))
    return ms.value, n.value


def pool_elems(dims, n_pages):
    """Number of storage elements of a KV pool with n_pages pages."""
    return n_pages * dims.n_layers * 2 * dims.n_kv_heads * dims.page_size * dims.head_dim
