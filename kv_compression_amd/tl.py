"""Python binding of libtl.so (include/tl.h): argument marshalling only.

Every function here forwards to the C ABI of the same name; every step of the
decode path runs in the library's HIP kernels. PyTorch supplies device memory
(``torch.empty`` on the GPU) and the current HIP stream. There is no fallback:
if the library or a GPU is missing, loading fails with an error.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libtl.so")

TL_OK, TL_E_ARG, TL_E_UNSUPPORTED, TL_E_CAPACITY, TL_E_CACHE_GAP, TL_E_HIP = range(6)
MODES = {"kv": 0, "f32": 1, "f16": 2, "int8": 3, "int4": 4, "delta8": 5}
DTYPES = {"f32": 0, "f16": 1}
ATTN_ORDERS = {"explicit": 0, "absorbed": 1}
LANE_OK, LANE_ABORTED = 0, 1
MAX_BATCH, MAX_CHUNK = 256, 512

_STATUS_NAMES = {0: "TL_OK", 1: "TL_E_ARG", 2: "TL_E_UNSUPPORTED", 3: "TL_E_CAPACITY",
                 4: "TL_E_CACHE_GAP", 5: "TL_E_HIP"}


class TLError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__("%s: %s" % (_STATUS_NAMES.get(status, status), msg))
        self.status = status


class tl_config(ctypes.Structure):
    _fields_ = [("d_model", ctypes.c_int32), ("n_heads", ctypes.c_int32),
                ("d_head", ctypes.c_int32), ("d_mlp", ctypes.c_int32),
                ("n_pre", ctypes.c_int32), ("vocab", ctypes.c_int32),
                ("norm_eps", ctypes.c_float), ("dtype", ctypes.c_int32)]


class tl_layer_weights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("norm1", "w_qkv", "w_o", "norm2", "w_up", "w_down")]


class tl_weights(ctypes.Structure):
    _fields_ = [("embed", ctypes.c_void_p), ("final_norm", ctypes.c_void_p),
                ("lm_head", ctypes.c_void_p), ("layers", ctypes.POINTER(tl_layer_weights))]


_lib = None
EXPORTS = ("tl_version", "tl_last_error", "tl_model_create", "tl_model_destroy",
           "tl_cache_bytes", "tl_workspace_bytes", "tl_cache_alloc", "tl_cache_free",
           "tl_prefill_chunk", "tl_decode_step", "tl_residual_norms", "tl_lane_residual",
           "tl_cache_write_h", "tl_cache_fill_synthetic", "tl_cache_set_length",
           "tl_cache_read", "tl_cache_reset_lane", "tl_profile_start", "tl_profile_stop",
           "tl_prefill_chunk_x", "tl_extend_depth", "tl_spec_step", "tl_cache_set_attention",
           "tl_decode_step_static")


def load(path: str = LIB_PATH):
    """Load libtl.so and declare the C signatures (no GPU call is made)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError("libtl.so not built (%s); run python -m kv_compression_amd.build" % path)
    L = ctypes.CDLL(path)
    P, I, S, F, U = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t, ctypes.c_float, ctypes.c_uint32
    cfgp = ctypes.POINTER(tl_config)
    sig = {
        "tl_version": (I, []),
        "tl_last_error": (ctypes.c_char_p, []),
        "tl_model_create": (I, [cfgp, ctypes.POINTER(tl_weights), ctypes.POINTER(P)]),
        "tl_model_destroy": (None, [P]),
        "tl_cache_bytes": (S, [cfgp, I, I, I, I]),
        "tl_workspace_bytes": (S, [cfgp, I, I, I, I]),
        "tl_cache_alloc": (I, [P, I, I, I, I, P, S, P, S, P, ctypes.POINTER(P)]),
        "tl_cache_free": (None, [P]),
        "tl_prefill_chunk": (I, [P, I, I, P, I, P, P, P]),
        "tl_prefill_chunk_x": (I, [P, I, I, P, I, P, P, P, P]),
        "tl_extend_depth": (I, [P, I, I, I, I, I, P, P, P, P]),
        "tl_decode_step": (I, [P, I, P, P, P, F, P, P, P, P]),
        "tl_decode_step_static": (I, [P, I, P, P, P, F, P, P, P, P]),
        "tl_spec_step": (I, [P, I, I, I, I, P, P, ctypes.POINTER(I), P]),
        "tl_cache_set_attention": (I, [P, I]),
        "tl_residual_norms": (I, [P, I, P, P]),
        "tl_lane_residual": (I, [P, I, P, P]),
        "tl_cache_write_h": (I, [P, I, I, I, I, P, P]),
        "tl_cache_fill_synthetic": (I, [P, I, I, I, I, U, P]),
        "tl_cache_set_length": (I, [P, I, I, I, P]),
        "tl_cache_read": (I, [P, I, I, I, I, P, P, P, P]),
        "tl_cache_reset_lane": (I, [P, I, P]),
        "tl_profile_start": (I, [P]),
        "tl_profile_stop": (I, [P, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(I)]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    _lib = L
    return L


def _check(status: int):
    if status != TL_OK:
        raise TLError(status, _lib.tl_last_error().decode())


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    return t.data_ptr()


def _stream(stream=None) -> Optional[int]:
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def make_config(shape) -> tl_config:
    """tl_config from a shape with d_model, n_heads, d_head, d_mlp, n_pre, vocab, dtype, norm_eps."""
    return tl_config(shape.d_model, shape.n_heads, shape.d_head, shape.d_mlp, shape.n_pre,
                     shape.vocab, shape.norm_eps, DTYPES[shape.dtype])


# ---------------------------------------------------------------------------
# same-name wrappers of the C ABI
# ---------------------------------------------------------------------------
def tl_cache_bytes(cfg: tl_config, mode: str, n_lanes: int, max_seq: int, l_max: int) -> int:
    return load().tl_cache_bytes(ctypes.byref(cfg), MODES[mode], n_lanes, max_seq, l_max)


def tl_workspace_bytes(cfg: tl_config, mode: str, n_lanes: int, max_seq: int, l_max: int) -> int:
    return load().tl_workspace_bytes(ctypes.byref(cfg), MODES[mode], n_lanes, max_seq, l_max)


class Model:
    """tl_model_create over device weight tensors (kept alive by this object)."""

    def __init__(self, shape, weights_dev: dict):
        L = load()
        self.shape = shape
        self.cfg = make_config(shape)
        self._w = weights_dev
        n_unique = shape.n_pre + 1
        self._layers = (tl_layer_weights * n_unique)()
        for u in range(n_unique):
            lw = weights_dev["layers"][u]
            self._layers[u] = tl_layer_weights(*(lw[k].data_ptr() for k in
                                                 ("norm1", "w_qkv", "w_o", "norm2", "w_up", "w_down")))
        tw = tl_weights(weights_dev["embed"].data_ptr(), weights_dev["final_norm"].data_ptr(),
                        weights_dev["lm_head"].data_ptr(), self._layers)
        h = ctypes.c_void_p()
        _check(L.tl_model_create(ctypes.byref(self.cfg), ctypes.byref(tw), ctypes.byref(h)))
        self.handle = h

    def __del__(self):
        if getattr(self, "handle", None) and _lib is not None:
            _lib.tl_model_destroy(self.handle)
            self.handle = None


def upload_weights(shape, weights_np: dict, device="cuda"):
    """Copy numpy weights (synth.make_weights layout) to device tensors."""
    import torch

    def t(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(device)
    return {
        "embed": t(weights_np["embed"]), "final_norm": t(weights_np["final_norm"]),
        "lm_head": t(weights_np["lm_head"]),
        "layers": [{k: t(v) for k, v in lw.items()} for lw in weights_np["layers"]],
    }


class Cache:
    """tl_cache_alloc over torch-allocated cache and workspace buffers."""

    def __init__(self, model: Model, mode: str, n_lanes: int, max_seq: int, l_max: int,
                 stream=None):
        import torch
        L = load()
        self.model, self.mode = model, mode
        self.n_lanes, self.max_seq, self.l_max = n_lanes, max_seq, l_max
        cb = tl_cache_bytes(model.cfg, mode, n_lanes, max_seq, l_max)
        wb = tl_workspace_bytes(model.cfg, mode, n_lanes, max_seq, l_max)
        if cb == 0 or wb == 0:
            raise TLError(TL_E_UNSUPPORTED, "no layout for this shape / mode")
        self.cache_bytes, self.workspace_bytes = cb, wb
        self.d_cache = torch.empty(cb + 256, dtype=torch.uint8, device="cuda")
        self.d_ws = torch.empty(wb + 256, dtype=torch.uint8, device="cuda")
        cp = (self.d_cache.data_ptr() + 255) // 256 * 256
        wp = (self.d_ws.data_ptr() + 255) // 256 * 256
        h = ctypes.c_void_p()
        _check(L.tl_cache_alloc(model.handle, MODES[mode], n_lanes, max_seq, l_max, cp, cb, wp, wb,
                                _stream(stream), ctypes.byref(h)))
        self.handle = h

    def __del__(self):
        if getattr(self, "handle", None) and _lib is not None:
            _lib.tl_cache_free(self.handle)
            self.handle = None

    # -- the ABI calls -------------------------------------------------------
    def tl_prefill_chunk(self, lane, loops, d_tokens, next_token=None, last_logits=None, stream=None):
        _check(_lib.tl_prefill_chunk(self.handle, lane, loops, _ptr(d_tokens), d_tokens.numel(),
                                     _ptr(next_token), _ptr(last_logits), _stream(stream)))

    def tl_prefill_chunk_x(self, lane, loops, d_tokens, x_out=None, next_token=None, last_logits=None,
                           stream=None):
        _check(_lib.tl_prefill_chunk_x(self.handle, lane, loops, _ptr(d_tokens), d_tokens.numel(),
                                       _ptr(x_out), _ptr(next_token), _ptr(last_logits), _stream(stream)))

    def tl_extend_depth(self, lane, pos0, n, old_loops, new_loops, d_x, next_token=None,
                        last_logits=None, stream=None):
        _check(_lib.tl_extend_depth(self.handle, lane, pos0, n, old_loops, new_loops, _ptr(d_x),
                                    _ptr(next_token), _ptr(last_logits), _stream(stream)))

    def tl_decode_step(self, lanes: Sequence[int], loops: Sequence[int], d_tokens_in, threshold,
                       d_tokens_out, d_logits, d_lane_status, stream=None):
        n = len(lanes)
        la = (ctypes.c_int32 * n)(*lanes)
        lo = (ctypes.c_int32 * n)(*loops)
        _check(_lib.tl_decode_step(self.handle, n, la, lo, _ptr(d_tokens_in), float(threshold),
                                   _ptr(d_tokens_out), _ptr(d_logits), _ptr(d_lane_status),
                                   _stream(stream)))

    def tl_decode_step_static(self, lanes: Sequence[int], loops: Sequence[int], d_tokens_in, threshold,
                              d_tokens_out, d_logits, d_lane_status, stream=None):
        n = len(lanes)
        la = (ctypes.c_int32 * n)(*lanes)
        lo = (ctypes.c_int32 * n)(*loops)
        _check(_lib.tl_decode_step_static(self.handle, n, la, lo, _ptr(d_tokens_in), float(threshold),
                                          _ptr(d_tokens_out), _ptr(d_logits), _ptr(d_lane_status),
                                          _stream(stream)))

    def tl_spec_step(self, lane, draft_loops, verify_loops, draft_ahead, d_token_in, d_tokens_out,
                     stream=None) -> int:
        n = ctypes.c_int()
        _check(_lib.tl_spec_step(self.handle, lane, draft_loops, verify_loops, draft_ahead,
                                 _ptr(d_token_in), _ptr(d_tokens_out), ctypes.byref(n), _stream(stream)))
        return n.value

    def tl_cache_set_attention(self, order: str):
        """order: "explicit" (rebuild K/V) or "absorbed" (W_k^T q against h')."""
        _check(_lib.tl_cache_set_attention(self.handle, ATTN_ORDERS[order]))

    def tl_residual_norms(self, lane, stream=None) -> np.ndarray:
        out = np.empty(self.l_max, np.float32)
        _check(_lib.tl_residual_norms(self.handle, lane, out.ctypes.data, _stream(stream)))
        return out

    def tl_lane_residual(self, lane, d_out, stream=None):
        _check(_lib.tl_lane_residual(self.handle, lane, _ptr(d_out), _stream(stream)))

    def tl_cache_write_h(self, lane, layer, pos0, d_h, stream=None):
        _check(_lib.tl_cache_write_h(self.handle, lane, layer, pos0, d_h.shape[0], _ptr(d_h),
                                     _stream(stream)))

    def tl_cache_fill_synthetic(self, lane, layer, pos0, n, seed, stream=None):
        _check(_lib.tl_cache_fill_synthetic(self.handle, lane, layer, pos0, n, seed, _stream(stream)))

    def tl_cache_set_length(self, lane, length, layers_valid, stream=None):
        _check(_lib.tl_cache_set_length(self.handle, lane, length, layers_valid, _stream(stream)))

    def tl_cache_read(self, lane, layer, pos0, n, d_codes=None, d_scales=None, d_h=None, stream=None):
        _check(_lib.tl_cache_read(self.handle, lane, layer, pos0, n, _ptr(d_codes), _ptr(d_scales),
                                  _ptr(d_h), _stream(stream)))

    def tl_cache_reset_lane(self, lane, stream=None):
        _check(_lib.tl_cache_reset_lane(self.handle, lane, _stream(stream)))

    def tl_profile_start(self):
        _check(_lib.tl_profile_start(self.handle))

    def tl_profile_stop(self):
        ms = ctypes.c_double()
        n = ctypes.c_int()
        _check(_lib.tl_profile_stop(self.handle, ctypes.byref(ms), ctypes.byref(n)))
        return ms.value, n.value

    # -- conveniences built from the calls above --------------------------------
    def prefill(self, lane: int, tokens, loops: int, chunk: int = MAX_CHUNK):
        """Prefill a whole prompt in chunks; returns (next_token, last_logits) device tensors."""
        import torch
        tok = torch.as_tensor(np.asarray(tokens, np.int32)).to("cuda")
        nxt = torch.empty(1, dtype=torch.int32, device="cuda")
        lg = torch.empty(self.model.shape.vocab, dtype=torch.float32, device="cuda")
        for p in range(0, tok.numel(), chunk):
            self.tl_prefill_chunk(lane, loops, tok[p:p + chunk], nxt, lg)
        return nxt, lg

    def prefill_x(self, lane: int, tokens, loops: int, chunk: int = MAX_CHUNK):
        """prefill that also returns every prompt position's residual after its
        last layer (device f32 [n, d_model]): the state tl_extend_depth resumes from."""
        import torch
        tok = torch.as_tensor(np.asarray(tokens, np.int32)).to("cuda")
        x = torch.empty((tok.numel(), self.model.shape.d_model), dtype=torch.float32, device="cuda")
        nxt = torch.empty(1, dtype=torch.int32, device="cuda")
        lg = torch.empty(self.model.shape.vocab, dtype=torch.float32, device="cuda")
        for p in range(0, tok.numel(), chunk):
            self.tl_prefill_chunk_x(lane, loops, tok[p:p + chunk], x[p:p + chunk], nxt, lg)
        return nxt, lg, x

    def extend_depth(self, lane: int, x, old_loops: int, new_loops: int, chunk: int = MAX_CHUNK):
        """Deepen all of the lane's positions from old_loops to new_loops, chunk by
        chunk; x (device f32 [length, d_model]) is updated in place to the new
        residuals. Returns (next_token, last_logits) after the last position."""
        import torch
        nxt = torch.empty(1, dtype=torch.int32, device="cuda")
        lg = torch.empty(self.model.shape.vocab, dtype=torch.float32, device="cuda")
        n = x.shape[0]
        for p in range(0, n, chunk):
            m = min(chunk, n - p)
            self.tl_extend_depth(lane, p, m, old_loops, new_loops, x[p:p + m], nxt, lg)
        return nxt, lg

    def generate_speculative(self, lane: int, token: int, max_tokens: int, draft_loops: int,
                             verify_loops: int, draft_ahead: int):
        """Greedy tokens after ``token`` (the token at the lane's current length)
        by rounds of tl_spec_step until at least ``max_tokens`` are emitted.
        Returns (tokens, emitted per round) as host lists; the last token is at
        the lane's new length."""
        import torch
        tin = torch.tensor([token], dtype=torch.int32, device="cuda")
        tout = torch.empty(draft_ahead + 1, dtype=torch.int32, device="cuda")
        out, rounds = [], []
        while len(out) < max_tokens:
            n = self.tl_spec_step(lane, draft_loops, verify_loops, draft_ahead, tin, tout)
            rounds.append(n)
            if n == 0:
                break
            out.extend(int(t) for t in tout[:n].cpu())
            tin.copy_(tout[n - 1:n])
        return out, rounds
