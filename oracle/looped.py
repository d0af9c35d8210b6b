"""CPU oracle: one decode step of a weight-shared looped transformer with a
store-h KV cache, written as the plain definition in float64.

TEST INFRASTRUCTURE ONLY. This module is the parity reference for the HIP
library. Only the test suite, the package's smoke check and the benchmark's
CPU-baseline leg may import it; the product path never calls it and has no CPU
fallback. It shares no code with the HIP path: the only common inputs come from
the ``synth`` generators.

What it computes (TinyLoop documentation pages):
* Model (architecture-exclusive features page, introduction): n_pre unique
  layers, then one loop block applied L times; W_q, W_k, W_v, W_o, the norms
  and the MLP are the same arrays at every loop iteration.
* Store-h cache (same page, "Store-h KV cache"; novel-contributions page,
  "Store-h KV Cache"): the cache keeps h, the pre-QKV norm output, per token and
  per layer-iteration; attention rebuilds K = W_k h and V = W_v h from it with
  the layer's own weights. Modes: float h (fp32 or fp16), INT8-h and INT4-h,
  and the stored-K/V baseline (measured-benchmarks page, section 3, "FP16 KV
  baseline").
* Variable-L cache (features page, "Variable-L KV cache"): n_pre + L_max cache
  layers; layer n_pre + i is written only by loop iteration i, so it is valid
  for every L >= i + 1.
* Per-lane loops (features page, "L-aware batching"): every lane of a batch runs
  its own loop count; lanes never interact.
* Iteration-axis delta mode (features page, "4) Iteration-axis delta-KV"):
  the unique layers keep fp16 h, the last of them serving as the anchor h0;
  loop layer n_pre + i keeps the INT8 delta of its h against the previous
  layer's reconstruction, one fp16 scale per head; a loop layer's h' is
  fp16 of the FP32 prefix sum h0 + sum of s * q up to it.
* Safety check (novel-contributions page, "Per-Iteration Safety Check";
  features page, "Per-iteration safety check"): during decode, after every loop
  iteration, the FP32 residual L2 norm is compared with a threshold and the
  lane aborts when it exceeds it.

Readings of points the pages leave open (each one is also listed in the design
notes): RMSNorm with eps 1e-5 and real gains; no positional encoding; two-matrix
erf-GELU MLP; multi-head attention with scale 1/sqrt(d_head), causal including
the current token; untied LM head after a final RMSNorm; every layer (pre and
loop) stores h; the current token's h is appended before attention reads the
cache; INT8 one absmax scale per token, INT4 one per 32 consecutive d_model
elements, divisors 127 and 7, fp32 IEEE divide and round-half-to-even, clamps
[-127, 127] and [-8, 7], fp16 scales; the safety check fires iff
not (norm <= threshold), only on loop iterations during decode, and a +inf
threshold turns it off; an aborted lane emits no token and its length does not
advance; argmax ties go to the lowest index; delta mode: the anchor h0 is
the last unique layer's h, and the write side is closed-loop (each delta is
taken against the previous layer's FP32 prefix sum, which is what the
page's reconstruction-error table, falling as L grows, implies).

Rounding points (the storage and operand dtypes that define the cache and the
fp16 model; everything else is float64):
  R1  h rounded to the h dtype (model dtype);
  R2  the INT8 / INT4 / delta codec (float32 arithmetic, exactly as specified);
  R3  dequantised h' = fp16(q * s);
  R4  o, the norm-2 output, the GELU output and the final-norm output rounded
      to the model dtype before they enter a matrix product;
  R5  stored-K/V values rounded to the model dtype;
  R6  weights are exactly their model-dtype values.
``exact=True`` switches R1, R3, R4 and R5 off.
"""
from __future__ import annotations

import math
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np
from scipy.special import erf

__all__ = [
    "MODES", "LANE_OK", "LANE_ABORTED", "CacheGapError", "CapacityError",
    "rmsnorm", "gelu_erf", "encode_int", "decode_int", "int8_encode", "int4_encode",
    "attend", "entry_bytes", "cache_bytes", "LoopedOracle",
]

MODES = ("kv", "f32", "f16", "int8", "int4", "delta8")
LANE_OK, LANE_ABORTED = 0, 1
INT4_GROUP = 32


class CacheGapError(RuntimeError):
    """A lane asked for a cache layer that misses earlier positions."""


class CapacityError(RuntimeError):
    """Appending would exceed the cache's max_seq positions."""


# ---------------------------------------------------------------------------
# elementwise pieces
# ---------------------------------------------------------------------------
def rmsnorm(x: np.ndarray, g: np.ndarray, eps: float) -> np.ndarray:
    """RMSNorm over the last axis: g * x / sqrt(mean(x^2) + eps), float64."""
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return g * (x / np.sqrt(ms + eps))


def gelu_erf(x: np.ndarray) -> np.ndarray:
    """Exact GELU: x * Phi(x) = 0.5 x (1 + erf(x / sqrt 2)), float64."""
    return 0.5 * x * (1.0 + erf(x / math.sqrt(2.0)))


# ---------------------------------------------------------------------------
# h codec (R2, R3): symmetric absmax, fp16 scale, computed in float32
# ---------------------------------------------------------------------------
def encode_int(h16: np.ndarray, group: int, qmax: int, qmin: int) -> Tuple[np.ndarray, np.ndarray]:
    """Quantise fp16 rows [..., D] in groups of ``group`` along the last axis.

    s = fp16(absmax / qmax) (float32 divide, round to nearest even into fp16);
    q = clip(rint(h / s), qmin, qmax) in float32 with round-half-to-even; a
    group whose scale is zero (all-zero or underflowed) gets q = 0.
    Returns int8 codes [..., D] and fp16 scales [..., D / group].
    """
    return _encode_f32(np.asarray(h16, dtype=np.float16).astype(np.float32), group, qmax, qmin)


def _encode_f32(x: np.ndarray, group: int, qmax: int, qmin: int) -> Tuple[np.ndarray, np.ndarray]:
    """The rule of ``encode_int`` on float32 rows."""
    x = np.asarray(x, dtype=np.float32)
    D = x.shape[-1]
    assert D % group == 0
    hf = x.reshape(x.shape[:-1] + (D // group, group))
    am = np.max(np.abs(hf), axis=-1)
    s = (am / np.float32(qmax)).astype(np.float16)
    sf = s.astype(np.float32)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.rint(hf / sf)
    q = np.where(sf == 0, np.float32(0), np.clip(q, qmin, qmax))
    return q.astype(np.int8).reshape(x.shape), s


def decode_int(q: np.ndarray, s: np.ndarray) -> np.ndarray:
    """h' = fp16(q * s): the product is exact in float32, then rounded to fp16."""
    q = np.asarray(q, dtype=np.int8)
    D = q.shape[-1]
    group = D // s.shape[-1]
    qf = q.astype(np.float32).reshape(q.shape[:-1] + (D // group, group))
    # near the fp16 maximum the rounded product can overflow to +-inf (e.g. h = 65504:
    # s = fp16(65504 / 7) = 9360, q = 7, q * s = 65520); that is part of the codec
    with np.errstate(over="ignore"):
        return (qf * s.astype(np.float32)[..., None]).astype(np.float16).reshape(q.shape)


def int8_encode(h16):
    """INT8-h: one scale per token (group = d_model), divisor 127, clamp [-127, 127]."""
    h16 = np.asarray(h16, dtype=np.float16)
    return encode_int(h16, h16.shape[-1], 127, -127)


def int4_encode(h16):
    """INT4-h: one scale per 32 consecutive d_model elements, divisor 7, clamp [-8, 7]."""
    return encode_int(h16, INT4_GROUP, 7, -8)


# ---------------------------------------------------------------------------
# iteration-axis delta codec (features page, "4) Iteration-axis delta-KV")
# ---------------------------------------------------------------------------
def delta_encode(d32: np.ndarray, d_head: int) -> Tuple[np.ndarray, np.ndarray]:
    """INT8 codes of float32 delta rows [..., D] with one fp16 scale per head
    (the [T, n_heads] scale grid): the INT8 rule (divisor 127, clamp
    [-127, 127]) in groups of d_head."""
    return _encode_f32(d32, d_head, 127, -127)


def delta_accumulate(r: np.ndarray, q: np.ndarray, s: np.ndarray) -> np.ndarray:
    """One term of the FP32 prefix sum: r + s[head] * q, float32. The product
    of an fp16 scale and an 8-bit code is exact in float32, so the only
    rounding is the addition."""
    D = q.shape[-1]
    sf = np.repeat(s.astype(np.float32), D // s.shape[-1], axis=-1)
    return (np.asarray(r, np.float32) + sf * q.astype(np.float32)).astype(np.float32)


# ---------------------------------------------------------------------------
# attention over reconstructed K/V
# ---------------------------------------------------------------------------
def attend(q: np.ndarray, K: np.ndarray, V: np.ndarray, n_heads: int, pos0: int) -> np.ndarray:
    """Causal multi-head attention, float64.

    q [n, D] (already scaled by 1/sqrt(d_head)), K, V [T, D] with T = pos0 + n.
    Query i sits at position pos0 + i and sees positions 0 .. pos0 + i.
    Per head: s_j = q . K_j, p = softmax_j(s) (max subtracted), o = sum_j p_j V_j.
    """
    n, D = q.shape
    T = K.shape[0]
    d = D // n_heads
    qh = q.reshape(n, n_heads, d).transpose(1, 0, 2)            # [H, n, d]
    Kh = K.reshape(T, n_heads, d).transpose(1, 2, 0)            # [H, d, T]
    Vh = V.reshape(T, n_heads, d).transpose(1, 0, 2)            # [H, T, d]
    s = qh @ Kh                                                  # [H, n, T]
    visible = np.arange(T)[None, :] <= (pos0 + np.arange(n))[:, None]
    s = np.where(visible[None], s, -np.inf)
    s = s - np.max(s, axis=-1, keepdims=True)
    p = np.exp(s)
    p = p / np.sum(p, axis=-1, keepdims=True)
    o = p @ Vh                                                   # [H, n, d]
    return o.transpose(1, 0, 2).reshape(n, D)


# ---------------------------------------------------------------------------
# cache byte counts (closed form)
# ---------------------------------------------------------------------------
def entry_bytes(mode: str, d_model: int) -> int:
    """Bytes of one cache entry (one token, one layer-iteration); the delta mode
    has two kinds of entry and is counted by ``cache_bytes``."""
    D = d_model
    return {"kv": None, "f32": 4 * D, "f16": 2 * D, "int8": D + 2,
            "int4": D // 2 + 2 * (D // INT4_GROUP)}[mode]


def cache_bytes(mode: str, d_model: int, model_dtype: str, n_lanes: int, max_seq: int,
                l_max: int, n_pre: int, n_heads: int = 0) -> int:
    """Total cache payload for n_pre + L_max layers x lanes x max_seq positions.

    Delta mode: the n_pre unique layers keep fp16 h (the last one is the
    anchor h0), every loop layer INT8 codes plus one fp16 scale per head."""
    if mode == "delta8":
        per_token = n_pre * 2 * d_model + l_max * (d_model + 2 * n_heads)
        return n_lanes * max_seq * per_token
    if mode == "kv":
        per = 2 * d_model * (4 if model_dtype == "f32" else 2)
    else:
        per = entry_bytes(mode, d_model)
    return (n_pre + l_max) * n_lanes * max_seq * per


# ---------------------------------------------------------------------------
# the model
# ---------------------------------------------------------------------------
class LoopedOracle:
    """Float64 reference of the looped decoder with a per-lane, per-layer cache.

    ``weights`` is the dict from ``synth.make_weights`` (model-dtype arrays).
    """

    def __init__(self, shape, weights: dict, mode: str, n_lanes: int, max_seq: int,
                 l_max: int, exact: bool = False):
        if mode not in MODES:
            raise ValueError(mode)
        if shape.dtype == "f32" and mode not in ("f32", "kv"):
            raise ValueError("an fp32 model stores fp32 h or K/V")
        if shape.dtype == "f16" and mode == "f32":
            raise ValueError("an fp16 model stores fp16, INT8 or INT4 h, or fp16 K/V")
        if mode == "delta8" and (exact or shape.n_pre < 1):
            raise ValueError("the delta codec needs a pre layer for its anchor and rounds by definition")
        self.shape = shape
        self.mode = mode
        self.exact = exact
        self.n_lanes, self.max_seq, self.l_max = n_lanes, max_seq, l_max
        self.D, self.H, self.d = shape.d_model, shape.n_heads, shape.d_head
        self.n_pre = shape.n_pre
        self.eps = shape.norm_eps
        self.dt = np.float32 if shape.dtype == "f32" else np.float16
        f64 = lambda a: np.asarray(a, dtype=np.float64)
        D = self.D
        self.embed = f64(weights["embed"])
        self.lm_head = f64(weights["lm_head"])
        self.final_norm = f64(weights["final_norm"])
        self.layers = []
        for lw in weights["layers"]:
            wqkv = f64(lw["w_qkv"])
            self.layers.append(dict(
                wq=wqkv[:D], wk=wqkv[D:2 * D], wv=wqkv[2 * D:],
                wo=f64(lw["w_o"]), wup=f64(lw["w_up"]), wdown=f64(lw["w_down"]),
                g1=f64(lw["norm1"]), g2=f64(lw["norm2"])))
        self.cache: Dict[Tuple[int, int], dict] = {}
        self.length = [0] * n_lanes
        self.layers_valid = [0] * n_lanes          # layers filled for every position < length
        self.status = [LANE_OK] * n_lanes
        self.norms = [np.full(l_max, np.nan) for _ in range(n_lanes)]
        self.trace: Dict[int, list] = {}           # per-lane stage snapshots of the last call
        # Test hooks, inert unless a test sets them (they change no arithmetic):
        # h_log, when a dict, receives for every row write_h stores the h row in
        # the h dtype and the float32 row its codec is applied to (the h itself;
        # in the delta mode's loop layers h minus the reconstruction below), keyed
        # (layer, lane, pos); row_override maps (layer, lane, pos) to a row stored
        # in place of the encoded one: dict(q=int8 codes, s=fp16 scales) for the
        # INT codecs, dict(h=row) for float h.
        self.h_log: Optional[dict] = None
        self.row_override: Dict[Tuple[int, int, int], dict] = {}

    # -- rounding points ----------------------------------------------------
    def _rd(self, a: np.ndarray) -> np.ndarray:
        if self.exact:
            return a
        return a.astype(self.dt).astype(np.float64)

    def weights_for(self, layer: int) -> dict:
        """Unique layer ``layer`` for layer < n_pre, else the shared loop block."""
        return self.layers[min(layer, self.n_pre)]

    # -- cache storage --------------------------------------------------------
    def _slot(self, layer: int, lane: int) -> dict:
        key = (layer, lane)
        if key not in self.cache:
            S, D = self.max_seq, self.D
            if self.mode == "kv":
                dt = np.float64 if self.exact else self.dt
                slot = {"k": np.zeros((S, D), dt), "v": np.zeros((S, D), dt)}
            elif self.mode in ("f32", "f16") or (self.mode == "delta8" and layer < self.n_pre):
                slot = {"h": np.zeros((S, D), np.float64 if self.exact else self.dt)}
            elif self.mode == "delta8":
                slot = {"q": np.zeros((S, D), np.int8), "s": np.zeros((S, self.H), np.float16)}
            else:
                ng = 1 if self.mode == "int8" else D // INT4_GROUP
                slot = {"q": np.zeros((S, D), np.int8), "s": np.zeros((S, ng), np.float16)}
            self.cache[key] = slot
        return self.cache[key]

    def write_h(self, layer: int, lane: int, pos0: int, h: np.ndarray) -> None:
        """Store h rows (already in the h dtype, or float64 when exact) at pos0.."""
        slot = self._slot(layer, lane)
        n = h.shape[0]
        if pos0 + n > self.max_seq:
            raise CapacityError("cache full")
        codec_in = None
        if self.mode in ("f32", "f16"):
            slot["h"][pos0:pos0 + n] = h
        elif self.mode == "int8":
            q, s = int8_encode(h.astype(np.float16))
            slot["q"][pos0:pos0 + n], slot["s"][pos0:pos0 + n] = q, s
        elif self.mode == "int4":
            q, s = int4_encode(h.astype(np.float16))
            slot["q"][pos0:pos0 + n], slot["s"][pos0:pos0 + n] = q, s
        elif self.mode == "delta8":
            if layer < self.n_pre:
                slot["h"][pos0:pos0 + n] = h
            else:
                # closed loop: the delta is taken against the previous layer as
                # the reader rebuilds it, so quantisation errors do not pile up
                r_prev = self.delta_rec(layer - 1, lane, pos0, n)
                d = h.astype(np.float16).astype(np.float32) - r_prev
                codec_in = d
                q, s = delta_encode(d, self.d)
                slot["q"][pos0:pos0 + n], slot["s"][pos0:pos0 + n] = q, s
        else:
            W = self.weights_for(layer)
            hf = np.asarray(h, dtype=np.float64)
            slot["k"][pos0:pos0 + n] = self._rd(hf @ W["wk"].T)      # R5
            slot["v"][pos0:pos0 + n] = self._rd(hf @ W["wv"].T)
        if self.mode != "kv" and (self.h_log is not None or self.row_override):
            for r in range(n):
                key = (layer, lane, pos0 + r)
                if self.h_log is not None:
                    hr = np.asarray(h[r]) if self.exact else np.asarray(h[r]).astype(self.dt)
                    cin = codec_in[r] if codec_in is not None else hr.astype(np.float32)
                    self.h_log[key] = (hr.copy(), np.array(cin, np.float32))
                ov = self.row_override.get(key)
                if ov is not None:
                    if "h" in ov:
                        slot["h"][pos0 + r] = ov["h"]
                    else:
                        slot["q"][pos0 + r], slot["s"][pos0 + r] = ov["q"], ov["s"]

    def delta_rec(self, layer: int, lane: int, pos0: int, n: int) -> np.ndarray:
        """Delta mode, float32 rows of positions pos0..pos0+n-1: a unique layer's
        own h; a loop layer's FP32 prefix sum h0 + sum of s * q over the loop
        layers up to it, h0 being the last unique layer's h."""
        if layer < self.n_pre:
            return self._slot(layer, lane)["h"][pos0:pos0 + n].astype(np.float32)
        r = self._slot(self.n_pre - 1, lane)["h"][pos0:pos0 + n].astype(np.float32)
        for j in range(self.n_pre, layer + 1):
            sj = self._slot(j, lane)
            r = delta_accumulate(r, sj["q"][pos0:pos0 + n], sj["s"][pos0:pos0 + n])
        return r

    def read_h(self, layer: int, lane: int, T: int) -> np.ndarray:
        """Dequantised h' for positions 0..T-1 as float64 (R3; delta mode: the
        prefix sum rounded to fp16)."""
        slot = self._slot(layer, lane)
        if self.mode in ("f32", "f16") or (self.mode == "delta8" and layer < self.n_pre):
            return slot["h"][:T].astype(np.float64)
        if self.mode == "delta8":
            return self.delta_rec(layer, lane, 0, T).astype(np.float16).astype(np.float64)
        return decode_int(slot["q"][:T], slot["s"][:T]).astype(np.float64)

    def read_codes(self, layer: int, lane: int, pos0: int, n: int):
        slot = self._slot(layer, lane)
        return slot["q"][pos0:pos0 + n].copy(), slot["s"][pos0:pos0 + n].copy()

    def reconstruct_kv(self, layer: int, lane: int, T: int) -> Tuple[np.ndarray, np.ndarray]:
        """K = W_k h', V = W_v h' for positions 0..T-1 (stored K/V in the baseline mode)."""
        slot = self._slot(layer, lane)
        if self.mode == "kv":
            return slot["k"][:T].astype(np.float64), slot["v"][:T].astype(np.float64)
        W = self.weights_for(layer)
        hp = self.read_h(layer, lane, T)
        return hp @ W["wk"].T, hp @ W["wv"].T

    def prime_synthetic(self, lane: int, layers: Sequence[int], n: int, h_rows_fn) -> None:
        """Fill positions 0..n-1 of the given layers with synthetic h.

        ``h_rows_fn(layer)`` returns float32 [n, D]; it is rounded to the h dtype
        (R1) and then stored through the mode's codec. Sets the lane length.
        """
        for layer in layers:
            h = np.asarray(h_rows_fn(layer), dtype=np.float32)
            if not self.exact:
                h = h.astype(self.dt)
            self.write_h(layer, lane, 0, h)
        self.length[lane] = n
        self.layers_valid[lane] = len(layers)

    # -- one pass over new positions -------------------------------------------
    def _layers(self, lane: int, x: np.ndarray, pos0: int, layer_begin: int, layer_end: int,
                check_safety: bool, threshold: float, trace: Optional[list]):
        """Layers layer_begin .. layer_end-1 for the n rows of x at positions pos0...

        Every layer first appends the new h rows, then rebuilds K/V for
        positions 0 .. pos0+n-1 from the cache. Returns (x, norms, aborted_at).
        """
        n = x.shape[0]
        T = pos0 + n
        norms = np.full((n, self.l_max), np.nan)
        for layer in range(layer_begin, layer_end):
            W = self.weights_for(layer)
            h = rmsnorm(x, W["g1"], self.eps)
            h = h if self.exact else h.astype(self.dt)            # R1
            self.write_h(layer, lane, pos0, h)                     # appended before the read
            hq = np.asarray(h, dtype=np.float64)
            q = (hq @ W["wq"].T) / math.sqrt(self.d)
            K, V = self.reconstruct_kv(layer, lane, T)
            o = attend(q, K, V, self.H, pos0)
            x = x + self._rd(o) @ W["wo"].T                        # R4 on o
            u = self._rd(rmsnorm(x, W["g2"], self.eps))            # R4
            a = self._rd(gelu_erf(u @ W["wup"].T))                 # R4
            x = x + a @ W["wdown"].T
            if trace is not None:
                trace.append(("pre.%d" % layer if layer < self.n_pre
                              else "loop.%d" % (layer - self.n_pre), x.copy()))
            if layer >= self.n_pre:
                i = layer - self.n_pre
                norms[:, i] = np.sqrt(np.sum(x * x, axis=-1))
                if check_safety and not np.all(norms[:, i] <= threshold):
                    return x, norms, i
        return x, norms, None

    def _head(self, x: np.ndarray) -> np.ndarray:
        z = self._rd(rmsnorm(x, self.final_norm, self.eps))        # R4
        return z @ self.lm_head.T

    def forward(self, lane: int, tokens: Sequence[int], loops: int, check_safety: bool,
                threshold: float = math.inf, keep_trace: bool = False) -> dict:
        """Append new positions pos0 .. pos0+n-1 to ``lane`` (pos0 = its length)
        and run them through n_pre + loops layers.

        With ``check_safety`` (decode: n == 1) the residual norm after each loop
        iteration is compared with ``threshold``. Returns a dict: logits [n, V]
        (None when aborted), x [n, D] (the residual after the last layer run),
        norms [n, L_max] (NaN where not run), aborted_at (loop iteration or None).
        """
        n = len(tokens)
        pos0 = self.length[lane]
        if not (1 <= loops <= self.l_max):
            raise ValueError("loops out of range")
        if pos0 + n > self.max_seq:
            raise CapacityError("cache full")
        n_layers = self.n_pre + loops
        if pos0 > 0 and n_layers > self.layers_valid[lane]:
            raise CacheGapError("layers above %d miss earlier positions" % self.layers_valid[lane])
        x = self.embed[np.asarray(tokens, dtype=np.int64)].copy()
        trace = [("embed", x.copy())] if keep_trace else None
        x, norms, aborted_at = self._layers(lane, x, pos0, 0, n_layers, check_safety,
                                            threshold, trace)
        if keep_trace:
            trace.append(("final_ln", rmsnorm(x, self.final_norm, self.eps)))
            self.trace[lane] = trace
        if aborted_at is not None:
            return dict(logits=None, x=x, norms=norms, aborted_at=aborted_at)
        logits = self._head(x)
        self.length[lane] = pos0 + n
        self.layers_valid[lane] = n_layers if pos0 == 0 else min(self.layers_valid[lane], n_layers)
        return dict(logits=logits, x=x, norms=norms, aborted_at=None)

    def extend_depth(self, lane: int, x_saved: np.ndarray, old_loops: int, new_loops: int) -> dict:
        """Warm start (features page, "Warm-start mid-loop"): the lane's positions
        were run at ``old_loops`` and ``x_saved`` [length, D] is their residual
        after loop iteration old_loops-1; run only iterations old_loops ..
        new_loops-1 on them, filling the upper cache layers."""
        n = self.length[lane]
        if self.layers_valid[lane] != self.n_pre + old_loops or x_saved.shape[0] != n:
            raise ValueError("resume state does not match the lane")
        if not (old_loops < new_loops <= self.l_max):
            raise ValueError("loops out of range")
        x, norms, _ = self._layers(lane, np.array(x_saved, dtype=np.float64), 0,
                                   self.n_pre + old_loops, self.n_pre + new_loops,
                                   False, math.inf, None)
        self.layers_valid[lane] = self.n_pre + new_loops
        return dict(logits=self._head(x), x=x, norms=norms, aborted_at=None)

    # -- the ABI-shaped calls ----------------------------------------------------
    def prefill(self, lane: int, tokens: Sequence[int], loops: int) -> dict:
        """Append prompt tokens to ``lane``; norms are computed but never checked."""
        out = self.forward(lane, tokens, loops, check_safety=False)
        out["next_token"] = argmax_lowest(out["logits"][-1])
        return out

    def decode_step(self, lanes: Sequence[int], loops: Sequence[int], tokens: Sequence[int],
                    threshold: float = math.inf) -> dict:
        """One greedy decode step for a batch of lanes, each with its own loop count.

        A +inf threshold turns the safety check off. An aborted lane returns
        token -1 and status LANE_ABORTED, keeps its length, and is skipped by
        later steps until ``reset_lane``.
        """
        check = not (threshold == math.inf)
        V = self.shape.vocab
        out_tok = np.full(len(lanes), -1, dtype=np.int64)
        out_logits = np.full((len(lanes), V), np.nan)
        out_status = np.zeros(len(lanes), dtype=np.int64)
        out_x = np.full((len(lanes), self.D), np.nan)
        for k, (lane, L, tok) in enumerate(zip(lanes, loops, tokens)):
            if self.status[lane] == LANE_ABORTED:
                out_status[k] = LANE_ABORTED
                continue
            r = self.forward(lane, [tok], L, check_safety=check, threshold=threshold)
            self.norms[lane] = r["norms"][0].copy()
            out_x[k] = r["x"][0]
            if r["aborted_at"] is not None:
                self.status[lane] = LANE_ABORTED
                out_status[k] = LANE_ABORTED
                continue
            out_logits[k] = r["logits"][0]
            out_tok[k] = argmax_lowest(r["logits"][0])
        return dict(tokens=out_tok, logits=out_logits, status=out_status, x=out_x)

    def spec_step(self, lane: int, token: int, draft_loops: int, verify_loops: int,
                  draft_ahead: int) -> dict:
        """One round of self-speculative decoding in chain mode (features page,
        "Self-speculative decoding"): the same weights draft at the shallow depth
        and verify at the deep one.

        ``token`` sits at the lane's current length. The drafter proposes
        ``draft_ahead`` greedy tokens, one decode at ``draft_loops`` each; then the
        input token and the drafts go through ``verify_loops`` in one pass, which
        gives the verifier's greedy token after every one of them. The longest
        run of drafts that the verifier agrees with is kept, followed by the
        verifier's own token at the first disagreement (or after the last
        draft), so the emitted tokens are those greedy decoding at
        ``verify_loops`` produces (the greedy-equality claim of the page's "Tree
        speculative decoding" section, chain mode). The lane's length grows by
        the number emitted; cache entries past it are stale and get overwritten.
        """
        if not (1 <= draft_loops <= verify_loops <= self.l_max):
            raise ValueError("loops out of range")
        if not draft_ahead >= 1:
            raise ValueError("draft_ahead must be positive")
        pos0, valid = self.length[lane], self.layers_valid[lane]
        if pos0 + draft_ahead + 1 > self.max_seq:
            raise CapacityError("cache full")
        if pos0 > 0 and self.n_pre + verify_loops > valid:
            raise CacheGapError("layers above %d miss earlier positions" % valid)
        if self.status[lane] == LANE_ABORTED:
            return dict(tokens=[], drafts=[], verified=[], logits=None)
        drafts, t = [], token
        for _ in range(draft_ahead):
            r = self.forward(lane, [t], draft_loops, check_safety=False)
            t = argmax_lowest(r["logits"][0])
            drafts.append(t)
        # back to the round's start: the verification writes the same positions
        self.length[lane], self.layers_valid[lane] = pos0, valid
        r = self.forward(lane, [token] + drafts, verify_loops, check_safety=False)
        verified = [argmax_lowest(row) for row in r["logits"]]
        agree = 0
        while agree < draft_ahead and drafts[agree] == verified[agree]:
            agree += 1
        n = agree + 1
        self.length[lane] = pos0 + n
        return dict(tokens=verified[:n], drafts=drafts, verified=verified, logits=r["logits"][:n])

    def reset_lane(self, lane: int) -> None:
        self.length[lane] = 0
        self.layers_valid[lane] = 0
        self.status[lane] = LANE_OK
        self.norms[lane] = np.full(self.l_max, np.nan)
        for key in [k for k in self.cache if k[1] == lane]:
            del self.cache[key]


def argmax_lowest(v: np.ndarray) -> int:
    """Index of the maximum; ties go to the lowest index."""
    return int(np.argmax(v))
