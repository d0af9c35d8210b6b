"""Seeded synthetic inputs shared by the CPU oracle and the HIP path.

This module only *draws* inputs: model shapes, weights, prompt token ids and
prior hidden states. It holds none of the looped-transformer arithmetic (no
norm, codec, projection, attention or MLP), so the two implementations that
consume these inputs stay independent.

Shapes follow the workloads on the TinyLoop pages (architecture-exclusive
features page, "Store-h KV cache" and "L-aware batching"; measured-benchmarks
page, section 3 "decode throughput after the new cache modes"): a 407M-shaped
and a 2B-shaped weight-shared looped decoder plus a tiny fp32 one. The pages
never print those architectures, so the sizes below are the ones this project
fixes for them.

Random streams
--------------
* Weights: numpy PCG64 ``default_rng(seed)``; matrices drawn in a fixed order
  (embed; then for each unique layer u = 0..n_pre: w_qkv, w_o, w_up, w_down;
  then lm_head) as float64 N(0, 0.02) and rounded to the model dtype.
  RMSNorm gains are ones unless ``random_gains`` asks for 1 + 0.1*N(0, 1)
  (drawn after lm_head), which tests use so that a dropped gain is visible.
* Prompt ids: ``default_rng(seed).integers(0, vocab, size=(lanes, n))``.
* Prior hidden states h: a counter-based generator, Philox4x32-10 (Salmon,
  Moraes, Dror, Shaw, "Parallel random numbers: as easy as 1, 2, 3", SC'11),
  so that the GPU can fill tens of GB of cache without a host round trip and
  the oracle can regenerate any sampled row. Each element has its own
  counter (k, pos, lane, layer) under key (seed, 0x1F0E9D75); the 128 output
  bits are split into eight 16-bit uniforms whose centred sum (an
  Irwin-Hall(8) variate) is scaled to unit variance in one fp32 multiply.
  Every step is integer or a single correctly rounded fp32 operation, so both
  sides produce the same bits. The values are N(0, 1)-like: mean 0,
  variance 1, tails cut at about +-4.9.
"""
from __future__ import annotations

import concurrent.futures
import dataclasses
import os
from typing import Dict, List, Optional

import numpy as np

__all__ = [
    "ModelShape", "Workload", "SHAPES", "WORKLOADS", "workload",
    "make_weights", "make_prompts", "philox4x32_10", "prior_h",
    "PHILOX_H_KEY1", "NORMAL_SCALE_F32",
]


@dataclasses.dataclass(frozen=True)
class ModelShape:
    name: str
    d_model: int
    n_heads: int
    d_head: int
    d_mlp: int
    n_pre: int
    vocab: int
    dtype: str          # "f32" | "f16"
    norm_eps: float = 1e-5


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    shape: ModelShape
    modes: tuple        # cache modes the workload is run in ("int4", "int8", "f16", "f32", "kv", "delta8")
    lanes: int
    loops: tuple        # per-lane loop counts (cycled over lanes)
    l_max: int
    context: int        # prompt tokens (or prior positions) per lane
    prior_synthetic: bool   # True: context is synthetic prior h, not prompt tokens
    chunk: int          # prefill chunk (tokens) timed after the prior context, 0 = none
    steps: int          # greedy decode steps
    threshold: float    # safety-norm threshold for the decode steps
    seed_weights: int = 0
    seed_prompt: int = 1
    seed_prior: int = 2

    @property
    def max_seq(self) -> int:
        return self.context + self.chunk + self.steps

    def lane_loops(self) -> List[int]:
        return [self.loops[i % len(self.loops)] for i in range(self.lanes)]


SHAPES: Dict[str, ModelShape] = {
    "tiny": ModelShape("tiny", 128, 4, 32, 512, 1, 256, "f32"),
    "407m": ModelShape("407m", 1024, 16, 64, 4096, 2, 32000, "f16"),
    "2b": ModelShape("2b", 2048, 16, 128, 8192, 2, 32000, "f16"),
}

_INF = float("inf")

WORKLOADS: Dict[str, Workload] = {
    # one decode step after 64 synthetic prior positions, safety threshold 50
    "tiny-f32-ctx64": Workload("tiny-f32-ctx64", SHAPES["tiny"], ("f32", "kv"), 1, (2,), 2,
                               64, True, 0, 1, 50.0),
    # 1024-token prompt, 128 greedy steps, fp16 h
    "407m-f16h-ctx1024": Workload("407m-f16h-ctx1024", SHAPES["407m"], ("f16",), 1, (8,), 8,
                                  1024, False, 0, 128, _INF),
    # the headline: 4 lanes x 4096-token prompts, 128 greedy steps, INT4-h
    "407m-int4h-ctx4096-b4": Workload("407m-int4h-ctx4096-b4", SHAPES["407m"],
                                      ("int4", "int8", "f16", "kv", "delta8"), 4, (8,), 8,
                                      4096, False, 0, 128, _INF),
    # 48 lanes at loops [4, 16, 32] on one 34-layer cache, 2048-token prompts, 64 steps
    "2b-int4h-laware-b48": Workload("2b-int4h-laware-b48", SHAPES["2b"], ("int4",), 48,
                                    (4, 16, 32), 32, 2048, False, 0, 64, _INF),
    # 32768 synthetic prior positions, one 512-token chunk, 32 steps
    "2b-int4h-ctx32k-b8": Workload("2b-int4h-ctx32k-b8", SHAPES["2b"], ("int4",), 8, (8,), 8,
                                   32768, True, 512, 32, _INF),
}


def workload(name: str) -> Workload:
    return WORKLOADS[name]


def _np_dtype(dtype: str):
    return {"f32": np.float32, "f16": np.float16}[dtype]


def make_weights(shape: ModelShape, seed: int = 0, random_gains: bool = False,
                 std: float = 0.02) -> dict:
    """Draw the model's weights (numpy arrays in the model dtype).

    Layout (row-major, y = W @ x): embed [V, D]; layers[u] for u in 0..n_pre
    (u == n_pre is the shared loop block) with norm1 [D], w_qkv [3D, D] (rows
    q | k | v, head-major inside each), w_o [D, D], norm2 [D], w_up [F, D],
    w_down [D, F]; final_norm [D]; lm_head [V, D].
    """
    rng = np.random.default_rng(seed)
    dt = _np_dtype(shape.dtype)
    D, F, V = shape.d_model, shape.d_mlp, shape.vocab

    def draw(*size):
        return (rng.standard_normal(size, dtype=np.float64) * std).astype(dt)

    w = {"embed": draw(V, D), "layers": []}
    for _ in range(shape.n_pre + 1):
        w["layers"].append({
            "w_qkv": draw(3 * D, D),
            "w_o": draw(D, D),
            "w_up": draw(F, D),
            "w_down": draw(D, F),
        })
    w["lm_head"] = draw(V, D)

    def gain():
        if random_gains:
            return (1.0 + 0.1 * rng.standard_normal(D, dtype=np.float64)).astype(dt)
        return np.ones(D, dtype=dt)

    for layer in w["layers"]:
        layer["norm1"] = gain()
        layer["norm2"] = gain()
    w["final_norm"] = gain()
    return w


def make_prompts(vocab: int, lanes: int, n: int, seed: int = 1) -> np.ndarray:
    """Prompt token ids, uniform on [0, vocab), lane-major, int32 [lanes, n]."""
    rng = np.random.default_rng(seed)
    return rng.integers(0, vocab, size=(lanes, n)).astype(np.int32)


# --------------------------------------------------------------------------
# Philox4x32-10 (Salmon et al., SC'11): multipliers, Weyl key increments and
# the round function as published with the Random123 library.
# --------------------------------------------------------------------------
_PHILOX_M0 = np.uint64(0xD2511F53)
_PHILOX_M1 = np.uint64(0xCD9E8D57)
_PHILOX_W0 = np.uint32(0x9E3779B9)
_PHILOX_W1 = np.uint32(0xBB67AE85)
_MASK32 = np.uint64(0xFFFFFFFF)

PHILOX_H_KEY1 = 0x1F0E9D75
# fp32 constant 1 / (65536 * sqrt(2/3)), bit pattern 0x379CC471: scales the
# centred Irwin-Hall(8) sum of 16-bit uniforms to unit variance.
NORMAL_SCALE_F32 = np.array([0x379CC471], dtype=np.uint32).view(np.float32)[0]


def philox4x32_10(ctr, key):
    """Vectorised Philox4x32-10.

    ctr: uint32 array [..., 4]; key: uint32 array [..., 2] (broadcastable).
    Returns uint32 [..., 4].
    """
    c = np.asarray(ctr, dtype=np.uint32)
    k = np.asarray(key, dtype=np.uint32)
    c0, c1, c2, c3 = (c[..., i].astype(np.uint64) for i in range(4))
    k0 = np.broadcast_to(k[..., 0], c[..., 0].shape).astype(np.uint64)
    k1 = np.broadcast_to(k[..., 1], c[..., 0].shape).astype(np.uint64)
    for r in range(10):
        if r:
            k0 = (k0 + np.uint64(_PHILOX_W0)) & _MASK32
            k1 = (k1 + np.uint64(_PHILOX_W1)) & _MASK32
        p0 = _PHILOX_M0 * c0
        p1 = _PHILOX_M1 * c2
        hi0, lo0 = p0 >> np.uint64(32), p0 & _MASK32
        hi1, lo1 = p1 >> np.uint64(32), p1 & _MASK32
        c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0
    return np.stack([c0, c1, c2, c3], axis=-1).astype(np.uint32)


def prior_h(seed: int, layer: int, lane: int, positions, d_model: int) -> np.ndarray:
    """Synthetic prior hidden state rows as float32 [len(positions), d_model].

    Element (pos, k) uses counter (k, pos, lane, layer) and key
    (seed, PHILOX_H_KEY1). The float32 values are what the cache writer
    receives before it rounds them to the model dtype.
    """
    pos = np.asarray(positions, dtype=np.uint32).reshape(-1)
    k = np.arange(d_model, dtype=np.uint32)
    key = np.array([seed, PHILOX_H_KEY1], dtype=np.uint32)
    res = np.empty((pos.size, d_model), dtype=np.float32)
    # chunks of positions keep the generator's temporaries in cache; numpy
    # releases the interpreter lock inside its array operations, so large
    # requests run their chunks on a few threads (each chunk writes its own
    # rows, the values do not depend on the split)
    step = max(1, (1 << 16) // max(d_model, 1))

    def chunk(p0):
        pc = pos[p0:p0 + step]
        ctr = np.empty((pc.size, d_model, 4), dtype=np.uint32)
        ctr[..., 0] = k[None, :]
        ctr[..., 1] = pc[:, None]
        ctr[..., 2] = np.uint32(lane)
        ctr[..., 3] = np.uint32(layer)
        out = philox4x32_10(ctr, key)                     # [P, D, 4] uint32
        lo = (out & np.uint32(0xFFFF)).astype(np.int64)
        hi = (out >> np.uint32(16)).astype(np.int64)
        s = lo.sum(axis=-1) + hi.sum(axis=-1)             # sum of eight 16-bit uniforms
        centred = (s - 262140).astype(np.float32)         # exact: |value| < 2**24
        res[p0:p0 + pc.size] = centred * NORMAL_SCALE_F32  # one fp32 rounding

    starts = range(0, pos.size, step)
    workers = min(16, len(os.sched_getaffinity(0)), len(starts))
    if workers > 1 and pos.size * d_model >= (1 << 22):
        with concurrent.futures.ThreadPoolExecutor(max_workers=workers) as ex:
            list(ex.map(chunk, starts))
    else:
        for p0 in starts:
            chunk(p0)
    return res
