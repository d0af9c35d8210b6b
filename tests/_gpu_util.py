"""Helpers for the GPU parity tests: build the HIP model/cache from the seeded
inputs, and compare against the oracle with the parity rules."""
import math

import numpy as np

import synth

REL_TOL = 2e-3          # normwise-max relative error on fp32-accumulated floats
TIE_REL = 2e-3          # top-1 / top-2 logit margin that counts as a near-tie


def torch_gpu():
    import torch
    if not torch.cuda.is_available():
        import pytest
        pytest.skip("no GPU")
    return torch


def record(name: str, **kv):
    """Append a parity measurement to $TL_PARITY_LOG (JSON lines), if set."""
    import json
    import os
    path = os.environ.get("TL_PARITY_LOG")
    if path:
        with open(path, "a") as f:
            f.write(json.dumps(dict(name=name, **kv)) + "\n")


def rel_err(got, ref) -> float:
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.max(np.abs(ref))
    return float(np.max(np.abs(got - ref)) / (den if den > 0 else 1.0))


def token_ok(gpu_tok: int, ref_logits: np.ndarray) -> bool:
    """Argmax must match unless the oracle's top-2 margin is a near-tie."""
    ref_tok = int(np.argmax(ref_logits))
    if gpu_tok == ref_tok:
        return True
    srt = np.sort(ref_logits)
    margin = srt[-1] - srt[-2]
    return margin <= TIE_REL * np.max(np.abs(ref_logits)) and ref_logits[gpu_tok] >= srt[-2]


class GpuModel:
    def __init__(self, shape, weights_np):
        from kv_compression_amd import tl
        torch = torch_gpu()
        self.tl = tl
        self.torch = torch
        self.shape = shape
        self.w_dev = tl.upload_weights(shape, weights_np)
        self.model = tl.Model(shape, self.w_dev)

    def cache(self, mode, n_lanes, max_seq, l_max):
        return self.tl.Cache(self.model, mode, n_lanes, max_seq, l_max)


_MODELS = {}


def gpu_model(shape, seed=0, random_gains=False):
    """Seeded weights (numpy) and their device model, shared by the GPU tests."""
    key = (shape.name, seed, random_gains)
    if key not in _MODELS:
        w = synth.make_weights(shape, seed, random_gains=random_gains)
        _MODELS[key] = (w, GpuModel(shape, w))
    return _MODELS[key]


def decode(tlc, lanes, loops, tokens, threshold=math.inf, want_logits=True):
    """One tl_decode_step; returns host (tokens, logits, status)."""
    import torch
    n = len(lanes)
    tin = torch.tensor(np.asarray(tokens, np.int32), device="cuda")
    tout = torch.empty(n, dtype=torch.int32, device="cuda")
    st = torch.empty(n, dtype=torch.int32, device="cuda")
    lg = torch.empty((n, tlc.model.shape.vocab), dtype=torch.float32, device="cuda") if want_logits else None
    tlc.tl_decode_step(list(lanes), list(loops), tin, threshold, tout, lg, st)
    torch.cuda.synchronize()
    return (tout.cpu().numpy(), lg.cpu().numpy() if lg is not None else None, st.cpu().numpy())
