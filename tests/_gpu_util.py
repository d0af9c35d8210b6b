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


# ---------------------------------------------------------------------------
# INT / delta codes decided differently by FP32 (GPU) and FP64 (oracle) h
# ---------------------------------------------------------------------------
# cache modes whose rows are codes decided by rounding (the synced helpers'
# adoption applies to them only)
CODED_MODES = ("int4", "int8", "delta8")


def _codec(mode, shape):
    """(group, qmax, qmin) of the mode's codec."""
    if mode == "int4":
        return 32, 7, -8
    if mode == "int8":
        return shape.d_model, 127, -127
    return shape.d_head, 127, -127      # delta8: one scale per head


def flip_explained(h16, cin, gq, gs_bits, oq, os_bits, group, qmax, qmin, tol=REL_TOL):
    """True if every group whose GPU codes or scale differ from the oracle's is
    the codec's exact result for an h row within the float bar of the
    oracle's own: some h' with |h' - h| <= tol * max|h| elementwise (the
    normwise-max measure float results are held to). The codec is monotone in
    each element (q = clip(rint(c / s)) for s > 0), so under the GPU's scale
    s each element's admissible h' is an interval, and the scale must come
    back as fp16(absmax / qmax) for an absmax reachable from those intervals.
    h16: the oracle's h row (fp16); cin: the float32 row the oracle's codec
    was applied to (h itself, or h minus the reconstruction below in the delta
    mode), so a moved row is coded as h' - (h - cin)."""
    hf = np.asarray(h16, np.float16).astype(np.float64)
    off = hf - np.asarray(cin, np.float32).astype(np.float64)
    tau = tol * np.max(np.abs(hf))
    for g in range(hf.shape[0] // group):
        sl = slice(g * group, (g + 1) * group)
        if np.array_equal(gq[sl], oq[sl]) and gs_bits[g] == os_bits[g]:
            continue
        sg = float(np.array([gs_bits[g]], np.uint16).view(np.float16)[0])
        q = gq[sl].astype(np.float64)
        lo, hi = hf[sl] - tau, hf[sl] + tau
        if sg == 0:
            if np.any(q != 0):
                return False
            a, b = lo, hi
        else:
            # c / s in [q - 1/2, q + 1/2] codes to q (the clamps open the ends)
            ca = np.where(q <= qmin, -np.inf, (q - 0.5) * sg)
            cb = np.where(q >= qmax, np.inf, (q + 0.5) * sg)
            a = np.maximum(lo, ca + off[sl])
            b = np.minimum(hi, cb + off[sl])
            if np.any(a > b):
                return False
        # the absmax over the intervals ranges over [max of the smallest
        # |h'|, max of the largest |h'|]; the scale is monotone in it
        ca, cb = a - off[sl], b - off[sl]
        small = np.where((ca <= 0) & (cb >= 0), 0.0, np.minimum(np.abs(ca), np.abs(cb)))
        large = np.maximum(np.abs(ca), np.abs(cb))

        def scale(am):
            return float(np.array([am / qmax], np.float32).astype(np.float16)[0])
        if not scale(np.max(small)) <= sg <= scale(np.max(large)):
            return False
    return True


def _gpu_row(c, mode, lane, layer, pos, shape):
    """The GPU cache's entry at (lane, layer, pos): dict(q, s) of codes and fp16
    scale bits, or dict(h) of an fp16 h row (the delta mode's unique layers)."""
    import torch
    D = shape.d_model
    if mode == "delta8" and layer < shape.n_pre:
        h = torch.empty((1, D), dtype=torch.float16, device="cuda")
        c.tl_cache_read(lane, layer, pos, 1, d_h=h)
        torch.cuda.synchronize()
        return {"h": h.cpu().numpy()[0]}
    group, _, _ = _codec(mode, shape)
    q = torch.empty((1, D), dtype=torch.int8, device="cuda")
    s = torch.empty((1, D // group), dtype=torch.int16, device="cuda")
    c.tl_cache_read(lane, layer, pos, 1, q, s)
    torch.cuda.synchronize()
    return {"q": q.cpu().numpy()[0], "s": s.cpu().numpy()[0].view(np.uint16).copy()}


def _orc_row(orc, lane, layer, pos):
    slot = orc._slot(layer, lane)
    if "h" in slot:
        return {"h": slot["h"][pos].astype(np.float16)}
    return {"q": slot["q"][pos].copy(), "s": slot["s"][pos].view(np.uint16).copy()}


def decode_synced(c, orc, lanes, loops, toks, threshold=math.inf):
    """One decode step of `lanes` (the same lane ids on both sides) on the GPU
    and in the oracle. Where the GPU coded a cache group of the step's
    position differently, the group must be a rounding-boundary decision: the
    codec's exact result for an h within the 2e-3 float bar of the oracle's
    own (flip_explained; in the delta mode a unique layer's fp16 h may differ
    by the same bar). The oracle then adopts that row
    and runs the step again, lowest differing layer first, until both caches
    hold the same entries; the oracle's final result is returned with the
    GPU's (tokens, logits, status) and the number of rows adopted."""
    mode, sh = orc.mode, orc.shape
    if mode not in CODED_MODES:
        # fp16 / fp32 h and stored K/V: nothing is decided discretely
        t, lg, st = decode(c, lanes, loops, toks, threshold)
        return t, lg, st, orc.decode_step(lanes, loops, toks, threshold), 0
    group, qmax, qmin = _codec(mode, sh)
    t, lg, st = decode(c, lanes, loops, toks, threshold)
    pos = {k: orc.length[k] for k in lanes}
    nl = {k: sh.n_pre + L for k, L in zip(lanes, loops)}
    gpu = {(layer, k): _gpu_row(c, mode, k, layer, pos[k], sh) for k in lanes for layer in range(nl[k])}
    snap = (list(orc.length), list(orc.layers_valid), list(orc.status), [x.copy() for x in orc.norms])
    adopted = 0
    for _ in range(sum(nl.values()) + 1):
        orc.h_log = {}
        r = orc.decode_step(lanes, loops, toks, threshold)
        first = {}
        for k in lanes:
            for layer in range(nl[k]):
                if not _same(gpu[(layer, k)], _orc_row(orc, k, layer, pos[k])):
                    first[k] = layer
                    break
        if not first:
            orc.h_log = None
            return t, lg, st, r, adopted
        for k, layer in first.items():
            _adopt(orc, (layer, k, pos[k]), gpu[(layer, k)], _orc_row(orc, k, layer, pos[k]), group, qmax, qmin)
            adopted += 1
        orc.length, orc.layers_valid, orc.status = list(snap[0]), list(snap[1]), list(snap[2])
        orc.norms = [x.copy() for x in snap[3]]
    raise AssertionError("the caches did not agree after adopting every explained row")


def _same(g, o):
    if "h" in g:
        return np.array_equal(g["h"].view(np.uint16), o["h"].view(np.uint16))
    return np.array_equal(g["q"], o["q"]) and np.array_equal(g["s"], o["s"])


def _adopt(orc, key, g, o, group, qmax, qmin):
    """Check that the GPU's row g differs from the oracle's row o only by
    rounding-boundary decisions on an h within the float bar of the oracle's
    own (flip_explained; fp16 h rows: within the bar elementwise, relative to
    the row's largest element), then make the oracle store g."""
    h16, cin = orc.h_log[key]
    if "h" in g:
        ho = o["h"].astype(np.float64)
        assert np.all(np.abs(g["h"].astype(np.float64) - ho) <= REL_TOL * np.max(np.abs(ho))), ("h row", key)
        orc.row_override[key] = {"h": g["h"]}
    else:
        if not flip_explained(h16, cin, g["q"], g["s"], o["q"], o["s"], group, qmax, qmin):
            import os
            d = os.environ.get("TL_PARITY_DUMP")
            if d:
                os.makedirs(d, exist_ok=True)
                np.savez(os.path.join(d, "flip_%s_%d_%d_%d.npz" % ((orc.mode,) + key)), h16=h16, cin=cin,
                         gq=g["q"], gs=g["s"], oq=o["q"], os=o["s"])
            raise AssertionError(("codes not explained by an h within the float bar", orc.mode, key))
        orc.row_override[key] = {"q": g["q"], "s": g["s"].view(np.float16)}


def prefill_synced(c, orc, lane, tokens, loops):
    """Prefill `tokens` into `lane` on the GPU and in the oracle; as in
    decode_synced, every cache row the GPU coded differently (any position of
    the prompt) must be a rounding-boundary decision on the oracle's h, and the
    oracle adopts such rows, lowest layer first, re-running its prefill until
    both caches agree. Returns the GPU's next token and last logits, the
    oracle's result and the number of rows adopted."""
    mode, sh = orc.mode, orc.shape
    nxt, lg = c.prefill(lane, tokens, loops)
    g_next, g_last = int(nxt.cpu().numpy()[0]), lg.cpu().numpy()
    if mode not in CODED_MODES:
        return g_next, g_last, orc.prefill(lane, tokens, loops), 0
    group, qmax, qmin = _codec(mode, sh)
    n = len(tokens)
    pos0 = orc.length[lane]
    nl = sh.n_pre + loops
    gpu = {(layer, p): _gpu_row(c, mode, lane, layer, pos0 + p, sh) for layer in range(nl) for p in range(n)}
    snap = (orc.length[lane], orc.layers_valid[lane])
    adopted = 0
    for _ in range(nl + 1):
        orc.h_log = {}
        r = orc.prefill(lane, tokens, loops)
        for layer in range(nl):
            bad = [p for p in range(n) if not _same(gpu[(layer, p)], _orc_row(orc, lane, layer, pos0 + p))]
            if bad:
                break
        else:
            orc.h_log = None
            return g_next, g_last, r, adopted
        for p in bad:
            key = (layer, lane, pos0 + p)
            _adopt(orc, key, gpu[(layer, p)], _orc_row(orc, lane, layer, pos0 + p), group, qmax, qmin)
            adopted += 1
        orc.length[lane], orc.layers_valid[lane] = snap
    raise AssertionError("the caches did not agree after adopting every explained row")
