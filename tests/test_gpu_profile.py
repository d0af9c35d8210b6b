"""Kernel timing (tl_profile_start / tl_profile_stop), which the benchmark's
rooflines divide by: every decode attention launch is timed by a pair of
events attached to that launch. Checked: one timed launch per layer-iteration
of each step (all active rows share a launch), a positive total below the
steps' own wall time, and results bitwise equal to the same steps run
untimed from an identical cache, in every attention path (store-h
reconstruction in the explicit and absorbed orders, fp16-h, and the
stored-K/V baseline)."""
import numpy as np
import pytest

import synth
from tests._gpu_util import decode, gpu_model, torch_gpu

pytestmark = pytest.mark.gpu

S407 = synth.SHAPES["407m"]


def _filled_cache(gm, mode, lanes, ctx, L):
    n_layers = S407.n_pre + L
    c = gm.cache(mode, lanes, ctx + 8, L)
    for k in range(lanes):
        for layer in range(n_layers):
            c.tl_cache_fill_synthetic(k, layer, 0, ctx, 11 + k)
        c.tl_cache_set_length(k, ctx, n_layers)
    return c


@pytest.mark.parametrize("mode,order", [("int4", "explicit"), ("int4", "absorbed"),
                                        ("f16", "explicit"), ("kv", "explicit")])
def test_profile_times_each_attention_launch(mode, order):
    torch = torch_gpu()
    _, gm = gpu_model(S407)
    L, lanes, ctx, steps = 3, 2, 700, 3
    timed = _filled_cache(gm, mode, lanes, ctx, L)
    plain = _filled_cache(gm, mode, lanes, ctx, L)
    if order != "explicit":
        timed.tl_cache_set_attention(order)
        plain.tl_cache_set_attention(order)
    toks = [int(x) for x in synth.make_prompts(S407.vocab, lanes, 1, 3)[:, 0]]
    ta, tb = list(toks), list(toks)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    timed.tl_profile_start()
    e0.record()
    outs_timed = []
    for _ in range(steps):
        t, lg, st = decode(timed, list(range(lanes)), [L] * lanes, ta)
        outs_timed.append((t, lg, st))
        ta = [int(x) for x in t]
    e1.record()
    ms, n = timed.tl_profile_stop()
    torch.cuda.synchronize()
    wall_ms = e0.elapsed_time(e1)
    assert n == steps * (S407.n_pre + L)
    assert 0.0 < ms < wall_ms, (ms, wall_ms)
    for t_ref, lg_ref, st_ref in outs_timed:
        t, lg, st = decode(plain, list(range(lanes)), [L] * lanes, tb)
        assert np.array_equal(t, t_ref) and np.array_equal(st, st_ref)
        assert np.array_equal(lg, lg_ref)
        tb = [int(x) for x in t]
    # a second window starts from zero
    timed.tl_profile_start()
    decode(timed, list(range(lanes)), [L] * lanes, ta)
    ms2, n2 = timed.tl_profile_stop()
    assert n2 == S407.n_pre + L and ms2 > 0.0
