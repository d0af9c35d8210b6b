"""The no-allocation decode step (tl_decode_step_static: step scratch in a
static array of the library) against tl_decode_step, through the C ABI, from
the same cache state: tokens and lane status identical, logits and residual
norms bit for bit (the same kernels run on the same inputs; only the scratch
addresses differ), on two calls in a row, the second with fewer lanes. Steps
too large for the static array and the modes it does not cover are refused
before anything is enqueued."""
import math

import numpy as np
import pytest

import synth
from tests._gpu_util import gpu_model, torch_gpu

pytestmark = pytest.mark.gpu

S407 = synth.SHAPES["407m"]


def _step(c, fn, lanes, loops, toks, thr):
    import torch
    n = len(lanes)
    tin = torch.tensor(np.asarray(toks, np.int32), device="cuda")
    tout = torch.empty(n, dtype=torch.int32, device="cuda")
    st = torch.empty(n, dtype=torch.int32, device="cuda")
    lg = torch.empty((n, S407.vocab), dtype=torch.float32, device="cuda")
    fn(list(lanes), list(loops), tin, thr, tout, lg, st)
    torch.cuda.synchronize()
    return tout.cpu().numpy(), lg.cpu().numpy(), st.cpu().numpy()


def _both(c, lanes, loops, toks, lengths, nl, thr):
    """The plain step, then the static one from the same lane state."""
    a = _step(c, c.tl_decode_step, lanes, loops, toks, thr)
    na = [c.tl_residual_norms(k) for k in lanes]
    for k in lanes:
        c.tl_cache_set_length(k, lengths[k], nl)
    b = _step(c, c.tl_decode_step_static, lanes, loops, toks, thr)
    nb = [c.tl_residual_norms(k) for k in lanes]
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[2], b[2])
    assert np.array_equal(a[1].view(np.uint32), b[1].view(np.uint32))
    for x, y in zip(na, nb):
        assert np.array_equal(x.view(np.uint32), y.view(np.uint32))
    return b


@pytest.mark.parametrize("mode", ["int4", "f16", "kv"])
def test_static_step_matches_decode_step(mode):
    torch_gpu()
    w, gm = gpu_model(S407)
    n_lanes, ctx, L = 4, 300, 3
    nl = S407.n_pre + L
    c = gm.cache(mode, n_lanes, ctx + 8, L)
    for k in range(n_lanes):
        for layer in range(nl):
            c.tl_cache_fill_synthetic(k, layer, 0, ctx, 2)
        c.tl_cache_set_length(k, ctx, nl)
    lengths = {k: ctx for k in range(n_lanes)}
    toks = [int(x) for x in synth.make_prompts(S407.vocab, n_lanes, 1, 4)[:, 0]]
    loops = [3, 1, 2, 3]
    t, lg, st = _both(c, [0, 1, 2, 3], loops, toks, lengths, nl, 1e4)
    assert np.all(st == 0) and np.all(np.isfinite(lg))
    # a second call with fewer lanes, from the state the static step left
    for k in range(n_lanes):
        lengths[k] = ctx + 1
    t2, lg2, st2 = _both(c, [2, 0], [2, 3], [int(t[2]), int(t[0])], lengths, nl, 1e4)
    assert np.all(st2 == 0)
    # and the plain step goes on from the static one's state
    t3, _, st3 = _step(c, c.tl_decode_step, [0, 2], [3, 2], [int(t2[1]), int(t2[0])], 1e4)
    assert np.all(st3 == 0) and np.all(t3 >= 0)


def test_static_step_refusals():
    from kv_compression_amd import tl
    torch = torch_gpu()
    w, gm = gpu_model(S407)
    # 256 lanes: about 39 MB of step scratch, past the 16 MiB array
    n = 256
    c = gm.cache("int4", n, 4, 1)
    toks = torch.zeros(n, dtype=torch.int32, device="cuda")
    tout = torch.empty(n, dtype=torch.int32, device="cuda")
    st = torch.empty(n, dtype=torch.int32, device="cuda")
    with pytest.raises(tl.TLError) as e:
        c.tl_decode_step_static(list(range(n)), [1] * n, toks, math.inf, tout, None, st)
    assert e.value.status == tl.TL_E_CAPACITY and "static scratch" in str(e.value)
    c.tl_decode_step(list(range(n)), [1] * n, toks, math.inf, tout, None, st)   # the lanes were untouched
    torch.cuda.synchronize()
    assert np.all(st.cpu().numpy() == 0)
    del c
    # the absorbed order and the delta-KV mode are not covered
    c = gm.cache("int4", 1, 8, 1)
    c.tl_cache_set_attention("absorbed")
    with pytest.raises(tl.TLError) as e:
        c.tl_decode_step_static([0], [1], toks[:1], math.inf, tout[:1], None, st[:1])
    assert e.value.status == tl.TL_E_UNSUPPORTED
    c = gm.cache("delta8", 1, 8, 1)
    with pytest.raises(tl.TLError) as e:
        c.tl_decode_step_static([0], [1], toks[:1], math.inf, tout[:1], None, st[:1])
    assert e.value.status == tl.TL_E_UNSUPPORTED
