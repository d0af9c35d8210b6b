"""Warm start mid-loop on the GPU (features page, "Warm-start mid-loop"): a
prompt run at L = 4 and deepened to L = 8 from its saved residuals
(tl_prefill_chunk_x, tl_extend_depth).

* Parity with the oracle's extend_depth (fp16-h and stored K/V, whose codecs
  are exact, at a context of 40 positions; INT codes at so short a context
  are governed by the code-flip reading of the design notes).
* The GPU's own invariant, bit for bit: with the same chunking, the warm
  path leaves the same cache, logits and later decode steps as a fresh
  L = 8 prefill, because every chunk runs the same kernels on the same
  inputs (layers 0 .. n_pre+3 in the first pass, the rest from the saved
  residual in the second).
* Argument errors are refused before anything is enqueued."""
import numpy as np
import pytest

import oracle
import synth
from tests._gpu_util import REL_TOL, decode, gpu_model, record, rel_err, token_ok, torch_gpu

pytestmark = pytest.mark.gpu

S407 = synth.SHAPES["407m"]
N_PROMPT, CHUNK = 40, 16


def _prompt(seed=5):
    return [int(t) for t in synth.make_prompts(S407.vocab, 1, N_PROMPT, seed)[0]]


@pytest.mark.parametrize("mode", ["f16", "kv"])
def test_extend_depth_matches_oracle(mode):
    torch_gpu()
    w, gm = gpu_model(S407, random_gains=True)
    pr = _prompt()
    c = gm.cache(mode, 1, 64, 8)
    _, _, x = c.prefill_x(0, pr, 4, chunk=CHUNK)
    nxt, lg = c.extend_depth(0, x, 4, 8, chunk=CHUNK)
    orc = oracle.LoopedOracle(S407, w, mode, 1, 64, 8)
    r4 = orc.forward(0, pr, 4, check_safety=False)
    r8 = orc.extend_depth(0, r4["x"], 4, 8)
    e = rel_err(lg.cpu().numpy(), r8["logits"][-1])
    record("resume_logits", mode=mode, rel=e)
    assert e <= REL_TOL, e
    ex = rel_err(x.cpu().numpy(), r8["x"])
    record("resume_residual", mode=mode, rel=ex)
    assert ex <= REL_TOL, ex
    tok = int(nxt.cpu().numpy()[0])
    assert token_ok(tok, r8["logits"][-1])
    for step in range(3):
        t, lgd, st = decode(c, [0], [8], [tok])
        r = orc.decode_step([0], [8], [tok])
        assert st[0] == 0 and r["status"][0] == oracle.LANE_OK
        e = rel_err(lgd[0], r["logits"][0])
        record("resume_decode", mode=mode, step=step, rel=e)
        assert e <= REL_TOL, (step, e)
        assert token_ok(int(t[0]), r["logits"][0])
        tok = int(t[0])


def test_extend_depth_bitwise_equals_fresh_prefill():
    torch = torch_gpu()
    w, gm = gpu_model(S407, random_gains=True)
    pr = _prompt(6)
    fresh = gm.cache("int4", 1, 64, 8)
    nf, lf = fresh.prefill(0, pr, 8, chunk=CHUNK)
    warm = gm.cache("int4", 1, 64, 8)
    _, _, x = warm.prefill_x(0, pr, 4, chunk=CHUNK)
    nw, lw = warm.extend_depth(0, x, 4, 8, chunk=CHUNK)
    torch.cuda.synchronize()
    assert np.array_equal(lf.cpu().numpy().view(np.uint32), lw.cpu().numpy().view(np.uint32))
    assert int(nf.cpu()[0]) == int(nw.cpu()[0])
    D = S407.d_model
    for layer in range(S407.n_pre + 8):
        got = []
        for cache in (fresh, warm):
            codes = torch.empty((N_PROMPT, D), dtype=torch.int8, device="cuda")
            scales = torch.empty((N_PROMPT, D // 32), dtype=torch.int16, device="cuda")
            cache.tl_cache_read(0, layer, 0, N_PROMPT, codes, scales)
            torch.cuda.synchronize()
            got.append((codes.cpu().numpy(), scales.cpu().numpy()))
        assert np.array_equal(got[0][0], got[1][0]) and np.array_equal(got[0][1], got[1][1]), layer
    tf = tw = int(nf.cpu()[0])
    for _ in range(3):
        a = decode(fresh, [0], [8], [tf])
        b = decode(warm, [0], [8], [tw])
        assert np.array_equal(a[1].view(np.uint32), b[1].view(np.uint32))
        tf, tw = int(a[0][0]), int(b[0][0])


def test_extend_depth_errors():
    from kv_compression_amd import tl
    torch = torch_gpu()
    w, gm = gpu_model(S407)
    c = gm.cache("int4", 2, 64, 8)
    x = torch.zeros((N_PROMPT, S407.d_model), dtype=torch.float32, device="cuda")
    with pytest.raises(tl.TLError) as e:           # empty lane
        c.tl_extend_depth(0, 0, CHUNK, 4, 8, x[:CHUNK])
    assert e.value.status == tl.TL_E_ARG
    _, _, x = c.prefill_x(0, _prompt(), 4, chunk=CHUNK)
    with pytest.raises(tl.TLError) as e:           # the lane holds n_pre + 4 layers, not n_pre + 3
        c.tl_extend_depth(0, 0, CHUNK, 3, 8, x[:CHUNK])
    assert e.value.status == tl.TL_E_CACHE_GAP
    with pytest.raises(tl.TLError) as e:           # loops must grow
        c.tl_extend_depth(0, 0, CHUNK, 4, 4, x[:CHUNK])
    assert e.value.status == tl.TL_E_ARG
    with pytest.raises(tl.TLError) as e:           # chunks start at position 0
        c.tl_extend_depth(0, CHUNK, CHUNK, 4, 8, x[CHUNK:2 * CHUNK])
    assert e.value.status == tl.TL_E_ARG
    c.tl_extend_depth(0, 0, CHUNK, 4, 8, x[:CHUNK])
    with pytest.raises(tl.TLError) as e:           # no decode while the extension is half done
        decode(c, [0], [8], [1])
    assert e.value.status == tl.TL_E_ARG
    tok = torch.tensor([1], dtype=torch.int32, device="cuda")
    with pytest.raises(tl.TLError) as e:           # nor prefill
        c.tl_prefill_chunk(0, 8, tok)
    assert e.value.status == tl.TL_E_ARG
    with pytest.raises(tl.TLError) as e:           # nor a chunk of another extension
        c.tl_extend_depth(0, CHUNK, CHUNK, 4, 7, x[CHUNK:2 * CHUNK])
    assert e.value.status == tl.TL_E_ARG
    c.tl_extend_depth(0, CHUNK, N_PROMPT - CHUNK, 4, 8, x[CHUNK:])
    t, _, st = decode(c, [0], [8], [1])           # deepened: decodes at L = 8
    assert st[0] == 0 and 0 <= int(t[0]) < S407.vocab
