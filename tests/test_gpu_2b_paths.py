"""The delta-KV codec, warm start mid-loop and self-speculative decoding at the
2B shape (d_model 2048, 16 heads of 128, MLP 8192), whose kernels take the
other head width and element counts per thread than at 407M. Short contexts
keep the oracle quick; the bars are those of the 407M tests."""
import numpy as np
import pytest

import oracle
import synth
from tests._gpu_util import REL_TOL, decode, gpu_model, record, rel_err, token_ok, torch_gpu

pytestmark = pytest.mark.gpu

S2B = synth.SHAPES["2b"]


def _prompt(n, seed):
    return [int(t) for t in synth.make_prompts(S2B.vocab, 1, n, seed)[0]]


def test_2b_delta_prefill_and_decode():
    torch_gpu()
    w, gm = gpu_model(S2B, random_gains=True)
    pr = _prompt(90, 31)
    c = gm.cache("delta8", 1, 100, 3)
    orc = oracle.LoopedOracle(S2B, w, "delta8", 1, 100, 3)
    nxt, lg = c.prefill(0, pr, 3, chunk=64)
    ro = orc.prefill(0, pr, 3)
    e = rel_err(lg.cpu().numpy(), ro["logits"][-1])
    record("2b_delta_prefill", rel=e)
    assert e <= REL_TOL, e
    tok = int(nxt.cpu()[0])
    assert token_ok(tok, ro["logits"][-1])
    for step in range(2):
        t, lgd, st = decode(c, [0], [3], [tok])
        r = orc.decode_step([0], [3], [tok])
        e = rel_err(lgd[0], r["logits"][0])
        record("2b_delta_decode", step=step, rel=e)
        assert st[0] == 0 and e <= REL_TOL, (step, e)
        assert token_ok(int(t[0]), r["logits"][0])
        tok = int(t[0])


def test_2b_warm_start_bitwise():
    torch = torch_gpu()
    w, gm = gpu_model(S2B, random_gains=True)
    pr = _prompt(40, 32)
    fresh = gm.cache("int4", 1, 48, 4)
    nf, lf = fresh.prefill(0, pr, 4, chunk=16)
    warm = gm.cache("int4", 1, 48, 4)
    _, _, x = warm.prefill_x(0, pr, 2, chunk=16)
    nw, lw = warm.extend_depth(0, x, 2, 4, chunk=16)
    torch.cuda.synchronize()
    assert np.array_equal(lf.cpu().numpy().view(np.uint32), lw.cpu().numpy().view(np.uint32))
    assert int(nf.cpu()[0]) == int(nw.cpu()[0])
    tf = tw = int(nf.cpu()[0])
    for _ in range(2):
        a = decode(fresh, [0], [4], [tf])
        b = decode(warm, [0], [4], [tw])
        assert np.array_equal(a[1].view(np.uint32), b[1].view(np.uint32))
        tf, tw = int(a[0][0]), int(b[0][0])


def test_2b_speculative_matches_oracle_greedy():
    torch_gpu()
    w, gm = gpu_model(S2B, random_gains=True)
    pr = _prompt(24, 33)
    c = gm.cache("f16", 1, 64, 4)
    nxt, _ = c.prefill(0, pr, 4, chunk=16)
    t0 = int(nxt.cpu()[0])
    got, rounds = c.generate_speculative(0, t0, 8, 1, 4, 3)
    record("2b_spec_rounds", rounds=rounds)
    orc = oracle.LoopedOracle(S2B, w, "f16", 1, 64, 4)
    r = orc.prefill(0, pr, 4)
    assert token_ok(t0, r["logits"][-1])
    prev = t0
    for i, g in enumerate(got):
        r = orc.decode_step([0], [4], [prev])
        assert token_ok(g, r["logits"][0]), (i, g)
        prev = g


@pytest.mark.parametrize("mode", ["kv", "f16", "int8"])
def test_2b_chunked_prefill_and_decode(mode):
    """The prefill attention at 128-wide heads: fp16 stored K|V (no lo half)
    and fp32 K|V rebuilt from h (hi and lo halves), over three chunks of 128
    tokens (later chunks attend over earlier ones), then two decode steps
    (INT8: the reconstruction kernel's 256-row variant at 128-wide heads)."""
    torch_gpu()
    w, gm = gpu_model(S2B, random_gains=True)
    pr = _prompt(300, 34)
    c = gm.cache(mode, 1, 310, 2)
    orc = oracle.LoopedOracle(S2B, w, mode, 1, 310, 2)
    nxt, lg = c.prefill(0, pr, 2, chunk=128)
    ro = orc.prefill(0, pr, 2)
    e = rel_err(lg.cpu().numpy(), ro["logits"][-1])
    record("2b_chunked_prefill", mode=mode, rel=e)
    assert e <= REL_TOL, (mode, e)
    tok = int(nxt.cpu()[0])
    assert token_ok(tok, ro["logits"][-1])
    for step in range(2):
        t, lgd, st = decode(c, [0], [2], [tok])
        r = orc.decode_step([0], [2], [tok])
        e = rel_err(lgd[0], r["logits"][0])
        record("2b_chunked_decode", mode=mode, step=step, rel=e)
        assert st[0] == 0 and e <= REL_TOL, (mode, step, e)
        assert token_ok(int(t[0]), r["logits"][0])
        tok = int(t[0])
