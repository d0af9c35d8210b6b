"""Chunked prefill whose causal attention is split over key ranges (chunks
late in a long prompt): every position's residual after the last layer, the
last logits and the decode steps that follow match the oracle.

Chunk plans and the key splits they get: 300 tokens in one chunk (2 splits),
200 + 100 (the second chunk 2), and 512 + 512 + 76 of an 1100-token prompt
(the last chunk 7 splits of 160 keys, the second 8 of 128)."""
import pytest

import oracle
import synth
from tests._gpu_util import REL_TOL, decode, gpu_model, record, rel_err, token_ok, torch_gpu

pytestmark = pytest.mark.gpu

S407 = synth.SHAPES["407m"]


@pytest.mark.parametrize("mode,n,chunk", [("f16", 300, 300), ("kv", 300, 200), ("f16", 1100, 512)])
def test_prefill_key_splits_match_oracle(mode, n, chunk):
    torch_gpu()
    w, gm = gpu_model(S407, random_gains=True)
    pr = [int(t) for t in synth.make_prompts(S407.vocab, 1, n, 21)[0]]
    c = gm.cache(mode, 1, n + 8, 8)
    nxt, lg, x = c.prefill_x(0, pr, 8, chunk=chunk)
    orc = oracle.LoopedOracle(S407, w, mode, 1, n + 8, 8)
    r = orc.prefill(0, pr, 8)
    ex = rel_err(x.cpu().numpy(), r["x"])
    el = rel_err(lg.cpu().numpy(), r["logits"][-1])
    record("prefill_split", mode=mode, n=n, chunk=chunk, rel_x=ex, rel_logits=el)
    assert ex <= REL_TOL, ex
    assert el <= REL_TOL, el
    tok = int(nxt.cpu()[0])
    assert token_ok(tok, r["logits"][-1])
    for _ in range(2):
        t, lgd, st = decode(c, [0], [8], [tok])
        rd = orc.decode_step([0], [8], [tok])
        e = rel_err(lgd[0], rd["logits"][0])
        assert st[0] == 0 and e <= REL_TOL, e
        assert token_ok(int(t[0]), rd["logits"][0])
        tok = int(t[0])
