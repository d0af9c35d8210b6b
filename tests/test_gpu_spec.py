"""Self-speculative decoding on the GPU (features page, "Self-speculative
decoding"; the greedy-equality claim of its "Tree speculative decoding"
section, chain mode), through tl_spec_step.

* Every emitted token is the oracle's greedy token at the verify depth given
  the same prefix (teacher-forced replay on the oracle, near-tie rule), and
  after the rounds the lane decodes like the oracle's plainly decoded lane
  (the rewrites past rejected drafts left the cache a plain run would leave).
* A model whose drafts agree part of the time exercises rounds that accept
  some drafts and rewind past the rest.
* With equal draft and verify depths every draft is accepted, and the tokens
  equal plain GPU decoding of the same prompt, also at the full 4096-position
  INT4-h context.
* An aborted lane emits nothing; argument errors are refused before anything
  is enqueued and leave the lane usable."""
import numpy as np
import pytest

import oracle
import synth
from tests._gpu_util import REL_TOL, decode, gpu_model, record, rel_err, token_ok, torch_gpu

pytestmark = pytest.mark.gpu

S407 = synth.SHAPES["407m"]
N_PROMPT = 24


def _prompt(seed=11, n=N_PROMPT):
    return [int(t) for t in synth.make_prompts(S407.vocab, 1, n, seed)[0]]


def _replay(orc, pr, t0, got, verify):
    """Decode the oracle plainly along the GPU's tokens; every GPU token must be
    the oracle's greedy choice (or a near-tie of it)."""
    if pr:
        r = orc.prefill(0, pr, verify)
        assert token_ok(t0, r["logits"][-1])
    prev = t0
    for i, g in enumerate(got):
        r = orc.decode_step([0], [verify], [prev])
        assert token_ok(g, r["logits"][0]), (i, g, int(np.argmax(r["logits"][0])))
        prev = g


@pytest.mark.parametrize("mode,draft,ahead", [("f16", 2, 4), ("kv", 2, 4), ("f16", 1, 7)])
def test_spec_matches_oracle_greedy(mode, draft, ahead):
    torch = torch_gpu()
    w, gm = gpu_model(S407, random_gains=True)
    pr = _prompt()
    c = gm.cache(mode, 1, 96, 8)
    nxt, _ = c.prefill(0, pr, 8, chunk=16)
    t0 = int(nxt.cpu()[0])
    got, rounds = c.generate_speculative(0, t0, 16, draft, 8, ahead)
    record("spec_rounds", mode=mode, draft=draft, ahead=ahead, rounds=rounds)
    assert min(rounds) >= 1 and sum(rounds) == len(got)
    assert min(rounds) < ahead + 1            # rejections happened and were rewound
    orc = oracle.LoopedOracle(S407, w, mode, 1, 96, 8)
    _replay(orc, pr, t0, got, 8)
    # the lane continues like the oracle's plainly decoded one
    t, lg, st = decode(c, [0], [8], [got[-1]])
    r = orc.decode_step([0], [8], [got[-1]])
    assert st[0] == 0
    e = rel_err(lg[0], r["logits"][0])
    record("spec_then_decode", mode=mode, draft=draft, rel=e)
    assert e <= REL_TOL, e
    torch.cuda.synchronize()


def test_spec_partial_acceptance():
    """A model whose loop block barely moves the residual (its output
    projections scaled by 0.03) makes shallow drafts agree with the verifier
    part of the time: rounds that accept some but not all drafts rewind to
    the first disagreement, and the tokens stay the oracle's greedy ones."""
    from tests._gpu_util import GpuModel
    torch_gpu()
    w, _ = gpu_model(S407, random_gains=True)
    wq = dict(w)
    wq["layers"] = [dict(lw) for lw in w["layers"]]
    lb = wq["layers"][S407.n_pre]
    for k in ("w_o", "w_down"):
        lb[k] = (lb[k].astype(np.float32) * 0.03).astype(lb[k].dtype)
    gm = GpuModel(S407, wq)
    pr = _prompt()
    c = gm.cache("f16", 1, 96, 8)
    nxt, _ = c.prefill(0, pr, 8, chunk=16)
    t0 = int(nxt.cpu()[0])
    got, rounds = c.generate_speculative(0, t0, 24, 2, 8, 4)
    record("spec_partial_rounds", rounds=rounds)
    assert any(1 < n < 5 for n in rounds), rounds
    orc = oracle.LoopedOracle(S407, wq, "f16", 1, 96, 8)
    _replay(orc, pr, t0, got, 8)
    t, lg, st = decode(c, [0], [8], [got[-1]])
    r = orc.decode_step([0], [8], [got[-1]])
    e = rel_err(lg[0], r["logits"][0])
    record("spec_partial_then_decode", rel=e)
    assert e <= REL_TOL, e


def test_spec_from_empty_lane():
    torch_gpu()
    w, gm = gpu_model(S407, random_gains=True)
    c = gm.cache("f16", 1, 32, 8)
    t0 = 17
    got, rounds = c.generate_speculative(0, t0, 8, 2, 8, 3)
    orc = oracle.LoopedOracle(S407, w, "f16", 1, 32, 8)
    _replay(orc, [], t0, got, 8)


def test_spec_equal_depths_accepts_everything():
    torch = torch_gpu()
    w, gm = gpu_model(S407, random_gains=True)
    pr = _prompt(12)
    c = gm.cache("f16", 2, 96, 8)
    t0 = None
    for lane in (0, 1):
        nxt, _ = c.prefill(lane, pr, 8, chunk=16)
        t0 = int(nxt.cpu()[0])
    got, rounds = c.generate_speculative(0, t0, 15, 8, 8, 4)
    assert rounds == [5, 5, 5]
    plain, t = [], t0
    for _ in range(len(got)):
        t = int(decode(c, [1], [8], [t])[0][0])
        plain.append(t)
    assert got == plain
    torch.cuda.synchronize()


def test_spec_full_size_int4_equal_depths():
    """The 407M INT4-h workload's context (4096 prior positions in all 10
    layers): with equal depths every draft is accepted and the tokens equal
    plain decoding of the same lane (decoded first, then rewound to 4096)."""
    torch_gpu()
    w, gm = gpu_model(S407)
    ctx, L, ahead = 4096, 8, 4
    c = gm.cache("int4", 1, ctx + 32, L)
    for layer in range(S407.n_pre + L):
        c.tl_cache_fill_synthetic(0, layer, 0, ctx, 1234 + layer)
    c.tl_cache_set_length(0, ctx, S407.n_pre + L)
    t0 = 4242
    plain, t = [], t0
    for _ in range(10):
        t = int(decode(c, [0], [L], [t], want_logits=False)[0][0])
        plain.append(t)
    c.tl_cache_set_length(0, ctx, S407.n_pre + L)
    got, rounds = c.generate_speculative(0, t0, 10, L, L, ahead)
    record("spec_full_size", rounds=rounds, agree=int(np.sum(np.array(got[:10]) == np.array(plain))))
    assert rounds == [ahead + 1] * len(rounds)
    assert got[:10] == plain


def test_spec_aborted_lane_emits_nothing():
    torch = torch_gpu()
    w, gm = gpu_model(S407)
    c = gm.cache("int4", 1, 64, 8)
    nxt, _ = c.prefill(0, _prompt(), 8, chunk=16)
    t0 = int(nxt.cpu()[0])
    _, _, st = decode(c, [0], [8], [t0], threshold=1e-6)
    assert st[0] == 1
    tin = torch.tensor([t0], dtype=torch.int32, device="cuda")
    tout = torch.zeros(4, dtype=torch.int32, device="cuda")
    assert c.tl_spec_step(0, 2, 8, 3, tin, tout) == 0
    assert tout.cpu().tolist() == [-1, -1, -1, -1]


def test_spec_errors():
    from kv_compression_amd import tl
    torch = torch_gpu()
    w, gm = gpu_model(S407)
    c = gm.cache("int4", 2, 36, 8)
    pr = _prompt(13)
    nxt, _ = c.prefill(0, pr, 8, chunk=16)
    tin = nxt.clone()
    tout = torch.empty(16, dtype=torch.int32, device="cuda")

    def refused(status, *args):
        with pytest.raises(tl.TLError) as e:
            c.tl_spec_step(*args)
        assert e.value.status == status, e.value

    refused(tl.TL_E_ARG, 0, 2, 8, 0, tin, tout)        # draft_ahead 0
    refused(tl.TL_E_ARG, 0, 2, 8, 16, tin, tout)       # draft_ahead above 15
    refused(tl.TL_E_ARG, 0, 4, 3, 2, tin, tout)        # draft deeper than verify
    refused(tl.TL_E_ARG, 0, 2, 9, 2, tin, tout)        # verify above l_max
    refused(tl.TL_E_ARG, 2, 2, 8, 2, tin, tout)        # lane out of range
    refused(tl.TL_E_CAPACITY, 0, 2, 8, 15, tin, tout)  # 24 + 16 > 36
    c.prefill(1, pr[:4], 2)
    refused(tl.TL_E_CACHE_GAP, 1, 2, 8, 2, tin, tout)  # lane 1 holds n_pre + 2 layers
    # the refusals left lane 0 as it was: a round still runs from length 24
    got, rounds = c.generate_speculative(0, int(tin.cpu()[0]), 3, 2, 8, 2)
    assert len(got) >= 3
    orc = oracle.LoopedOracle(S407, w, "int4", 1, 36, 8)
    r = orc.prefill(0, pr, 8)
    # (INT codes at 24 positions can flip, so only the first token is checked)
    assert token_ok(int(tin.cpu()[0]), r["logits"][-1])
