"""GPU parity of the safety check on a degenerate state and of argmax ties,
through the C ABI, against the oracle.

* A NaN residual fires the check (novel-contributions page, "Per-Iteration
  Safety Check": the check catches degenerate hidden states; the comparison
  is not (norm <= threshold)). An infinite embedding element makes the first
  norm's output NaN, so the residual is NaN by loop iteration 0.
* Argmax ties go to the lowest index: an LM head whose top logits tie exactly
  (each logit a single exact product), with tied indices close together and
  far apart in the vocabulary (the same and different threads, waves and
  load batches of the step's end kernel).
"""
import numpy as np
import pytest

import synth
import oracle
from tests._gpu_util import GpuModel, decode, rel_err, token_ok, torch_gpu, REL_TOL
from tests.test_oracle_pins import tie_head

pytestmark = pytest.mark.gpu

S407 = synth.SHAPES["407m"]
BAD = 4242          # token whose embedding holds an infinite element


def _nan_weights():
    w = synth.make_weights(S407, 0)
    w["embed"] = w["embed"].copy()
    w["embed"][BAD, 5] = np.float16(np.inf)
    return w


@pytest.mark.parametrize("mode,order", [("int4", "explicit"), ("f16", "explicit"), ("kv", "explicit"),
                                        ("int4", "absorbed")])
def test_nan_residual_aborts_lane(mode, order):
    torch = torch_gpu()
    w = _nan_weights()
    gm = GpuModel(S407, w)
    L = 3
    prompts = synth.make_prompts(S407.vocab, 2, 260, 31)
    c = gm.cache(mode, 2, 300, L)
    if order != "explicit":
        # the stopped lane's rows leave the absorbed kernels early, its batch mate is unaffected
        c.tl_cache_set_attention(order)
    o = oracle.LoopedOracle(S407, w, mode, 2, 300, L)
    first = []
    for k in range(2):
        nxt, _ = c.prefill(k, prompts[k], L)
        first.append(int(nxt.cpu()[0]))
        o.prefill(k, prompts[k], L)
    thr = 1e30
    toks, lg, st = decode(c, [0, 1], [L, L], [BAD, first[1]], thr)
    ref = o.decode_step([0, 1], [L, L], [BAD, first[1]], thr)
    assert ref["status"].tolist() == [oracle.LANE_ABORTED, oracle.LANE_OK]
    assert st.tolist() == [oracle.LANE_ABORTED, oracle.LANE_OK]
    assert toks[0] == -1 and np.all(np.isnan(lg[0]))
    norms0 = c.tl_residual_norms(0)[:L]
    assert np.all(np.isnan(norms0)), norms0
    assert rel_err(lg[1], ref["logits"][1]) <= REL_TOL
    assert token_ok(int(toks[1]), ref["logits"][1])
    assert np.allclose(c.tl_residual_norms(1)[:L], o.norms[1][:L], rtol=REL_TOL)
    # the aborted lane is skipped by the next step and keeps its length; its
    # batch mate goes on
    t1 = int(ref["tokens"][1])
    toks2, lg2, st2 = decode(c, [0, 1], [L, L], [first[0], t1], thr)
    ref2 = o.decode_step([0, 1], [L, L], [first[0], t1], thr)
    assert st2.tolist() == [oracle.LANE_ABORTED, oracle.LANE_OK]
    assert toks2[0] == -1
    assert rel_err(lg2[1], ref2["logits"][1]) <= REL_TOL
    assert token_ok(int(toks2[1]), ref2["logits"][1])
    # after a reset the lane starts over and decodes normally
    c.tl_cache_reset_lane(0)
    nxt, _ = c.prefill(0, prompts[0][:40], L)
    toks3, lg3, st3 = decode(c, [0], [L], [int(nxt.cpu()[0])], thr)
    assert st3.tolist() == [oracle.LANE_OK] and toks3[0] >= 0 and np.all(np.isfinite(lg3[0]))


@pytest.mark.parametrize("ties,lowest", [((20000, 1000, 999, 31999), 999),
                                         ((1998, 1500, 1999, 25000), 1500)])
def test_argmax_tie_lowest_index(ties, lowest):
    torch = torch_gpu()
    w = synth.make_weights(S407, 0)
    L = 2
    prompt = synth.make_prompts(S407.vocab, 1, 260, 33)[0]
    tok = 17
    # the final-norm output of the step (it does not depend on the LM head)
    o = oracle.LoopedOracle(S407, w, "int4", 1, 300, L)
    o.prefill(0, prompt, L)
    o.forward(0, [tok], L, check_safety=False, keep_trace=True)
    z = dict(o.trace[0])["final_ln"][0]
    k = int(np.argmax(np.abs(z)))
    w["lm_head"] = tie_head(S407.vocab, S407.d_model, k, np.sign(z[k]), ties).astype(np.float16)
    o = oracle.LoopedOracle(S407, w, "int4", 1, 300, L)
    o.prefill(0, prompt, L)
    ref = o.decode_step([0], [L], [tok])
    assert ref["tokens"][0] == lowest
    gm = GpuModel(S407, w)
    c = gm.cache("int4", 1, 300, L)
    c.prefill(0, prompt, L)
    toks, lg, st = decode(c, [0], [L], [tok])
    top = np.max(lg[0])
    assert [float(lg[0][t]) for t in ties] == [float(top)] * len(ties)
    assert int(np.sum(lg[0] == top)) == len(ties)
    assert int(toks[0]) == lowest
    assert rel_err(lg[0], ref["logits"][0]) <= REL_TOL
