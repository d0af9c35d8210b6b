"""The INT4 / INT8 decode attention merges its own 256-position tiles: the
last workgroup of each (row, head group) to finish combines the row's tile
partials, counted by a per-(row, head group) tile counter that it zeroes again
for the next launch. These cases change what a counter slot stands for from
one launch to the next and check every step against the oracle:

* rows that move to other lanes, with 1, 2 and 3 tiles in one launch and a
  different row count each step;
* a lane that aborts in the middle of a step (its later launches skip the
  row, so its counters must stay untouched) while its batch mate goes on."""
import math

import numpy as np
import pytest

import oracle
import synth
from tests._gpu_util import REL_TOL, decode, gpu_model, record, rel_err, token_ok

pytestmark = pytest.mark.gpu

S407 = synth.SHAPES["407m"]


def _both(gm, w, mode, prompts, loops, max_seq, l_max):
    orc = oracle.LoopedOracle(S407, w, mode, len(prompts), max_seq, l_max)
    c = gm.cache(mode, len(prompts), max_seq, l_max)
    toks = []
    for lane, pr in enumerate(prompts):
        ro = orc.prefill(lane, pr, loops[lane])
        nxt, _ = c.prefill(lane, pr, loops[lane])
        t = int(nxt.cpu().numpy()[0])
        assert token_ok(t, ro["logits"][-1])
        toks.append(t)
    return orc, c, toks


@pytest.mark.parametrize("mode", ["int4", "int8"])
def test_rows_change_lanes_and_tile_counts(mode):
    w, gm = gpu_model(S407)
    # 1, 2 and 3 position tiles; INT4 codes flipped by upstream rounding move
    # the logits of a context of a few dozen positions by more than 2e-3 (in
    # either evaluation order), so the shortest lane still has 250
    lens = [250, 300, 700]
    prompts = [synth.make_prompts(S407.vocab, 1, n, 20 + i)[0] for i, n in enumerate(lens)]
    loops = [2, 3, 1]
    orc, c, toks = _both(gm, w, mode, prompts, loops, 710, 3)
    for step, lanes in enumerate([[0, 1, 2], [2, 0], [1], [1, 2, 0]]):
        lp = [loops[k] for k in lanes]
        tin = [toks[k] for k in lanes]
        r = orc.decode_step(lanes, lp, tin)
        t, lg, st = decode(c, lanes, lp, tin)
        for i, k in enumerate(lanes):
            assert st[i] == 0
            e = rel_err(lg[i], r["logits"][i])
            record("fused_merge_rows", mode=mode, step=step, lane=k, rel=e)
            assert e <= REL_TOL, (mode, step, k, e)
            assert token_ok(int(t[i]), r["logits"][i]), (mode, step, k)
            toks[k] = int(t[i])


def test_abort_mid_step_leaves_counters_clean():
    w, gm = gpu_model(S407)
    L = 4
    # prompts whose lanes' largest residual norms of the first decode step are
    # at least 1 % apart (probed on the GPU), so a threshold between them
    # aborts one lane and not the other
    for seed in range(30, 40):
        prompts = [synth.make_prompts(S407.vocab, 1, n, seed + 100 * i)[0] for i, n in enumerate([300, 520])]
        probe = gm.cache("int4", 2, 540, L)
        toks = [int(probe.prefill(lane, pr, L)[0].cpu().numpy()[0]) for lane, pr in enumerate(prompts)]
        decode(probe, [0, 1], [L, L], toks)
        n0, n1 = probe.tl_residual_norms(0)[:L], probe.tl_residual_norms(1)[:L]
        del probe
        if max(n0.max(), n1.max()) > 1.01 * min(n0.max(), n1.max()):
            break
    else:
        raise AssertionError("no prompt pair separates the lanes' norms")
    hi, lo = (1, 0) if n1.max() > n0.max() else (0, 1)
    nh, nl = (n1, n0) if hi == 1 else (n0, n1)
    # the lane with the larger norm aborts at the first iteration above thr
    thr = float(np.float32(0.5 * (nl.max() + nh.max())))
    assert not np.any(nl > thr)
    orc, c, toks = _both(gm, w, "int4", prompts, [L, L], 540, L)
    r = orc.decode_step([0, 1], [L, L], toks, thr)
    t, lg, st = decode(c, [0, 1], [L, L], toks, thr)
    assert st[hi] == oracle.LANE_ABORTED == r["status"][hi] and t[hi] == -1
    assert st[lo] == 0 == r["status"][lo]
    assert rel_err(lg[lo], r["logits"][lo]) <= REL_TOL
    assert token_ok(int(t[lo]), r["logits"][lo])
    tok = int(t[lo])
    for step in range(3):
        r = orc.decode_step([0, 1], [L, L], [tok, tok], math.inf)
        t, lg, st = decode(c, [0, 1], [L, L], [tok, tok])
        assert st[hi] == oracle.LANE_ABORTED and t[hi] == -1
        e = rel_err(lg[lo], r["logits"][lo])
        record("fused_merge_abort", step=step, rel=e)
        assert st[lo] == 0 and e <= REL_TOL, (step, e)
        assert token_ok(int(t[lo]), r["logits"][lo])
        tok = int(t[lo])
