"""The fp16 models' decode attention (INT4, INT8 and fp16 h) merges its own
256-position tiles: the last workgroup of each (row, head group) to finish
combines the row's tile partials, counted by a per-(row, head group) tile
counter that it zeroes again for the next launch. These cases change what a counter slot stands for from
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
from tests._gpu_util import REL_TOL, decode, decode_synced, gpu_model, prefill_synced, record, rel_err, token_ok

pytestmark = pytest.mark.gpu

S407 = synth.SHAPES["407m"]


def _both(gm, w, mode, prompts, loops, max_seq, l_max):
    orc = oracle.LoopedOracle(S407, w, mode, len(prompts), max_seq, l_max)
    c = gm.cache(mode, len(prompts), max_seq, l_max)
    toks = []
    for lane, pr in enumerate(prompts):
        t, last, ro, _ = prefill_synced(c, orc, lane, pr, loops[lane])
        assert rel_err(last, ro["logits"][-1]) <= REL_TOL
        assert token_ok(t, ro["logits"][-1])
        toks.append(t)
    return orc, c, toks


@pytest.mark.parametrize("mode", ["int4", "int8", "f16"])
def test_rows_change_lanes_and_tile_counts(mode):
    w, gm = gpu_model(S407)
    # 1, 2 and 3 position tiles; at a context of a few dozen positions a code
    # decided on the other side of a rounding boundary is not diluted, so
    # every such group is proven a rounding-boundary decision on the oracle's
    # h and adopted by the oracle
    # (prefill_synced, decode_synced)
    lens = [40, 300, 700]
    prompts = [synth.make_prompts(S407.vocab, 1, n, 20 + i)[0] for i, n in enumerate(lens)]
    loops = [2, 3, 1]
    orc, c, toks = _both(gm, w, mode, prompts, loops, 710, 3)
    for step, lanes in enumerate([[0, 1, 2], [2, 0], [1], [1, 2, 0]]):
        lp = [loops[k] for k in lanes]
        tin = [toks[k] for k in lanes]
        t, lg, st, r, _ = decode_synced(c, orc, lanes, lp, tin)
        for i, k in enumerate(lanes):
            assert st[i] == 0
            e = rel_err(lg[i], r["logits"][i])
            record("fused_merge_rows", mode=mode, step=step, lane=k, rel=e)
            assert e <= REL_TOL, (mode, step, k, e)
            assert token_ok(int(t[i]), r["logits"][i]), (mode, step, k)
            toks[k] = int(t[i])


@pytest.mark.parametrize("mode", ["int4", "int8"])
def test_tail_tiles_across_tile_boundaries(mode):
    """INT4 and INT8 at 64-wide heads: a last position tile of at most 32 positions is
    computed with its row blocks dealt over the four waves (the tail split),
    one of 33 or more as an ordinary partial tile. One launch mixes rows on
    both sides of that boundary (prompts of 256, 287, 288 and 543 tokens:
    contexts 257, 288, 289 and 544 at the first step, one more each step),
    rows leave and rejoin, and every step is checked against the oracle."""
    w, gm = gpu_model(S407)
    lens = [256, 287, 288, 543]
    prompts = [synth.make_prompts(S407.vocab, 1, n, 40 + i)[0] for i, n in enumerate(lens)]
    loops = [2, 1, 3, 2]
    orc, c, toks = _both(gm, w, mode, prompts, loops, 560, 3)
    for step, lanes in enumerate([[0, 1, 2, 3], [3, 1], [2, 0, 3], [1, 2, 3, 0]]):
        lp = [loops[k] for k in lanes]
        tin = [toks[k] for k in lanes]
        t, lg, st, r, _ = decode_synced(c, orc, lanes, lp, tin)
        for i, k in enumerate(lanes):
            assert st[i] == 0
            e = rel_err(lg[i], r["logits"][i])
            record("tail_tiles", mode=mode, step=step, lane=k, T=int(orc.length[k]), rel=e)
            assert e <= REL_TOL, (step, k, e)
            assert token_ok(int(t[i]), r["logits"][i]), (step, k)
            toks[k] = int(t[i])


@pytest.mark.parametrize("mode", ["int4", "int8", "f16"])
def test_abort_mid_step_leaves_counters_clean(mode):
    w, gm = gpu_model(S407)
    L = 4
    # prompts whose lanes' largest residual norms of the first decode step are
    # at least 1 % apart (probed on the GPU), so a threshold between them
    # aborts one lane and not the other
    for seed in range(30, 40):
        prompts = [synth.make_prompts(S407.vocab, 1, n, seed + 100 * i)[0] for i, n in enumerate([300, 520])]
        probe = gm.cache(mode, 2, 540, L)
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
    orc, c, toks = _both(gm, w, mode, prompts, [L, L], 540, L)
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
        record("fused_merge_abort", mode=mode, step=step, rel=e)
        assert st[lo] == 0 and e <= REL_TOL, (step, e)
        assert token_ok(int(t[lo]), r["logits"][lo])
        tok = int(t[lo])


@pytest.mark.parametrize("mode", ["f16", "delta8"])
def test_fp16_h_tiles_at_mixed_lengths(mode):
    """fp16 h (and the delta mode's fp16 view) with enough rows and position
    tiles for the regular configuration (8 waves, the W and h tiles copied
    into the LDS ring): 4 lanes at contexts 2049, 2100, 2280 and 2304 (a last
    tile of 1, 52 and 232 positions, and none), every lane against the oracle
    over two steps."""
    w, gm = gpu_model(S407)
    L, seed = 3, 77
    n_layers = S407.n_pre + L
    ctxs = [2049, 2100, 2280, 2304]
    c = gm.cache(mode, 4, 2312, L)
    orc = oracle.LoopedOracle(S407, w, mode, 4, 2312, L)
    for k, n in enumerate(ctxs):
        for layer in range(n_layers):
            c.tl_cache_fill_synthetic(k, layer, 0, n, seed)
        c.tl_cache_set_length(k, n, n_layers)
        orc.prime_synthetic(k, range(n_layers), n,
                            lambda layer, k=k, n=n: synth.prior_h(seed, layer, k, np.arange(n), S407.d_model))
    toks = [int(x) for x in synth.make_prompts(S407.vocab, 4, 1, 9)[:, 0]]
    for step in range(2):
        t, lg, st = decode(c, [0, 1, 2, 3], [L] * 4, toks)
        r = orc.decode_step([0, 1, 2, 3], [L] * 4, toks)
        for k in range(4):
            assert st[k] == 0
            e = rel_err(lg[k], r["logits"][k])
            record("fp16_h_mixed_lengths", mode=mode, step=step, lane=k, rel=e)
            assert e <= REL_TOL, (mode, step, k, e)
            assert token_ok(int(t[k]), r["logits"][k]), (mode, step, k)
            assert rel_err(c.tl_residual_norms(k)[:L], orc.norms[k][:L]) <= REL_TOL
        toks = [int(x) for x in t]


def test_fp16_h_many_short_lanes():
    """fp16 h with many rows at short contexts, so the regular configuration
    runs (rows x tiles x head groups fill the CUs) with every tile partial and
    most waves holding no position: 32 lanes at contexts 1 .. 32 (decoding
    at 2 .. 33, one or two tiles of 256), every lane against the oracle."""
    w, gm = gpu_model(S407)
    L, seed, lanes = 2, 91, 32
    n_layers = S407.n_pre + L
    c = gm.cache("f16", lanes, 40, L)
    orc = oracle.LoopedOracle(S407, w, "f16", lanes, 40, L)
    for k in range(lanes):
        n = k + 1
        for layer in range(n_layers):
            c.tl_cache_fill_synthetic(k, layer, 0, n, seed)
        c.tl_cache_set_length(k, n, n_layers)
        orc.prime_synthetic(k, range(n_layers), n,
                            lambda layer, k=k, n=n: synth.prior_h(seed, layer, k, np.arange(n), S407.d_model))
    toks = [int(x) for x in synth.make_prompts(S407.vocab, lanes, 1, 5)[:, 0]]
    for step in range(2):
        t, lg, st = decode(c, list(range(lanes)), [L] * lanes, toks)
        r = orc.decode_step(list(range(lanes)), [L] * lanes, toks)
        for k in range(lanes):
            assert st[k] == 0
            e = rel_err(lg[k], r["logits"][k])
            record("fp16_h_short_lanes", step=step, lane=k, rel=e)
            assert e <= REL_TOL, (step, k, e)
            assert token_ok(int(t[k]), r["logits"][k]), (step, k)
        toks = [int(x) for x in t]
