"""Absorbed evaluation order of the decode attention (tl_cache_set_attention
ABSORBED; the novel-contributions page relates store-h to MLA): scores
(W_k,h^T q_h) . h' and outputs W_v,h sum p h', with no K or V formed. The
oracle is the same plain definition (the order changes rounding only), so the
same 2e-3 bar and near-tie rule apply.

Covered: the 4096-position 4-lane INT4-h workload shape (all lanes against
the oracle), 300 positions in INT4, INT8, fp16-h and delta-KV with per-lane
loop counts, a lane's first tokens, switching order between steps, the 2B
shape (the 48-lane L-aware workload, and 600 positions in every h mode), and
the models and modes the order does not cover being refused."""
import numpy as np
import pytest

import oracle
import synth
from tests._gpu_util import REL_TOL, decode, decode_synced, gpu_model, record, rel_err, token_ok, torch_gpu

pytestmark = pytest.mark.gpu

S407 = synth.SHAPES["407m"]
def test_absorbed_ctx4096_b4_decode():
    torch_gpu()
    wl = synth.workload("407m-int4h-ctx4096-b4")
    sh, L, ctx, lanes = wl.shape, 8, wl.context, 4
    n_layers = sh.n_pre + L
    w, gm = gpu_model(sh)
    c = gm.cache("int4", lanes, ctx + 4, L)
    for k in range(lanes):
        for layer in range(n_layers):
            c.tl_cache_fill_synthetic(k, layer, 0, ctx, wl.seed_prior)
        c.tl_cache_set_length(k, ctx, n_layers)
    c.tl_cache_set_attention("absorbed")
    orc = oracle.LoopedOracle(sh, w, "int4", lanes, ctx + 4, L)
    for k in range(lanes):
        orc.prime_synthetic(k, range(n_layers), ctx,
                            lambda layer, k=k: synth.prior_h(wl.seed_prior, layer, k, np.arange(ctx), sh.d_model))
    toks = [int(x) for x in synth.make_prompts(sh.vocab, lanes, 1, wl.seed_prompt)[:, 0]]
    for step in range(2):
        t, lg, st = decode(c, list(range(lanes)), [L] * lanes, toks)
        r = orc.decode_step(list(range(lanes)), [L] * lanes, toks)
        for k in range(lanes):
            assert st[k] == 0
            e = rel_err(lg[k], r["logits"][k])
            record("absorbed_ctx4096", step=step, lane=k, rel=e)
            assert e <= REL_TOL, (step, k, e)
            assert token_ok(int(t[k]), r["logits"][k])
            assert rel_err(c.tl_residual_norms(k)[:L], orc.norms[k][:L]) <= REL_TOL
        toks = [int(x) for x in t]


@pytest.mark.parametrize("mode", ["int4", "int8", "f16", "delta8"])
def test_absorbed_prefill_then_decode(mode):
    torch_gpu()
    w, gm = gpu_model(S407)
    prompts = synth.make_prompts(S407.vocab, 2, 300, 1)
    loops = [3, 2]
    orc = oracle.LoopedOracle(S407, w, mode, 2, 320, 3)
    c = gm.cache(mode, 2, 320, 3)
    toks = []
    for lane in range(2):
        ro = orc.prefill(lane, prompts[lane], loops[lane])
        nxt, _ = c.prefill(lane, prompts[lane], loops[lane])
        t = int(nxt.cpu().numpy()[0])
        assert token_ok(t, ro["logits"][-1])
        toks.append(t)
    c.tl_cache_set_attention("absorbed")
    for step in range(3):
        r = orc.decode_step([0, 1], loops, toks)
        t, lg, st = decode(c, [0, 1], loops, toks)
        for k in range(2):
            assert st[k] == 0
            e = rel_err(lg[k], r["logits"][k])
            record("absorbed_decode", mode=mode, step=step, lane=k, rel=e)
            assert e <= REL_TOL, (mode, step, k, e)
            assert token_ok(int(t[k]), r["logits"][k])
        toks = [int(x) for x in t]


@pytest.mark.parametrize("mode", ["f16", "int4"])
def test_absorbed_first_tokens(mode):
    torch_gpu()
    w, gm = gpu_model(S407)
    c = gm.cache(mode, 2, 24, 3)
    c.tl_cache_set_attention("absorbed")
    orc = oracle.LoopedOracle(S407, w, mode, 2, 24, 3)
    toks = [17, 31999]
    for step in range(12):
        # INT4: codes decided on the other side of a rounding boundary are
        # proven rounding-boundary decisions on the oracle's h and adopted by
        # the oracle
        if mode == "f16":
            t, lg, st = decode(c, [0, 1], [3, 1], toks)
            r = orc.decode_step([0, 1], [3, 1], toks)
        else:
            t, lg, st, r, _ = decode_synced(c, orc, [0, 1], [3, 1], toks)
        assert np.all(st == 0)
        for k in range(2):
            ref = r["logits"][k]
            e = rel_err(lg[k], ref)
            record("absorbed_first_tokens", mode=mode, lane=k, step=step, rel=e)
            assert e <= REL_TOL, (mode, step, k, e)
            assert token_ok(int(t[k]), ref)
        toks = [int(x) for x in t]


def test_switch_order_between_steps():
    torch_gpu()
    w, gm = gpu_model(S407)
    pr = synth.make_prompts(S407.vocab, 1, 200, 2)[0]
    c = gm.cache("int4", 1, 210, 4)
    orc = oracle.LoopedOracle(S407, w, "int4", 1, 210, 4)
    orc.prefill(0, pr, 4)
    nxt, _ = c.prefill(0, pr, 4)
    tok = int(nxt.cpu()[0])
    for step, order in enumerate(["absorbed", "explicit", "absorbed", "explicit"]):
        c.tl_cache_set_attention(order)
        t, lg, st = decode(c, [0], [4], [tok])
        r = orc.decode_step([0], [4], [tok])
        e = rel_err(lg[0], r["logits"][0])
        assert st[0] == 0 and e <= REL_TOL, (order, e)
        assert token_ok(int(t[0]), r["logits"][0])
        tok = int(t[0])


def test_absorbed_2b_laware_b48_decode():
    """The 2B L-aware workload shape (48 lanes, loops [4, 16, 32] on one
    34-layer cache, 2048 prior positions) in the absorbed order; one lane of
    each loop tier recomputed by the oracle."""
    torch_gpu()
    wl = synth.workload("2b-int4h-laware-b48")
    sh, ctx = wl.shape, wl.context
    loops = wl.lane_loops()
    w, gm = gpu_model(sh)
    c = gm.cache("int4", wl.lanes, ctx + 2, wl.l_max)
    layers_of = lambda k: sh.n_pre + loops[k]
    for k in range(wl.lanes):
        for layer in range(layers_of(k)):
            c.tl_cache_fill_synthetic(k, layer, 0, ctx, wl.seed_prior)
        c.tl_cache_set_length(k, ctx, layers_of(k))
    c.tl_cache_set_attention("absorbed")
    sampled = [0, 1, 2]
    orc = oracle.LoopedOracle(sh, w, "int4", wl.lanes, ctx + 2, wl.l_max)
    for k in sampled:
        orc.prime_synthetic(k, range(layers_of(k)), ctx,
                            lambda layer, k=k: synth.prior_h(wl.seed_prior, layer, k, np.arange(ctx), sh.d_model))
    toks = [int(x) for x in synth.make_prompts(sh.vocab, wl.lanes, 1, wl.seed_prompt)[:, 0]]
    t, lg, st = decode(c, list(range(wl.lanes)), loops, toks)
    assert np.all(st == 0)
    r = orc.decode_step(sampled, [loops[k] for k in sampled], [toks[k] for k in sampled])
    for i, k in enumerate(sampled):
        e = rel_err(lg[k], r["logits"][i])
        record("absorbed_2b_laware", lane=k, loops=loops[k], rel=e)
        assert e <= REL_TOL, (k, e)
        assert token_ok(int(t[k]), r["logits"][i])


@pytest.mark.parametrize("mode", ["int4", "int8", "f16", "delta8"])
def test_absorbed_2b_prefill_then_decode(mode):
    torch_gpu()
    s2 = synth.SHAPES["2b"]
    w, gm = gpu_model(s2, random_gains=True)
    # 600 positions: INT4 codes that upstream rounding flips at a context of
    # ~150 move the logits by ~2e-3 in either order; here they are diluted
    pr = [int(x) for x in synth.make_prompts(s2.vocab, 1, 600, 7)[0]]
    orc = oracle.LoopedOracle(s2, w, mode, 1, 610, 3)
    c = gm.cache(mode, 1, 610, 3)
    ro = orc.prefill(0, pr, 3)
    nxt, _ = c.prefill(0, pr, 3)
    tok = int(nxt.cpu()[0])
    assert token_ok(tok, ro["logits"][-1])
    c.tl_cache_set_attention("absorbed")
    for step in range(2):
        r = orc.decode_step([0], [3], [tok])
        t, lg, st = decode(c, [0], [3], [tok])
        e = rel_err(lg[0], r["logits"][0])
        record("absorbed_2b_decode", mode=mode, step=step, rel=e)
        assert st[0] == 0 and e <= REL_TOL, (mode, step, e)
        assert token_ok(int(t[0]), r["logits"][0])
        tok = int(t[0])


def test_absorbed_refused_where_not_covered():
    from kv_compression_amd import tl
    torch_gpu()
    _, gm = gpu_model(S407)
    c = gm.cache("kv", 1, 16, 2)
    with pytest.raises(tl.TLError) as e:
        c.tl_cache_set_attention("absorbed")
    assert e.value.status == tl.TL_E_UNSUPPORTED
    _, gt = gpu_model(synth.SHAPES["tiny"])              # an fp32 model
    ct = gt.cache("f32", 1, 16, 2)
    with pytest.raises(tl.TLError) as e:
        ct.tl_cache_set_attention("absorbed")
    assert e.value.status == tl.TL_E_UNSUPPORTED
    c.tl_cache_set_attention("explicit")
    with pytest.raises(tl.TLError) as e:           # an order that does not exist
        tl._check(tl.load().tl_cache_set_attention(c.handle, 7))
    assert e.value.status == tl.TL_E_ARG
