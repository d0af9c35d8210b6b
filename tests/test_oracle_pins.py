"""Pins of the CPU oracle against facts fixed outside it: published
known-answer vectors, hand-worked examples, closed forms, brute force on tiny
shapes, the pages' measured codec error, and the invariants the pages state."""
import json
import math
import os

import numpy as np
import pytest

import synth
import oracle
from oracle import looped
from tests import _bruteforce

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------- generators
def test_philox_known_answers():
    rows = [l.split() for l in open(os.path.join(GOLDEN, "philox4x32_10_kat.txt"))
            if l.strip() and not l.startswith("#")]
    assert len(rows) == 3
    for r in rows:
        v = [int(t, 16) for t in r]
        out = synth.philox4x32_10(np.array(v[:4], np.uint32), np.array(v[4:6], np.uint32))
        assert [int(t) for t in out] == v[6:]


def test_prior_h_moments_and_determinism():
    h = synth.prior_h(2, 3, 1, np.arange(512), 256)
    assert h.dtype == np.float32 and h.shape == (512, 256)
    assert abs(float(h.mean())) < 0.01 and abs(float(h.var()) - 1.0) < 0.02
    assert np.abs(h).max() < 4.95
    h2 = synth.prior_h(2, 3, 1, np.arange(100, 140), 256)
    assert np.array_equal(h[100:140], h2)
    assert not np.array_equal(h, synth.prior_h(2, 4, 1, np.arange(512), 256))


# ---------------------------------------------------------------- codec
@pytest.mark.parametrize("kind", ["int4", "int8"])
def test_codec_hand_cases(kind):
    cases = _golden("codec_hand_cases.json")[kind]
    D = 32 if kind == "int4" else 64
    for c in cases:
        h = np.zeros(D, np.float16)
        h[:len(c["h_head"])] = np.array(c["h_head"], np.float64).astype(np.float16)
        assert np.array_equal(h[:len(c["h_head"])].astype(np.float64), np.array(c["h_head"])), c["note"]
        q, s = looped.int4_encode(h) if kind == "int4" else looped.int8_encode(h)
        assert float(s[0]) == c["scale"], c["note"]
        assert list(q[:len(c["q_head"])]) == c["q_head"], c["note"]
        assert np.all(q[len(c["q_head"]):][h[len(c["q_head"]):] == 0] == 0)


def test_codec_int4_is_nearest_code_bruteforce():
    """Every code is the nearest of the 16 representable levels q*s (ties to the
    even code), found by exhaustive search rather than by the formula."""
    rng = np.random.default_rng(5)
    h = (rng.standard_normal((400, 32)) * rng.uniform(0.01, 30, size=(400, 1))).astype(np.float16)
    h[::7, 3] = 0
    q, s = looped.int4_encode(h)
    levels = np.arange(-8, 8, dtype=np.float64)
    for r in range(h.shape[0]):
        sf = float(s[r, 0])
        assert sf == float(np.float16(np.float32(np.abs(h[r].astype(np.float32)).max()) / np.float32(7)))
        for k in range(32):
            x = float(h[r, k]) / sf
            dist = np.abs(levels - x)
            best = levels[dist == dist.min()]
            want = best[0] if len(best) == 1 else best[best % 2 == 0][0]
            assert q[r, k] == int(want), (r, k, x)
        # the absmax element maps to +-7 (scale rounding is within half an fp16 ulp)
        k = int(np.argmax(np.abs(h[r].astype(np.float64))))
        assert abs(int(q[r, k])) == 7 or int(q[r, k]) == -8


def test_codec_decode_roundtrip_exact_levels():
    """Dequantisation is fp16(q*s): decode(encode(h)) of an h that already
    lies on the grid returns h bit for bit."""
    s = np.float16(0.375)
    q = np.tile(np.arange(-7, 8), 3)[:32].astype(np.int8)
    q[0] = 7
    h = (q.astype(np.float32) * np.float32(s)).astype(np.float16)
    q2, s2 = looped.int4_encode(h)
    assert s2[0] == s and np.array_equal(q2, q)
    assert np.array_equal(looped.decode_int(q2, s2), h)


def test_codec_error_matches_pages():
    """Relative L2 error of h' and of K = W_k h' against the pages' measured
    store-h quality table (INT8-h ~0.6 %, INT4-h ~10 %). On N(0,1) h this
    codec gives about 0.78 % and 9.7 %; the bands allow for the pages'
    real activations."""
    pages = _golden("pages_store_h_table.json")["kv_rel_l2_error"]
    rng = np.random.default_rng(11)
    D = 1024
    h = rng.standard_normal((256, D)).astype(np.float16)
    wk = (rng.standard_normal((D, D)) * 0.02).astype(np.float16).astype(np.float64)
    hf = h.astype(np.float64)
    for kind, lo, hi in (("int8", 0.004, 0.012), ("int4", 0.08, 0.12)):
        q, s = looped.int4_encode(h) if kind == "int4" else looped.int8_encode(h)
        hp = looped.decode_int(q, s).astype(np.float64)
        e_h = np.linalg.norm(hp - hf) / np.linalg.norm(hf)
        e_k = np.linalg.norm((hp - hf) @ wk.T) / np.linalg.norm(hf @ wk.T)
        assert lo < e_h < hi and lo < e_k < hi, (kind, e_h, e_k)
        assert 0.5 * pages[kind] < e_k < 2.0 * pages[kind]


# ---------------------------------------------------------------- elementwise
def test_rmsnorm_closed_form():
    x = np.array([[3.0, 4.0]])
    g = np.array([1.0, 2.0])
    r = looped.rmsnorm(x, g, 1e-5)
    inv = 1.0 / math.sqrt(12.5 + 1e-5)          # mean(9, 16) = 12.5
    assert np.allclose(r, [[3.0 * inv, 8.0 * inv]], rtol=0, atol=1e-15)


def test_gelu_values():
    # Phi(1) = 0.8413447460685429 (standard normal CDF table value)
    assert abs(looped.gelu_erf(np.array(1.0)) - 0.8413447460685429) < 1e-15
    assert abs(looped.gelu_erf(np.array(-1.0)) + 0.15865525393145707) < 1e-15
    x = np.linspace(-6, 6, 101)
    assert np.allclose(looped.gelu_erf(x) - looped.gelu_erf(-x), x, atol=1e-14)
    assert looped.gelu_erf(np.array(0.0)) == 0.0


# ---------------------------------------------------------------- attention
def test_attention_hand_case():
    c = _golden("attention_hand_case.json")
    K, V = np.array(c["K"]), np.array(c["V"])
    o = looped.attend(np.array(c["q"]), K, V, c["n_heads"], c["pos0"])
    assert np.allclose(o, c["o"], atol=1e-14)
    o0 = looped.attend(np.array(c["q_at_pos0"]), K[:1], V[:1], c["n_heads"], 0)
    assert np.allclose(o0, c["o_at_pos0"], atol=1e-14)


def test_attention_special_cases():
    rng = np.random.default_rng(3)
    H, d, T = 4, 8, 9
    D = H * d
    q = rng.standard_normal((1, D))
    K = rng.standard_normal((T, D))
    V = rng.standard_normal((T, D))
    # a query at position 0 sees only itself: o = V_0
    assert np.allclose(looped.attend(q, K[:1], V[:1], H, 0), V[:1], atol=1e-14)
    # identical keys -> uniform weights -> o = mean V
    Ks = np.tile(K[:1], (T, 1))
    assert np.allclose(looped.attend(q, Ks, V, H, T - 1), V.mean(0, keepdims=True), atol=1e-13)
    # causal: rows after the query's position do not matter
    V2 = V.copy()
    V2[5:] = 1e6
    K2 = K.copy()
    K2[5:] = -3.0
    qq = rng.standard_normal((3, D))
    o1 = looped.attend(qq, K[:5], V[:5], H, 2)
    o2 = looped.attend(qq, K2[:5], V2[:5], H, 2)
    assert np.allclose(o1, o2)
    # heads do not mix: changing head 1's V leaves head 0's output alone
    V3 = V.copy()
    V3[:, d:2 * d] += 10
    a, b = looped.attend(q, K, V, H, T - 1), looped.attend(q, K, V3, H, T - 1)
    assert np.allclose(a[:, :d], b[:, :d]) and not np.allclose(a[:, d:2 * d], b[:, d:2 * d])


# ---------------------------------------------------------------- whole model
TINY = synth.ModelShape("bf-tiny", 4, 2, 2, 8, 1, 7, "f32")


def _tiny_weights(seed=0):
    return synth.make_weights(TINY, seed, random_gains=True, std=0.5)


def test_bruteforce_tiny_model_matches_oracle():
    w = _tiny_weights()
    toks = [3, 1, 6, 0, 2]
    wl = {
        "embed": w["embed"].astype(float).tolist(),
        "lm_head": w["lm_head"].astype(float).tolist(),
        "final_norm": w["final_norm"].astype(float).tolist(),
        "layers": [{k: v.astype(float).tolist() for k, v in lw.items()} for lw in w["layers"]],
    }
    bf_logits, bf_h = _bruteforce.run_sequence(wl, TINY.n_heads, TINY.n_pre, 2, toks, TINY.norm_eps)
    for mode in ("f32", "kv"):
        o = oracle.LoopedOracle(TINY, w, mode, 1, 8, 2, exact=True)
        # prefill 3 then two decode steps (teacher forced)
        r = o.prefill(0, toks[:3], 2)
        got = [r["logits"][i] for i in range(3)]
        for t in toks[3:]:
            got.append(o.decode_step([0], [2], [t])["logits"][0])
        for p in range(len(toks)):
            assert np.allclose(got[p], bf_logits[p], rtol=0, atol=1e-12), (mode, p)
        if mode == "f32":
            for (layer, p), h in bf_h.items():
                assert np.allclose(o.read_h(layer, 0, 5)[p], h, atol=1e-12)


def _run(shape, w, mode, lanes, loops, prompts, steps, exact=False, l_max=None, thr=math.inf):
    l_max = l_max or max(loops)
    o = oracle.LoopedOracle(shape, w, mode, len(lanes), prompts.shape[1] + steps + 1, l_max, exact)
    toks = []
    for k, lane in enumerate(lanes):
        toks.append(o.prefill(lane, prompts[k], loops[k])["next_token"])
    out = [list(toks)]
    logits = []
    for _ in range(steps):
        r = o.decode_step(lanes, loops, toks, thr)
        toks = list(r["tokens"])
        out.append(toks)
        logits.append(r["logits"])
    return o, np.array(out), np.array(logits)


SMALL16 = synth.ModelShape("small16", 64, 4, 16, 128, 2, 97, "f16")


def test_store_h_equals_stored_kv_exact():
    """Store-h attention is ordinary attention with K = W_k h, V = W_v h: with
    the rounding points off, the h modes and the stored-K/V mode agree to
    float64 rounding (the pages' 'FP16-h: K/V bit-exact')."""
    for shape, mode in ((synth.SHAPES["tiny"], "f32"), (SMALL16, "f16")):
        w = synth.make_weights(shape, 1, random_gains=True)
        pr = synth.make_prompts(shape.vocab, 1, 6, 4)
        _, t_h, l_h = _run(shape, w, mode, [0], [3], pr, 3, exact=True)
        _, t_kv, l_kv = _run(shape, w, "kv", [0], [3], pr, 3, exact=True)
        assert np.array_equal(t_h, t_kv)
        assert np.max(np.abs(l_h - l_kv)) <= 1e-12 * np.max(np.abs(l_kv))


def test_variable_L_layer_reuse_bitwise():
    """Cache layer n_pre + i is written only by loop iteration i, so for the
    same tokens it is identical at L = i + 1 and at L_max."""
    w = synth.make_weights(SMALL16, 2, random_gains=True)
    pr = synth.make_prompts(SMALL16.vocab, 1, 5, 7)
    seq = list(pr[0]) + [11, 23, 5]
    caches = {}
    for L in (2, 5):
        o = oracle.LoopedOracle(SMALL16, w, "int4", 1, 16, 5)
        o.prefill(0, seq[:5], L)
        for t in seq[5:]:
            o.decode_step([0], [L], [t])
        caches[L] = o
    for layer in range(SMALL16.n_pre + 2):
        a = caches[2].read_codes(layer, 0, 0, 8)
        b = caches[5].read_codes(layer, 0, 0, 8)
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_resume_equals_fresh_run():
    """Warm start: a prompt run at L=4, extended to L=8 from its saved residual,
    then decoded at L=8, is bit-identical to a fresh L=8 run."""
    w = synth.make_weights(SMALL16, 3, random_gains=True)
    pr = synth.make_prompts(SMALL16.vocab, 1, 6, 8)[0]
    fresh = oracle.LoopedOracle(SMALL16, w, "int4", 1, 16, 8)
    rf = fresh.prefill(0, pr, 8)
    warm = oracle.LoopedOracle(SMALL16, w, "int4", 1, 16, 8)
    r4 = warm.forward(0, pr, 4, check_safety=False)
    r8 = warm.extend_depth(0, r4["x"], 4, 8)
    assert np.array_equal(r8["logits"], rf["logits"])
    tf, tw = rf["next_token"], oracle.argmax_lowest(r8["logits"][-1])
    assert tf == tw
    for _ in range(4):
        a = fresh.decode_step([0], [8], [tf])
        b = warm.decode_step([0], [8], [tw])
        assert np.array_equal(a["logits"], b["logits"])
        tf, tw = a["tokens"][0], b["tokens"][0]
    for layer in range(SMALL16.n_pre + 8):
        ca, cb = fresh.read_codes(layer, 0, 0, 10), warm.read_codes(layer, 0, 0, 10)
        assert np.array_equal(ca[0], cb[0]) and np.array_equal(ca[1], cb[1])


def test_lanes_are_independent():
    """A mixed-loops batch equals each lane run alone (the pages' L-aware
    batching check), bit for bit."""
    w = synth.make_weights(SMALL16, 4, random_gains=True)
    pr = synth.make_prompts(SMALL16.vocab, 3, 5, 9)
    loops = [1, 3, 6]
    _, t_b, l_b = _run(SMALL16, w, "int8", [0, 1, 2], loops, pr, 3, l_max=6)
    for k in range(3):
        _, t_1, l_1 = _run(SMALL16, w, "int8", [0], [loops[k]], pr[k:k + 1], 3, l_max=6)
        assert np.array_equal(t_b[:, k], t_1[:, 0])
        assert np.array_equal(l_b[:, k], l_1[:, 0])


def test_safety_threshold_bracket():
    """The check fires exactly when a loop iteration's residual norm exceeds
    the threshold; the aborted lane emits no token and keeps its length."""
    w = synth.make_weights(SMALL16, 5, random_gains=True)
    pr = synth.make_prompts(SMALL16.vocab, 1, 4, 10)[0]
    L = 5

    def fresh():
        o = oracle.LoopedOracle(SMALL16, w, "int4", 1, 12, L)
        t = o.prefill(0, pr, L)["next_token"]
        return o, t

    o, t = fresh()
    r = o.decode_step([0], [L], [t])
    norms = o.norms[0][:L].copy()
    assert np.all(np.isfinite(norms)) and r["status"][0] == oracle.LANE_OK
    assert np.isclose(norms[-1], np.linalg.norm(r["x"][0]), rtol=1e-15)
    # threshold = max norm: never strictly exceeded
    o, t = fresh()
    r = o.decode_step([0], [L], [t], float(norms.max()))
    assert r["status"][0] == oracle.LANE_OK and r["tokens"][0] >= 0
    for i in range(L):
        thr = float(norms[i]) * (1 - 1e-6)
        first = int(np.argmax(norms > thr))
        o, t = fresh()
        r = o.decode_step([0], [L], [t], thr)
        assert r["status"][0] == oracle.LANE_ABORTED and r["tokens"][0] == -1
        assert o.length[0] == len(pr)
        ran = o.norms[0]
        assert np.all(np.isfinite(ran[:first + 1])) and np.all(np.isnan(ran[first + 1:]))
        # the aborted lane is skipped by the next step
        r2 = o.decode_step([0], [L], [t], math.inf)
        assert r2["status"][0] == oracle.LANE_ABORTED and o.length[0] == len(pr)


def test_cache_gap_rejected():
    w = synth.make_weights(SMALL16, 6)
    o = oracle.LoopedOracle(SMALL16, w, "int4", 1, 12, 8)
    t = o.prefill(0, [1, 2, 3], 2)["next_token"]
    o.decode_step([0], [1], [t])                  # a lower L is allowed
    with pytest.raises(oracle.CacheGapError):
        o.decode_step([0], [2], [t])              # layer n_pre+1 misses the last position


def test_prefill_equals_token_by_token():
    w = synth.make_weights(SMALL16, 7, random_gains=True)
    pr = synth.make_prompts(SMALL16.vocab, 1, 7, 12)[0]
    a = oracle.LoopedOracle(SMALL16, w, "f16", 1, 8, 3)
    ra = a.prefill(0, pr, 3)
    b = oracle.LoopedOracle(SMALL16, w, "f16", 1, 8, 3)
    b.prefill(0, pr[:1], 3)
    last = None
    for t in pr[1:]:
        last = b.decode_step([0], [3], [t])["logits"][0]
    assert np.allclose(ra["logits"][-1], last, rtol=0, atol=1e-12 * np.abs(last).max())


# ------------------------------------------------------- delta codec (f2)
def test_delta_codec_hand_case():
    """Features page, "4) Iteration-axis delta-KV", worked by hand on D = 4,
    two heads of 2: anchor h0 = (1, 2, 3, 4), next h = (1.5, 2, 3, 4.25).
    delta = (0.5, 0, 0, 0.25); head scales fp16(0.5/127) = 1032 * 2^-18 and
    fp16(0.25/127) = 1032 * 2^-19; codes rint(127.0077) = 127 and 0; the FP32
    prefix sum is 1 + 127 * 1032 * 2^-18 = 49151/32768 and 4 + 127 * 1032 * 2^-19,
    both exact in fp32, which round to fp16 1.5 and 4.25."""
    h0 = np.array([[1, 2, 3, 4]], np.float16)
    h1 = np.array([[1.5, 2, 3, 4.25]], np.float16)
    d = h1.astype(np.float32) - h0.astype(np.float32)
    q, sc = looped.delta_encode(d, 2)
    assert q.tolist() == [[127, 0, 0, 127]]
    assert sc.astype(np.float64).tolist() == [[1032 * 2.0 ** -18, 1032 * 2.0 ** -19]]
    r = looped.delta_accumulate(h0.astype(np.float32), q, sc)
    assert r.astype(np.float64).tolist() == [[49151 / 32768, 2, 3, 4 + 127 * 1032 * 2.0 ** -19]]
    assert r.astype(np.float16).tolist() == [[1.5, 2, 3, 4.25]]


DELTA16 = synth.ModelShape("delta16", 64, 4, 16, 128, 2, 97, "f16")


def _trajectory(n_pos, n_layers, seed):
    """fp16 h rows per layer that settle geometrically, like the loop's
    converging trajectory (the relative step shrinks by 0.6 per layer)."""
    rng = np.random.default_rng(seed)
    base = rng.standard_normal((n_pos, 64)).astype(np.float32)
    out, step = [], 1.0
    for _ in range(n_layers):
        base = base + np.float32(step) * rng.standard_normal((n_pos, 64)).astype(np.float32)
        out.append(base.astype(np.float16))
        step *= 0.6
    return out


def test_delta_closed_loop_error_is_one_step():
    """Closed loop: every loop layer's FP32 reconstruction is within half of its
    own head scale of its h (one quantisation, no pile-up of the earlier,
    much coarser steps), and h' is that reconstruction rounded to fp16."""
    o = oracle.LoopedOracle(DELTA16, synth.make_weights(DELTA16, 1), "delta8", 1, 8, 10)
    hs = _trajectory(6, DELTA16.n_pre + 10, 3)
    for layer, h in enumerate(hs):
        o.write_h(layer, 0, 0, h)
    first_step = None
    for layer in range(DELTA16.n_pre, len(hs)):
        r = o.delta_rec(layer, 0, 0, 6).astype(np.float64)
        _, sc = o.read_codes(layer, 0, 0, 6)
        half = np.repeat(sc.astype(np.float64), 16, axis=-1) / 2
        err = np.abs(r - hs[layer].astype(np.float64))
        assert np.all(err <= half * (1 + 2.0 ** -10) + 4 * np.spacing(np.abs(r).astype(np.float32))), layer
        if first_step is None:
            first_step = float(np.max(half))
        assert np.array_equal(o.read_h(layer, 0, 6), r.astype(np.float32).astype(np.float16).astype(np.float64))
    assert float(np.max(half)) < first_step / 50      # the last steps are far finer than the first


def test_delta_open_loop_would_pile_up():
    """The same trajectory coded open-loop (deltas of the exact h) misses the
    one-step bound at the last layer: the closed-loop reading is what the
    bound above pins."""
    hs = _trajectory(6, DELTA16.n_pre + 10, 3)
    r = hs[DELTA16.n_pre - 1].astype(np.float32)
    for layer in range(DELTA16.n_pre, len(hs)):
        d = hs[layer].astype(np.float32) - hs[layer - 1].astype(np.float32)
        q, sc = looped.delta_encode(d, 16)
        r = looped.delta_accumulate(r, q, sc)
    half = np.repeat(sc.astype(np.float64), 16, axis=-1) / 2
    assert np.any(np.abs(r.astype(np.float64) - hs[-1].astype(np.float64)) > half * 1.01)


def test_delta_identical_layer_codes_zero():
    """A first loop layer equal to the anchor has a zero delta: zero codes,
    zero scales, and h' equal to the anchor bit for bit."""
    o = oracle.LoopedOracle(DELTA16, synth.make_weights(DELTA16, 1), "delta8", 1, 4, 2)
    h = _trajectory(3, 1, 5)[0]
    o.write_h(0, 0, 0, h)
    o.write_h(1, 0, 0, h)
    o.write_h(2, 0, 0, h)
    q, sc = o.read_codes(2, 0, 0, 3)
    assert not q.any() and not sc.astype(np.float32).any()
    assert np.array_equal(o.read_h(2, 0, 3), h.astype(np.float64))


def test_delta_variable_L_reuse_and_resume():
    """Delta mode keeps the variable-L property (loop layer n_pre + i depends
    only on earlier layers of the same position) and warm start equals a
    fresh run, bit for bit."""
    w = synth.make_weights(DELTA16, 2, random_gains=True)
    seq = list(synth.make_prompts(DELTA16.vocab, 1, 5, 7)[0]) + [11, 23, 5]
    caches = {}
    for L in (2, 5):
        o = oracle.LoopedOracle(DELTA16, w, "delta8", 1, 16, 5)
        o.prefill(0, seq[:5], L)
        for t in seq[5:]:
            o.decode_step([0], [L], [t])
        caches[L] = o
    for layer in range(DELTA16.n_pre + 2):
        assert np.array_equal(caches[2].read_h(layer, 0, 8), caches[5].read_h(layer, 0, 8))
    fresh = oracle.LoopedOracle(DELTA16, w, "delta8", 1, 16, 5)
    rf = fresh.prefill(0, seq[:6], 5)
    warm = oracle.LoopedOracle(DELTA16, w, "delta8", 1, 16, 5)
    r2 = warm.forward(0, seq[:6], 2, check_safety=False)
    r5 = warm.extend_depth(0, r2["x"], 2, 5)
    assert np.array_equal(r5["logits"], rf["logits"])


def _greedy(o, lane, token, loops, n):
    out = []
    while len(out) < n:
        token = int(o.decode_step([lane], [loops], [token])["tokens"][0])
        out.append(token)
    return out


@pytest.mark.parametrize("draft,verify,ahead", [(1, 4, 3), (2, 3, 4), (4, 4, 2)])
def test_self_speculative_equals_greedy(draft, verify, ahead):
    """Chain-mode self-speculation emits exactly the greedy tokens of plain
    decoding at the verify depth (features page, "Tree speculative decoding",
    chain mode), and leaves the cache a plain run would leave; with equal
    depths every draft is accepted."""
    w = synth.make_weights(SMALL16, 8, random_gains=True)
    pr = synth.make_prompts(SMALL16.vocab, 1, 5, 13)[0]
    n_tok = 14
    plain = oracle.LoopedOracle(SMALL16, w, "f16", 1, 40, 4, exact=True)
    t0 = plain.prefill(0, pr, verify)["next_token"]
    ref = _greedy(plain, 0, t0, verify, n_tok)
    spec = oracle.LoopedOracle(SMALL16, w, "f16", 1, 40, 4, exact=True)
    assert spec.prefill(0, pr, verify)["next_token"] == t0
    got, rounds, t = [], [], t0
    while len(got) < n_tok:
        r = spec.spec_step(0, t, draft, verify, ahead)
        got.extend(r["tokens"])
        rounds.append(len(r["tokens"]))
        t = r["tokens"][-1]
    if draft == verify:
        assert all(n == ahead + 1 for n in rounds)
    else:
        assert min(rounds) < ahead + 1          # the rejection path ran
    # the rounds may overshoot n_tok: decode plainly to the same point
    extra = len(got) - n_tok
    if extra:
        ref += _greedy(plain, 0, ref[-1], verify, extra)
    assert got == ref
    # the state a plain run leaves: same length, same h in every layer it ran
    T = len(pr) + len(got)
    assert plain.length[0] == T and spec.length[0] == T
    for layer in range(SMALL16.n_pre + verify):
        a, b = plain.read_h(layer, 0, T), spec.read_h(layer, 0, T)
        assert np.allclose(a, b, rtol=0, atol=1e-12 * np.abs(a).max()), layer


def test_self_speculative_on_aborted_lane():
    w = synth.make_weights(SMALL16, 9)
    o = oracle.LoopedOracle(SMALL16, w, "int4", 1, 20, 4)
    t = o.prefill(0, [3, 1, 4], 4)["next_token"]
    assert o.decode_step([0], [4], [t], 1e-6)["status"][0] == oracle.LANE_ABORTED
    r = o.spec_step(0, t, 1, 4, 3)
    assert r["tokens"] == [] and o.length[0] == 3


def test_cache_bytes_closed_form_delta():
    # 407M shape, 2 unique layers + 8 loop layers: 2 * 2048 + 8 * (1024 + 2 * 16) bytes a token
    assert looped.cache_bytes("delta8", 1024, "f16", 1, 1, 8, 2, 16) == 12544
    assert looped.cache_bytes("delta8", 1024, "f16", 3, 5, 8, 2, 16) == 15 * 12544


def test_cache_bytes_closed_form():
    # per-entry bytes at d_model 1024: fp16 K/V 4096, fp16-h 2048, INT8-h 1026, INT4-h 576
    assert looped.cache_bytes("kv", 1024, "f16", 1, 1, 1, 0) == 4096
    assert looped.entry_bytes("f16", 1024) == 2048
    assert looped.entry_bytes("int8", 1024) == 1026
    assert looped.entry_bytes("int4", 1024) == 576
    assert looped.entry_bytes("int4", 2048) == 1152
    # 4 lanes x 10 layers x 4224 positions x 576 B
    assert looped.cache_bytes("int4", 1024, "f16", 4, 4224, 8, 2) == 97_320_960
    assert looped.cache_bytes("kv", 1024, "f16", 4, 4224, 8, 2) == 692_060_160


# ------------------------------------------------ rounding points of the fp16 model
BF16 = synth.ModelShape("bf-f16", 64, 2, 32, 128, 1, 13, "f16")
BF16_POINTS = {
    "f16": frozenset(("R1", "R4o", "R4u", "R4a", "R4z")),
    "kv": frozenset(("R1", "R4o", "R4u", "R4a", "R4z", "R5")),
    "int4": frozenset(("R1", "R3", "R4o", "R4u", "R4a", "R4z")),
    "int8": frozenset(("R1", "R3", "R4o", "R4u", "R4a", "R4z")),
}


def _as_lists(w):
    return {
        "embed": w["embed"].astype(float).tolist(),
        "lm_head": w["lm_head"].astype(float).tolist(),
        "final_norm": w["final_norm"].astype(float).tolist(),
        "layers": [{k: v.astype(float).tolist() for k, v in lw.items()} for lw in w["layers"]],
    }


def _oracle_sequence_logits(shape, w, mode, toks, L, n_prefill=3):
    o = oracle.LoopedOracle(shape, w, mode, 1, len(toks) + 1, L)
    r = o.prefill(0, toks[:n_prefill], L)
    got = [r["logits"][i] for i in range(n_prefill)]
    for t in toks[n_prefill:]:
        got.append(o.decode_step([0], [L], [t])["logits"][0])
    return np.array(got)


@pytest.mark.parametrize("mode", ["f16", "kv", "int4", "int8"])
def test_bruteforce_fp16_model_rounding_points(mode):
    """The fp16 model rounds at fixed points: h before it is stored and
    projected (R1), the codec's h' = fp16(q s) (R3), o, the norm-2 output, the
    GELU output and the final-norm output before their products (R4), and
    stored K/V (R5). A scalar brute force that rounds through the standard
    library's binary16 packing, and codes INT4 / INT8 h by its own scalar
    codec, matches the oracle to float64 rounding; and dropping any one of
    those points moves the brute force's logits by far more than that
    tolerance, so the comparison sees every rounding point."""
    w = synth.make_weights(BF16, 3, random_gains=True, std=0.3)
    wl = _as_lists(w)
    toks = [3, 11, 0, 7, 5]
    L = 2
    points = BF16_POINTS[mode]
    bf, _ = _bruteforce.run_sequence(wl, BF16.n_heads, BF16.n_pre, L, toks, BF16.norm_eps,
                                     rounding=points, mode=mode if mode != "f16" else "h")
    bf = np.array(bf)
    scale = np.max(np.abs(bf))
    got = _oracle_sequence_logits(BF16, w, mode, toks, L)
    assert np.max(np.abs(got - bf)) <= 1e-12 * scale
    for p in sorted(points):
        alt, _ = _bruteforce.run_sequence(wl, BF16.n_heads, BF16.n_pre, L, toks, BF16.norm_eps,
                                          rounding=points - {p}, mode=mode if mode != "f16" else "h")
        assert np.max(np.abs(np.array(alt) - bf)) > 1e-8 * scale, p


def test_bruteforce_codec_matches_oracle_codec():
    """The brute force's scalar codec gives the oracle's codes and scales
    (both INT widths, groups along d_model), so its end-to-end INT runs test
    the oracle's model, not a second reading of the codec."""
    rng = np.random.default_rng(21)
    h = (rng.standard_normal((6, 64)) * rng.uniform(0.05, 20, size=(6, 1))).astype(np.float16)
    h[2, :32] = 0
    for kind, enc, group, qmax, qmin in (("int4", looped.int4_encode, 32, 7, -8),
                                         ("int8", looped.int8_encode, 64, 127, -127)):
        q, s = enc(h)
        hp = looped.decode_int(q, s)
        for r in range(h.shape[0]):
            codes, scales, out = _bruteforce.codec_roundtrip([float(t) for t in h[r]], group, qmax, qmin)
            assert codes == q[r].tolist(), kind
            assert scales == s[r].astype(float).tolist(), kind
            assert [_bruteforce.f16(t) for t in out] == hp[r].astype(float).tolist(), kind


# ------------------------------------------------ safety check on a degenerate state
def test_safety_fires_on_nan_residual():
    """A degenerate hidden state fires the check (novel-contributions page,
    'Per-Iteration Safety Check': the check exists to catch degenerate states).
    An infinite embedding element makes the first norm's output NaN, so the
    residual is NaN by loop iteration 0; not (NaN <= threshold) holds, so the
    lane aborts there with no token and keeps its length, while its batch mate
    decodes exactly as it would alone."""
    w = synth.make_weights(SMALL16, 5, random_gains=True)
    bad = 7
    w["embed"] = w["embed"].copy()
    w["embed"][bad, 3] = np.inf
    L = 3
    o = oracle.LoopedOracle(SMALL16, w, "int4", 2, 12, L)
    t0 = o.prefill(0, [1, 2, 3, 4], L)["next_token"]
    t1 = o.prefill(1, [5, 6, 8, 9], L)["next_token"]
    r = o.decode_step([0, 1], [L, L], [bad, t1], 1e30)
    assert r["status"].tolist() == [oracle.LANE_ABORTED, oracle.LANE_OK]
    assert r["tokens"][0] == -1 and o.length[0] == 4 and o.length[1] == 5
    assert np.all(np.isnan(o.norms[0]))
    # the lane ran iteration 0 and stopped there
    o2 = oracle.LoopedOracle(SMALL16, w, "int4", 1, 12, L)
    o2.prefill(0, [1, 2, 3, 4], L)
    f = o2.forward(0, [bad], L, check_safety=True, threshold=1e30)
    assert f["aborted_at"] == 0 and f["logits"] is None
    assert np.isnan(f["norms"][0, 0]) and np.all(np.isnan(f["norms"][0, 1:]))
    alone = oracle.LoopedOracle(SMALL16, w, "int4", 1, 12, L)
    assert alone.prefill(0, [5, 6, 8, 9], L)["next_token"] == t1
    ra = alone.decode_step([0], [L], [t1], 1e30)
    assert np.array_equal(ra["logits"][0], r["logits"][1]) and ra["tokens"][0] == r["tokens"][1]


# ------------------------------------------------ argmax ties
def test_argmax_ties_lowest_index():
    assert oracle.argmax_lowest(np.array([1.0, 3.0, -2.0, 3.0, 3.0])) == 1
    assert oracle.argmax_lowest(np.zeros(9)) == 0
    assert oracle.argmax_lowest(np.array([-1.0, -5.0, -1.0])) == 0


def tie_head(vocab, d_model, k, sign, ties, value=5.0, others=(1.0, 2.0, 3.0, 4.0)):
    """An LM head whose logits tie exactly at the top: row r is c_r times the
    unit vector on coordinate k, so logit r = c_r * z_k is one exact product
    (the other terms are zeros). c_r = value at the rows in ``ties``, a
    smaller value at every other row; ``sign`` (the sign of z_k) makes the
    tied rows the largest."""
    head = np.zeros((vocab, d_model), np.float64)
    c = np.array([others[r % len(others)] for r in range(vocab)], np.float64)
    c[list(ties)] = value
    head[:, k] = sign * c
    return head


def test_decode_argmax_tie_goes_to_lowest_index():
    """End to end: with an LM head whose top logits tie exactly, the decode
    step emits the lowest tied index."""
    w = synth.make_weights(SMALL16, 11, random_gains=True)
    L = 2
    o = oracle.LoopedOracle(SMALL16, w, "f16", 1, 8, L)
    o.prefill(0, [4, 2, 9], L)
    f = o.forward(0, [17], L, check_safety=False, keep_trace=True)
    z = dict(o.trace[0])["final_ln"][0]
    k = int(np.argmax(np.abs(z)))
    ties = (40, 13, 88)
    w["lm_head"] = tie_head(SMALL16.vocab, SMALL16.d_model, k, np.sign(z[k]), ties).astype(np.float16)
    o = oracle.LoopedOracle(SMALL16, w, "f16", 1, 8, L)
    t = o.prefill(0, [4, 2, 9], L)["next_token"]
    r = o.decode_step([0], [L], [17])
    lg = r["logits"][0]
    assert lg[13] == lg[40] == lg[88] == np.max(lg) and np.sum(lg == np.max(lg)) == 3
    assert r["tokens"][0] == 13
