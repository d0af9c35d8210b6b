"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Bars: codec integers, dequantised h and argmax tokens bit-exact (tokens with
the near-tie rule); fp32-accumulated logits, norms and residuals within 2e-3
normwise-max relative error."""
import math

import numpy as np
import pytest

import synth
import oracle
from oracle import looped
from tests._gpu_util import decode, gpu_model, record, rel_err, token_ok, torch_gpu, REL_TOL

pytestmark = pytest.mark.gpu

S407 = synth.SHAPES["407m"]
S2B = synth.SHAPES["2b"]
TINY = synth.SHAPES["tiny"]

# ------------------------------------------------------------------ codec
@pytest.mark.parametrize("mode", ["int4", "int8", "f16"])
def test_codec_bitexact_on_identical_input(mode):
    torch = torch_gpu()
    w, gm = gpu_model(S407)
    rng = np.random.default_rng(21)
    n, D = 96, S407.d_model
    h = (rng.standard_normal((n, D)) * rng.uniform(1e-3, 50, size=(n, 1))).astype(np.float16)
    h[1] = 0                                   # all-zero row / groups
    h[2, :32] = np.float16(2.0 ** -24)         # scale underflow
    h[3, :32] = np.float16(65504.0)            # largest fp16
    h[3, 32:64] = -np.float16(65504.0)
    h[4, :64] = np.linspace(-7.5, 7.5, 64).astype(np.float16)   # exact .5 ties at s = 1
    h[4, 0] = 7.0
    h[5, :32] = np.float16(17 * 2.0 ** -24)    # subnormal scale, +-8.5 -> (7, -8)
    h[5, 1] = -np.float16(17 * 2.0 ** -24)
    c = gm.cache(mode, 2, 128, 1)
    d_h = torch.from_numpy(h).cuda()
    c.tl_cache_write_h(1, 2, 7, d_h)
    hp = torch.empty((n, D), dtype=torch.float16, device="cuda")
    if mode == "f16":
        c.tl_cache_read(1, 2, 7, n, d_h=hp)
        torch.cuda.synchronize()
        assert np.array_equal(hp.cpu().numpy().view(np.uint16), h.view(np.uint16))
        return
    G = D // 32 if mode == "int4" else 1
    codes = torch.empty((n, D), dtype=torch.int8, device="cuda")
    scales = torch.empty((n, G), dtype=torch.int16, device="cuda")
    c.tl_cache_read(1, 2, 7, n, codes, scales, hp)
    torch.cuda.synchronize()
    q_ref, s_ref = (looped.int4_encode(h) if mode == "int4" else looped.int8_encode(h))
    assert np.array_equal(codes.cpu().numpy(), q_ref)
    assert np.array_equal(scales.cpu().numpy().view(np.uint16), s_ref.view(np.uint16))
    hp_ref = looped.decode_int(q_ref, s_ref)
    assert np.array_equal(hp.cpu().numpy().view(np.uint16), hp_ref.view(np.uint16))


@pytest.mark.parametrize("mode", ["f16", "int4"])
def test_synthetic_fill_matches_generator(mode):
    torch = torch_gpu()
    w, gm = gpu_model(S407)
    c = gm.cache(mode, 3, 300, 2)
    c.tl_cache_fill_synthetic(2, 3, 0, 300, 2)
    pos = np.arange(0, 300, 7)
    ref16 = synth.prior_h(2, 3, 2, np.arange(300), S407.d_model).astype(np.float16)
    hp = torch.empty((300, S407.d_model), dtype=torch.float16, device="cuda")
    c.tl_cache_read(2, 3, 0, 300, d_h=hp)
    torch.cuda.synchronize()
    got = hp.cpu().numpy()
    if mode == "f16":
        bad = np.argwhere(got.view(np.uint16) != ref16.view(np.uint16))
        detail = [(int(p), int(k), float(got[p, k]), float(ref16[p, k]),
                   float(synth.prior_h(2, 3, 2, [p], S407.d_model)[0, k])) for p, k in bad[:8]]
        assert bad.shape[0] == 0, (bad.shape[0], detail)
    else:
        q, s = looped.int4_encode(ref16)
        assert np.array_equal(got.view(np.uint16), looped.decode_int(q, s).view(np.uint16))
    del pos


# ------------------------------------------------------------------ tiny fp32 (one decode step)
@pytest.mark.parametrize("mode", ["f32", "kv"])
def test_tiny_fp32_decode_step(mode):
    wl = synth.workload("tiny-f32-ctx64")
    sh = wl.shape
    w, gm = gpu_model(sh, random_gains=True)
    n_layers = sh.n_pre + wl.l_max
    ctx = wl.context
    orc = oracle.LoopedOracle(sh, w, mode, 1, ctx + 2, wl.l_max)
    orc.prime_synthetic(0, range(n_layers), ctx,
                        lambda layer: synth.prior_h(wl.seed_prior, layer, 0, np.arange(ctx), sh.d_model))
    c = gm.cache(mode, 1, ctx + 2, wl.l_max)
    for layer in range(n_layers):
        c.tl_cache_fill_synthetic(0, layer, 0, ctx, wl.seed_prior)
    c.tl_cache_set_length(0, ctx, n_layers)
    tok = int(synth.make_prompts(sh.vocab, 1, 1, wl.seed_prompt)[0, 0])
    r = orc.decode_step([0], [2], [tok], wl.threshold)
    t, lg, st = decode(c, [0], [2], [tok], wl.threshold)
    assert st[0] == oracle.LANE_OK == r["status"][0]
    record("decode_logits", shape="tiny", mode=mode, rel=rel_err(lg[0], r["logits"][0]))
    assert rel_err(lg[0], r["logits"][0]) <= REL_TOL
    assert token_ok(int(t[0]), r["logits"][0])
    norms = c.tl_residual_norms(0)
    assert rel_err(norms[:2], orc.norms[0][:2]) <= REL_TOL
    torch = torch_gpu()
    xr = torch.empty(sh.d_model, dtype=torch.float32, device="cuda")
    c.tl_lane_residual(0, xr)
    assert rel_err(xr.cpu().numpy(), r["x"][0]) <= REL_TOL


# ------------------------------------------------------------------ 407M shape, short context
def _prefill_both(gm, w, shape, mode, lanes_prompts, loops, max_seq, l_max):
    orc = oracle.LoopedOracle(shape, w, mode, len(lanes_prompts), max_seq, l_max)
    c = gm.cache(mode, len(lanes_prompts), max_seq, l_max)
    toks, ref = [], []
    for lane, pr in enumerate(lanes_prompts):
        ro = orc.prefill(lane, pr, loops[lane])
        nxt, lg = c.prefill(lane, pr, loops[lane])
        g_lg = lg.cpu().numpy()
        e = rel_err(g_lg, ro["logits"][-1])
        record("prefill_logits", shape=shape.name, mode=mode, lane=lane, n=len(pr), rel=e)
        assert e <= REL_TOL, (mode, lane, e)
        g_t = int(nxt.cpu().numpy()[0])
        assert token_ok(g_t, ro["logits"][-1])
        toks.append(g_t)
    return orc, c, toks


@pytest.mark.parametrize("mode", ["int4", "int8", "f16", "kv"])
def test_407m_prefill_and_decode(mode):
    w, gm = gpu_model(S407)
    prompts = synth.make_prompts(S407.vocab, 2, 300, 1)      # two 256-position tiles + a ragged tail
    loops = [3, 2]
    orc, c, toks = _prefill_both(gm, w, S407, mode, list(prompts), loops, 320, 3)
    for step in range(3):
        r = orc.decode_step([0, 1], loops, toks)
        t, lg, st = decode(c, [0, 1], loops, toks)
        for k in range(2):
            assert st[k] == 0
            e = rel_err(lg[k], r["logits"][k])
            record("decode_logits", shape="407m", mode=mode, step=step, lane=k, rel=e)
            assert e <= REL_TOL, (mode, step, k, e)
            assert token_ok(int(t[k]), r["logits"][k])
        for k in range(2):
            n_ref = orc.norms[k][:loops[k]]
            assert rel_err(c.tl_residual_norms(k)[:loops[k]], n_ref) <= REL_TOL
        toks = [int(x) for x in t]          # teacher-force the GPU's tokens into both


def test_2b_decode_int4_short():
    w, gm = gpu_model(S2B)
    prompts = synth.make_prompts(S2B.vocab, 1, 200, 3)
    orc, c, toks = _prefill_both(gm, w, S2B, "int4", list(prompts), [2], 210, 2)
    for step in range(2):
        r = orc.decode_step([0], [2], toks)
        t, lg, st = decode(c, [0], [2], toks)
        record("decode_logits", shape="2b", mode="int4", step=step, rel=rel_err(lg[0], r["logits"][0]))
        assert rel_err(lg[0], r["logits"][0]) <= REL_TOL
        assert token_ok(int(t[0]), r["logits"][0])
        toks = [int(t[0])]


# ------------------------------------------------------------------ layer 0 codes, end to end
def test_layer0_codes_bitexact_end_to_end():
    """Layer 0's h depends only on the token embedding, so its codes match the
    oracle's wherever the oracle's h is not within fp32 rounding of an fp16
    rounding boundary."""
    torch = torch_gpu()
    w, gm = gpu_model(S407)
    pr = synth.make_prompts(S407.vocab, 1, 64, 5)[0]
    orc, c, _ = _prefill_both(gm, w, S407, "int4", [pr], [1], 64, 1)
    codes = torch.empty((64, S407.d_model), dtype=torch.int8, device="cuda")
    scales = torch.empty((64, S407.d_model // 32), dtype=torch.int16, device="cuda")
    c.tl_cache_read(0, 0, 0, 64, codes, scales)
    torch.cuda.synchronize()
    q_ref, s_ref = orc.read_codes(0, 0, 0, 64)
    q, s = codes.cpu().numpy(), scales.cpu().numpy().view(np.uint16)
    mism = np.any((q != q_ref).reshape(64, -1, 32), axis=-1) | (s != s_ref.view(np.uint16))
    assert mism.mean() <= 1e-3, mism.mean()


# ------------------------------------------------------------------ safety check
def test_safety_threshold_bracket_gpu():
    w, gm = gpu_model(S407)
    pr = synth.make_prompts(S407.vocab, 1, 40, 6)[0]
    L = 4

    def fresh():
        c = gm.cache("int4", 1, 50, L)
        nxt, _ = c.prefill(0, pr, L)
        return c, int(nxt.cpu().numpy()[0])

    c, t0 = fresh()
    t, _, st = decode(c, [0], [L], [t0], math.inf)
    norms = c.tl_residual_norms(0)[:L].astype(np.float64)
    assert st[0] == 0 and np.all(np.isfinite(norms))
    for i in range(L):
        thr = float(np.float32(norms[i] * (1 - 1e-4)))
        first = int(np.argmax(norms > thr))
        c, t0 = fresh()
        t, lg, st = decode(c, [0], [L], [t0], thr)
        assert st[0] == oracle.LANE_ABORTED and t[0] == -1
        got = c.tl_residual_norms(0)
        assert np.all(np.isfinite(got[:first + 1])) and np.all(np.isnan(got[first + 1:L]))
        assert np.all(np.isnan(lg[0]))
        # skipped by the next step, length unchanged
        t2, _, st2 = decode(c, [0], [L], [t0], math.inf)
        assert st2[0] == oracle.LANE_ABORTED and t2[0] == -1
    c, t0 = fresh()
    t, _, st = decode(c, [0], [L], [t0], float(np.float32(norms.max() * (1 + 1e-4))))
    assert st[0] == 0 and t[0] >= 0


def test_last_iteration_check_at_step_end():
    """Each row's last loop iteration is checked at the end of the step, on
    its final residual, with the row's own iteration index (rows of 1 and 3
    loops in one step): a threshold just under the 1-loop row's only norm
    stops that row there (status, token -1, NaN logits, the norm recorded),
    while its batch mate stops exactly where its own norms first exceed the
    threshold, or decodes bitwise as without the check."""
    w, gm = gpu_model(S407)
    prompts = synth.make_prompts(S407.vocab, 2, 60, 12)
    loops = [1, 3]

    def fresh():
        c = gm.cache("int4", 2, 80, 3)
        toks = [int(c.prefill(k, prompts[k], loops[k])[0].cpu().numpy()[0]) for k in range(2)]
        return c, toks

    c, toks = fresh()
    t, lg, st = decode(c, [0, 1], loops, toks, math.inf)
    assert np.all(st == 0)
    n0 = c.tl_residual_norms(0)[:1].astype(np.float64)
    n1 = c.tl_residual_norms(1)[:3].astype(np.float64)
    assert np.all(np.isfinite(n0)) and np.all(np.isfinite(n1))
    thr = float(np.float32(n0[0] * (1 - 1e-4)))
    c, toks2 = fresh()
    assert toks2 == toks
    t2, lg2, st2 = decode(c, [0, 1], loops, toks, thr)
    assert st2[0] == oracle.LANE_ABORTED and t2[0] == -1 and np.all(np.isnan(lg2[0]))
    assert c.tl_residual_norms(0)[0] == np.float32(n0[0])
    if np.any(n1 > thr):
        first = int(np.argmax(n1 > thr))
        got = c.tl_residual_norms(1)
        assert st2[1] == oracle.LANE_ABORTED and t2[1] == -1
        assert np.all(np.isfinite(got[:first + 1])) and np.all(np.isnan(got[first + 1:3]))
    else:
        assert st2[1] == 0 and t2[1] == t[1]
        assert np.array_equal(lg2[1].view(np.uint32), lg[1].view(np.uint32))


# ------------------------------------------------------------------ invariants on the GPU
def test_lane_result_independent_of_batch_mates():
    """A mixed-loops batch gives each lane exactly (bitwise) what it gets alone."""
    w, gm = gpu_model(S407)
    prompts = synth.make_prompts(S407.vocab, 3, 90, 8)
    loops = [1, 3, 2]
    c = gm.cache("int4", 3, 100, 3)
    toks = []
    for k in range(3):
        nxt, _ = c.prefill(k, prompts[k], loops[k])
        toks.append(int(nxt.cpu().numpy()[0]))
    tb, lb, _ = decode(c, [0, 1, 2], loops, toks)
    for k in range(3):
        c1 = gm.cache("int4", 1, 100, 3)
        nxt, _ = c1.prefill(0, prompts[k], loops[k])
        assert int(nxt.cpu().numpy()[0]) == toks[k]
        t1, l1, _ = decode(c1, [0], [loops[k]], [toks[k]])
        assert t1[0] == tb[k]
        assert np.array_equal(l1[0].view(np.uint32), lb[k].view(np.uint32))


def test_variable_L_layer_reuse_gpu_bitwise():
    torch = torch_gpu()
    w, gm = gpu_model(S407)
    pr = synth.make_prompts(S407.vocab, 1, 70, 9)[0]
    got = {}
    for L in (2, 5):
        c = gm.cache("int4", 1, 80, 5)
        nxt, _ = c.prefill(0, pr, L)
        t = [int(nxt.cpu().numpy()[0])]
        for _ in range(2):
            tt, _, _ = decode(c, [0], [L], [17])
        codes = torch.empty((72, S407.d_model), dtype=torch.int8, device="cuda")
        res = []
        for layer in range(S407.n_pre + 2):
            c.tl_cache_read(0, layer, 0, 72, codes)
            torch.cuda.synchronize()
            res.append(codes.cpu().numpy().copy())
        got[L] = res
    for a, b in zip(got[2], got[5]):
        assert np.array_equal(a, b)


def test_run_twice_bitwise():
    w, gm = gpu_model(S407)
    pr = synth.make_prompts(S407.vocab, 2, 120, 10)
    outs = []
    for _ in range(2):
        c = gm.cache("int4", 2, 130, 3)
        toks = []
        for k in range(2):
            nxt, _ = c.prefill(k, pr[k], 3)
            toks.append(int(nxt.cpu().numpy()[0]))
        t, lg, _ = decode(c, [0, 1], [3, 3], toks)
        outs.append(lg)
    assert np.array_equal(outs[0].view(np.uint32), outs[1].view(np.uint32))


def test_abi_errors_do_not_enqueue():
    from kv_compression_amd import tl
    w, gm = gpu_model(S407)
    c = gm.cache("int4", 2, 16, 2)
    torch = torch_gpu()
    with pytest.raises(tl.TLError) as e:
        decode(c, [0], [3], [1])
    assert e.value.status == tl.TL_E_ARG
    c.prefill(0, list(range(16)), 1)
    with pytest.raises(tl.TLError) as e:
        decode(c, [0], [1], [1])
    assert e.value.status == tl.TL_E_CAPACITY
    c.prefill(1, [1, 2], 1)
    with pytest.raises(tl.TLError) as e:
        decode(c, [1], [2], [1])
    assert e.value.status == tl.TL_E_CACHE_GAP
    with pytest.raises(tl.TLError) as e:
        decode(c, [1, 1], [1, 1], [1, 1])
    assert e.value.status == tl.TL_E_ARG


@pytest.mark.parametrize("mode", ["f32", "kv"])
def test_tiny_fp32_chunked_prefill(mode):
    """The fp32 model's prefill: the fp32-MFMA attention kernel, and chunks of
    20 tokens late in a 300-token prompt, whose keys are split over
    workgroups and merged row-parallel; then two decode steps."""
    w, gm = gpu_model(TINY)
    pr = synth.make_prompts(TINY.vocab, 1, 300, 12)[0]
    c = gm.cache(mode, 1, 310, 2)
    orc = oracle.LoopedOracle(TINY, w, mode, 1, 310, 2)
    nxt, lg = c.prefill(0, pr, 2, chunk=20)
    ro = orc.prefill(0, pr, 2)
    e = rel_err(lg.cpu().numpy(), ro["logits"][-1])
    record("tiny_chunked_prefill", mode=mode, rel=e)
    assert e <= REL_TOL, (mode, e)
    tok = int(nxt.cpu().numpy()[0])
    assert token_ok(tok, ro["logits"][-1])
    for step in range(2):
        t, lgd, st = decode(c, [0], [2], [tok])
        r = orc.decode_step([0], [2], [tok])
        assert st[0] == 0 and rel_err(lgd[0], r["logits"][0]) <= REL_TOL, (mode, step)
        assert token_ok(int(t[0]), r["logits"][0])
        tok = int(t[0])
