"""The C-ABI library loads without a GPU and exports every function that
include/tl.h declares; the closed-form byte counts need no device."""
import os
import re

import pytest

import synth
from oracle import looped

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "tl.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(tl_[a-z_0-9]+)\s*\(", src)))


def test_header_declares_the_core_calls():
    names = _declared()
    for n in ("tl_cache_alloc", "tl_decode_step", "tl_prefill_chunk", "tl_residual_norms"):
        assert n in names


def test_library_exports_every_declared_symbol():
    from kv_compression_amd import tl
    L = tl.load()
    missing = [n for n in _declared() if not hasattr(L, n)]
    assert not missing, missing
    assert set(tl.EXPORTS) == set(_declared())


@pytest.mark.parametrize("name", ["tiny", "407m", "2b"])
def test_cache_bytes_match_closed_form(name):
    from kv_compression_amd import tl
    sh = synth.SHAPES[name]
    cfg = tl.make_config(sh)
    modes = ("f32", "kv") if sh.dtype == "f32" else ("f16", "int8", "int4", "kv", "delta8")
    for mode in modes:
        for lanes, seq, lmax in ((1, 1, 1), (4, 4224, 8), (3, 77, 32)):
            want = looped.cache_bytes(mode, sh.d_model, sh.dtype, lanes, seq, lmax, sh.n_pre,
                                      sh.n_heads)
            assert tl.tl_cache_bytes(cfg, mode, lanes, seq, lmax) == want
    # modes a model dtype does not support have no layout
    for bad in (("int4", "delta8") if sh.dtype == "f32" else ("f32",)):
        assert tl.tl_cache_bytes(cfg, bad, 1, 16, 1) == 0


@pytest.mark.parametrize("mode,limit", [("int8", 1 << 20), ("int4", 1 << 21), ("f16", 1 << 19),
                                        ("kv", 1 << 18), ("delta8", 1 << 19)])
def test_cache_slab_limit_refused(mode, limit):
    """At d_model 2048 one (layer, lane) slab of code rows reaches 2^31 bytes
    at `limit` positions (2^31 / row bytes: INT8 2048, INT4 1024, fp16-h 4096,
    fp16 K|V 8192; the delta mode's anchor rows are 4096 bytes): the byte counts are 0 and tl_cache_alloc refuses with
    TL_E_UNSUPPORTED before it touches any buffer (the pointers passed are
    never dereferenced), so no GPU is needed."""
    import ctypes
    from kv_compression_amd import tl
    L = tl.load()
    sh = synth.SHAPES["2b"]
    cfg = tl.make_config(sh)
    assert tl.tl_cache_bytes(cfg, mode, 1, limit - 1, 8) == looped.cache_bytes(
        mode, sh.d_model, sh.dtype, 1, limit - 1, 8, sh.n_pre, sh.n_heads)
    assert tl.tl_workspace_bytes(cfg, mode, 1, limit - 1, 8) > 0
    for seq in (limit, 1_100_000 if mode == "int8" else limit + 1):
        assert tl.tl_cache_bytes(cfg, mode, 1, seq, 8) == 0
        assert tl.tl_workspace_bytes(cfg, mode, 1, seq, 8) == 0
    fake = 1 << 20
    layers = (tl.tl_layer_weights * (sh.n_pre + 1))(
        *[tl.tl_layer_weights(fake, fake, fake, fake, fake, fake) for _ in range(sh.n_pre + 1)])
    w = tl.tl_weights(fake, fake, fake, layers)
    m = ctypes.c_void_p()
    assert L.tl_model_create(ctypes.byref(cfg), ctypes.byref(w), ctypes.byref(m)) == tl.TL_OK
    try:
        out = ctypes.c_void_p()
        seq = 1_100_000 if mode == "int8" else limit
        st = L.tl_cache_alloc(m, tl.MODES[mode], 1, seq, 8, fake, 1 << 44, fake, 1 << 44, None,
                              ctypes.byref(out))
        assert st == tl.TL_E_UNSUPPORTED and out.value is None
        assert b"2^31" in L.tl_last_error()
    finally:
        L.tl_model_destroy(m)
