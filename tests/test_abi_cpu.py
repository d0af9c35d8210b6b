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
