"""Calls every host-side path of the C ABI that needs no GPU and prints the
results as one JSON object: the closed-form byte counts over a grid of
configurations, modes and sizes (valid, degenerate and refused), model
creation with valid and broken configurations, every validation branch of
tl_cache_alloc (and, on a machine without a GPU, its full handle
construction up to the first launch, which fails there), and the null-handle
checks of the other entry points. Device pointers are fake and never
dereferenced. Run: python tests/_asan_driver.py LIBRARY"""
import ctypes
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

from kv_compression_amd import tl  # noqa: E402
import synth  # noqa: E402

FAKE = 1 << 20   # a 256-byte aligned address that is never dereferenced


def weights(n_pre, bad_layer=-1):
    ls = [tl.tl_layer_weights(*([0 if u == bad_layer else FAKE] * 6)) for u in range(n_pre + 1)]
    return tl.tl_weights(FAKE, FAKE, FAKE, (tl.tl_layer_weights * (n_pre + 1))(*ls))


def main(path):
    L = tl.load(path)
    res = {"version": L.tl_version()}
    err = lambda: L.tl_last_error().decode()

    # closed-form sizes
    sizes = []
    cfgs = {name: tl.make_config(sh) for name, sh in synth.SHAPES.items()}
    broken = []
    for field, val in (("d_model", 0), ("n_heads", 3), ("d_head", 48), ("d_mlp", 100), ("vocab", 15),
                       ("dtype", 7), ("n_pre", -1), ("norm_eps", float("nan")), ("d_model", 4096)):
        c = tl.make_config(synth.SHAPES["407m"])
        setattr(c, field, val)
        broken.append(("407m-%s=%s" % (field, val), c))
    for name, cfg in list(cfgs.items()) + broken:
        for mode in range(-1, 8):
            for lanes, seq, lmax in ((1, 1, 1), (4, 4224, 8), (3, 77, 32), (0, 16, 1), (1, 0, 1), (1, 16, 0),
                                     (-1, 16, 1), (1, 1 << 24, 1), (1, (1 << 24) + 1, 1), (1 << 20, 1, 1),
                                     ((1 << 20) + 1, 1, 1), (1, 16, 4096), (1, 16, 4097), (2, 1 << 21, 2)):
                sizes.append([name, mode, lanes, seq, lmax,
                              L.tl_cache_bytes(ctypes.byref(cfg), mode, lanes, seq, lmax),
                              L.tl_workspace_bytes(ctypes.byref(cfg), mode, lanes, seq, lmax)])
    sizes.append(["null-config", 4, 1, 16, 1, L.tl_cache_bytes(None, 4, 1, 16, 1),
                  L.tl_workspace_bytes(None, 4, 1, 16, 1)])
    res["sizes"] = sizes

    # model creation
    mc = []
    for name, cfg in list(cfgs.items()) + broken:
        n_pre = max(cfg.n_pre, 0)
        for bad in (-1, 0, n_pre):
            m = ctypes.c_void_p()
            w = weights(n_pre, bad)
            st = L.tl_model_create(ctypes.byref(cfg), ctypes.byref(w), ctypes.byref(m))
            mc.append([name, bad, st, err() if st else "", m.value is not None])
            if m.value:
                L.tl_model_destroy(m)
    m = ctypes.c_void_p()
    mc.append(["null-weights", L.tl_model_create(ctypes.byref(cfgs["407m"]), None, ctypes.byref(m)), err()])
    w = weights(cfgs["407m"].n_pre)
    mc.append(["null-out", L.tl_model_create(ctypes.byref(cfgs["407m"]), ctypes.byref(w), None), err()])
    L.tl_model_destroy(None)
    res["model_create"] = mc

    # cache allocation: every refusal, then the full construction where no GPU
    # can run its first launch
    gpu_here = os.path.exists("/dev/kfd")
    al = []
    for name in ("tiny", "407m", "2b"):
        cfg = cfgs[name]
        m = ctypes.c_void_p()
        w = weights(cfg.n_pre)
        assert L.tl_model_create(ctypes.byref(cfg), ctypes.byref(w), ctypes.byref(m)) == tl.TL_OK
        for mode in range(-1, 7):
            need = L.tl_cache_bytes(ctypes.byref(cfg), mode, 2, 64, 2)
            wneed = L.tl_workspace_bytes(ctypes.byref(cfg), mode, 2, 64, 2)
            cases = [("ok", 2, 64, 2, FAKE, need, FAKE, wneed), ("dims", 0, 64, 2, FAKE, need, FAKE, wneed),
                     ("slab", 1, 1 << 22, 2, FAKE, 1 << 44, FAKE, 1 << 44),
                     ("small-cache", 2, 64, 2, FAKE, max(need - 1, 0), FAKE, wneed),
                     ("small-ws", 2, 64, 2, FAKE, need, FAKE, max(wneed - 1, 0)),
                     ("null-cache", 2, 64, 2, 0, need, FAKE, wneed),
                     ("misaligned", 2, 64, 2, FAKE + 8, need, FAKE, wneed)]
            for tag, lanes, seq, lmax, dc, cb, dw, wb in cases:
                if tag == "ok" and (gpu_here or need == 0):
                    continue
                out = ctypes.c_void_p()
                st = L.tl_cache_alloc(m, mode, lanes, seq, lmax, dc, cb, dw, wb, None, ctypes.byref(out))
                al.append([name, mode, tag, st, err() if st else "", out.value is not None])
                if out.value:
                    L.tl_cache_free(out)
        out = ctypes.c_void_p()
        al.append([name, "null-out", L.tl_cache_alloc(m, 4, 1, 16, 1, FAKE, 1 << 40, FAKE, 1 << 40, None, None)])
        al.append([name, "null-model", L.tl_cache_alloc(None, 4, 1, 16, 1, FAKE, 1 << 40, FAKE, 1 << 40, None,
                                                          ctypes.byref(out))])
        L.tl_model_destroy(m)
    L.tl_cache_free(None)
    res["cache_alloc"] = al

    # null cache handles
    nh = []
    i32 = ctypes.c_int32(0)
    d = ctypes.c_double(0)
    ii = ctypes.c_int(0)
    calls = {
        "reset_lane": lambda: L.tl_cache_reset_lane(None, 0, None),
        "set_length": lambda: L.tl_cache_set_length(None, 0, 0, 0, None),
        "write_h": lambda: L.tl_cache_write_h(None, 0, 0, 0, 1, FAKE, None),
        "fill_synthetic": lambda: L.tl_cache_fill_synthetic(None, 0, 0, 0, 1, 1, None),
        "read": lambda: L.tl_cache_read(None, 0, 0, 0, 1, FAKE, FAKE, None, None),
        "residual_norms": lambda: L.tl_residual_norms(None, 0, FAKE, None),
        "lane_residual": lambda: L.tl_lane_residual(None, 0, FAKE, None),
        "prefill_chunk": lambda: L.tl_prefill_chunk(None, 0, 1, FAKE, 1, FAKE, FAKE, None),
        "extend_depth": lambda: L.tl_extend_depth(None, 0, 0, 1, 1, 2, FAKE, FAKE, FAKE, None),
        "decode_step": lambda: L.tl_decode_step(None, 1, ctypes.byref(i32), ctypes.byref(i32), FAKE,
                                                float("inf"), FAKE, None, FAKE, None),
        "decode_step_static": lambda: L.tl_decode_step_static(None, 1, ctypes.byref(i32), ctypes.byref(i32),
                                                              FAKE, float("inf"), FAKE, None, FAKE, None),
        "spec_step": lambda: L.tl_spec_step(None, 0, 1, 2, 1, FAKE, FAKE, ctypes.byref(ii), None),
        "set_attention": lambda: L.tl_cache_set_attention(None, 0),
        "profile_start": lambda: L.tl_profile_start(None),
        "profile_stop": lambda: L.tl_profile_stop(None, ctypes.byref(d), ctypes.byref(ii)),
    }
    for k, f in calls.items():
        nh.append([k, f(), err()])
    res["null_handles"] = nh
    print(json.dumps(res))


if __name__ == "__main__":
    main(sys.argv[1])
