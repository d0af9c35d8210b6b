"""The host code of the C-ABI layer (argument validation, cache and workspace
layout, handle lifetime, error strings) under AddressSanitizer and
UndefinedBehaviorSanitizer: tests/_asan_driver.py calls every host path that
needs no GPU, once on the regular library and once on the sanitized build
(kv_compression_amd/build_asan.py, tl_api.hip's host code instrumented) with
the sanitizer runtime preloaded. The sanitized run must report nothing and
return exactly the regular run's results."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
DRIVER = os.path.join(ROOT, "tests", "_asan_driver.py")


def _run(lib, env_extra):
    env = dict(os.environ)
    env.update(env_extra)
    return subprocess.run([sys.executable, DRIVER, lib], capture_output=True, text=True, env=env, timeout=600)


def test_host_paths_clean_under_sanitizers():
    from kv_compression_amd import build as B
    from kv_compression_amd import build_asan
    if not os.path.exists(build_asan.ASAN_LIB):
        if not os.path.exists(B.LIB):
            B.build()
        build_asan.build_asan()
    plain = _run(B.LIB, {})
    assert plain.returncode == 0, plain.stderr[-3000:]
    san = _run(build_asan.ASAN_LIB, {
        "LD_PRELOAD": build_asan.asan_runtime(),
        # the interpreter itself is not instrumented and keeps its allocations
        "ASAN_OPTIONS": "detect_leaks=0:exitcode=86",
        "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
    })
    assert san.returncode == 0, san.stderr[-4000:]
    assert "Sanitizer" not in san.stderr and "runtime error" not in san.stderr, san.stderr[-4000:]
    assert san.stdout == plain.stdout
