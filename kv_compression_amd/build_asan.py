"""Host-side AddressSanitizer and UndefinedBehaviorSanitizer build of the C-ABI
layer, for CPU tests.

tl_api.hip (argument validation, cache and workspace layout, handle
lifetime, error strings) is compiled again with both sanitizers on its host
code only (undefined behaviour aborts), and linked with the regular objects of the kernels into
_build/libtl_asan.so. Loading it needs the sanitizer runtime preloaded
(asan_runtime() names it); no GPU code is instrumented.
Run: python -m kv_compression_amd.build_asan (after kv_compression_amd.build).
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys

from kv_compression_amd import build as B

ASAN_LIB = os.path.join(B.BUILD, "libtl_asan.so")
# sanitizer flags apply to the host compilation only
HOST_SAN = ["-Xarch_host", "-fsanitize=address,undefined", "-Xarch_host", "-fno-sanitize-recover=undefined",
            "-Xarch_host", "-fno-omit-frame-pointer"]


def asan_runtime() -> str:
    """The clang AddressSanitizer runtime of the ROCm toolchain."""
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not hits:
        raise RuntimeError("no libclang_rt.asan-x86_64.so under /opt/rocm/llvm/lib/clang")
    return hits[-1]


def build_asan(verbose: bool = True) -> str:
    os.makedirs(os.path.join(B.BUILD, "asan"), exist_ok=True)
    srcs = B.sources()
    objs = []
    for src in srcs:
        name = os.path.basename(src)[:-4] + ".o"
        if os.path.basename(src) == "tl_api.hip":
            obj = os.path.join(B.BUILD, "asan", name)
            r = subprocess.run([B.HIPCC, *B.CFLAGS, *HOST_SAN, "-c", src, "-o", obj],
                               capture_output=True, text=True)
            if r.returncode != 0:
                raise RuntimeError("hipcc (asan) failed for %s:\n%s" % (src, r.stderr[-6000:]))
        else:
            obj = os.path.join(B.BUILD, name)
            if not os.path.exists(obj):
                raise RuntimeError("%s is missing: run kv_compression_amd.build first" % obj)
        objs.append(obj)
    tmp = ASAN_LIB + ".tmp"
    r = subprocess.run([B.HIPCC, "--offload-arch=" + B.ARCH, "-shared", "-fPIC", *HOST_SAN, "-o", tmp, *objs],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link (asan) failed:\n" + r.stderr[-4000:])
    os.replace(tmp, ASAN_LIB)
    if verbose:
        print("built", ASAN_LIB)
    return ASAN_LIB


if __name__ == "__main__":
    build_asan()
    sys.exit(0)
