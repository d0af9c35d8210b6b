"""Build libtl.so (the HIP library behind include/tl.h) for gfx950, in-tree.

Each .hip source under csrc/ is compiled to an object with hipcc in parallel,
then linked into kv_compression_amd/libtl.so; probe/hbm_read.hip and
probe/mfma_rate.hip, the streaming-read and MFMA-rate reference programs, are
built beside it as probe/hbm_read and probe/mfma_rate.
Run: python -m kv_compression_amd.build
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libtl.so")
# the streaming-read and MFMA-rate reference programs (no part of the library)
PROBES = [(os.path.join(HERE, "probe", name + ".hip"), os.path.join(HERE, "probe", name))
          for name in ("hbm_read", "mfma_rate")]
ARCH = os.environ.get("TL_OFFLOAD_ARCH", "gfx950")

HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
CFLAGS = [
    "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
    "-Wno-unused-variable", "-Wno-unused-but-set-variable",
    # no packed-fp32 instructions anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # every float operation rounds where the source says it does (no implicit
    # fusing, e.g. of fp16(fp32(a*b)) into one mixed-precision FMA); kernels
    # that want fused multiply-adds call fmaf explicitly
    "-ffp-contract=off",
]


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src)[:-4] + ".o")
    cmd = [HIPCC, *CFLAGS, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s" % (src, r.stderr[-6000:]))
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    jobs = min(len(srcs), int(os.environ.get("MAX_JOBS", "8")))
    with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stderr[-4000:])
    os.replace(tmp, LIB)
    for src, exe in PROBES:
        ptmp = exe + ".tmp"
        r = subprocess.run([HIPCC, *CFLAGS, "-o", ptmp, src], capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError("hipcc failed for %s:\n%s" % (src, r.stderr[-4000:]))
        os.replace(ptmp, exe)
    if verbose:
        print("built", LIB, "from", len(srcs), "sources, and", ", ".join(exe for _, exe in PROBES))
    return LIB


if __name__ == "__main__":
    build()
    sys.exit(0)
