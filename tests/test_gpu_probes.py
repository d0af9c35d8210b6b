"""GPU checks of the two reference programs the benchmark's rooflines are read
against: the streaming-read probe (bytes a kernel that only reads moves per
second) and the MFMA-rate probe (fp16 flops MFMAs alone sustain, and the
shader clock). Each runs as a child process, as in bench.py; the checks are
on the shape and plausibility of what they report, not on speed."""
import json
import os
import subprocess

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PROBE = os.path.join(ROOT, "kv_compression_amd", "probe")


def _run(name, *args):
    exe = os.path.join(PROBE, name)
    assert os.path.exists(exe), "%s not built (python -m kv_compression_amd.build)" % exe
    r = subprocess.run([exe, *map(str, args)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr[-2000:]
    return [json.loads(line) for line in r.stdout.splitlines() if line.startswith("{")]


def test_mfma_rate_probe():
    (res,) = _run("mfma_rate", 2000)
    assert res["cus"] > 0 and res["workgroups"] == 2 * res["cus"] and res["iters"] == 2000
    assert res["us_per_launch"] > 0
    # flops of the launch over its time, and a shader clock within what a GPU runs at
    flops = res["workgroups"] * 4 * res["iters"] * 8 * 32 * 32 * 16 * 2
    assert res["tflops"] == pytest.approx(flops / (res["us_per_launch"] * 1e-6) / 1e12, rel=2e-3)
    assert 0.3 < res["shader_ghz"] < 3.5
    assert res["wall_clock_khz"] > 0


def test_mfma_rate_refuses_bad_count():
    r = subprocess.run([os.path.join(PROBE, "mfma_rate"), "0"], capture_output=True, text=True, timeout=60)
    assert r.returncode == 2


def test_hbm_read_probe():
    res = _run("hbm_read", 8, 64)
    assert [x["bytes"] for x in res] == [8 << 20, 64 << 20]
    for x in res:
        assert x["us_single"] > 0 and x["us_back_to_back"] > 0
        for k in ("single", "back_to_back"):
            assert x["GBs_" + k] == pytest.approx(x["bytes"] / (x["us_" + k] * 1e-6) / 1e9, rel=1e-2)
