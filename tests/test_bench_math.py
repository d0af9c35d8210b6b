"""The benchmark's measurement arithmetic (host logic, no GPU): the attention
kernel's algorithmic flops, bytes and launch counts over decode steps, the
absorbed order's HBM bytes, and the traffic figure read from the committed
counter summary, against hand-computed values."""
import os

import pytest

import bench
import synth


def test_recon_flops_bytes_one_loop_count():
    sh = synth.SHAPES["407m"]            # D 1024, n_pre 2
    D = sh.d_model
    t_values = [4097, 4098]
    flops, hbytes, launches = bench.recon_flops_bytes(sh, 576, [0, 1, 2, 3], [8] * 4, t_values)
    # every one of the 10 layers has all 4 lanes active at each step
    assert launches == 2 * 10
    expect = sum(40 * (4.0 * T * D * D + 4.0 * T * D) for T in t_values)
    assert flops == pytest.approx(expect, rel=1e-15)
    assert hbytes == pytest.approx(sum(40 * T * 576 for T in t_values), rel=1e-15)


def test_recon_flops_bytes_per_lane_loops():
    sh = synth.SHAPES["2b"]              # D 2048, n_pre 2
    D = sh.d_model
    loops = [4, 16, 32] * 2              # 6 lanes, layers 0 .. 33
    flops, hbytes, launches = bench.recon_flops_bytes(sh, 1152, None, loops, [2049])
    assert launches == 2 + 32
    # lane-layers: layers 0..5 all 6 lanes, 6..17 four lanes, 18..33 two lanes
    lane_layers = 6 * 6 + 12 * 4 + 16 * 2
    assert lane_layers == sum(2 + L for L in loops)
    assert flops == pytest.approx(lane_layers * (4.0 * 2049 * D * D + 4.0 * 2049 * D), rel=1e-15)
    assert hbytes == pytest.approx(lane_layers * 2049 * 1152, rel=1e-15)


def test_absorbed_roofline_bytes():
    sh = synth.SHAPES["407m"]
    kern_ms = 1.0
    r = bench.absorbed_roofline(sh, [8] * 4, [4097], kern_ms, 576)
    rows = 4 * 10
    abytes = rows * 4097 * 576 + rows * 2 * sh.n_heads * sh.d_model * 4
    assert r["achieved"] == pytest.approx(round(abytes / 1e-3 / 1e9, 1))
    assert r["bound"] == "hbm" and r["peak"] == bench.PEAK_HBM_GBS
    assert r["frac"] == pytest.approx(round(abytes / 1e-3 / 1e9 / bench.PEAK_HBM_GBS, 4))


def test_traffic_summary_read_only_for_current_sources():
    # the committed counter summary is read only while it describes the
    # attention kernel's current sources; otherwise the figure is null
    path = os.path.join(bench.ROOT, "profiles", "recon_attn_407m-int4h-ctx4096-b4_int4_traffic.txt")
    with open(path) as f:
        text = f.read()
    t = bench.load_traffic("407m-int4h-ctx4096-b4", "int4")
    if "kernel_sources_sha256: " + bench.kernel_sources_sha256() in text:
        # at least the algorithmic bytes of a launch (13.6 MB), at most 10x
        assert t is not None and 13637248 < t < 10 * 13637248
    else:
        assert t is None
    assert bench.load_traffic("no-such-workload", "int4") is None
