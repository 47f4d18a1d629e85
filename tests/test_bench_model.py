"""Host logic of bench.py (no GPU): the cost models behind the bench line's
fractions, the kernel-path thresholds it prices by, and its one-GPU rule.

Expected values are worked out by hand from the definitions in the
docstrings of bench.py, not by calling the functions under test again."""

from __future__ import annotations

import os
import subprocess
import sys

import pytest

import bench
import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
W = workloads.WORKLOADS


def test_stream_model_of_the_fused_skinny_workload():
    """74 x [24,10240], bf16 G, float32 W, bf16 X, k = 5: 2 + 8 + 2*4 + 17*2
    = 52 bytes per element, plus k m^2 (8 + 2*2) = 34560 bytes per slice;
    its flops, 74 * 5 * (4 * 576 * 10240 + 2 * 13824), are far below the
    matrix cores' share, so T_roof is the bytes over 8 TB/s."""
    b, t = bench.stream_model(W["fused_74x24x10240"], "bf16")
    expect_b = 74 * (24 * 10240 * 52 + 5 * 576 * 12)
    assert b == pytest.approx(expect_b, rel=1e-12)
    assert t == pytest.approx(expect_b / 8e12, rel=1e-12)
    assert t * 1e6 == pytest.approx(118.5, abs=0.1)


def test_stream_model_of_the_8192_share_is_matrix_core_bound():
    """4 x [8192,8192] and 4 x [16384,4096] (oriented [4096,16384]): each
    bucket's flops over 2.5 PFLOP/s exceed its bytes over 8 TB/s."""
    _, t = bench.stream_model(W["large_share"], "bf16")
    f = 4 * 5 * (4 * 8192.0 ** 3 + 2 * 8192.0 ** 3) + 4 * 5 * (4 * 4096.0 ** 2 * 16384 + 2 * 4096.0 ** 3)
    assert t == pytest.approx(f / 2.5e15, rel=1e-12)
    assert t * 1e3 == pytest.approx(36.3, abs=0.05)


def test_stream_model_fp32_uses_four_byte_x_and_the_fp32_peak():
    """[128,256], float32 G and W, fp32 mode: 4 + 8 + 8 + 17*4 = 88 bytes
    per element plus 5 * 128^2 * 16; flops over 157.3 TFLOP/s."""
    b, t = bench.stream_model(W["single_128x256"], "fp32")
    expect_b = 128 * 256 * 88 + 5 * 128 * 128 * 16
    assert b == pytest.approx(expect_b, rel=1e-12)
    f = 5 * (4.0 * 128 * 128 * 256 + 2.0 * 128 ** 3)
    assert t == pytest.approx(max(f / 157.3e12, expect_b / 8e12), rel=1e-12)


def test_own_work_counts_each_symmetric_product_once_on_the_large_tiles():
    """A [4096,4096] slice on the large tiles: Gram m(m+1)n and A^2 m^2(m+1)
    per round, apply 2 m^2 n; the same slice in fp32 mode takes the tiled
    products, full squares."""
    wl = workloads.Workload(99, "one_4096", (workloads.ParamSpec((4096, 4096)),), grad_std=1e-3, mode="bf16")
    m = n = 4096
    total, cls = bench.own_work_flops(wl, "bf16")
    assert cls["gram"] == 5 * m * (m + 1) * n and cls["poly"] == 5 * m * m * (m + 1)
    assert cls["apply"] == 5 * 2 * m * m * n
    total32, cls32 = bench.own_work_flops(wl, "fp32")
    assert cls32["gram"] == 5 * 2 * m * m * n and cls32["poly"] == 5 * 2 * m ** 3
    assert total32 == wl.flops() and total < total32


def test_own_work_of_the_skinny_path_is_the_gram_space_count():
    """[24,10240]: one Gram m(m+1)n, per round A^2 and P^2 (m^2(m+1) each)
    and two m^3 products (2 m^3 each), one apply 2 m^2 n."""
    wl = workloads.Workload(98, "one_skinny", (workloads.ParamSpec((24, 10240)),), grad_std=1e-3, mode="bf16")
    _, cls = bench.own_work_flops(wl, "bf16")
    assert cls["skinny_gram"] == 24 * 25 * 10240
    assert cls["skinny_poly"] == 5 * (2 * 576 * 25 + 4 * 24 ** 3)
    assert cls["skinny_apply"] == 2 * 576 * 10240


@pytest.mark.parametrize("m,mode,path", [(1, "bf16", "skinny"), (32, "fp32", "skinny"), (33, "bf16", "stream"),
                                         (128, "bf16", "stream"), (129, "bf16", "large"), (129, "fp32", "stream"),
                                         (8192, "bf16", "large"), (8192, "fp32", "stream")])
def test_paths_follow_the_planner_thresholds(m, mode, path):
    assert bench.path_of(m, mode) == path


def test_paths_agree_with_the_planner():
    """bench.path_of prices each slice by the path the planner gives it:
    compare with muon_plan_describe on shapes around the thresholds."""
    import muon_newton_schulz_05_amd as pkg
    if not os.path.exists(pkg.LIB_PATH):
        pytest.skip("libmuon.so not built")
    shapes = [(24, 300), (32, 300), (33, 300), (128, 300), (129, 300), (600, 700)]
    for mode in ("bf16", "fp32"):
        d = pkg.make_descs(shapes, ["f32"] * len(shapes), ["bf16"] * len(shapes))
        info = pkg.info_dict(pkg.muon_plan_describe(d, pkg.make_opts(mode=mode)))
        planner = {b["m"]: b["path"] for b in info["buckets"]}
        for m, _ in shapes:
            p = bench.path_of(m, mode)
            assert planner[m] == ("skinny" if p == "skinny" else "stream"), (m, mode)
        launches = info["launches_per_ns"]
        groups = {bench.path_of(m, mode) for m, _ in shapes} - {"skinny"}
        small_or_tiled = {("small" if m <= 256 else "tiled") for m, _ in shapes
                          if bench.path_of(m, mode) == "stream"}
        assert launches == 3 * (len(small_or_tiled) + ("large" in groups))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, cwd=ROOT, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stdout
