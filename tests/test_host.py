"""Host-side tests (no GPU): the C-ABI library loads, exports what the header
declares, its structs match the C layout, the planner groups each workload as
intended and every argument error is reported with its code."""

from __future__ import annotations

import ctypes
import os
import re
import subprocess
import tempfile

import pytest

import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "muon.h")


@pytest.fixture(scope="module")
def m():
    import muon_newton_schulz_05_amd as pkg
    if not os.path.exists(pkg.LIB_PATH):
        pytest.skip("libmuon.so not built (run __graft_entry__.build())")
    pkg.load_library()
    return pkg


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(muon_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_function(m):
    declared = header_functions()
    assert set(declared) == set(m.EXPORTED)
    lib = ctypes.CDLL(m.LIB_PATH)
    for name in declared:
        assert hasattr(lib, name), name


def test_struct_layout_matches_c(m):
    src = r'''
#include <stddef.h>
#include <stdio.h>
#include "muon.h"
int main(void) {
  printf("%zu %zu %zu %zu\n", sizeof(muon_param_desc_t), sizeof(muon_plan_opts_t),
         sizeof(muon_bucket_info_t), sizeof(muon_plan_info_t));
  printf("%zu %zu %zu %zu\n", offsetof(muon_param_desc_t, shape), offsetof(muon_plan_opts_t, workspace_limit),
         offsetof(muon_plan_opts_t, n_cu), offsetof(muon_plan_info_t, buckets));
  printf("%zu %zu\n", offsetof(muon_bucket_info_t, workspace_bytes), offsetof(muon_plan_info_t, launches_per_ns));
  printf("%zu %zu %zu %zu\n", offsetof(muon_plan_opts_t, nesterov), offsetof(muon_plan_opts_t, update_scale),
         offsetof(muon_plan_opts_t, weight_decay), offsetof(muon_plan_opts_t, large_min_m));
  return 0;
}
'''
    with tempfile.TemporaryDirectory() as d:
        c = os.path.join(d, "t.c")
        exe = os.path.join(d, "t")
        open(c, "w").write(src)
        subprocess.run(["gcc", "-std=c99", "-I", os.path.join(ROOT, "include"), c, "-o", exe], check=True)
        vals = [int(x) for x in subprocess.run([exe], capture_output=True, text=True, check=True).stdout.split()]
    from muon_newton_schulz_05_amd import binding as b
    got = [ctypes.sizeof(b.ParamDesc), ctypes.sizeof(b.PlanOpts), ctypes.sizeof(b.BucketInfo),
           ctypes.sizeof(b.PlanInfo), b.ParamDesc.shape.offset, b.PlanOpts.workspace_limit.offset,
           b.PlanOpts.n_cu.offset, b.PlanInfo.buckets.offset, b.BucketInfo.workspace_bytes.offset,
           b.PlanInfo.launches_per_ns.offset, b.PlanOpts.nesterov.offset, b.PlanOpts.update_scale.offset,
           b.PlanOpts.weight_decay.offset, b.PlanOpts.large_min_m.offset]
    assert got == vals


def describe(m, wl, **opts):
    d = m.make_descs([p.shape for p in wl.params], [p.param_dtype for p in wl.params],
                     [p.grad_dtype for p in wl.params])
    opts.setdefault("mode", wl.mode)
    return m.info_dict(m.muon_plan_describe(d, m.make_opts(**opts)))


def bucket_keys(info):
    return [(b["m"], b["n"], b["count"], b["n_transposed"], b["path"]) for b in info["buckets"]]


def test_plans_of_the_workloads(m):
    W = workloads.WORKLOADS
    assert bucket_keys(describe(m, W["single_128x256"])) == [(128, 256, 1, 0, "stream")]
    info = describe(m, W["fused_74x24x10240"])
    assert bucket_keys(info) == [(24, 10240, 74, 0, "skinny")]
    assert info["buckets"][0]["chunks"] == 40
    assert info["launches_fixed"] == 3 and info["launches_per_ns"] == 0   # three kernels (eager: no prologue)
    assert bucket_keys(describe(m, W["moe_experts"])) == [(24, 10240, 32, 0, "skinny"),
                                                          (1408, 2048, 64, 0, "stream")]
    info = describe(m, W["dense_h4096_l8"])
    assert bucket_keys(info) == [(4096, 12288, 8, 0, "stream"), (4096, 4096, 8, 0, "stream"),
                                 (4096, 16384, 16, 8, "stream")]
    assert info["launches_fixed"] == 3 * 2 and info["launches_per_ns"] == 3   # phases grouped over the buckets
    assert bucket_keys(describe(m, W["large_share"])) == [(8192, 8192, 4, 0, "stream"),
                                                          (4096, 16384, 4, 4, "stream")]
    assert describe(m, W["large_share"])["n_matrices"] == 8


def test_graph_plans_count_the_scalar_prologue(m):
    """Eager steps let the first kernel write the step's scalars; a graph
    replay needs one extra kernel ahead of the graph for them."""
    W = workloads.WORKLOADS
    eager = describe(m, W["fused_74x24x10240"])
    graph = describe(m, W["fused_74x24x10240"], use_graph=True)
    assert graph["launches_fixed"] == eager["launches_fixed"] + 1


def test_large_bucket_workspace_is_padded_to_the_big_tile(m):
    """bf16 buckets with m >= 129 are padded to 256 (1408 -> 1536); their
    workspace holds X and X^T twice, A (float32), E and R (bf16), the
    diagonal and the two tile tables."""
    d = m.make_descs([(1408, 2048)], ["f32"], ["bf16"])
    big = m.info_dict(m.muon_plan_describe(d, m.make_opts(mode="bf16")))["buckets"][0]["workspace_bytes"]
    mp, np_ = 1536, 2048
    assert big >= 4 * mp * np_ * 2 + mp * mp * (4 + 2 + 2) + mp * 4
    small = m.info_dict(m.muon_plan_describe(d, m.make_opts(mode="fp32")))["buckets"][0]["workspace_bytes"]
    assert small >= 4 * 1408 * 2048 * 4 + 1408 * 1408 * (4 + 4)


def test_chunks_depend_on_shape_not_batch(m):
    """A slice's work split must not depend on the batch size (bitwise fusion)."""
    one = m.info_dict(m.muon_plan_describe(m.make_descs([(24, 10240)], ["f32"], ["bf16"]), m.make_opts()))
    many = m.info_dict(m.muon_plan_describe(m.make_descs([(24, 10240)] * 200, ["f32"] * 200, ["bf16"] * 200),
                                            m.make_opts()))
    assert one["buckets"][0]["chunks"] == many["buckets"][0]["chunks"] == 40
    fp32 = describe(m, workloads.WORKLOADS["fused_74x24x10240"], mode="fp32")
    assert fp32["buckets"][0]["chunks"] == 40 and fp32["buckets"][0]["path"] == "skinny"


def test_large_shape_groups_split_into_buckets_the_grid_can_index(m):
    """Launches index a bucket's slices in a grid dimension of at most 65535
    entries, so 70000 slices of one shape become two buckets."""
    info = m.info_dict(m.muon_plan_describe(m.make_descs([(70000, 8, 16)], ["f32"], ["bf16"]), m.make_opts()))
    assert bucket_keys(info) == [(8, 16, 65535, 0, "skinny"), (8, 16, 70000 - 65535, 0, "skinny")]
    assert info["n_matrices"] == 70000


def test_skinny_buckets_share_three_launches(m):
    """Every skinny shape of a plan runs in the same three launches."""
    shapes = [(24, 10240), (16, 4096), (4, 32, 700), (100, 8), (24, 10240)]
    d = m.make_descs(shapes, ["f32"] * 5, ["bf16"] * 5)
    info = m.info_dict(m.muon_plan_describe(d, m.make_opts()))
    assert [b["path"] for b in info["buckets"]] == ["skinny"] * 4
    assert info["launches_fixed"] == 3 and info["launches_per_ns"] == 0


def test_streamed_groups_share_three_launches_per_round(m):
    """The streamed buckets run their rounds in groups, three launches per
    round each: the small buckets (padded m <= 256), the other buckets that
    do not take the large tiles, and the large-tile buckets (bf16 mode,
    m >= 129 by default)."""
    shapes = [(100, 300), (200, 150), (64, 64), (3, 40, 500), (256, 1000)]
    d = m.make_descs(shapes, ["f32"] * 5, ["bf16"] * 5)
    for mode, launches in (("bf16", 3 + 3), ("fp32", 3)):
        info = m.info_dict(m.muon_plan_describe(d, m.make_opts(mode=mode)))
        assert [b["path"] for b in info["buckets"]] == ["stream"] * 5
        assert info["launches_per_ns"] == launches, mode
    small = m.make_descs([(100, 300), (64, 64), (3, 40, 500), (128, 4000)], ["f32"] * 4, ["bf16"] * 4)
    assert m.info_dict(m.muon_plan_describe(small, m.make_opts(mode="bf16")))["launches_per_ns"] == 3
    mixed = m.make_descs(shapes + [(300, 520), (600, 700), (1000, 1100)], ["f32"] * 8, ["bf16"] * 8)
    info = m.info_dict(m.muon_plan_describe(mixed, m.make_opts(mode="bf16")))
    assert info["launches_per_ns"] == 3 + 3 and info["launches_fixed"] == 2 * 8
    assert m.info_dict(m.muon_plan_describe(mixed, m.make_opts(mode="fp32")))["launches_per_ns"] == 3 + 3
    # large_min_m moves the threshold (-1: no large tiles)
    off = m.info_dict(m.muon_plan_describe(mixed, m.make_opts(mode="bf16", large_min_m=-1)))
    assert off["launches_per_ns"] == 3 + 3
    high = m.info_dict(m.muon_plan_describe(mixed, m.make_opts(mode="bf16", large_min_m=301)))
    assert high["launches_per_ns"] == 3 + 3 + 3   # small group, [300,520] in the other group, the rest large
    low = m.info_dict(m.muon_plan_describe(small, m.make_opts(mode="bf16", large_min_m=65)))
    assert low["launches_per_ns"] == 3 + 3        # m = 64 and 40 stay small; m = 100 and 128 go large
    assert m.info_dict(m.muon_plan_describe(small, m.make_opts(mode="bf16", large_min_m=33)))["launches_per_ns"] == 3


def test_skinny_path_can_be_disabled(m):
    info = describe(m, workloads.WORKLOADS["fused_74x24x10240"], skinny_max_m=-1)
    assert info["buckets"][0]["path"] == "stream"


def test_3d_slices_and_orientation(m):
    d = m.make_descs([(3, 50, 20), (20, 50), (50, 20)], ["f32"] * 3, ["f32"] * 3)
    info = m.info_dict(m.muon_plan_describe(d, m.make_opts(skinny_max_m=-1)))
    assert info["n_matrices"] == 5
    assert bucket_keys(info) == [(20, 50, 5, 4, "stream")]


def expect_error(m, code, shapes, pd=None, gd=None, **opts):
    d = m.make_descs(shapes, pd or ["f32"] * len(shapes), gd or ["f32"] * len(shapes))
    with pytest.raises(m.MuonError) as ei:
        m.muon_plan_describe(d, m.make_opts(**opts))
    assert ei.value.code == code, m.muon_last_error()
    assert m.muon_last_error()


def test_argument_errors(m):
    INV, UNS, OOM = 1, 2, 4
    expect_error(m, INV, [(5,)])
    expect_error(m, INV, [(2, 2, 2, 2)])
    expect_error(m, INV, [(0, 4)])
    expect_error(m, INV, [(4, -1)])
    expect_error(m, INV, [(1 << 31, 2)])
    expect_error(m, INV, [(4, 4)], pd=[7])
    expect_error(m, INV, [(4, 4)], gd=[9])
    expect_error(m, INV, [(4, 4)], mode=5)
    expect_error(m, INV, [(4, 4)], eps=-1.0)
    expect_error(m, INV, [(4, 4)], eps=float("nan"))
    expect_error(m, INV, [(4, 4)], max_ns_steps=-2)
    expect_error(m, INV, [(4, 4)], skinny_max_m=33)
    expect_error(m, INV, [(4, 4)], large_min_m=32)
    expect_error(m, INV, [(4, 4)], large_min_m=-2)
    expect_error(m, INV, [(4, 4)], nesterov=2)
    expect_error(m, INV, [(4, 4)], update_scale=3)
    expect_error(m, INV, [(4, 4)], weight_decay=-0.1)
    expect_error(m, INV, [(4, 4)], weight_decay=float("inf"))
    expect_error(m, OOM, [(256, 256)], workspace_limit=1024)
    expect_error(m, UNS, [(40 + i, 100) for i in range(65)])


def test_zero_params_and_null_pointers(m):
    lib = m.load_library()
    info = m.PlanInfo()
    assert lib.muon_plan_describe(m.make_descs([(4, 4)]), 0, None, ctypes.byref(info)) == 1
    assert lib.muon_plan_describe(None, 1, None, ctypes.byref(info)) == 1
    assert lib.muon_plan_describe(m.make_descs([(4, 4)]), 1, None, None) == 1


def test_create_validates_before_touching_the_device(m):
    lib = m.load_library()
    h = ctypes.c_void_p()
    d = m.make_descs([(2, 2, 2, 2)])
    assert lib.muon_plan_create(d, 1, None, ctypes.byref(h)) == 1
    assert not h.value
    assert lib.muon_plan_create(d, 1, None, None) == 1


def test_invalid_handles(m):
    lib = m.load_library()
    P = ctypes.c_void_p * 1
    assert lib.muon_plan_destroy(None) == 0
    assert lib.muon_step(None, P(1), P(1), P(1), 0.1, 0.9, 5, 1.0, 0.0, 0.0, None) == 1
    assert lib.muon_plan_query(None, ctypes.byref(m.PlanInfo())) == 1
    bogus = ctypes.create_string_buffer(64)
    assert lib.muon_step(ctypes.cast(bogus, ctypes.c_void_p), P(1), P(1), P(1), 0.1, 0.9, 5, 1.0, 0.0, 0.0,
                         None) == 1
    assert lib.muon_plan_status(None, None) == 1


def test_default_opts(m):
    o = m.muon_default_opts()
    assert o.mode == m.MUON_MODE_BF16_MFMA and abs(o.eps - 1e-7) < 1e-12 and o.max_ns_steps == 16
    assert o.use_graph == 0 and o.timing == 0 and o.workspace_limit == 0


def test_workspace_grows_with_batch(m):
    a = m.info_dict(m.muon_plan_describe(m.make_descs([(100, 300)] * 2), None))
    b = m.info_dict(m.muon_plan_describe(m.make_descs([(100, 300)] * 4), None))
    assert b["workspace_bytes"] > a["workspace_bytes"]


TABLE_HARNESS = r"""
#include <cstdio>
#include <vector>
#include "planner.h"
int main(int argc, char** argv) {
  // argv: mode, then triples rows cols count (2-D or stacked 3-D shapes)
  std::vector<muon_param_desc_t> d;
  for (int i = 2; i + 2 < argc; i += 3) {
    muon_param_desc_t x{};
    long e = std::atol(argv[i + 2]);
    x.ndim = e > 1 ? 3 : 2;
    x.param_dtype = MUON_F32;
    x.grad_dtype = MUON_BF16;
    if (e > 1) { x.shape[0] = e; x.shape[1] = std::atol(argv[i]); x.shape[2] = std::atol(argv[i + 1]); }
    else { x.shape[0] = std::atol(argv[i]); x.shape[1] = std::atol(argv[i + 1]); }
    d.push_back(x);
  }
  muon_plan_opts_t o;
  muon::default_opts(&o);
  o.mode = (muon_mode_t)std::atoi(argv[1]);
  muon::Plan p;
  std::string err;
  if (muon::make_plan(d.data(), (int)d.size(), &o, 256, &p, &err) != 0) { std::printf("ERR %s\n", err.c_str()); return 1; }
  std::printf("big %zu\n", p.big.size());
  for (size_t i = 0; i < p.big.size(); ++i) {
    const auto& b = p.buckets[p.big[i]];
    std::printf("bucket %zu %lld %lld %lld %lld %zu\n", i, (long long)b.m, (long long)b.n, (long long)b.mp,
                (long long)b.np, b.slices.size());
  }
  for (int ph = 0; ph < 3; ++ph) {
    std::printf("table %d %zu\n", ph, p.big_tab[ph].size());
    for (auto& t : p.big_tab[ph]) std::printf("%u %u\n", t.bz, t.mn);
  }
  return 0;
}
"""


def _tables(shapes):
    """Run the planner (compiled from source with g++) on large bf16 shapes and
    return its buckets and the three tile tables."""
    import tempfile
    src = os.path.join(ROOT, "muon_newton_schulz_05_amd", "csrc")
    with tempfile.TemporaryDirectory() as d:
        c = os.path.join(d, "t.cpp")
        exe = os.path.join(d, "t")
        open(c, "w").write(TABLE_HARNESS)
        subprocess.run(["g++", "-std=c++17", "-O1", "-I", src, c, os.path.join(src, "planner.cpp"), "-o", exe],
                       check=True)
        args = [exe, "1"] + [str(v) for s in shapes for v in s]
        out = subprocess.run(args, capture_output=True, text=True, check=True).stdout.split("\n")
    buckets, tables, k = [], [], 0
    nb = int(out[0].split()[1])
    for i in range(nb):
        f = out[1 + i].split()
        buckets.append(tuple(int(x) for x in f[2:]))
    k = 1 + nb
    for _ in range(3):
        n = int(out[k].split()[2])
        tables.append([tuple(int(x) for x in out[k + 1 + j].split()) for j in range(n)])
        k += 1 + n
    return buckets, tables


def test_large_tile_tables_cover_every_tile_once():
    """Each phase's table lists every output tile of every large slice exactly
    once (upper triangle for X X^T and E E), pads only with the empty marker,
    has a length that is a multiple of 8, and its 8 XCD stretches carry work
    within one block of each other.  Work is counted as the kernel spends it:
    the contraction length per tile, half of it for the symmetric phases'
    half tiles (the last tile row of a slice with at most 128 rows inside m;
    on such a slice the kernel takes the table's column index as the row)."""
    shapes = [(4096, 12288, 2), (4096, 4096, 3), (16384, 4096, 1), (1408, 2048, 5), (600, 700, 1)]
    buckets, tables = _tables(shapes)
    assert [b[:2] for b in buckets] == [(4096, 12288), (4096, 4096), (4096, 16384), (1408, 2048), (600, 700)]
    no_tile = 0xFFFFFFFF
    for ph, tab in enumerate(tables):
        assert len(tab) % 8 == 0
        seen = set()
        for bz, mn in tab:
            if bz == no_tile:
                continue
            key = (bz >> 24, bz & 0xFFFFFF, mn & 0xFFFF, mn >> 16)
            assert key not in seen
            seen.add(key)
        want = set()
        for bi, (m, n, mp, np_, cnt) in enumerate(buckets):
            assert mp % 256 == 0 and np_ % 256 == 0 and mp >= m and np_ >= n
            tm, tn = mp // 256, (np_ // 256 if ph == 2 else mp // 256)
            for z in range(cnt):
                for i in range(tm):
                    for j in range(tn):
                        if ph == 2 or j >= i:
                            want.add((bi, z, i, j))
        assert seen == want
        # work per XCD stretch
        def half(bucket, j):
            m, n, mp, np_, cnt = bucket
            return ph != 2 and j == mp // 256 - 1 and m - (mp - 256) <= 128
        L = len(tab) // 8
        work = []
        for x in range(8):
            w = 0
            for bz, mn in tab[x * L:(x + 1) * L]:
                if bz != no_tile:
                    bk = buckets[bz >> 24]
                    k = bk[3] if ph == 0 else bk[2]
                    w += k // 2 if half(bk, mn >> 16) else k
            work.append(w)
        if ph != 2:  # [1408,2048]: the 6 tiles of the last tile row of each of its 5 slices are half tiles
            n_half = sum(1 for bz, mn in tab if bz != no_tile and half(buckets[bz >> 24], mn >> 16))
            assert n_half == 5 * 6 + 1 * 3  # and the 3 of [600,700]'s last row
        biggest_block = 32 * max((b[3] if ph == 0 else b[2]) for b in buckets)
        assert max(work) - min(work) <= biggest_block


def test_overlong_slices_leave_the_large_tile_products(m):
    """The large-tile products address a 256-row operand panel with 32-bit
    lane offsets (255 rows of n bf16 must stay below 2^32 bytes), so a slice
    whose padded n exceeds 2^23 takes the general products; its neighbours
    keep the large tiles."""
    buckets, tables = _tables([(600, 9_000_000, 1), (600, 700, 1)])
    assert [b[:2] for b in buckets] == [(600, 700)]
    d = m.make_descs([(600, 9_000_000), (600, 700)], ["f32"] * 2, ["bf16"] * 2)
    info = m.info_dict(m.muon_plan_describe(d, m.make_opts(mode="bf16")))
    assert info["launches_per_ns"] == 3 + 3  # its own three launches + the grouped large launches
    buckets, _ = _tables([(600, (1 << 23) - 256, 1)])
    assert [b[:2] for b in buckets] == [(600, (1 << 23) - 256)]


def test_noalloc_checks_on_the_host_before_any_device_call(m):
    """muon_step_noalloc refuses a step larger than its fixed scratch, and the
    options that need a plan, before touching any device (so this runs
    without a GPU)."""
    lib = m.load_library()
    P = ctypes.c_void_p * 1
    ptr = P(16)
    big = m.make_descs([(4096, 4096)], ["f32"], ["bf16"])
    assert lib.muon_step_noalloc(big, 1, ctypes.byref(m.make_opts()), ptr, ptr, ptr, 0.02, 0.95, 5,
                                 *workloads.QUINTIC, None, None) == 2
    assert "scratch" in m.muon_last_error()
    small = m.make_descs([(24, 100)], ["f32"], ["bf16"])
    for kw in (dict(use_graph=True), dict(timing=True)):
        assert lib.muon_step_noalloc(small, 1, ctypes.byref(m.make_opts(**kw)), ptr, ptr, ptr, 0.02, 0.95, 5,
                                     *workloads.QUINTIC, None, None) == 1
    assert lib.muon_step_noalloc(m.make_descs([(2, 2, 2, 2)]), 1, None, ptr, ptr, ptr, 0.02, 0.95, 5,
                                 *workloads.QUINTIC, None, None) == 1
    # A step that fits but has a misaligned pointer is refused before any launch.
    bad = P(8)
    assert lib.muon_step_noalloc(small, 1, None, bad, bad, bad, 0.02, 0.95, 5, *workloads.QUINTIC, None,
                                 None) == 1
    assert m.MUON_NOALLOC_SCRATCH_BYTES == 64 << 20
