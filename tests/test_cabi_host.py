"""The C ABI library on the host (no GPU): exports, planning, validation and error paths.

Nothing here launches a kernel; every call either is host-only
(muon_version, muon_workspace_size, muon_describe, muon_last_error) or is
rejected by argument validation before any HIP call is made.
"""
import ctypes
import os
import re
from collections import Counter

import pytest

from muon_newton_schulz_03_amd import _lib, describe, inputs
from muon_newton_schulz_03_amd._lib import MatrixDesc, Options

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        from muon_newton_schulz_03_amd.build import build_library
        build_library()
    return _lib.load()


def header_functions():
    text = open(os.path.join(ROOT, "include", "muon.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(muon_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_symbol(lib):
    names = header_functions()
    assert set(names) == set(_lib.EXPORTS)
    for name in names:
        assert hasattr(lib, name), name


def test_version(lib):
    assert lib.muon_version().decode().startswith("muon-mi355x")


def descs(shapes, ptrs=False, **kw):
    arr = (MatrixDesc * len(shapes))()
    for i, (r, c) in enumerate(shapes):
        d = arr[i]
        d.rows, d.cols, d.ld_w, d.ld_g = r, c, c, c
        d.w_dtype = kw.get("w_dtype", _lib.MUON_DTYPE_F32)
        d.g_dtype = kw.get("g_dtype", _lib.MUON_DTYPE_BF16)
        if ptrs:
            base = 0x100000 * (i + 1)
            d.weight, d.grad, d.momentum = base, base + 0x40000, base + 0x80000
    return arr


def test_workspace_size_model(lib):
    # 768x768 bf16 path with the low bytes of X: X lo + 2 bf16 X + A + B, each 256-aligned, plus tables
    arr = descs([(768, 768)])
    ws = lib.muon_workspace_size(arr, 1, None)
    x = 768 * 768
    assert ws >= x + 2 * x * 2 + 2 * x * 2
    assert ws < x + 4 * x * 2 + (1 << 20)
    # no low bytes: 1 byte per element less
    ws0 = lib.muon_workspace_size(arr, 1, ctypes.byref(Options(0, 0, 0, 0)))
    assert ws - ws0 == x
    # fp32 path: 4-byte operands, no master and no words for B's diagonal (one
    # fp32 per row on the bf16 path); its 128 x 128 tile tables are longer than
    # the bf16 path's 256 x 128 ones (a few 256-byte blocks)
    wsf = lib.muon_workspace_size(arr, 1, ctypes.byref(Options(1, -1, 0, 0)))
    assert 0 <= wsf - (ws0 - 4 * 768) - 4 * x * 2 < 4096
    g = inputs.workload("gpt2_small")
    d, _ = describe(g.shapes)
    assert 0.59e9 < d["workspace_bytes"] < 0.60e9


def expected_tiles(shapes, kind, path="bf16"):
    """Tiles of one launch kind.  fp32 products (short side < 128, or the fp32 path):
    128 x 128 tiles over the upper triangle (A, B) or the whole X.  bf16 products:
    the Gram product takes 128 x 128 tiles on or above the diagonal; the polynomial
    and the update take 256 x 128 tiles (256-row panel a, 128-column panel b), the
    polynomial's with b >= 2a (they reach the upper triangle)."""
    expect = set()
    for i, (r, c) in enumerate(shapes):
        m, n = min(r, c), max(r, c)
        f32 = path == "f32" or m < 128
        mp, np_ = -(-m // (128 if f32 else 256)) * (128 if f32 else 256), -(-n // 128) * 128
        if kind == _lib.KIND_MOMENTUM:
            expect |= {(i, a, b) for a in range(mp // 64) for b in range(np_ // 64)}
        elif f32 and kind == _lib.KIND_UPDATE:
            expect |= {(i, a, b) for a in range(mp // 128) for b in range(np_ // 128)}
        elif f32 or kind == _lib.KIND_GRAM:
            expect |= {(i, a, b) for a in range(mp // 128) for b in range(a, mp // 128)}
        elif kind == _lib.KIND_UPDATE:
            expect |= {(i, a, b) for a in range(mp // 256) for b in range(np_ // 128)}
        else:
            expect |= {(i, a, b) for a in range(mp // 256) for b in range(2 * a, mp // 128)}
    return expect


@pytest.mark.parametrize("shapes", [[(768, 768)], [(4, 8), (8, 4), (1, 1), (257, 129), (130, 1000)],
                                    inputs.workload("gpt2_small").shapes[:12]])
@pytest.mark.parametrize("groups", [0, 1, 3, 4])
def test_tile_lists_cover_each_tile_once(shapes, groups):
    for kind in (_lib.KIND_MOMENTUM, _lib.KIND_GRAM, _lib.KIND_POLY, _lib.KIND_UPDATE):
        info, tiles = describe(shapes, kind=kind, groups=groups)
        real = [t for t in tiles if t[0] >= 0]
        cnt = Counter(real)
        assert all(v == 1 for v in cnt.values())
        assert set(cnt) == expected_tiles(shapes, kind)
        assert info["blocks"][kind] == len(tiles)
        assert info["bf16_tile_rows"] == 256 and info["bf16_tile_cols"] == 128 and info["tile"] == 128


def tile_cost(shapes, kind, tile):
    """Host cost of one bf16 tile in 32-element K slabs: a Gram tile (128 x 128)
    costs its K; a polynomial tile (256 x 128) with b == 2a computes only its upper
    half and counts half."""
    mat, a, b = tile
    r, c = shapes[mat]
    if kind == _lib.KIND_GRAM:
        return max(r, c) // 32
    k = min(r, c) // 32
    return k if kind == _lib.KIND_POLY and b == 2 * a else 2 * k


def test_block_loads_are_balanced():
    # Product launches run 512 blocks; block b takes entries b, b + 512, ...
    # Inside each XCD each tile in turn (longest first) goes to the least-loaded
    # block, so the loads of an XCD's blocks differ by at most one tile.
    g = inputs.workload("gpt2_small")
    grid = 512
    for kind in (_lib.KIND_GRAM, _lib.KIND_POLY, _lib.KIND_UPDATE):
        _, tiles = describe(g.shapes, kind=kind, groups=1)
        load = Counter()
        biggest = 0
        for e, tl in enumerate(tiles):
            if tl[0] < 0:
                continue
            cost = tile_cost(g.shapes, kind, tl)
            load[e % grid] += cost
            biggest = max(biggest, cost)
        for x in range(8):
            per_block = [load[b] for b in range(x, grid, 8)]
            assert max(per_block) - min(per_block) <= biggest
        # every XCD holds the long (K = 3072) Gram tiles as well as the short ones
        if kind == _lib.KIND_GRAM:
            for x in range(8):
                costs = {max(g.shapes[m]) for e, (m, _, _) in enumerate(tiles) if m >= 0 and e % 8 == x}
                assert costs == {768, 3072}


def test_xcd_runs_are_balanced():
    g = inputs.workload("gpt2_small")
    for kind in (_lib.KIND_GRAM, _lib.KIND_POLY, _lib.KIND_UPDATE):
        _, tiles = describe(g.shapes, kind=kind)
        load = Counter()
        biggest = 0
        for b, tl in enumerate(tiles):
            if tl[0] < 0:
                continue
            cost = tile_cost(g.shapes, kind, tl)
            load[b % 8] += cost
            biggest = max(biggest, cost)
        # each launch's table is cut into equal-cost runs at tile granularity:
        # the XCD loads differ by at most one tile per launch (two groups)
        assert max(load.values()) - min(load.values()) <= 2 * biggest
        assert max(load.values()) / min(load.values()) < 1.05
        # each XCD works on a contiguous run of matrices: a matrix spans at most 2 XCDs
        xcds = {}
        for b, (mat, _, _) in enumerate(tiles):
            if mat >= 0:
                xcds.setdefault(mat, set()).add(b % 8)
        assert max(len(v) for v in xcds.values()) <= 2


def test_short_matrices_take_fp32_products():
    d, _ = describe([(4, 8), (127, 1000), (64, 64), (128, 128), (768, 768), (3000, 40)])
    assert d["n_f32_matrices"] == 4
    d, _ = describe([(4, 8), (768, 768)], path="f32")
    assert d["n_f32_matrices"] == 2
    # each precision has its own launch: the lists hold both sets of tiles
    _, tiles = describe([(4, 8), (768, 768)], kind=_lib.KIND_UPDATE)
    assert {t[0] for t in tiles if t[0] >= 0} == {0, 1}


def test_groups_option():
    g = inputs.workload("gpt2_small")
    d, _ = describe(g.shapes)
    assert d["n_groups"] == 2
    d, _ = describe(g.shapes, groups=1)
    assert d["n_groups"] == 1
    d, _ = describe([(768, 768)])
    assert d["n_groups"] == 1  # one matrix: one group
    # both groups of the default plan cover every matrix once, contiguously and by equal cost
    d1, t1 = describe(g.shapes, kind=_lib.KIND_UPDATE, groups=1)
    d2, t2 = describe(g.shapes, kind=_lib.KIND_UPDATE)
    assert sorted(t for t in t1 if t[0] >= 0) == sorted(t for t in t2 if t[0] >= 0)
    # up to 4 groups; more matrices than groups fill all of them, fewer leave some empty
    for ng in (3, 4):
        d, t = describe(g.shapes, kind=_lib.KIND_UPDATE, groups=ng)
        assert d["n_groups"] == ng
        assert sorted(x for x in t if x[0] >= 0) == sorted(x for x in t1 if x[0] >= 0)
    assert describe([(768, 768), (768, 3072)], groups=4)[0]["n_groups"] == 2
    lib = _lib.load()
    arr = descs([(64, 64)])
    info = _lib.PlanInfo()
    rc = lib.muon_describe(arr, 1, ctypes.byref(Options(0, -1, 0, 0, 5)), ctypes.byref(info), -1, None, 0, None)
    assert rc == _lib.MUON_E_INVAL and "groups" in _lib.last_error()


def test_master_iters_option():
    d, _ = describe([(64, 64)], x_master_iters=-1)
    assert d["x_master_iters"] == 3
    d, _ = describe([(64, 64)], x_master_iters=5)
    assert d["x_master_iters"] == 5
    d, _ = describe([(64, 64)], path="f32")
    assert d["x_master_iters"] == 0


def expect_error(code, fn, *args, match=None):
    rc = fn(*args)
    assert rc == code, (rc, _lib.last_error())
    if match:
        assert re.search(match, _lib.last_error()), _lib.last_error()


def test_validation_errors(lib):
    plan = ctypes.c_void_p()
    ws = ctypes.c_void_p(0x10000000)  # never touched: validation fails first
    E = _lib
    expect_error(E.MUON_E_INVAL, lib.muon_init, None, 1, None, ws, 1 << 30, None, ctypes.byref(plan))
    expect_error(E.MUON_E_INVAL, lib.muon_init, descs([(4, 4)], True), 0, None, ws, 1 << 30, None,
                 ctypes.byref(plan), match="count")
    bad = descs([(4, 4)], True)
    bad[0].rows = 0
    expect_error(E.MUON_E_INVAL, lib.muon_init, bad, 1, None, ws, 1 << 30, None, ctypes.byref(plan),
                 match="positive")
    bad = descs([(4, 4)], True)
    bad[0].ld_g = 8
    expect_error(E.MUON_E_UNSUPPORTED, lib.muon_init, bad, 1, None, ws, 1 << 30, None, ctypes.byref(plan),
                 match="ld_g")
    bad = descs([(4, 4)], True, g_dtype=7)
    expect_error(E.MUON_E_UNSUPPORTED, lib.muon_init, bad, 1, None, ws, 1 << 30, None, ctypes.byref(plan))
    bad = descs([(4, 4)], False)
    expect_error(E.MUON_E_INVAL, lib.muon_init, bad, 1, None, ws, 1 << 30, None, ctypes.byref(plan),
                 match="null")
    bad = descs([(4, 4)], True)
    bad[0].grad = bad[0].weight
    expect_error(E.MUON_E_INVAL, lib.muon_init, bad, 1, None, ws, 1 << 30, None, ctypes.byref(plan),
                 match="distinct")
    bad = descs([(4, 4)], True)
    bad[0].scale = float("nan")
    expect_error(E.MUON_E_INVAL, lib.muon_init, bad, 1, None, ws, 1 << 30, None, ctypes.byref(plan))
    bad = descs([(4, 4)], True)
    bad[0].reserved = 1
    expect_error(E.MUON_E_INVAL, lib.muon_init, bad, 1, None, ws, 1 << 30, None, ctypes.byref(plan))
    ok = descs([(4, 4)], True)
    expect_error(E.MUON_E_WORKSPACE, lib.muon_init, ok, 1, None, None, 1 << 30, None, ctypes.byref(plan))
    expect_error(E.MUON_E_WORKSPACE, lib.muon_init, ok, 1, None, ctypes.c_void_p(0x10000010), 1 << 30, None,
                 ctypes.byref(plan), match="aligned")
    expect_error(E.MUON_E_WORKSPACE, lib.muon_init, ok, 1, None, ws, 1024, None, ctypes.byref(plan),
                 match="needs")
    expect_error(E.MUON_E_UNSUPPORTED, lib.muon_init, ok, 1, ctypes.byref(Options(9, 0, 0, 0)), ws, 1 << 30,
                 None, ctypes.byref(plan))
    expect_error(E.MUON_E_INVAL, lib.muon_init, ok, 1, None, ws, 1 << 30, None, None)
    assert not plan.value
    assert lib.muon_workspace_size(bad, 1, None) == 0


def test_size_limits(lib):
    """Sides up to 2^20 and buffers below 2 GiB are accepted (the largest
    shapes the GPU limit tests run); one element more on a side, or a padded
    buffer of 2 GiB, is refused before anything is allocated."""
    for shape in [(128, 1 << 20), (1 << 20, 128), (100, (1 << 20) - 1), (512, 1048447), (1024, 524160),
                  (23040, 23040)]:
        ws = lib.muon_workspace_size(descs([shape]), 1, None)
        assert ws > 0, (shape, _lib.last_error())
    for shape, why in [((128, (1 << 20) + 1), "limit per side"), (((1 << 20) + 1, 1), "limit per side"),
                       ((1024, 524289), "2 GiB"), ((23296, 23296), "2 GiB"), ((512, 1048577), "limit per side")]:
        assert lib.muon_workspace_size(descs([shape]), 1, None) == 0, shape
        assert why in _lib.last_error(), (shape, _lib.last_error())
    # the tile tables index tiles with 16 bits: the longest side's lists still cover every tile
    d, t = describe([(512, 1048447)], kind=_lib.KIND_UPDATE)
    assert len([x for x in t if x[0] >= 0]) == 2 * 8191
    d, t = describe([(512, 1048447)], kind=_lib.KIND_MOMENTUM)
    assert len([x for x in t if x[0] >= 0]) == 8 * 16382


def test_step_and_destroy_on_null_plan(lib):
    expect_error(_lib.MUON_E_INVAL, lib.muon_step, None, None, 0, 1.0, 1.0, 1.0, 5, 0.9, 1, 0.1, None,
                 match="plan")
    coeffs = (ctypes.c_float * 6)(3.4445, -4.775, 2.0315, 3.4445, -4.775, 2.0315)
    expect_error(_lib.MUON_E_INVAL, lib.muon_step_schedule, None, None, 0, coeffs, 2, 0.9, 1, 0.1, None,
                 match="NULL")
    expect_error(_lib.MUON_E_INVAL, lib.muon_step_schedule, None, None, 0, None, 2, 0.9, 1, 0.1, None,
                 match="coeffs is NULL")
    assert lib.muon_destroy(None) == 0
    expect_error(_lib.MUON_E_INVAL, lib.muon_profile_enable, None, 1)
    expect_error(_lib.MUON_E_INVAL, lib.muon_profile_select, None, 1)
    expect_error(_lib.MUON_E_INVAL, lib.muon_profile_read, None, None, None)
    # errors are per thread and cleared by the next successful call
    assert lib.muon_destroy(None) == 0 and _lib.last_error() == ""


def test_binding_rejects_host_tensors():
    import torch
    from muon_newton_schulz_03_amd import MuonStep
    w = torch.zeros(4, 4)
    with pytest.raises(ValueError, match="device"):
        MuonStep([w], [w.clone()], [w.clone()])


def test_init_reports_hip_failures(lib):
    """Where a HIP runtime call fails (here: no device at all), muon_init returns
    MUON_E_HIP, names the call and keeps the runtime's own message."""
    import torch
    if torch.cuda.device_count() > 0:
        pytest.skip("a device is present: this case needs a host without one")
    plan = ctypes.c_void_p()
    ok = descs([(64, 64)], True)
    ws = lib.muon_workspace_size(ok, 1, None)
    expect_error(_lib.MUON_E_HIP, lib.muon_init, ok, 1, None, ctypes.c_void_p(0x10000000), ws, None,
                 ctypes.byref(plan), match=r"^hip\w+\(.*\): .+ \(\d+\)$")
    assert not plan.value
    assert "device" in _lib.last_error()


FUSED_SETS = [
    inputs.workload("gpt2_small").shapes,
    [(300, 700), (700, 300), (129, 4100), (1000, 130), (64, 64), (100, 333), (256, 256), (512, 1536)],
    [(768, 768)],
    [(4, 8), (100, 100)],  # only fp32 products: an empty queue
]


@pytest.mark.parametrize("shapes", FUSED_SETS, ids=["gpt2_small", "mixed", "one", "fp32_only"])
def test_fused_queues(shapes):
    """The fused plan's per-XCD queues: every bf16 matrix's tiles of each
    product exactly once, all on one XCD, each XCD's entries product by
    product (Gram 1, polynomial 2, update 3), every tile inside its matrix (the
    ranges the kernel checks before it runs an entry), no fp32 matrix."""
    d, q = describe(shapes, kind=_lib.KIND_FUSED, fused=True)
    assert d["fused"] == 1 and d["n_groups"] == 1
    assert d["blocks"][_lib.KIND_FUSED] == len(q)
    xcd_of = {}
    per = {}
    last_product = {}
    for x, prod, i, ti, tj in q:
        assert 0 <= x < 8 and prod in (1, 2, 3)
        assert xcd_of.setdefault(i, x) == x, f"matrix {i} on two XCDs"
        assert prod >= last_product.get(x, 1), f"XCD {x}: product {prod} after {last_product[x]}"
        last_product[x] = prod
        per.setdefault((i, prod), []).append((ti, tj))
    kinds = {1: _lib.KIND_GRAM, 2: _lib.KIND_POLY, 3: _lib.KIND_UPDATE}
    for i, (r, c) in enumerate(shapes):
        m, n = min(r, c), max(r, c)
        if m < 128:
            assert i not in xcd_of
            continue
        mp, np_ = -(-m // 256) * 256, -(-n // 128) * 128
        for prod, kind in kinds.items():
            got = per[(i, prod)]
            assert len(got) == len(set(got))
            assert {(0, a, b) for a, b in got} == expected_tiles([(r, c)], kind)  # the staged plan's tiles
            for ti, tj in got:
                if prod == 1:
                    assert ti <= tj < mp // 128
                elif prod == 2:
                    assert 2 * ti <= tj < mp // 128
                else:
                    assert ti < mp // 256 and tj < np_ // 128


def test_fused_queues_balance_gpt2_small():
    """The 72 GPT-2 small matrices spread over the 8 XCDs with equal work
    (3 of 768 x 3072 and 6 of 768 x 768 on each)."""
    shapes = inputs.workload("gpt2_small").shapes
    _, q = describe(shapes, kind=_lib.KIND_FUSED, fused=True)
    mats = {}
    for x, prod, i, ti, tj in q:
        mats.setdefault(x, set()).add(i)
    assert len(mats) == 8
    for x, s in mats.items():
        big = sum(1 for i in s if max(shapes[i]) == 3072)
        assert (big, len(s) - big) == (3, 6), f"XCD {x}: {big} large, {len(s) - big} small"


def test_fused_entry_points_reject_bad_arguments(lib):
    assert lib.muon_check(None, None) == _lib.MUON_E_INVAL
    assert lib.muon_fused_limits(None, 1, 0) == _lib.MUON_E_INVAL
    d, _ = describe([(768, 768)], fused=False)
    assert d["fused"] == 0 and d["blocks"][_lib.KIND_FUSED] == 0
