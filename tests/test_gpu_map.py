"""GPU kernel map vs the CPU oracle: bit-exact neighbour table, masks, mask
order, pair lists and per-tap offsets, on every workload and on edge sets."""
import numpy as np
import pytest

import synth
from _util import assert_map_equal, config, oracle_map, oracle_map_of, to_dev_i32

pytestmark = pytest.mark.gpu

smc = pytest.importorskip("submanifold_sparse_convolution_amd")


def auto_route(grid, pad=1):
    """The route the library picks for a fresh handle: dense when the padded
    grid's int32 ids and two occupancy bitmaps (4.25 bytes a cell) fit 1/16 of
    the device's memory, at most 16 GiB, and half the memory free now."""
    import torch
    # tall grids (Z + 2 pad >= 256) in whole bricks of 8 x 8 x 16 cells
    if grid[2] + 2 * pad >= 256:
        cells = float(np.prod([-(-(g + 2 * pad) // d) * d for g, d in zip(grid, (8, 8, 16))]))
    else:
        cells = float(np.prod([g + 2 * pad for g in grid]))
    budget = min(16 << 30, torch.cuda.get_device_properties(0).total_memory // 16)
    budget = min(budget, torch.cuda.mem_get_info()[0] / 2)
    return "dense" if cells * 4.25 <= budget and cells < 2.0 ** 36 else "sorted"


def gpu_map(coords, route="auto", spatial_shape=None, batch_size=0, ncols=4):
    c = coords if ncols == 4 else coords[:, 1:]
    m = smc.KernelMap().build(to_dev_i32(c), spatial_shape=spatial_shape, batch_size=batch_size,
                              route=route)
    out = m.export()
    out["info"] = m.info()
    m.close()
    return out


@pytest.mark.parametrize("name", ["tiny", "lidar", "deep", "wide", "stage"])
def test_workload_map_bit_exact(name):
    w, coords = config(name)
    print(f"map parity {name} n={len(coords)}", flush=True)
    got = gpu_map(coords, spatial_shape=w.grid)
    assert_map_equal(got, oracle_map(name), name)
    info = got["info"]
    assert info["pairs"] == len(oracle_map(name)["pair_in"])
    assert info["route"] == auto_route(w.grid)
    assert info["pairs_padded"] % info["tile_m"] == 0


@pytest.mark.parametrize("name", ["tiny", "lidar", "deep", "wide"])
def test_dense_equals_sorted(name):
    w, coords = config(name)
    a = gpu_map(coords, route="dense", spatial_shape=w.grid)
    b = gpu_map(coords, route="sorted", spatial_shape=w.grid)
    assert a["info"]["route"] == "dense" and b["info"]["route"] == "sorted"
    assert b["info"]["key_bits"] <= 32          # 32-bit key path
    assert_map_equal(a, b, name)


def test_sorted_derived_shape_32bit_keys():
    """Keys are cells of the padded grid: the wide set's box (2095 x 2095 x 695 at
    most, 2 cells of padding per axis) needs 32 bits, not the 34 of bit fields."""
    _, coords = config("wide")
    got = gpu_map(coords, route="sorted")      # bounding box derived on the device
    ext = coords[:, 1:].max(0) - coords[:, 1:].min(0) + 1
    cells = int(np.prod(ext.astype(np.int64) + 2))
    assert got["info"]["route"] == "sorted"
    assert got["info"]["key_bits"] == (cells - 1).bit_length() <= 32
    assert_map_equal(got, oracle_map("wide"), "wide/derived")


def test_sorted_64bit_keys():
    """A padded grid of more than 2^32 cells: 64-bit keys."""
    rng = np.random.default_rng(5)
    parts = []
    for i, off in enumerate([(0, 0, 0), (4000, 0, 0), (0, 4000, 9), (4000, 4000, 1000)]):
        c = synth.tiny_coords(seed=5 + i, n=700, side=12)       # dense clusters, far apart
        c[:, 1:] += np.array(off, np.int32)
        parts.append(c)
    coords = np.concatenate(parts)
    coords = coords[rng.permutation(len(coords))].astype(np.int32)
    got = gpu_map(coords)
    assert got["info"]["route"] == "sorted" and got["info"]["key_bits"] > 32
    assert_map_equal(got, oracle_map_of(coords), "64-bit keys")


def test_derived_shape_dense():
    _, coords = config("deep")
    got = gpu_map(coords, route="dense")
    assert_map_equal(got, oracle_map("deep"), "deep/derived")


@pytest.mark.parametrize("n", [1, 7, 16, 17, 63, 64, 65, 255, 256, 257, 4097])
@pytest.mark.parametrize("route", ["dense", "sorted"])
def test_small_and_ragged(n, route):
    coords = synth.tiny_coords(seed=n, n=n, side=max(3, int(round((4 * n) ** (1 / 3)))))
    got = gpu_map(coords, route=route, spatial_shape=None)
    assert_map_equal(got, oracle_map_of(coords), f"n={n} {route}")


@pytest.mark.parametrize("route", ["dense", "sorted"])
def test_full_boxes(route):
    for abc in [(3, 3, 3), (1, 1, 1), (5, 4, 3), (1, 1, 40), (17, 9, 5)]:
        coords = synth.box_coords(*abc, origin=(2, 3, 4), seed=sum(abc))
        got = gpu_map(coords, route=route, spatial_shape=(30, 30, 50))
        want = oracle_map_of(coords)
        assert_map_equal(got, want, f"box {abc} {route}")
        a, b, c = abc
        assert got["info"]["pairs"] == (3 * a - 2) * (3 * b - 2) * (3 * c - 2)


@pytest.mark.parametrize("route", ["dense", "sorted"])
def test_isolated_voxels(route):
    coords = synth.isolated_coords(3000, spacing=2, seed=4)
    got = gpu_map(coords, route=route)
    assert (got["mask"] == (1 << 13)).all()
    assert_map_equal(got, oracle_map_of(coords), "isolated")


@pytest.mark.parametrize("route", ["dense", "sorted"])
def test_two_batches(route):
    a = synth.tiny_coords(seed=5, n=900, side=12)
    b = synth.tiny_coords(seed=6, n=700, side=12)
    b[:, 0] = 1
    coords = np.concatenate([a, b])
    coords = coords[np.random.default_rng(0).permutation(len(coords))]
    want = oracle_map_of(coords)
    assert_map_equal(gpu_map(coords, route=route, spatial_shape=(12, 12, 12), batch_size=2),
                     want, "batches explicit")
    assert_map_equal(gpu_map(coords, route=route), want, "batches derived")


def test_three_column_coords():
    _, coords = config("tiny")
    got = gpu_map(coords, ncols=3, spatial_shape=(24, 24, 24))
    assert_map_equal(got, oracle_map("tiny"), "ncols=3")


def test_empty_map():
    import torch
    m = smc.KernelMap().build(torch.zeros((0, 4), dtype=torch.int32, device="cuda"),
                              spatial_shape=(4, 4, 4))
    info = m.info()
    assert info["n"] == 0 and info["pairs"] == 0
    x = torch.zeros((0, 16), dtype=torch.bfloat16, device="cuda")
    w = torch.zeros((27, 16, 16), dtype=torch.bfloat16, device="cuda")
    y = m.forward(x, smc.pack_weights(w))
    assert tuple(y.shape) == (0, 16)


@pytest.mark.parametrize("pairs,sort", [(True, True), (True, False), (False, True), (False, False)])
def test_rebuild_reuses_handle_and_keeps_grid_clean(pairs, sort):
    """One handle, several builds of different sets: each must match. Whichever
    pass ends the build (compaction, mask histogram) must leave the dense grid
    empty for the next build."""
    m = smc.KernelMap()
    for seed in (1, 2, 3):
        coords = synth.ground_box_coords(3000, (200, 200, 12), seed=seed, n_boxes=20)
        print(f"rebuild seed {seed} pairs={pairs} sort={sort}", flush=True)
        m.build(to_dev_i32(coords), spatial_shape=(200, 200, 12), pairs=pairs, sort=sort)
        got = m.export(pairs=pairs, perm=sort)
        assert_map_equal(got, oracle_map_of(coords), f"rebuild {seed}")
        assert m.info()["pairs"] == int(oracle_map_of(coords)["tap_off"][-1])
    m.close()


def test_route_switches_and_sizes_on_one_handle():
    """Dense builds alternate between two presence grids and clear the previous
    build's cells; a sorted build in between clears them too. Every build on one
    handle must still match the oracle, whatever the order of routes and sizes."""
    m = smc.KernelMap()
    plan = [("dense", 3000, 1), ("dense", 500, 2), ("sorted", 2000, 3), ("dense", 4000, 4),
            ("dense", 100, 5), ("dense", 4000, 4), ("sorted", 700, 6), ("sorted", 900, 7),
            ("dense", 2500, 8)]
    for route, n, seed in plan:
        coords = synth.ground_box_coords(n, (200, 200, 12), seed=seed, n_boxes=20)
        print(f"route {route} n {n} seed {seed}", flush=True)
        for pairs, sort in ((True, False), (True, True), (False, True)):
            m.build(to_dev_i32(coords), spatial_shape=(200, 200, 12), route=route, pairs=pairs,
                    sort=sort)
            assert_map_equal(m.export(pairs=pairs, perm=sort), oracle_map_of(coords),
                             f"{route} n={n} pairs={pairs} sort={sort}")
    m.close()


def test_dense_rebuilds_beyond_2_31_cells():
    """Dense builds on a 2095 x 2095 x 695 grid (3.06e9 padded cells): cell
    indices past 2^31, bitmap words past 2^26. Sets near the far corner and near
    the origin alternate on one handle, so each build's first kernel clears the
    previous build's words in the other bitmap."""
    grid = (2095, 2095, 695)
    m = smc.KernelMap()
    for seed, far in ((1, True), (2, False), (3, True), (4, True)):
        coords = synth.ground_box_coords(2000, (60, 60, 20), seed=seed, n_boxes=6)
        if far:
            coords[:, 1:] += np.array([2095 - 60, 2095 - 60, 695 - 20], np.int32)
        print(f"huge dense seed {seed} far={far}", flush=True)
        m.build(to_dev_i32(coords), spatial_shape=grid, route="dense")
        assert m.info()["route"] == "dense" and m.info()["grid_cells"] > 2 ** 31
        assert_map_equal(m.export(), oracle_map_of(coords), f"seed {seed}")
    m.close()


def tall_grid_coords(seed, batch=1):
    """Two boxes in a 40 x 40 x 300 grid (302 padded cells along z: the dense
    route's bricked layout), spanning several 16-cell bricks along z and 8-cell
    bricks along x and y, sparsified so masks vary."""
    rng = np.random.default_rng(seed)
    a = synth.box_coords(9, 10, 40, origin=(3, 5, 10), batch=0)
    b = synth.box_coords(12, 7, 25, origin=(20, 14, 270), batch=batch - 1)
    c = np.concatenate([a, b])
    c = c[rng.random(len(c)) < 0.6]
    return c[rng.permutation(len(c))].astype(np.int32)


@pytest.mark.parametrize("seed", [1, 2])
def test_bricked_dense_grid(seed):
    """A tall grid maps through bricks of 8 x 8 x 16 cells; rows next to brick
    faces read their column bits from two bricks. Bit-exact against the oracle
    and the sorted route, with a rebuild on the same handle in between."""
    coords = tall_grid_coords(seed)
    want = oracle_map_of(coords)
    m = smc.KernelMap()
    for rep in range(2):
        m.build(to_dev_i32(coords), spatial_shape=(40, 40, 300), route="dense")
        info = m.info()
        assert info["route"] == "dense"
        assert info["grid_cells"] == 48 * 48 * 304      # 6 x 6 x 19 bricks of 1,024 cells
        assert_map_equal(m.export(), want, f"bricked seed {seed} build {rep}")
    m.close()
    assert_map_equal(gpu_map(coords, route="sorted", spatial_shape=(40, 40, 300)), want,
                     f"sorted seed {seed}")


def test_map_is_deterministic():
    _, coords = config("stage")
    a = gpu_map(coords, spatial_shape=(1440, 1440, 41))
    b = gpu_map(coords, spatial_shape=(1440, 1440, 41))
    assert_map_equal(a, b, "determinism")


@pytest.mark.parametrize("name", ["tiny", "lidar", "stage"])
@pytest.mark.parametrize("table", [False, True])
def test_pair_only_build_with_and_without_the_table(name, table):
    """The dense 3x3x3 build with pair lists and no mask order leaves the
    neighbour table out of device memory unless asked (SMC_BUILD_TABLE): the
    pair lists and masks are the same either way, and the exported table (from
    the device, or filled on the host from the pair lists) equals the oracle's."""
    w, coords = config(name)
    m = smc.KernelMap().build(to_dev_i32(coords), spatial_shape=w.grid, sort=False, table=table)
    got = m.export(perm=False)
    m.close()
    want = dict(oracle_map(name))
    want.pop("perm")
    assert_map_equal(got, want, f"{name} table={table}")
