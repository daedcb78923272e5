"""Strided (downsampling) layer on the GPU vs the CPU oracle.

"Sparse convolution in FP32" (DriveRT), section "Calibrated bit order": the
strided layers change the coordinate set and run as mask-sorted tiles. The
reading (kernel 3, stride 2, padding 1, outputs ordered by (b, x, y, z)) is
the oracle's build_strided_map. Output coordinates, neighbour table, masks,
mask order and the output rows' pair lists (the centre a tap like the others)
must match bit for bit on both routes; outputs of both forward algorithms
(pair lists and mask tiles) exactly with integer inputs, within the bf16 /
float32 tolerances otherwise.
"""
import numpy as np
import pytest

import synth
from oracle import smconv_oracle as so
from _util import bf16_bits_of, check_bf16_output, check_f32_acc, to_dev_bf16, to_dev_i32

pytestmark = pytest.mark.gpu

smc = pytest.importorskip("submanifold_sparse_convolution_amd")


def oracle_strided(coords, shape):
    oc, oshape, nbr, mask = so.build_strided_map(coords, shape)
    return dict(out_coords=oc, out_shape=oshape, nbr=nbr, mask=mask,
                perm=so.mask_sort(mask)[None, :])


def gpu_strided(coords, shape=None, route="auto", batch_size=0, ncols=4, sync=True):
    c = coords if ncols == 4 else coords[:, 1:]
    m = smc.KernelMap().build_strided(to_dev_i32(c), spatial_shape=shape, route=route,
                                      batch_size=batch_size, sync=sync)
    ex = m.export(pairs=False)
    ex["out_coords"] = m.out_coords()
    ex["info"] = m.info()
    m.close()
    return ex


def check_map(got, want, label):
    for key in ("out_coords", "nbr", "mask", "perm"):
        g, w = np.asarray(got[key]), np.asarray(want[key])
        assert g.shape == w.shape, f"{label} {key}: shape {g.shape} != {w.shape}"
        assert np.array_equal(g.astype(np.int64), w.astype(np.int64)), f"{label} {key}"
    assert got["info"]["strided"] and got["info"]["n"] == len(want["out_coords"])
    assert tuple(got["info"]["out_extent"]) == tuple(want["out_shape"])


def random_cells(shape, n, seed, batch=0):
    rng = np.random.default_rng(seed)
    cells = rng.choice(int(np.prod(shape)), size=n, replace=False)
    xyz = np.stack(np.unravel_index(cells, shape), axis=1)
    return np.concatenate([np.full((n, 1), batch), xyz], axis=1).astype(np.int32)


@pytest.mark.parametrize("route", ["dense", "sorted"])
@pytest.mark.parametrize("shape,n,seed", [((8, 8, 8), 1, 1), ((8, 8, 8), 7, 2),
                                          ((9, 7, 5), 120, 3), ((1, 6, 11), 30, 4),
                                          ((24, 24, 24), 3000, 5), ((31, 17, 40), 2500, 6)])
def test_strided_map_small(shape, n, seed, route):
    coords = random_cells(shape, n, seed)
    print(f"strided map {shape} n={n} {route}", flush=True)
    check_map(gpu_strided(coords, shape, route=route), oracle_strided(coords, shape),
              f"{shape} n={n} {route}")


@pytest.mark.parametrize("route", ["dense", "sorted"])
def test_strided_batches_derived_shape_ncols3(route):
    a = random_cells((20, 20, 20), 900, 7, 0)
    b = random_cells((20, 20, 20), 700, 8, 2)
    coords = np.concatenate([a, b])
    coords = coords[np.random.default_rng(1).permutation(len(coords))]
    want = oracle_strided(coords, (20, 20, 20))
    check_map(gpu_strided(coords, (20, 20, 20), route=route, batch_size=3), want, "batches")
    mx = tuple(int(v) + 1 for v in coords[:, 1:].max(0))
    check_map(gpu_strided(coords, None, route=route), oracle_strided(coords, mx), "derived")
    check_map(gpu_strided(a, (20, 20, 20), route=route, ncols=3),
              oracle_strided(a, (20, 20, 20)), "ncols=3")


@pytest.mark.parametrize("name", ["lidar", "deep", "wide"])
def test_strided_map_workloads(name):
    """Output grids of at most 2^30 cells take the output bitmap: lidar and
    deep (small), wide (1048 x 1048 x 348 = 382M cells, a 48 MB bitmap). The
    candidate sort of larger grids is covered by the 64-bit-key test below."""
    w = synth.workload(name)
    coords = synth.make_coords(w)
    print(f"strided map {name} n={w.n}", flush=True)
    want = oracle_strided(coords, w.grid)
    got = gpu_strided(coords, w.grid)
    check_map(got, want, name)
    got2 = gpu_strided(coords, w.grid, route="sorted", sync=False)
    check_map(got2, want, name + " sorted")


def strided_forward(coords, shape, xb, wb, relu=False, out_f32=False, route="auto", algo="pairs"):
    m = smc.KernelMap().build_strided(to_dev_i32(coords), spatial_shape=shape, route=route,
                                      pairs=algo == "pairs", sort=algo == "mask_tiles")
    y = m.forward(to_dev_bf16(xb), smc.pack_weights(to_dev_bf16(wb)), relu=relu, out_f32=out_f32,
                  algo=algo)
    out = y.cpu().numpy() if out_f32 else bf16_bits_of(y)
    m.close()
    return out


@pytest.mark.parametrize("algo", ["pairs", "mask_tiles"])
@pytest.mark.parametrize("route", ["dense", "sorted"])
@pytest.mark.parametrize("ci,co", [(16, 16), (64, 48), (200, 136), (1, 1), (128, 128), (520, 64)])
def test_strided_layer_integer_exact(ci, co, route, algo):
    coords = random_cells((30, 30, 30), 4000, 11)
    print(f"strided layer {ci}x{co} {route} {algo}", flush=True)
    xb = synth.int_features(4000, ci, 5)
    wb = synth.int_weights(ci, co, 5)
    r = so.strided_conv(coords, (30, 30, 30), xb, wb)
    acc = strided_forward(coords, (30, 30, 30), xb, wb, out_f32=True, route=route, algo=algo)
    assert np.array_equal(acc.astype(np.float64), r["acc"])
    y = strided_forward(coords, (30, 30, 30), xb, wb, relu=True, route=route, algo=algo)
    assert np.array_equal(so.bf16_bits_to_f64(y), np.maximum(so.round_to_bf16(r["acc"]), 0.0))


@pytest.mark.parametrize("algo", ["pairs", "mask_tiles"])
@pytest.mark.parametrize("name", ["lidar", "deep"])
def test_strided_layer_workloads(name, algo):
    w = synth.workload(name)
    coords = synth.make_coords(w)
    c = w.channels
    xb = synth.features(w.n, c, w.seed)
    wb = synth.weights(c, c, w.seed)
    r = so.strided_conv(coords, w.grid, xb, wb)
    x, wt = so.bf16_bits_to_f64(xb), so.bf16_bits_to_f64(wb)
    s_abs = so.conv_accumulate(np.abs(x), np.abs(wt), r["pair_in"], r["pair_out"], r["tap_off"],
                               len(r["out_coords"]))
    print(f"strided layer {name}: {w.n} -> {len(r['out_coords'])} rows, {algo}", flush=True)
    y = strided_forward(coords, w.grid, xb, wb, algo=algo)
    check_bf16_output(y, r["acc"], name, abs_ref=s_abs, n_terms=27 * c)
    acc = strided_forward(coords, w.grid, xb, wb, out_f32=True, algo=algo)
    check_f32_acc(acc, r["acc"], name, abs_ref=s_abs, n_terms=27 * c)


@pytest.mark.parametrize("route", ["dense", "sorted"])
@pytest.mark.parametrize("case", ["small", "ragged", "lidar"])
def test_strided_pair_lists(case, route):
    """The output rows' pair lists, the centre tap (input at 2 o) a tap like
    the others, bit for bit against the oracle's compaction of its table."""
    if case == "lidar":
        w = synth.workload("lidar")
        coords, shape = synth.make_coords(w), w.grid
    elif case == "ragged":
        coords, shape = random_cells((31, 17, 40), 2500, 6), (31, 17, 40)
    else:
        coords, shape = random_cells((9, 7, 5), 120, 3), (9, 7, 5)
    print(f"strided pair lists {case} {route}", flush=True)
    want = oracle_strided(coords, shape)
    pin, pout, toff = so.compact_pairs(want["nbr"], want["mask"])
    m = smc.KernelMap().build_strided(to_dev_i32(coords), spatial_shape=shape, route=route,
                                      sort=False)
    ex = m.export(perm=False)
    m.close()
    assert np.array_equal(ex["tap_off"], toff)
    assert np.array_equal(ex["pair_in"], pin) and np.array_equal(ex["pair_out"], pout)
    assert np.array_equal(ex["nbr"], want["nbr"]) and np.array_equal(ex["mask"], want["mask"])


def test_strided_build_without_pairs_or_sort():
    """A pairs-only map refuses mask tiles; a sort-only map runs mask tiles
    whatever the algorithm asked for (a strided map without pair lists has
    only them); both give the same exact integers."""
    coords = random_cells((20, 20, 20), 1500, 21)
    xb, wb = synth.int_features(1500, 32, 2), synth.int_weights(32, 24, 3)
    r = so.strided_conv(coords, (20, 20, 20), xb, wb)
    x, wp = to_dev_bf16(xb), smc.pack_weights(to_dev_bf16(wb))
    only_pairs = smc.KernelMap().build_strided(to_dev_i32(coords), spatial_shape=(20, 20, 20),
                                               sort=False)
    only_sort = smc.KernelMap().build_strided(to_dev_i32(coords), spatial_shape=(20, 20, 20),
                                              pairs=False)
    with pytest.raises(smc.SmconvError):
        only_pairs.forward(x, wp, algo="mask_tiles")
    a = only_pairs.forward(x, wp, out_f32=True).cpu().numpy()
    b = only_sort.forward(x, wp, out_f32=True, algo="mask_tiles").cpu().numpy()
    c = only_sort.forward(x, wp, out_f32=True, algo="pairs").cpu().numpy()
    assert np.array_equal(a.astype(np.float64), r["acc"]) and np.array_equal(b, a)
    assert np.array_equal(c, b)
    only_pairs.close()
    only_sort.close()


def test_strided_errors_and_handle_reuse():
    import torch
    m = smc.KernelMap()
    neg = np.array([[0, -1, 2, 3], [0, 4, 4, 4]], np.int32)
    with pytest.raises(smc.SmconvError):
        m.build_strided(to_dev_i32(neg))
    with pytest.raises(smc.SmconvError):
        m.build_strided(to_dev_i32(random_cells((8, 8, 8), 10, 1)), kernel_size=5)
    dup = np.array([[0, 1, 2, 3], [0, 5, 5, 5], [0, 1, 2, 3]], np.int32)
    for route in ("dense", "sorted"):
        with pytest.raises(smc.SmconvError):
            m.build_strided(to_dev_i32(dup), spatial_shape=(8, 8, 8), route=route)
    # strided, submanifold and strided again on one handle
    coords = random_cells((16, 16, 16), 800, 3)
    for step in range(3):
        if step == 1:
            m.build(to_dev_i32(coords), spatial_shape=(16, 16, 16))
            assert m.n == 800 and not m.info()["strided"]
            continue
        m.build_strided(to_dev_i32(coords), spatial_shape=(16, 16, 16))
        want = oracle_strided(coords, (16, 16, 16))
        ex = m.export(pairs=False)
        ex["out_coords"] = m.out_coords()
        ex["info"] = m.info()
        check_map(ex, want, f"reuse {step}")
        xb = synth.int_features(800, 8, step)
        wb = synth.int_weights(8, 8, step)
        y = m.forward(to_dev_bf16(xb), smc.pack_weights(to_dev_bf16(wb)), out_f32=True)
        assert np.array_equal(y.cpu().numpy().astype(np.float64),
                              so.strided_conv(coords, (16, 16, 16), xb, wb)["acc"])
        with pytest.raises(ValueError):
            m.forward(torch.zeros((ex["info"]["n"], 8), dtype=torch.bfloat16, device="cuda"),
                      smc.pack_weights(to_dev_bf16(wb)))
    empty = m.build_strided(torch.zeros((0, 4), dtype=torch.int32, device="cuda"),
                            spatial_shape=(8, 8, 8))
    assert empty.n == 0
    m.close()


def test_strided_candidate_sort_route():
    """An output grid above 2^30 cells (1050 x 1050 x 1000): output cells from
    the candidate sort (480k keys), on both routes."""
    coords = synth.ground_box_coords(60000, (2100, 2100, 2000), seed=7, n_boxes=60)
    print(f"strided candidate sort n={len(coords)}", flush=True)
    want = oracle_strided(coords, (2100, 2100, 2000))
    check_map(gpu_strided(coords, (2100, 2100, 2000)), want, "candidates")
    check_map(gpu_strided(coords, (2100, 2100, 2000), route="sorted"), want, "candidates sorted")


def test_strided_sorted_64bit_keys():
    """A padded input grid of more than 2^32 cells: the sorted route with 64-bit keys
    (dense clusters far apart, so every query plane has neighbours to find)."""
    parts = []
    for i, off in enumerate([(0, 0, 0), (4000, 0, 0), (0, 4000, 9), (4000, 4000, 1000)]):
        c = synth.tiny_coords(seed=11 + i, n=600, side=12)
        c[:, 1:] += np.array(off, np.int32)
        parts.append(c)
    coords = np.concatenate(parts)
    coords = coords[np.random.default_rng(12).permutation(len(coords))].astype(np.int32)
    shape = tuple(int(v) + 1 for v in coords[:, 1:].max(0))
    got = gpu_strided(coords, shape)
    assert got["info"]["route"] == "sorted" and got["info"]["key_bits"] > 32
    check_map(got, oracle_strided(coords, shape), "64-bit keys")


def test_deferred_output_count_readers():
    """A strided pair-list build leaves its output count on the device (the
    lookup and compaction after it are sized by the bound 8 n); every reader
    of the count resolves it: the map info, the forward, the coordinate export,
    also for a build nobody read before the next one started."""
    import ctypes
    import torch
    L = smc.lib()
    cases = [(random_cells((30, 30, 30), 3000, 31), (30, 30, 30)),
             (random_cells((24, 24, 24), 1200, 32), (24, 24, 24))]
    refs = [so.strided_conv(c, shp, synth.int_features(len(c), 16, 3),
                            synth.int_weights(16, 24, 4)) for c, shp in cases]
    m = smc.KernelMap()
    keep = []

    def build_async(k):
        coords, shp = cases[k]
        d = to_dev_i32(coords)
        keep.append(d)
        shape = (ctypes.c_int32 * 3)(*shp)
        rc = L.smc_map_build_strided(m._h, ctypes.c_void_p(d.data_ptr()), len(coords), 4, shape,
                                     0, 3, 2, 0, smc.SMC_BUILD_ASYNC | smc.SMC_BUILD_NO_SORT,
                                     None)
        assert rc == 0

    # two builds back to back, the first count never read: the second's is reported
    build_async(0)
    build_async(1)
    assert m.info()["n"] == len(refs[1]["out_coords"])
    # the forward as the first reader, then the coordinate export
    build_async(0)
    n0 = len(refs[0]["out_coords"])
    coords0, _ = cases[0]
    x = to_dev_bf16(synth.int_features(len(coords0), 16, 3))
    wp = smc.pack_weights(to_dev_bf16(synth.int_weights(16, 24, 4)))
    y = torch.empty((n0, 24), dtype=torch.float32, device="cuda")
    rc = L.smc_conv_forward(m._h, ctypes.c_void_p(x.data_ptr()), 16, ctypes.c_void_p(wp.buf.data_ptr()),
                            24, ctypes.c_void_p(y.data_ptr()), smc.SMC_FWD_OUT_F32, None)
    assert rc == 0
    torch.cuda.synchronize()
    assert np.array_equal(y.cpu().numpy().astype(np.float64), refs[0]["acc"])
    m.n = n0
    assert np.array_equal(m.out_coords(), refs[0]["out_coords"])
    m.close()


def test_strided_above_the_deferred_bound():
    """1.1M inputs: a bound of 8 n above 2^23 rows, so a pair-list build reads
    its output count back and sizes by it (the fused lookup and compaction
    without a device count). Its map and an integer-valued layer equal those
    of a build that also sorts the masks (its own compaction, compared with
    the oracle in the tests above) exactly."""
    rng = np.random.default_rng(3)
    shape = (120, 120, 100)
    cells = rng.choice(int(np.prod(shape)), size=1_100_000, replace=False)
    xyz = np.stack(np.unravel_index(cells, shape), axis=1)
    coords = np.concatenate([np.zeros((len(xyz), 1)), xyz], axis=1).astype(np.int32)
    print(f"strided above the bound: n={len(coords)}", flush=True)
    d = to_dev_i32(coords)
    xb = synth.int_features(len(coords), 16, 7)
    wb = synth.int_weights(16, 16, 8)
    out = []
    for sort in (False, True):
        m = smc.KernelMap().build_strided(d, spatial_shape=shape, sort=sort)
        ex = m.export(perm=False)
        y = m.forward(to_dev_bf16(xb), smc.pack_weights(to_dev_bf16(wb)), out_f32=True)
        out.append((m.n, ex, y.cpu().numpy()))
        m.close()
    (na, ea, ya), (nb, eb, yb) = out
    assert na == nb
    for key in ("tap_off", "pair_in", "pair_out", "mask", "nbr"):
        assert np.array_equal(np.asarray(ea[key]), np.asarray(eb[key])), key
    assert np.array_equal(ya, yb)
