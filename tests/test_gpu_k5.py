"""5 x 5 x 5 kernels and batched coordinates on the GPU vs the CPU oracle.

"[Kernel] Add submanifold sparse 3D convolution (bf16 implicit GEMM, gfx950)",
"Test plan": kernel sizes 3 and 5 and batched [N, 4] coordinates are part of
the operation. Maps (125-column neighbour table, 4-word masks, pair lists,
per-tap offsets) must equal the oracle's bit for bit on both routes; layer
outputs must match it exactly with integer inputs and within the bf16 /
float32 tolerances otherwise. Neighbours never cross batches.
"""
import numpy as np
import pytest

import synth
from oracle import smconv_oracle as so
from _util import (assert_map_equal, bf16_bits_of, check_bf16_output, check_f32_acc,
                   oracle_map_of, to_dev_bf16, to_dev_i32)

pytestmark = pytest.mark.gpu

smc = pytest.importorskip("submanifold_sparse_convolution_amd")


def oracle_map5(coords):
    nbr, mask = so.build_kernel_map(coords, 5)
    pin, pout, toff = so.compact_pairs(nbr, mask)
    return dict(nbr=nbr, mask=mask, pair_in=pin, pair_out=pout, tap_off=toff)


def gpu_map5(coords, route="auto", spatial_shape=None, batch_size=0, ncols=4):
    c = coords if ncols == 4 else coords[:, 1:]
    m = smc.KernelMap().build(to_dev_i32(c), spatial_shape=spatial_shape, batch_size=batch_size,
                              route=route, kernel_size=5)
    out = m.export(perm=False)
    out["info"] = m.info()
    m.close()
    return out


def batched(seeds, n, side, kind="uniform"):
    parts = []
    for b, seed in enumerate(seeds):
        if kind == "uniform":
            c = synth.tiny_coords(seed=seed, n=n, side=side)
        else:
            c = synth.ground_box_coords(n, (side, side, 12), seed=seed, n_boxes=20)
        c[:, 0] = b
        parts.append(c)
    coords = np.concatenate(parts)
    return coords[np.random.default_rng(len(seeds)).permutation(len(coords))]


@pytest.mark.parametrize("route", ["dense", "sorted"])
@pytest.mark.parametrize("n,side", [(1, 3), (7, 4), (255, 9), (256, 9), (257, 9), (1500, 14)])
def test_k5_map_small_and_ragged(n, side, route):
    coords = synth.tiny_coords(seed=n, n=n, side=side)
    print(f"k5 map n={n} {route}", flush=True)
    got = gpu_map5(coords, route=route)
    assert got["info"]["kernel_size"] == 5 and got["info"]["taps"] == 125
    assert got["mask"].shape == (n, 4)
    assert_map_equal(got, oracle_map5(coords), f"k5 n={n} {route}")


@pytest.mark.parametrize("route", ["dense", "sorted"])
def test_k5_full_boxes(route):
    for abc in [(5, 5, 5), (1, 1, 9), (6, 3, 4)]:
        coords = synth.box_coords(*abc, origin=(2, 3, 4), seed=sum(abc))
        got = gpu_map5(coords, route=route, spatial_shape=(20, 20, 20))
        assert_map_equal(got, oracle_map5(coords), f"k5 box {abc} {route}")
        per_axis = [sum(max(e - abs(d), 0) for d in range(-2, 3)) for e in abc]
        assert got["info"]["pairs"] == per_axis[0] * per_axis[1] * per_axis[2]


def test_k5_dense_equals_sorted_and_ncols3():
    coords = synth.ground_box_coords(6000, (300, 300, 12), seed=7, n_boxes=40)
    a = gpu_map5(coords, route="dense", spatial_shape=(300, 300, 12))
    b = gpu_map5(coords, route="sorted", spatial_shape=(300, 300, 12))
    c = gpu_map5(coords, ncols=3, spatial_shape=(300, 300, 12))
    assert a["info"]["route"] == "dense" and b["info"]["route"] == "sorted"
    assert_map_equal(a, b, "k5 dense vs sorted")
    assert_map_equal(a, c, "k5 ncols=3")
    assert_map_equal(a, oracle_map5(coords), "k5 vs oracle")


def test_k5_bricked_dense_grid():
    """5 x 5 x 5 taps on a tall grid (bricked dense layout): each column's
    5-cell run crosses a 16-cell brick face for a quarter of the rows."""
    rng = np.random.default_rng(9)
    a = synth.box_coords(10, 9, 44, origin=(2, 6, 7), batch=0)
    coords = a[rng.random(len(a)) < 0.5]
    coords = coords[rng.permutation(len(coords))].astype(np.int32)
    got = gpu_map5(coords, route="dense", spatial_shape=(24, 24, 260))
    assert got["info"]["route"] == "dense"
    assert_map_equal(got, oracle_map5(coords), "k5 bricked")


def test_k5_wide_grid_64bit_keys():
    """A grid too large for the dense route: 64-bit packed keys with two cells of
    padding per field."""
    rng = np.random.default_rng(3)
    base = synth.tiny_coords(seed=3, n=2000, side=14)
    base[:, 1:] = base[:, 1:] * np.array([200, 200, 60]) + rng.integers(0, 2, (2000, 3))
    coords = np.unique(base, axis=0)
    coords = coords[rng.permutation(len(coords))].astype(np.int32)
    got = gpu_map5(coords)
    assert got["info"]["route"] == "sorted" and got["info"]["key_bits"] > 32
    assert_map_equal(got, oracle_map5(coords), "k5 64-bit keys")


@pytest.mark.parametrize("ksize", [3, 5])
@pytest.mark.parametrize("route", ["dense", "sorted"])
def test_batched_maps(ksize, route):
    """Four batches with overlapping xyz: neighbours stay inside their batch;
    explicit and derived batch counts agree."""
    coords = batched([11, 12, 13, 14], 1200, 14)
    want = oracle_map5(coords) if ksize == 5 else oracle_map_of(coords)
    print(f"batched k={ksize} {route} n={len(coords)}", flush=True)
    for bs, shape in ((4, (14, 14, 14)), (0, None)):
        m = smc.KernelMap().build(to_dev_i32(coords), spatial_shape=shape, batch_size=bs,
                                  route=route, kernel_size=ksize)
        got = m.export(perm=False)
        assert m.info()["batch"] == 4
        m.close()
        assert_map_equal(got, want, f"batched k={ksize} {route} bs={bs}")
    nbr = want["nbr"]
    b = coords[:, 0]
    ok = nbr >= 0
    assert (b[np.nonzero(ok)[0]] == b[nbr[ok]]).all()


def oracle_acc(coords, xb, wb):
    ksize = {27: 3, 125: 5}[wb.shape[0]]
    om = oracle_map5(coords) if ksize == 5 else oracle_map_of(coords)
    x, w = so.bf16_bits_to_f64(xb), so.bf16_bits_to_f64(wb)
    acc = so.conv_accumulate(x, w, om["pair_in"], om["pair_out"], om["tap_off"], x.shape[0])
    s_abs = so.conv_accumulate(np.abs(x), np.abs(w), om["pair_in"], om["pair_out"],
                               om["tap_off"], x.shape[0])
    return acc, s_abs


def gpu_forward(coords, xb, wb, relu=False, out_f32=False, route="auto", spatial_shape=None,
                batch_size=0):
    ksize = {27: 3, 125: 5}[wb.shape[0]]
    m = smc.KernelMap().build(to_dev_i32(coords), spatial_shape=spatial_shape, route=route,
                              batch_size=batch_size, kernel_size=ksize)
    y = m.forward(to_dev_bf16(xb), smc.pack_weights(to_dev_bf16(wb)), relu=relu, out_f32=out_f32)
    out = y.cpu().numpy() if out_f32 else bf16_bits_of(y)
    m.close()
    return out


def int_weights5(ci, co, seed):
    w = np.random.default_rng(seed).integers(-2, 3, (125, ci, co)).astype(np.float32)
    return synth.bf16_bits_from_f32(w)


def weights5(ci, co, seed):
    w = np.random.default_rng(seed).standard_normal((125, ci, co)).astype(np.float32)
    return synth.bf16_bits_from_f32(w / np.float32(np.sqrt(125 * ci)))


@pytest.mark.parametrize("route", ["dense", "sorted"])
@pytest.mark.parametrize("ci,co", [(16, 16), (64, 48), (200, 136), (1, 1)])
def test_k5_integer_exact(ci, co, route):
    coords = synth.tiny_coords(seed=3, n=2000, side=16)
    print(f"k5 int exact {ci}x{co} {route}", flush=True)
    xb = synth.int_features(2000, ci, 3)
    wb = int_weights5(ci, co, 3)
    ref, _ = oracle_acc(coords, xb, wb)
    acc = gpu_forward(coords, xb, wb, out_f32=True, route=route)
    assert np.array_equal(acc.astype(np.float64), ref)
    y = gpu_forward(coords, xb, wb, relu=True, route=route)
    assert np.array_equal(so.bf16_bits_to_f64(y), np.maximum(so.round_to_bf16(ref), 0.0))


@pytest.mark.parametrize("c", [32, 128])
def test_k5_random_within_tolerance(c):
    coords = synth.ground_box_coords(8000, (300, 300, 12), seed=9, n_boxes=40)
    xb = synth.features(8000, c, 9)
    wb = weights5(c, c, 9)
    ref, s_abs = oracle_acc(coords, xb, wb)
    print(f"k5 random c={c} pairs/voxel={int(oracle_map5(coords)['tap_off'][-1]) / 8000:.2f}",
          flush=True)
    y = gpu_forward(coords, xb, wb, spatial_shape=(300, 300, 12))
    check_bf16_output(y, ref, f"k5 c={c}", abs_ref=s_abs, n_terms=125 * c)
    acc = gpu_forward(coords, xb, wb, out_f32=True, spatial_shape=(300, 300, 12))
    check_f32_acc(acc, ref, f"k5 c={c}", abs_ref=s_abs, n_terms=125 * c)


@pytest.mark.parametrize("ksize", [3, 5])
def test_batched_layer(ksize):
    coords = batched([21, 22, 23], 3000, 200, kind="ground_box")
    n = len(coords)
    xb = synth.features(n, 64, 4)
    wb = weights5(64, 64, 4) if ksize == 5 else synth.weights(64, 64, 4)
    ref, s_abs = oracle_acc(coords, xb, wb)
    y = gpu_forward(coords, xb, wb)
    check_bf16_output(y, ref, f"batched k={ksize}", abs_ref=s_abs, n_terms=ksize ** 3 * 64)
    # each batch alone gives the same rows
    for b in range(3):
        sel = np.nonzero(coords[:, 0] == b)[0]
        yb = gpu_forward(coords[sel], xb[sel], wb)
        assert np.array_equal(yb, y[sel]), f"batch {b} alone"


def test_kernel_size_mismatch_and_mask_tiles_refused():
    import torch
    coords = synth.tiny_coords(seed=1, n=300, side=10)
    m = smc.KernelMap().build(to_dev_i32(coords), kernel_size=5)
    assert m.info()["n_groups"] == 0                 # no mask order on a 5x5x5 map
    w3 = smc.pack_weights(torch.zeros((27, 8, 8), dtype=torch.bfloat16, device="cuda"))
    w5 = smc.pack_weights(torch.zeros((125, 8, 8), dtype=torch.bfloat16, device="cuda"))
    x = torch.zeros((300, 8), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):
        m.forward(x, w3)
    with pytest.raises(smc.SmconvError):
        m.forward(x, w5, algo="mask_tiles")
    with pytest.raises(smc.SmconvError):
        m.calibrate(1)
    y = m.forward(x, w5)
    assert float(y.float().abs().sum()) == 0.0
    m.close()


def test_kernel_size_switches_on_one_handle():
    m = smc.KernelMap()
    for i, (k, route, n) in enumerate([(3, "dense", 900), (5, "dense", 1200), (5, "sorted", 400),
                                       (3, "sorted", 1500), (5, "dense", 300), (3, "dense", 800)]):
        coords = synth.tiny_coords(seed=30 + i, n=n, side=14)
        m.build(to_dev_i32(coords), route=route, kernel_size=k)
        want = oracle_map5(coords) if k == 5 else oracle_map_of(coords)
        assert_map_equal(m.export(perm=False), want, f"step {i} k={k} {route}")
        xb = synth.int_features(n, 16, i)
        wb = int_weights5(16, 8, i) if k == 5 else synth.int_weights(16, 8, i)
        y = m.forward(to_dev_bf16(xb), smc.pack_weights(to_dev_bf16(wb)), out_f32=True)
        ref, _ = oracle_acc(coords, xb, wb)
        assert np.array_equal(y.cpu().numpy().astype(np.float64), ref), f"step {i}"
    m.close()
