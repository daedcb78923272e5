"""GPU layer output vs the CPU oracle.

bf16 output: |y - bf16(ref)| <= 2e-2 (1 + |ref|) elementwise, and inside the
rigorous float32-summation + bf16-rounding bound; float32 accumulator:
within 1e-3 (1 + |ref|) elementwise, 1e-3 in relative L2, and inside the
float32 summation bound. Integer-valued and one-hot inputs are exact in any
summation order, so there the comparison is bit-exact. Neither algorithm
uses atomics, so two runs of one layer are bit-identical.
"""
import numpy as np
import pytest

import synth
from oracle import smconv_oracle as so
from _util import (bf16_bits_of, check_bf16_output, check_f32_acc, config, oracle_map,
                   oracle_map_of, to_dev_bf16, to_dev_i32)

pytestmark = pytest.mark.gpu

smc = pytest.importorskip("submanifold_sparse_convolution_amd")


def oracle_acc(om, xb, wb):
    x = so.bf16_bits_to_f64(xb)
    w = so.bf16_bits_to_f64(wb)
    return so.conv_accumulate(x, w, om["pair_in"], om["pair_out"], om["tap_off"], x.shape[0])


def oracle_abs(om, xb, wb):
    """sum |x| |w| per output: the scale of float32 summation error."""
    x = np.abs(so.bf16_bits_to_f64(xb))
    w = np.abs(so.bf16_bits_to_f64(wb))
    return so.conv_accumulate(x, w, om["pair_in"], om["pair_out"], om["tap_off"], x.shape[0])


ALGOS = ["pairs", "mask_tiles"]


def run_gpu(coords, xb, wb, spatial_shape=None, route="auto", relu=False, out_f32=False,
            algo="pairs"):
    m = smc.KernelMap().build(to_dev_i32(coords), spatial_shape=spatial_shape, route=route,
                              pairs=(algo == "pairs"), sort=(algo == "mask_tiles"))
    wp = smc.pack_weights(to_dev_bf16(wb))
    y = m.forward(to_dev_bf16(xb), wp, relu=relu, out_f32=out_f32, algo=algo)
    out = y.cpu().numpy() if out_f32 else bf16_bits_of(y)
    m.close()
    return out


@pytest.mark.parametrize("algo", ALGOS)
@pytest.mark.parametrize("name", ["tiny", "lidar", "deep", "wide"])
def test_workload_layer(name, algo):
    w, coords = config(name)
    c = w.channels
    xb = synth.features(w.n, c, w.seed)
    wb = synth.weights(c, c, w.seed)
    print(f"conv parity {name} n={w.n} c={c} {algo}", flush=True)
    om = oracle_map(name)
    ref = oracle_acc(om, xb, wb)
    s_abs = oracle_abs(om, xb, wb)
    y = run_gpu(coords, xb, wb, spatial_shape=w.grid, algo=algo)
    check_bf16_output(y, ref, name, abs_ref=s_abs, n_terms=27 * c)
    acc = run_gpu(coords, xb, wb, spatial_shape=w.grid, out_f32=True, algo=algo)
    check_f32_acc(acc, ref, name, abs_ref=s_abs, n_terms=27 * c)


@pytest.mark.parametrize("algo", ALGOS)
@pytest.mark.parametrize("route", ["dense", "sorted"])
def test_integer_inputs_exact(route, algo):
    coords = synth.tiny_coords(seed=3, n=3000, side=20)
    xb = synth.int_features(3000, 64, 3)
    wb = synth.int_weights(64, 48, 3)
    ref = oracle_acc(oracle_map_of(coords), xb, wb)
    acc = run_gpu(coords, xb, wb, route=route, out_f32=True, algo=algo)
    assert np.array_equal(acc.astype(np.float64), ref)
    y = run_gpu(coords, xb, wb, route=route, algo=algo)
    assert np.array_equal(so.bf16_bits_to_f64(y), so.round_to_bf16(ref))


@pytest.mark.parametrize("algo", ALGOS)
def test_integer_inputs_exact_c512(algo):
    w, coords = config("deep")
    xb = synth.int_features(w.n, 512, 3)
    wb = synth.int_weights(512, 512, 3)
    ref = oracle_acc(oracle_map("deep"), xb, wb)
    acc = run_gpu(coords, xb, wb, spatial_shape=w.grid, out_f32=True, algo=algo)
    assert np.array_equal(acc.astype(np.float64), ref)


@pytest.mark.parametrize("algo", ALGOS)
@pytest.mark.parametrize("k", [0, 4, 12, 13, 14, 22, 26])
def test_one_hot_tap_is_shifted_copy(k, algo):
    coords = synth.tiny_coords(seed=9, n=2500, side=18)
    c = 32
    xb = synth.features(2500, c, 9)
    w = np.zeros((27, c, c), np.float32)
    w[k] = np.eye(c, dtype=np.float32)
    y = run_gpu(coords, xb, synth.bf16_bits_from_f32(w), algo=algo)
    om = oracle_map_of(coords)
    j = om["nbr"][:, k]
    want = np.where((j >= 0)[:, None], xb[np.maximum(j, 0)], 0).astype(np.uint16)
    assert np.array_equal(y, want)


@pytest.mark.parametrize("algo", ALGOS)
@pytest.mark.parametrize("cin,cout", [(1, 1), (3, 5), (8, 8), (16, 16), (20, 36), (32, 32),
                                      (40, 24), (64, 128), (128, 64), (96, 160), (256, 256),
                                      (200, 72), (384, 96), (456, 48), (520, 64), (300, 40)])
def test_channel_shapes(cin, cout, algo):
    coords = synth.tiny_coords(seed=cin * 7 + cout, n=1500, side=16)
    xb = synth.features(1500, cin, cin)
    wb = synth.weights(cin, cout, cout)
    om = oracle_map_of(coords)
    ref = oracle_acc(om, xb, wb)
    s_abs = oracle_abs(om, xb, wb)
    check_bf16_output(run_gpu(coords, xb, wb, algo=algo), ref, f"{cin}x{cout}", abs_ref=s_abs,
                      n_terms=27 * cin)
    check_f32_acc(run_gpu(coords, xb, wb, out_f32=True, algo=algo), ref, f"{cin}x{cout}",
                  abs_ref=s_abs, n_terms=27 * cin)


@pytest.mark.parametrize("algo", ALGOS)
def test_relu_flag(algo):
    w, coords = config("tiny")
    om = oracle_map("tiny")
    # integer inputs: exact in any summation order, so ReLU output == max(plain output, 0)
    xi, wi = synth.int_features(w.n, 16, 7), synth.int_weights(16, 16, 7)
    yr = so.bf16_bits_to_f64(run_gpu(coords, xi, wi, relu=True, algo=algo))
    yp = so.bf16_bits_to_f64(run_gpu(coords, xi, wi, algo=algo))
    assert (yr >= 0).all() and (yp < 0).any()
    assert np.array_equal(yr, np.maximum(yp, 0))
    assert np.array_equal(yr, np.maximum(so.round_to_bf16(oracle_acc(om, xi, wi)), 0))
    # random inputs: within the rounding bound of max(ref, 0)
    xb, wb = synth.features(w.n, 16, 1), synth.weights(16, 16, 1)
    ref = oracle_acc(om, xb, wb)
    y = run_gpu(coords, xb, wb, relu=True, algo=algo)
    check_bf16_output(y, np.maximum(ref, 0), "relu", abs_ref=oracle_abs(om, xb, wb), n_terms=27 * 16)


@pytest.mark.parametrize("algo", ALGOS)
def test_full_cube_and_single_voxel(algo):
    for coords in (synth.box_coords(3, 3, 3), np.array([[0, 5, 6, 7]], np.int32),
                   synth.box_coords(9, 7, 5, seed=3), synth.tiny_coords(seed=4, n=65, side=5)):
        n = len(coords)
        xb = synth.features(n, 16, 2)
        wb = synth.weights(16, 16, 2)
        ref = oracle_acc(oracle_map_of(coords), xb, wb)
        check_bf16_output(run_gpu(coords, xb, wb, algo=algo), ref, f"n={n}")


def test_layers_share_one_map():
    """Several forwards on one map (the slab grows with c_out): each equals a fresh
    single-layer run."""
    w, coords = config("tiny")
    m = smc.KernelMap().build(to_dev_i32(coords), spatial_shape=w.grid)
    om = oracle_map("tiny")
    for layer in range(4):
        c_out = 16 if layer % 2 == 0 else 48
        xb = synth.features(w.n, 16, 10 + layer)
        wb = synth.weights(16, c_out, 1, layer)
        y = bf16_bits_of(m.forward(to_dev_bf16(xb), smc.pack_weights(to_dev_bf16(wb))))
        check_bf16_output(y, oracle_acc(om, xb, wb), f"layer {layer}")
    m.close()


@pytest.mark.parametrize("algo", ALGOS)
def test_stage_six_layers(algo):
    """Six layers on one map with ReLU between them (the stage workload)."""
    w, coords = config("stage")
    c = w.channels
    om = oracle_map("stage")
    m = smc.KernelMap().build(to_dev_i32(coords), spatial_shape=w.grid, pairs=(algo == "pairs"),
                              sort=(algo == "mask_tiles"))
    hb = synth.features(w.n, c, w.seed)
    h_dev = to_dev_bf16(hb)
    ref_h = so.bf16_bits_to_f64(hb)
    for layer in range(6):
        wb = synth.weights(c, c, w.seed, layer)
        relu = layer < 5
        # teacher-forced: the oracle gets the GPU's own bf16 input of this layer
        gpu_in = bf16_bits_of(h_dev)
        ref = oracle_acc(om, gpu_in, wb)
        h_dev = m.forward(h_dev, smc.pack_weights(to_dev_bf16(wb)), relu=relu, algo=algo)
        got = bf16_bits_of(h_dev)
        want = np.maximum(ref, 0) if relu else ref
        check_bf16_output(got, want, f"stage layer {layer}")
        # end to end: the oracle's own chain
        ref_h = so.round_to_bf16(so.conv_accumulate(ref_h, so.bf16_bits_to_f64(wb), om["pair_in"],
                                                    om["pair_out"], om["tap_off"], w.n))
        if relu:
            ref_h = np.maximum(ref_h, 0)
    got = so.bf16_bits_to_f64(bf16_bits_of(h_dev))
    assert (np.abs(got - ref_h) <= 2e-2 * (1 + np.abs(ref_h))).all()
    m.close()


def test_both_algorithms_agree_and_map_without_pairs():
    w, coords = config("lidar")
    xi, wi = synth.int_features(w.n, 128, 5), synth.int_weights(128, 128, 5)
    a = run_gpu(coords, xi, wi, spatial_shape=w.grid, algo="pairs", out_f32=True)
    b = run_gpu(coords, xi, wi, spatial_shape=w.grid, algo="mask_tiles", out_f32=True)
    assert np.array_equal(a, b)
    m = smc.KernelMap().build(to_dev_i32(coords), spatial_shape=w.grid, pairs=False)
    ex = m.export(pairs=False)
    om = oracle_map("lidar")
    for key in ("nbr", "mask", "perm", "tap_off"):
        assert np.array_equal(np.asarray(ex[key], np.int64), np.asarray(om[key], np.int64)), key
    with pytest.raises(smc.SmconvError):
        m.export(pairs=True)
    with pytest.raises(smc.SmconvError):
        m.forward(to_dev_bf16(xi), smc.pack_weights(to_dev_bf16(wi)), algo="pairs")
    m.close()
    # a map without the mask order: pair lists exact, perm and mask tiles refused
    m = smc.KernelMap().build(to_dev_i32(coords), spatial_shape=w.grid, sort=False)
    ex = m.export(pairs=True, perm=False)
    for key in ("nbr", "mask", "pair_in", "pair_out", "tap_off"):
        assert np.array_equal(np.asarray(ex[key], np.int64), np.asarray(om[key], np.int64)), key
    with pytest.raises(smc.SmconvError):
        m.export(pairs=False, perm=True)
    with pytest.raises(smc.SmconvError):
        m.forward(to_dev_bf16(xi), smc.pack_weights(to_dev_bf16(wi)), algo="mask_tiles")
    m.close()


@pytest.mark.parametrize("algo", ALGOS)
def test_async_build_then_forward(algo):
    """Forward enqueued right behind an asynchronous build (no host read of the counts)."""
    w, coords = config("lidar")
    xb = synth.features(w.n, w.channels, w.seed)
    wb = synth.weights(w.channels, w.channels, w.seed)
    m = smc.KernelMap().build(to_dev_i32(coords), spatial_shape=w.grid, batch_size=1, sync=False,
                              pairs=(algo == "pairs"), sort=(algo == "mask_tiles"))
    y = m.forward(to_dev_bf16(xb), smc.pack_weights(to_dev_bf16(wb)), algo=algo)
    m.sync()
    om = oracle_map("lidar")
    check_bf16_output(bf16_bits_of(y), oracle_acc(om, xb, wb), "async lidar",
                      abs_ref=oracle_abs(om, xb, wb), n_terms=27 * w.channels)
    m.close()


@pytest.mark.parametrize("algo", ALGOS)
def test_repeat_runs_bit_identical(algo):
    """No atomics: the same layer twice gives the same bits (random values, deep)."""
    w, coords = config("deep")
    xb = synth.features(w.n, w.channels, w.seed)
    wb = synth.weights(w.channels, w.channels, w.seed)
    a = run_gpu(coords, xb, wb, spatial_shape=w.grid, algo=algo, out_f32=True)
    b = run_gpu(coords, xb, wb, spatial_shape=w.grid, algo=algo, out_f32=True)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
