"""The one-kernel pair-list forward (3x3x3 maps, C_in and C_out <= 64, C_in a
multiple of 8: the chunk's slab rows in LDS) against the two-kernel form (slab
in device memory, forced with algo="pairs_slab") and against the CPU oracle.
Shapes past those bounds run the two-kernel form under both names.

Both forms add the same float32 products in the same order (the centre
product, then the row's slab rows in slab order), so their outputs must be
equal bit for bit; integer-valued inputs are exact in any order, so there the
output must equal the oracle's exactly.
"""
import numpy as np
import pytest

import synth
from oracle import smconv_oracle as so
from _util import (bf16_bits_of, check_bf16_output, config, oracle_map, oracle_map_of, to_dev_bf16,
                   to_dev_i32)

pytestmark = pytest.mark.gpu

smc = pytest.importorskip("submanifold_sparse_convolution_amd")


def oracle_acc(om, xb, wb):
    x = so.bf16_bits_to_f64(xb)
    w = so.bf16_bits_to_f64(wb)
    return so.conv_accumulate(x, w, om["pair_in"], om["pair_out"], om["tap_off"], x.shape[0])


def both_forms(m, xb, wb, relu=False, out_f32=False):
    """Outputs of the one-kernel and the two-kernel form on one map."""
    wp = smc.pack_weights(to_dev_bf16(wb))
    x = to_dev_bf16(xb)
    outs = []
    for algo in ("pairs", "pairs_slab"):
        y = m.forward(x, wp, relu=relu, out_f32=out_f32, algo=algo)
        outs.append(y.cpu().numpy() if out_f32 else bf16_bits_of(y))
    return outs


def assert_same(a, b, label):
    a, b = np.asarray(a), np.asarray(b)
    assert a.shape == b.shape, label
    if a.dtype == np.float32:
        a, b = a.view(np.uint32), b.view(np.uint32)
    bad = np.nonzero(a != b)
    assert bad[0].size == 0, f"{label}: {bad[0].size} differing values, first at {bad[0][0]}"


@pytest.mark.parametrize("name", ["tiny", "lidar", "wide", "stage"])
def test_one_kernel_equals_two_kernels_on_workloads(name):
    w, coords = config(name)
    c = min(w.channels, 64)
    print(f"rows vs slab {name} n={w.n} c={c}", flush=True)
    m = smc.KernelMap().build(to_dev_i32(coords), spatial_shape=w.grid)
    xb = synth.features(w.n, c, w.seed)
    wb = synth.weights(c, c, w.seed)
    for relu in (False, True):
        a, b = both_forms(m, xb, wb, relu=relu)
        assert_same(a, b, f"{name} relu={relu}")
    a, b = both_forms(m, xb, wb, out_f32=True)
    assert_same(a, b, f"{name} f32")
    om = oracle_map(name)
    check_bf16_output(both_forms(m, xb, wb)[0], oracle_acc(om, xb, wb), f"{name} c={c}")
    m.close()


@pytest.mark.parametrize("cin,cout", [(8, 1), (8, 16), (16, 17), (24, 33), (32, 32), (40, 48),
                                      (56, 64), (64, 40), (64, 64), (64, 72), (72, 64),
                                      (128, 128)])
def test_channel_shapes_integer_exact(cin, cout):
    coords = synth.tiny_coords(seed=cin + 3 * cout, n=1500, side=16)
    print(f"rows channels {cin}x{cout}", flush=True)
    xi = synth.int_features(len(coords), cin, cin)
    wi = synth.int_weights(cin, cout, cout)
    m = smc.KernelMap().build(to_dev_i32(coords))
    a, b = both_forms(m, xi, wi)
    assert_same(a, b, f"{cin}x{cout}")
    want = so.round_to_bf16(oracle_acc(oracle_map_of(coords), xi, wi))
    got = so.bf16_bits_to_f64(a)
    assert np.array_equal(got, want), f"{cin}x{cout}: {np.count_nonzero(got != want)} differ"
    af, bf = both_forms(m, xi, wi, out_f32=True)
    assert_same(af, bf, f"{cin}x{cout} f32")
    m.close()


@pytest.mark.parametrize("route", ["dense", "sorted"])
def test_dense_box_takes_several_passes(route):
    """A full 24 x 24 x 24 box: most rows have 26 off-centre pairs, so a
    256-row chunk has up to 6656 slab rows, more than one LDS window holds."""
    coords = synth.box_coords(24, 24, 24)
    n = len(coords)
    print(f"rows box n={n} {route}", flush=True)
    m = smc.KernelMap().build(to_dev_i32(coords), route=route)
    for cin, cout in ((64, 64), (16, 16)):
        xi = synth.int_features(n, cin, 5)
        wi = synth.int_weights(cin, cout, 6)
        a, b = both_forms(m, xi, wi, relu=True)
        assert_same(a, b, f"box {cin}x{cout}")
        want = np.maximum(so.round_to_bf16(oracle_acc(oracle_map_of(coords), xi, wi)), 0)
        assert np.array_equal(so.bf16_bits_to_f64(a), want)
    m.close()


@pytest.mark.parametrize("n", [1, 15, 255, 256, 257, 1000, 4097])
def test_ragged_row_counts(n):
    coords = synth.tiny_coords(seed=n, n=n, side=20)
    print(f"rows ragged n={n}", flush=True)
    xi = synth.int_features(n, 64, n)
    wi = synth.int_weights(64, 64, n + 1)
    m = smc.KernelMap().build(to_dev_i32(coords))
    a, b = both_forms(m, xi, wi)
    assert_same(a, b, f"n={n}")
    want = so.round_to_bf16(oracle_acc(oracle_map_of(coords), xi, wi))
    assert np.array_equal(so.bf16_bits_to_f64(a), want)
    m.close()


def test_async_build_then_forward_and_rebuilds():
    """Builds of different sizes on one handle, each forward enqueued right
    after an asynchronous build (the kernel reads the chunk table and counts on
    the device)."""
    m = smc.KernelMap()
    for n, seed in ((3000, 1), (700, 2), (5000, 3)):
        coords = synth.tiny_coords(seed=seed, n=n, side=22)
        print(f"rows async n={n}", flush=True)
        m.build(to_dev_i32(coords), sync=False)
        xi = synth.int_features(n, 32, seed)
        wi = synth.int_weights(32, 48, seed)
        a, b = both_forms(m, xi, wi)
        assert_same(a, b, f"async n={n}")
        want = so.round_to_bf16(oracle_acc(oracle_map_of(coords), xi, wi))
        assert np.array_equal(so.bf16_bits_to_f64(a), want)
    m.sync()
    m.close()
