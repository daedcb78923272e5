"""The wide-input GEMMs (C_in 136 .. 576, a multiple of 8: a tap's column-tile
weight slab resident in LDS, eight waves streaming 16-row fragments through
it) against the CPU oracle, exactly, on integer-valued inputs (every float32
partial sum is an integer below 2^24, so any summation order gives the same
bits). The shapes cover every column-block width of the wave tile (1, 2, 4
and 8 blocks of 16), odd and ragged output widths, the shortest and longest
k loops, row counts around the 16-row fragment, the off-centre work items of
one tap and of many, and a strided map, which sends every tap through the
off-centre kernel.
"""
import numpy as np
import pytest

import synth
from oracle import smconv_oracle as so
from _util import bf16_bits_of, oracle_map_of, to_dev_bf16, to_dev_i32

pytestmark = pytest.mark.gpu

smc = pytest.importorskip("submanifold_sparse_convolution_amd")


def oracle_acc(om, xb, wb):
    x = so.bf16_bits_to_f64(xb)
    w = so.bf16_bits_to_f64(wb)
    return so.conv_accumulate(x, w, om["pair_in"], om["pair_out"], om["tap_off"], x.shape[0])


def run(m, xi, wi, relu=False, out_f32=False):
    wp = smc.pack_weights(to_dev_bf16(wi))
    y = m.forward(to_dev_bf16(xi), wp, relu=relu, out_f32=out_f32)
    return y.cpu().numpy() if out_f32 else bf16_bits_of(y)


@pytest.mark.parametrize("cin,cout", [(136, 8), (136, 128), (256, 33), (256, 256), (264, 200),
                                      (384, 96), (392, 17), (504, 40), (512, 16), (512, 512),
                                      (576, 24), (576, 130)])
def test_channel_shapes_integer_exact(cin, cout):
    coords = synth.tiny_coords(seed=cin + cout, n=1100, side=15)
    n = len(coords)
    print(f"wide {cin}x{cout} n={n}", flush=True)
    xi = synth.int_features(n, cin, cin)
    wi = synth.int_weights(cin, cout, cout)
    ref = oracle_acc(oracle_map_of(coords), xi, wi)
    m = smc.KernelMap().build(to_dev_i32(coords))
    got = so.bf16_bits_to_f64(run(m, xi, wi))
    want = so.round_to_bf16(ref)
    assert np.array_equal(got, want), f"{cin}x{cout}: {np.count_nonzero(got != want)} differ"
    gf = run(m, xi, wi, out_f32=True)
    assert np.array_equal(gf.astype(np.float64), ref)
    gr = so.bf16_bits_to_f64(run(m, xi, wi, relu=True))
    assert np.array_equal(gr, np.maximum(want, 0))
    m.close()


@pytest.mark.parametrize("n", [1, 2, 15, 16, 17, 95, 1000])
def test_ragged_row_counts(n):
    coords = synth.tiny_coords(seed=n + 11, n=n, side=12)
    print(f"wide ragged n={n}", flush=True)
    for cin, cout in ((512, 64), (200, 72)):
        xi = synth.int_features(n, cin, n)
        wi = synth.int_weights(cin, cout, n + 1)
        m = smc.KernelMap().build(to_dev_i32(coords))
        got = so.bf16_bits_to_f64(run(m, xi, wi))
        want = so.round_to_bf16(oracle_acc(oracle_map_of(coords), xi, wi))
        assert np.array_equal(got, want), f"n={n} {cin}x{cout}"
        m.close()


def test_dense_box_many_items_per_tap():
    """A full 14 x 14 x 14 box: every tap holds hundreds of pairs, so a tap's
    work spans many 128-pair items and a block's item range crosses taps."""
    coords = synth.box_coords(14, 14, 14)
    n = len(coords)
    xi = synth.int_features(n, 256, 4)
    wi = synth.int_weights(256, 96, 5)
    m = smc.KernelMap().build(to_dev_i32(coords))
    got = so.bf16_bits_to_f64(run(m, xi, wi))
    want = so.round_to_bf16(oracle_acc(oracle_map_of(coords), xi, wi))
    assert np.array_equal(got, want)
    m.close()


def test_strided_wide_integer_exact():
    """A strided map: every tap, the centre included, goes through the
    off-centre kernel (rows with one pair written by it directly)."""
    coords = synth.tiny_coords(seed=21, n=1400, side=18)
    n = len(coords)
    xi = synth.int_features(n, 264, 8)
    wi = synth.int_weights(264, 72, 9)
    r = so.strided_conv(coords, (18, 18, 18), xi, wi)
    m = smc.KernelMap().build_strided(to_dev_i32(coords), spatial_shape=(18, 18, 18))
    wp = smc.pack_weights(to_dev_bf16(wi))
    acc = m.forward(to_dev_bf16(xi), wp, out_f32=True).cpu().numpy()
    assert np.array_equal(acc.astype(np.float64), r["acc"])
    y = bf16_bits_of(m.forward(to_dev_bf16(xi), wp, relu=True))
    assert np.array_equal(so.bf16_bits_to_f64(y), np.maximum(so.round_to_bf16(r["acc"]), 0.0))
    m.close()
