"""Calibrated bit order and offset groups of the mask-tile path on the GPU.

"Sparse convolution in FP32" (DriveRT), sections "Calibrated bit order" and
"Offset-group partitioning": the row orders the map exports must equal the
oracle's group_row_orders bit for bit, the library's calibration must choose
the same order and groups as the oracle's calibrate_order, and the grouped
mask-tile forward must match the oracle like the one-group path does
(integer inputs: exactly; bf16 inputs: within 2e-2 (1 + |ref|) and the
float32 summation bound), with the ReLU reaching every row.
"""
import numpy as np
import pytest

import synth
from oracle import smconv_oracle as so
from _util import (bf16_bits_of, check_bf16_output, check_f32_acc, config, oracle_map,
                   oracle_map_of, to_dev_bf16, to_dev_i32)

pytestmark = pytest.mark.gpu

smc = pytest.importorskip("submanifold_sparse_convolution_amd")

_SHUF = [int(t) for t in np.random.default_rng(21).permutation(27)]
_RUNS3 = [t for t in _SHUF if t != 13]
_GROUPS_RUNS3 = [0] * 27
for _p, _t in enumerate(_RUNS3):
    _GROUPS_RUNS3[_t] = (_p * 3) // 26
_GROUPS_RUNS3[13] = 2

CASES = {
    "plain": (None, None),
    "reversed": (list(range(27)), None),
    "shuffled": (_SHUF, None),
    "dx_slabs": (None, [{0: 0, 2: 1, 1: 2}[k // 9] for k in range(27)]),
    "runs3_shuffled": (_SHUF, _GROUPS_RUNS3),
    "four_groups": (list(range(27)), [k % 4 if k != 13 else 3 for k in range(27)]),
    "one_tap_first": (None, [0 if k == 0 else 1 for k in range(27)]),
}


def build(coords, bo, go, route="auto", spatial_shape=None, sync=True):
    m = smc.KernelMap().set_order(bo, go)
    m.build(to_dev_i32(coords), spatial_shape=spatial_shape, route=route, sync=sync)
    return m


def check_orders(m, mask, bo, go, label):
    ex = m.export(pairs=False)
    want, counts = so.group_row_orders(mask, bo, go)
    assert ex["perm"].shape == want.shape, label
    assert np.array_equal(ex["perm"], want), f"{label}: row orders"
    assert np.array_equal(ex["group_rows"], counts), f"{label}: group row counts"
    assert np.array_equal(ex["mask"], mask), f"{label}: masks"


@pytest.mark.parametrize("route", ["dense", "sorted"])
@pytest.mark.parametrize("case", list(CASES))
def test_group_orders_bit_exact(case, route):
    bo, go = CASES[case]
    for n, seed in ((3000, 3), (1001, 4)):
        coords = synth.tiny_coords(seed=seed, n=n, side=20)
        print(f"orders {case} {route} n={n}", flush=True)
        _, mask = so.build_kernel_map(coords)
        m = build(coords, bo, go, route=route)
        check_orders(m, mask, bo, go, f"{case}/{route}/{n}")
        m.close()


@pytest.mark.parametrize("name", ["lidar", "deep", "wide", "stage"])
def test_calibrated_orders_on_workloads(name):
    w, coords = config(name)
    mask = oracle_map(name)["mask"]
    m = smc.KernelMap().build(to_dev_i32(coords), spatial_shape=w.grid, pairs=False)
    bo, go = m.calibrate(3)
    print(f"calibrated {name}: {bo} {go}", flush=True)
    m.set_order(bo, go).build(to_dev_i32(coords), spatial_shape=w.grid, pairs=False)
    check_orders(m, mask, bo, go, name)
    m.close()


@pytest.mark.parametrize("n_groups", [1, 3])
def test_calibration_matches_oracle(n_groups):
    coords = synth.tiny_coords(seed=1, n=2048, side=24)
    _, mask = so.build_kernel_map(coords)
    m = smc.KernelMap().build(to_dev_i32(coords), spatial_shape=(24, 24, 24))
    got = m.calibrate(n_groups)
    m.close()
    want = so.calibrate_order(mask, n_groups, 64)
    assert list(got[0]) == list(want[0]), "bit order"
    assert list(got[1]) == list(want[1]), "groups"


def test_calibration_reduces_tile_work():
    w, coords = config("deep")
    mask = oracle_map("deep")["mask"]
    m = smc.KernelMap().build(to_dev_i32(coords), spatial_shape=w.grid, pairs=False)
    bo, go = m.calibrate(3)
    m.close()
    cnt = [int(((mask >> np.uint32(t)) & 1).sum()) for t in range(27)]
    start = sorted((t for t in range(27) if t != 13), key=lambda t: (cnt[t], t)) + [13]
    o1, c1 = so.group_row_orders(mask, bo)
    o0, c0 = so.group_row_orders(mask, start)
    plain, cp = so.group_row_orders(mask)
    w1 = so.tile_work(mask, o1[0], c1[0])
    assert w1 <= so.tile_work(mask, o0[0], c0[0])
    assert w1 < so.tile_work(mask, plain[0], cp[0])
    og, cg = so.group_row_orders(mask, bo, go)
    wg = sum(so.tile_work(mask, og[g], cg[g], [t for t in range(27) if go[t] == g])
             for g in range(3))
    assert wg < w1


def grouped_forward(coords, xb, wb, bo, go, relu=False, out_f32=False, spatial_shape=None,
                    route="auto", sync=True):
    m = build(coords, bo, go, route=route, spatial_shape=spatial_shape, sync=sync)
    y = m.forward(to_dev_bf16(xb), smc.pack_weights(to_dev_bf16(wb)), relu=relu,
                  out_f32=out_f32, algo="mask_tiles")
    out = y.cpu().numpy() if out_f32 else bf16_bits_of(y)
    m.close()
    return out


def oracle_acc(coords, xb, wb):
    om = oracle_map_of(coords)
    x, w = so.bf16_bits_to_f64(xb), so.bf16_bits_to_f64(wb)
    return so.conv_accumulate(x, w, om["pair_in"], om["pair_out"], om["tap_off"], x.shape[0])


@pytest.mark.parametrize("case", list(CASES))
def test_grouped_forward_integer_exact(case):
    bo, go = CASES[case]
    coords = synth.tiny_coords(seed=3, n=3000, side=20)
    for ci, co in ((64, 48), (16, 16), (200, 136)):
        print(f"grouped forward {case} c={ci}x{co}", flush=True)
        xb = synth.int_features(3000, ci, 3)
        wb = synth.int_weights(ci, co, 3)
        ref = oracle_acc(coords, xb, wb)
        acc = grouped_forward(coords, xb, wb, bo, go, out_f32=True)
        assert np.array_equal(acc.astype(np.float64), ref), f"{case} {ci}x{co} float32"
        y = grouped_forward(coords, xb, wb, bo, go, relu=True)
        want = np.maximum(so.round_to_bf16(ref), 0.0)
        assert np.array_equal(so.bf16_bits_to_f64(y), want), f"{case} {ci}x{co} bf16 + relu"


@pytest.mark.parametrize("name", ["lidar", "deep", "wide"])
def test_grouped_forward_workloads(name):
    w, coords = config(name)
    c = w.channels
    xb = synth.features(w.n, c, w.seed)
    wb = synth.weights(c, c, w.seed)
    om = oracle_map(name)
    x, wt = so.bf16_bits_to_f64(xb), so.bf16_bits_to_f64(wb)
    ref = so.conv_accumulate(x, wt, om["pair_in"], om["pair_out"], om["tap_off"], w.n)
    s_abs = so.conv_accumulate(np.abs(x), np.abs(wt), om["pair_in"], om["pair_out"],
                               om["tap_off"], w.n)
    m = smc.KernelMap().build(to_dev_i32(coords), spatial_shape=w.grid, pairs=False)
    bo, go = m.calibrate(3)
    m.close()
    print(f"grouped forward {name} n={w.n} c={c}", flush=True)
    y = grouped_forward(coords, xb, wb, bo, go, spatial_shape=w.grid, relu=True)
    check_bf16_output(y, np.maximum(ref, 0.0), name, abs_ref=s_abs, n_terms=27 * c)
    acc = grouped_forward(coords, xb, wb, bo, go, spatial_shape=w.grid, out_f32=True,
                          sync=False)
    check_f32_acc(acc, ref, name, abs_ref=s_abs, n_terms=27 * c)


def test_order_change_on_one_handle():
    """plain -> 4 groups -> calibrated 3 groups -> plain on one handle, sizes changing."""
    m = smc.KernelMap()
    steps = [(None, None, 500), (CASES["four_groups"][0], CASES["four_groups"][1], 3000),
             (_SHUF, _GROUPS_RUNS3, 1200), (None, None, 2500)]
    for i, (bo, go, n) in enumerate(steps):
        coords = synth.tiny_coords(seed=10 + i, n=n, side=20)
        _, mask = so.build_kernel_map(coords)
        m.set_order(bo, go).build(to_dev_i32(coords), pairs=(i % 2 == 0))
        check_orders(m, mask, bo, go, f"step {i}")
        xb = synth.int_features(n, 32, i)
        wb = synth.int_weights(32, 24, i)
        y = m.forward(to_dev_bf16(xb), smc.pack_weights(to_dev_bf16(wb)), out_f32=True,
                      algo="mask_tiles")
        assert np.array_equal(y.cpu().numpy().astype(np.float64), oracle_acc(coords, xb, wb))
    m.close()


def test_set_order_errors_keep_previous_order():
    m = smc.KernelMap()
    bad = [
        (list(range(26)) + [0], None),                        # not a permutation
        (None, [0] * 13 + [0] + [1] * 13),                    # centre not in the last group
        (None, [0] * 13 + [2] + [2] * 13),                    # empty group 1
        (None, [k % 5 for k in range(13)] + [4] + [0] * 13),  # five groups
        (None, [-1] + [0] * 26),
    ]
    good = CASES["dx_slabs"]
    m.set_order(*good)
    for bo, go in bad:
        with pytest.raises(smc.SmconvError):
            m.set_order(bo, go)
    coords = synth.tiny_coords(seed=5, n=700, side=12)
    _, mask = so.build_kernel_map(coords)
    m.build(to_dev_i32(coords))
    check_orders(m, mask, good[0], good[1], "previous order kept")
    with pytest.raises(smc.SmconvError):
        m.calibrate(5)
    m.close()
