"""Error paths of the C ABI that need a GPU (all force the condition from the
host side; every kernel still runs to completion)."""
import numpy as np
import pytest

import synth
from _util import to_dev_bf16, to_dev_i32

pytestmark = pytest.mark.gpu

smc = pytest.importorskip("submanifold_sparse_convolution_amd")


def status_of(fn):
    try:
        fn()
    except smc.SmconvError as e:
        return e.status
    return 0


@pytest.mark.parametrize("route", ["dense", "sorted"])
def test_duplicate_coordinates(route):
    coords = synth.tiny_coords(seed=1, n=500, side=10)
    coords[123] = coords[400]
    m = smc.KernelMap()
    assert status_of(lambda: m.build(to_dev_i32(coords), route=route)) == 2
    x = to_dev_bf16(synth.features(500, 16, 1))
    wp = smc.pack_weights(to_dev_bf16(synth.weights(16, 16, 1)))
    assert status_of(lambda: m.forward(x, wp)) == 7          # refused: build failed
    # the same handle recovers with a valid set
    good = synth.tiny_coords(seed=2, n=500, side=10)
    m.build(to_dev_i32(good), route=route)
    m.forward(x, wp)
    m.close()


@pytest.mark.parametrize("route", ["dense", "sorted"])
def test_out_of_range(route):
    coords = synth.tiny_coords(seed=1, n=300, side=10)
    coords[7, 3] = 10                                   # z == Z
    m = smc.KernelMap()
    assert status_of(lambda: m.build(to_dev_i32(coords), spatial_shape=(10, 10, 10),
                                      route=route)) == 3
    coords[7, 3] = -1
    assert status_of(lambda: m.build(to_dev_i32(coords), spatial_shape=(10, 10, 10),
                                      route=route)) == 3
    m.close()


def test_async_build_reports_on_sync():
    coords = synth.tiny_coords(seed=1, n=300, side=10)
    coords[5] = coords[6]
    m = smc.KernelMap()
    m.build(to_dev_i32(coords), sync=False)
    assert status_of(m.sync) == 2
    m.close()


def test_dense_forced_on_huge_grid():
    # 8194 x 8194 x 1026 padded cells: past 2^36, where a bitmap word index
    # would no longer fit an int32
    coords = np.array([[0, 0, 0, 0], [0, 8191, 8191, 1023]], np.int32)
    m = smc.KernelMap()
    assert status_of(lambda: m.build(to_dev_i32(coords), route="dense")) == 9
    m.build(to_dev_i32(coords))                          # auto picks the sorted route
    assert m.info()["route"] == "sorted"
    m.close()


def test_key_overflow():
    coords = np.array([[0, 0, 0, 0]], np.int32)
    m = smc.KernelMap()
    shape = (1 << 30, 1 << 30, 1 << 30)
    assert status_of(lambda: m.build(to_dev_i32(coords), spatial_shape=shape, batch_size=4)) == 4
    m.close()


def test_forward_before_build():
    import ctypes
    m = smc.KernelMap()
    x = to_dev_bf16(synth.features(10, 16, 1))
    y = to_dev_bf16(synth.features(10, 16, 2))
    wp = smc.pack_weights(to_dev_bf16(synth.weights(16, 16, 1)))
    rc = smc.lib().smc_conv_forward(m._h, ctypes.c_void_p(x.data_ptr()), 16,
                                    ctypes.c_void_p(wp.buf.data_ptr()), 16,
                                    ctypes.c_void_p(y.data_ptr()), 0, None)
    assert rc == 7
    m.close()


def test_forced_lookback_timeout_reports_hip_error():
    """The device-side look-back wait running out (forced from the host: the
    compaction waits for an epoch no block publishes, 64 polls at most) is
    latched and reported as SMC_ERR_HIP by the build; the forward refuses the
    map; with the hook off the same handle builds a correct map again."""
    from _util import assert_map_equal, oracle_map_of
    L = smc.lib()
    w = synth.workload("lidar")
    coords = synth.make_coords(w)
    m = smc.KernelMap()
    assert L.smc_test_force_lookback_timeout(m._h, 1) == 0
    assert status_of(lambda: m.build(to_dev_i32(coords), spatial_shape=w.grid, sort=False)) == 6
    assert b"ran out" in L.smc_last_error()
    x = to_dev_bf16(synth.features(len(coords), 128, 2))
    wp = smc.pack_weights(to_dev_bf16(synth.weights(128, 128, 2)))
    assert status_of(lambda: m.forward(x, wp)) == 7
    assert L.smc_test_force_lookback_timeout(m._h, 0) == 0
    m.build(to_dev_i32(coords), spatial_shape=w.grid, sort=False)
    got = m.export(perm=False)
    want = dict(oracle_map_of(coords))
    want.pop("perm")
    assert_map_equal(got, want, "after the forced timeout")
    m.close()


@pytest.mark.parametrize("route", ["dense", "sorted"])
def test_async_builds_do_not_lose_checks(route):
    """Asynchronous builds do not wait for each other: a failed check of an
    earlier one (duplicates) reaches the next wait through the sticky status
    word when the later build recycles its record; the wait after that is
    clean again."""
    bad = synth.tiny_coords(seed=1, n=400, side=10)
    bad[10] = bad[20]
    good = synth.tiny_coords(seed=2, n=400, side=10)
    m = smc.KernelMap()
    m.build(to_dev_i32(bad), route=route, sync=False)
    m.build(to_dev_i32(good), route=route, sync=False)
    m.build(to_dev_i32(good), route=route, sync=False)
    assert status_of(m.sync) == 2
    m.build(to_dev_i32(good), route=route, sync=False)
    m.sync()
    assert m.info()["status"] == 0
    m.close()
