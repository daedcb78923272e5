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
    coords = np.array([[0, 0, 0, 0], [0, 2094, 2094, 694]], np.int32)
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
