"""smc_conv_forward_noalloc through the C ABI: the same results as
smc_conv_forward on the same map (both run the same deterministic kernels, so
the outputs are compared bit for bit), over two calls in a row with the
second on a smaller voxel set, on the pair-list path (the one-kernel form,
which needs no scratch, and the two-kernel form, SMC_FWD_SLAB_IN_MEMORY,
whose slab lives in the fixed array) and the grouped mask-tile path (whose
partial sums also live there); a slab above the fixed 32 MiB is refused
before any work; and, with torch's caching allocator bound to the library,
the call takes no device memory while the allocating forward does."""
import ctypes

import numpy as np
import pytest

import synth
from _util import bf16_bits_of, to_dev_bf16, to_dev_i32

pytestmark = pytest.mark.gpu

smc = pytest.importorskip("submanifold_sparse_convolution_amd")
torch = pytest.importorskip("torch")

SMC_ERR_UNSUPPORTED = 8
SCRATCH_BYTES = 32 << 20
SLAB = 8                                                  # SMC_FWD_SLAB_IN_MEMORY


def call(fn, m, x, wp, y, flags=0):
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    return fn(m._h, ctypes.c_void_p(x.data_ptr()), wp.c_in, ctypes.c_void_p(wp.buf.data_ptr()),
              wp.c_out, ctypes.c_void_p(y.data_ptr()), flags, stream)


def both(m, x, wp, flags=0, out_f32=False):
    """(allocating forward's output, no-allocation forward's output) as bit patterns."""
    L = smc.lib()
    dt = torch.float32 if out_f32 else torch.bfloat16
    ya = torch.full((m.n, wp.c_out), 7.0, dtype=dt, device="cuda")
    yb = torch.full((m.n, wp.c_out), -5.0, dtype=dt, device="cuda")
    assert call(L.smc_conv_forward, m, x, wp, ya, flags) == 0, L.smc_last_error()
    assert call(L.smc_conv_forward_noalloc, m, x, wp, yb, flags) == 0, L.smc_last_error()
    torch.cuda.synchronize()
    if out_f32:
        return ya.cpu().numpy().view(np.uint32), yb.cpu().numpy().view(np.uint32)
    return bf16_bits_of(ya), bf16_bits_of(yb)


def inputs(n, grid, c, seed, n_boxes=40):
    coords = synth.ground_box_coords(n, grid, seed=seed, n_boxes=n_boxes)
    xb = synth.features(len(coords), c, seed)
    wb = synth.weights(c, c, seed)
    return to_dev_i32(coords), to_dev_bf16(xb), smc.pack_weights(to_dev_bf16(wb))


@pytest.mark.parametrize("route", ["dense", "sorted"])
def test_noalloc_equals_forward_on_two_calls_second_smaller(route):
    m = smc.KernelMap()
    # the first build is asynchronous: for the two-kernel form 26 pairs per row
    # would exceed the fixed array, so the call waits for the build's counts
    for n, grid, c, seed, sync in ((20000, (400, 400, 24), 128, 31, False),
                                   (3001, (120, 120, 12), 64, 32, True)):
        coords_d, x_d, wp = inputs(n, grid, c, seed)
        m.build(coords_d, spatial_shape=grid, route=route, sync=sync)
        # plain, ReLU, float32 out; one kernel, then two kernels with the slab
        for flags, f32 in ((0, False), (1, False), (2, True), (SLAB, False), (SLAB | 1, False),
                           (SLAB | 2, True)):
            a, b = both(m, x_d, wp, flags, f32)
            assert a.shape == (m.n, c)
            assert np.array_equal(a, b), (n, route, flags)
    m.close()


def test_noalloc_equals_forward_grouped_mask_tiles():
    m = smc.KernelMap()
    order = [t for t in range(27) if t != 13] + [13]
    groups = [t * 3 // 27 for t in range(27)]
    groups[13] = 2
    m.set_order(order, groups)
    for n, grid, c, seed in ((12000, (300, 300, 16), 64, 41), (2500, (100, 100, 10), 32, 42)):
        coords_d, x_d, wp = inputs(n, grid, c, seed)
        m.build(coords_d, spatial_shape=grid, pairs=False)
        assert m.info()["n_groups"] == 3
        a, b = both(m, x_d, wp, 4 | 1)                    # mask tiles, ReLU
        assert np.array_equal(a, b), n
    m.close()


def test_noalloc_refuses_a_slab_above_the_fixed_array():
    # a full 40^3 box: (3 * 40 - 2)^3 pairs, 1.58M off-centre, x 16 columns x 4 bytes
    coords = synth.box_coords(40, 40, 40)
    n = len(coords)
    off_centre = (3 * 40 - 2) ** 3 - n
    assert off_centre * 16 * 4 > SCRATCH_BYTES
    m = smc.KernelMap().build(to_dev_i32(coords), spatial_shape=(40, 40, 40))
    x = to_dev_bf16(synth.features(n, 16, 5))
    wp = smc.pack_weights(to_dev_bf16(synth.weights(16, 16, 5)))
    y = torch.full((n, 16), 3.0, dtype=torch.bfloat16, device="cuda")
    L = smc.lib()
    assert call(L.smc_conv_forward_noalloc, m, x, wp, y, SLAB) == SMC_ERR_UNSUPPORTED
    assert b"fixed scratch" in L.smc_last_error()
    torch.cuda.synchronize()
    assert bool((y == 3.0).all())                         # nothing ran
    # the allocating forward still serves this map, and the one-kernel form
    # (slab rows in LDS) needs no scratch at all
    assert call(L.smc_conv_forward, m, x, wp, y, SLAB) == 0
    y2 = torch.full((n, 16), 3.0, dtype=torch.bfloat16, device="cuda")
    assert call(L.smc_conv_forward_noalloc, m, x, wp, y2) == 0, L.smc_last_error()
    torch.cuda.synchronize()
    assert bool((y == y2).all())
    m.close()


def test_noalloc_takes_no_device_memory():
    grid = (200, 200, 16)
    coords_d, x_d, wp = inputs(8000, grid, 64, 51)
    L = smc.lib()
    smc.use_torch_allocator(True)
    try:
        m = smc.KernelMap().build(coords_d, spatial_shape=grid)
        y = torch.empty((m.n, 64), dtype=torch.bfloat16, device="cuda")
        torch.cuda.synchronize()
        before = torch.cuda.memory_allocated()
        for flags in (0, SLAB):
            assert call(L.smc_conv_forward_noalloc, m, x_d, wp, y, flags) == 0, L.smc_last_error()
        torch.cuda.synchronize()
        assert torch.cuda.memory_allocated() == before
        assert call(L.smc_conv_forward, m, x_d, wp, y, SLAB) == 0   # allocates the handle's slab
        torch.cuda.synchronize()
        assert torch.cuda.memory_allocated() > before
        m.close()
    finally:
        smc.use_torch_allocator(False)
