"""smc_set_allocator through the Python binding: with torch's caching
allocator bound, every device buffer of a map handle comes from torch's pool
(torch.cuda.memory_allocated grows by it) and goes back at destroy; results
are unchanged and a buffer made before the switch is freed by hipFree."""
import numpy as np
import pytest

import synth
from _util import oracle_map_of, to_dev_bf16, to_dev_i32
from oracle import smconv_oracle as so

pytestmark = pytest.mark.gpu

smc = pytest.importorskip("submanifold_sparse_convolution_amd")
torch = pytest.importorskip("torch")


def oracle_acc(om, xb, wb):
    x = so.bf16_bits_to_f64(xb)
    w = so.bf16_bits_to_f64(wb)
    return so.conv_accumulate(x, w, om["pair_in"], om["pair_out"], om["tap_off"], x.shape[0])


def layer(m, coords_d, x_d, wp, shape):
    m.build(coords_d, spatial_shape=shape)
    return m.forward(x_d, wp, out_f32=True).cpu().numpy()


def int_weights(c, seed):
    w = np.random.default_rng(seed).integers(-2, 3, (27, c, c)).astype(np.float32)
    return synth.bf16_bits_from_f32(w)


def test_torch_allocator_holds_and_returns_the_handle_memory():
    shape = (64, 64, 16)
    coords = synth.ground_box_coords(3000, shape, seed=11, n_boxes=20)
    xb, wb = synth.int_features(3000, 32, 11), int_weights(32, 11)
    ref = oracle_acc(oracle_map_of(coords), xb, wb)
    coords_d, x_d, wp = to_dev_i32(coords), to_dev_bf16(xb), smc.pack_weights(to_dev_bf16(wb))
    torch.cuda.synchronize()
    base = torch.cuda.memory_allocated()        # inputs and packed weights are held by torch
    smc.use_torch_allocator(True)
    try:
        m = smc.KernelMap()
        acc = layer(m, coords_d, x_d, wp, shape)
        assert np.array_equal(acc.astype(np.float64), ref)
        held = torch.cuda.memory_allocated() - base
        # at least the id grid of the padded shape, 4 bytes per cell
        assert held >= 4 * 66 * 66 * 18, held
        m.close()
        torch.cuda.synchronize()
        assert torch.cuda.memory_allocated() == base
    finally:
        smc.use_torch_allocator(False)


def test_allocator_switch_keeps_each_buffer_with_its_maker():
    small = synth.ground_box_coords(500, (40, 40, 10), seed=12, n_boxes=5)
    big = synth.ground_box_coords(5000, (80, 80, 16), seed=13, n_boxes=30)
    xs, xl, wb = synth.int_features(500, 16, 12), synth.int_features(5000, 16, 13), int_weights(16, 12)
    small_d, big_d = to_dev_i32(small), to_dev_i32(big)
    xs_d, xl_d, wp = to_dev_bf16(xs), to_dev_bf16(xl), smc.pack_weights(to_dev_bf16(wb))
    torch.cuda.synchronize()
    base = torch.cuda.memory_allocated()
    m = smc.KernelMap()
    a = layer(m, small_d, xs_d, wp, (40, 40, 10))    # hipMalloc buffers
    assert torch.cuda.memory_allocated() == base
    smc.use_torch_allocator(True)
    try:
        b = layer(m, big_d, xl_d, wp, (80, 80, 16))  # grown buffers come from torch
        assert torch.cuda.memory_allocated() > base
        assert np.array_equal(a.astype(np.float64), oracle_acc(oracle_map_of(small), xs, wb))
        assert np.array_equal(b.astype(np.float64), oracle_acc(oracle_map_of(big), xl, wb))
        m.close()                                     # hipFree for the old, torch for the new
        torch.cuda.synchronize()
        assert torch.cuda.memory_allocated() == base
    finally:
        smc.use_torch_allocator(False)


def test_allocator_returning_null_is_alloc_error():
    """A caller's allocator that returns NULL makes the call fail with
    SMC_ERR_ALLOC (a fresh handle at its first build, and an initialised
    handle whose buffers must grow); NULL, NULL restores hipMalloc and the
    same handles build again."""
    import ctypes
    L = smc.lib()
    null_alloc = smc._ALLOC_T(lambda ctx, nbytes, stream: None)
    no_free = smc._FREE_T(lambda ctx, ptr, stream: None)
    small = synth.ground_box_coords(500, (40, 40, 10), seed=21, n_boxes=5)
    big = synth.ground_box_coords(6000, (90, 90, 16), seed=22, n_boxes=30)
    grown = smc.KernelMap().build(to_dev_i32(small), spatial_shape=(40, 40, 10))  # hipMalloc
    fresh = smc.KernelMap()
    assert L.smc_set_allocator(ctypes.cast(null_alloc, ctypes.c_void_p),
                               ctypes.cast(no_free, ctypes.c_void_p), None) == 0
    try:
        for m, c, shape in ((fresh, small, (40, 40, 10)), (grown, big, (90, 90, 16))):
            with pytest.raises(smc.SmconvError) as e:
                m.build(to_dev_i32(c), spatial_shape=shape)
            assert e.value.status == 5, str(e.value)
            assert "NULL" in str(e.value)
    finally:
        assert L.smc_set_allocator(None, None, None) == 0
    for m, c, shape in ((fresh, small, (40, 40, 10)), (grown, big, (90, 90, 16))):
        m.build(to_dev_i32(c), spatial_shape=shape)
        assert m.info()["pairs"] == len(oracle_map_of(c)["pair_in"])
        m.close()
