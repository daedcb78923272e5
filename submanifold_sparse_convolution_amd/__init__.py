"""Submanifold sparse 3x3x3 convolution on MI355X: Python binding.

A thin ctypes layer over libsmconv.so (C ABI in include/smconv.h). It only
marshals arguments: torch tensors supply device memory and the current HIP
stream, every step of the computation runs in the library's HIP kernels.
There is no fallback: if the library is not built, every call raises.

    m = KernelMap()
    m.build(coords, spatial_shape=(1440, 1440, 41))     # int32 [N, 4] on the GPU
    wp = pack_weights(w)                                 # bf16 [27, C_in, C_out]
    y = m.forward(x, wp, relu=True)                      # bf16 [N, C_in] -> [N, C_out]
"""
from __future__ import annotations

import ctypes
import os

__all__ = ["KernelMap", "PackedWeights", "pack_weights", "subm_conv3d", "lib", "library_path",
           "SmconvError", "ROUTES", "EXPORTED_SYMBOLS", "use_torch_allocator", "probe_mfma_bf16",
           "probe_copy"]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libsmconv.so")

ROUTES = {"auto": 0, "dense": 1, "sorted": 2}
_ROUTE_NAMES = {v: k for k, v in ROUTES.items()}
SMC_BUILD_ASYNC = 1
SMC_FWD_RELU = 1
SMC_FWD_OUT_F32 = 2
SMC_FWD_MASK_TILES = 4
SMC_FWD_SLAB_IN_MEMORY = 8
SMC_BUILD_NO_PAIRS = 2
SMC_BUILD_NO_SORT = 4
SMC_BUILD_TABLE = 8
ALGOS = ("pairs", "pairs_slab", "mask_tiles")

EXPORTED_SYMBOLS = [
    "smc_map_create", "smc_map_destroy", "smc_map_build", "smc_map_sync", "smc_map_info",
    "smc_map_export", "smc_weight_packed_bytes", "smc_weight_pack", "smc_conv_forward",
    "smc_status_string", "smc_last_error", "smc_version", "smc_timing_enable", "smc_timing_read",
    "smc_map_set_order", "smc_map_calibrate", "smc_map_build_strided",
    "smc_map_export_out_coords", "smc_set_allocator", "smc_probe_mfma_out_bytes",
    "smc_probe_mfma_bf16", "smc_probe_copy", "smc_conv_forward_noalloc",
    "smc_test_force_lookback_timeout", "smc_map_rows",
]
STAGES = ["map", "neighbours", "mask_sort", "compact", "gemm", "centre"]


class SmconvError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(msg)
        self.status = status


class MapInfo(ctypes.Structure):
    _fields_ = [
        ("n", ctypes.c_int64), ("route", ctypes.c_int32), ("key_bits", ctypes.c_int32),
        ("origin", ctypes.c_int32 * 3), ("extent", ctypes.c_int32 * 3),
        ("batch", ctypes.c_int32), ("tile_m", ctypes.c_int32), ("grid_cells", ctypes.c_int64),
        ("pairs", ctypes.c_int64), ("pairs_padded", ctypes.c_int64), ("n_tiles", ctypes.c_int64),
        ("tap_count", ctypes.c_int64 * 125), ("status", ctypes.c_int32),
        ("n_groups", ctypes.c_int32), ("group_rows", ctypes.c_int64 * 4),
        ("kernel_size", ctypes.c_int32), ("taps", ctypes.c_int32),
        ("n_in", ctypes.c_int64), ("strided", ctypes.c_int32), ("out_extent", ctypes.c_int32 * 3),
    ]


_lib = None


def library_path() -> str:
    return _LIB_PATH


def lib():
    """Load libsmconv.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(f"{_LIB_PATH} is not built; run `python __graft_entry__.py build` "
                           "(hipcc --offload-arch=gfx950) first")
    # torch ships its own HIP runtime under the same soname (libamdhip64.so.7).
    # Importing torch first makes the library bind to that runtime, the one
    # that owns the tensors and streams handed over; loaded first, the library
    # would pull in a second runtime that cannot use them.
    import torch  # noqa: F401
    L = ctypes.CDLL(_LIB_PATH)
    vp, i32, i64, u32 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_uint
    L.smc_map_create.argtypes = [ctypes.POINTER(vp)]
    L.smc_map_destroy.argtypes = [vp]
    L.smc_map_build.argtypes = [vp, vp, i64, i32, vp, i32, i32, i32, u32, vp]
    L.smc_map_sync.argtypes = [vp]
    L.smc_map_info.argtypes = [vp, ctypes.POINTER(MapInfo)]
    L.smc_map_rows.argtypes = [vp, ctypes.POINTER(i64), ctypes.POINTER(i64)]
    L.smc_map_export.argtypes = [vp, vp, vp, vp, vp, vp, vp]
    L.smc_weight_packed_bytes.argtypes = [i32, i32, i32]
    L.smc_weight_packed_bytes.restype = ctypes.c_size_t
    L.smc_weight_pack.argtypes = [vp, i32, i32, i32, vp, vp]
    L.smc_conv_forward.argtypes = [vp, vp, i32, vp, i32, vp, u32, vp]
    L.smc_conv_forward_noalloc.argtypes = [vp, vp, i32, vp, i32, vp, u32, vp]
    L.smc_test_force_lookback_timeout.argtypes = [vp, i32]
    L.smc_status_string.argtypes = [i32]
    L.smc_status_string.restype = ctypes.c_char_p
    L.smc_last_error.argtypes = []
    L.smc_last_error.restype = ctypes.c_char_p
    L.smc_version.restype = i32
    L.smc_timing_enable.argtypes = [vp, i32]
    L.smc_timing_read.argtypes = [vp, vp, vp, i32]
    L.smc_map_set_order.argtypes = [vp, vp, vp]
    L.smc_map_calibrate.argtypes = [vp, i32, vp, vp]
    L.smc_map_build_strided.argtypes = [vp, vp, i64, i32, vp, i32, i32, i32, i32, u32, vp]
    L.smc_map_export_out_coords.argtypes = [vp, vp]
    L.smc_set_allocator.argtypes = [vp, vp, vp]
    L.smc_probe_mfma_out_bytes.argtypes = [i32]
    L.smc_probe_mfma_out_bytes.restype = ctypes.c_size_t
    L.smc_probe_mfma_bf16.argtypes = [i64, vp, ctypes.c_size_t, ctypes.POINTER(ctypes.c_double), vp]
    L.smc_probe_copy.argtypes = [vp, vp, ctypes.c_size_t, vp]
    for name in ("smc_map_create", "smc_map_destroy", "smc_map_build", "smc_map_sync",
                 "smc_map_info", "smc_map_export", "smc_weight_pack", "smc_conv_forward",
                 "smc_timing_enable", "smc_timing_read", "smc_map_set_order",
                 "smc_map_calibrate", "smc_map_build_strided", "smc_map_export_out_coords",
                 "smc_set_allocator", "smc_probe_mfma_bf16", "smc_probe_copy",
                 "smc_conv_forward_noalloc", "smc_test_force_lookback_timeout", "smc_map_rows"):
        getattr(L, name).restype = i32
    _lib = L
    return L


_ALLOC_T = ctypes.CFUNCTYPE(ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p)
_FREE_T = ctypes.CFUNCTYPE(None, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p)
_allocator_refs = []        # every callback pair ever handed over: buffers free through them


def use_torch_allocator(on: bool = True):
    """Take every device buffer that map handles allocate from now on (builds,
    forwards, growth) from torch's caching allocator, on the stream of the call
    that needs it, so that torch's pool holds all of the library's device
    memory; on=False goes back to hipMalloc/hipFree. Buffers keep the
    allocator that made them (smc_set_allocator)."""
    import torch
    L = lib()
    if not on:
        _check(L.smc_set_allocator(None, None, None))
        return

    def _alloc(ctx, nbytes, stream):
        try:
            return torch.cuda.caching_allocator_alloc(int(nbytes), stream=stream or None)
        except Exception:
            return None                # the library reports SMC_ERR_ALLOC

    def _free(ctx, ptr, stream):
        try:
            torch.cuda.caching_allocator_delete(ptr)
        except Exception:
            pass

    fa, ff = _ALLOC_T(_alloc), _FREE_T(_free)
    _allocator_refs.append((fa, ff))
    _check(L.smc_set_allocator(ctypes.cast(fa, ctypes.c_void_p), ctypes.cast(ff, ctypes.c_void_p),
                               None))


def _check(status: int):
    if status != 0:
        L = lib()
        raise SmconvError(status, f"{L.smc_status_string(status).decode()}: "
                                  f"{L.smc_last_error().decode()}")


def _stream(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _need(t, dtype, name, ndim=None):
    import torch
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA (HIP) torch tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


class PackedWeights:
    """Weights packed for the GEMM; holds the device buffer."""

    def __init__(self, buf, c_in: int, c_out: int, kernel_size: int = 3):
        self.buf, self.c_in, self.c_out, self.kernel_size = buf, c_in, c_out, kernel_size


_KSIZE_OF_TAPS = {27: 3, 125: 5}


def pack_weights(w, out: PackedWeights = None, stream=None) -> PackedWeights:
    """bf16 [K^3, C_in, C_out] CUDA tensor (K = 3 or 5) -> PackedWeights
    (into ``out`` if given)."""
    import torch
    _need(w, torch.bfloat16, "w", 3)
    if int(w.shape[0]) not in _KSIZE_OF_TAPS:
        raise ValueError("w must be [27, C_in, C_out] or [125, C_in, C_out]")
    k = _KSIZE_OF_TAPS[int(w.shape[0])]
    c_in, c_out = int(w.shape[1]), int(w.shape[2])
    L = lib()
    nbytes = L.smc_weight_packed_bytes(k, c_in, c_out)
    if out is not None:
        if (out.c_in, out.c_out, out.kernel_size) != (c_in, c_out, k):
            raise ValueError("out was packed for other channel counts or kernel size")
        buf = out.buf
    else:
        buf = torch.empty(nbytes, dtype=torch.uint8, device=w.device)
    _check(L.smc_weight_pack(ctypes.c_void_p(w.data_ptr()), k, c_in, c_out,
                             ctypes.c_void_p(buf.data_ptr()), _stream(stream)))
    return PackedWeights(buf, c_in, c_out, k)


class KernelMap:
    """A kernel map handle: built from coordinates, reused by every layer."""

    def __init__(self):
        self._h = ctypes.c_void_p()
        _check(lib().smc_map_create(ctypes.byref(self._h)))
        self.n = 0
        self.n_in = 0
        self.kernel_size = 3
        self.strided = False
        self._coords = None

    def close(self):
        """Destroy the handle (waits for its work) and drop the last coordinates."""
        if self._h:
            lib().smc_map_destroy(self._h)
            self._h = ctypes.c_void_p()
        self._coords = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def build(self, coords, spatial_shape=None, batch_size: int = 0, route: str = "auto",
              sync: bool = True, pairs: bool = True, sort: bool = True,
              kernel_size: int = 3, table: bool = False, stream=None) -> "KernelMap":
        """coords: int32 [N, 4] (b, x, y, z) or [N, 3] (x, y, z) CUDA tensor.

        pairs=False skips the per-tap pair lists (algo="pairs" then refuses the
        map); sort=False skips the mask-sorted row order (algo="mask_tiles"
        then refuses it). kernel_size 3 or 5 (a 5x5x5 map has pair lists and
        no mask order). table=True keeps the neighbour table in device memory
        where the build would leave it out (dense route, 3x3x3, pair lists
        without the mask order); export() returns the table either way."""
        import torch
        _need(coords, torch.int32, "coords", 2)
        n, ncols = int(coords.shape[0]), int(coords.shape[1])
        shape = None
        if spatial_shape is not None:
            shape = (ctypes.c_int32 * 3)(*[int(v) for v in spatial_shape])
        flags = ((0 if sync else SMC_BUILD_ASYNC) | (0 if pairs else SMC_BUILD_NO_PAIRS)
                 | (0 if sort else SMC_BUILD_NO_SORT) | (SMC_BUILD_TABLE if table else 0))
        if kernel_size == 5:
            flags |= SMC_BUILD_NO_SORT
        self._coords = coords          # keep alive while the stream reads it
        self.n = self.n_in = n
        self.strided = False
        _check(lib().smc_map_build(self._h, ctypes.c_void_p(coords.data_ptr() if n else 0), n,
                                   ncols, shape, int(batch_size), int(kernel_size), ROUTES[route],
                                   flags, _stream(stream)))
        self.kernel_size = int(kernel_size)
        return self

    def build_strided(self, coords, spatial_shape=None, batch_size: int = 0, route: str = "auto",
                      sync: bool = True, kernel_size: int = 3, stride: int = 2,
                      pairs: bool = True, sort: bool = True, stream=None) -> "KernelMap":
        """Downsampling map (kernel 3, stride 2, padding 1) of int32 [N, 4] / [N, 3]
        CUDA coordinates; outputs are new cells (``out_coords()``), ``n`` of them.
        pairs: per-tap pair lists over the output rows (forward algo "pairs");
        sort: the mask order of the output rows (forward algo "mask_tiles")."""
        import torch
        _need(coords, torch.int32, "coords", 2)
        n, ncols = int(coords.shape[0]), int(coords.shape[1])
        shape = None
        if spatial_shape is not None:
            shape = (ctypes.c_int32 * 3)(*[int(v) for v in spatial_shape])
        self._coords = coords
        self.n, self.n_in, self.strided = 0, n, True
        _check(lib().smc_map_build_strided(
            self._h, ctypes.c_void_p(coords.data_ptr() if n else 0), n, ncols, shape,
            int(batch_size), int(kernel_size), int(stride), ROUTES[route],
            (0 if sync else SMC_BUILD_ASYNC) | (0 if pairs else SMC_BUILD_NO_PAIRS)
            | (0 if sort else SMC_BUILD_NO_SORT), _stream(stream)))
        # the output count: waits for its own event only (the lookup and
        # compaction after it are still running)
        rows = ctypes.c_int64()
        _check(lib().smc_map_rows(self._h, ctypes.byref(rows), None))
        self.n, self.n_in, self.kernel_size, self.strided = rows.value, n, int(kernel_size), True
        return self

    def out_coords(self):
        """Output coordinates of a strided map: numpy int32 [n, 4] (b, x, y, z)."""
        import numpy as np
        out = np.empty((self.n, 4), np.int32)
        _check(lib().smc_map_export_out_coords(
            self._h, ctypes.c_void_p(out.ctypes.data) if out.size else None))
        return out

    def sync(self):
        _check(lib().smc_map_sync(self._h))

    def set_order(self, bit_order=None, group_of=None) -> "KernelMap":
        """Bit order (27 taps, most significant first) and offset groups (group
        of each tap) of the mask sort of later builds; None: plain / one group."""
        arr = {}
        for name, v in (("bit_order", bit_order), ("group_of", group_of)):
            if v is not None:
                v = [int(t) for t in v]
                if len(v) != 27:
                    raise ValueError(f"{name} must have 27 entries")
                arr[name] = (ctypes.c_int32 * 27)(*v)
        _check(lib().smc_map_set_order(self._h, arr.get("bit_order"), arr.get("group_of")))
        return self

    def calibrate(self, n_groups: int = 1):
        """(bit_order, group_of) chosen on this built map (see smc_map_calibrate)."""
        order = (ctypes.c_int32 * 27)()
        groups = (ctypes.c_int32 * 27)()
        _check(lib().smc_map_calibrate(self._h, int(n_groups), order, groups))
        return list(order), list(groups)

    def timing(self, on: bool = True):
        """Record HIP events around each stage of later builds and forwards."""
        _check(lib().smc_timing_enable(self._h, 1 if on else 0))

    def timing_read(self, reset: bool = True) -> dict:
        """{stage: (total_ms, calls)} of the timed work (waits for it)."""
        ms = (ctypes.c_double * len(STAGES))()
        calls = (ctypes.c_int64 * len(STAGES))()
        _check(lib().smc_timing_read(self._h, ms, calls, 1 if reset else 0))
        return {name: (ms[i], calls[i]) for i, name in enumerate(STAGES)}

    def info(self) -> dict:
        inf = MapInfo()
        _check(lib().smc_map_info(self._h, ctypes.byref(inf)))
        return dict(n=inf.n, route=_ROUTE_NAMES.get(inf.route, inf.route), key_bits=inf.key_bits,
                    origin=tuple(inf.origin), extent=tuple(inf.extent), batch=inf.batch,
                    tile_m=inf.tile_m, grid_cells=inf.grid_cells, pairs=inf.pairs,
                    pairs_padded=inf.pairs_padded, n_tiles=inf.n_tiles,
                    tap_count=list(inf.tap_count)[:inf.taps], status=inf.status,
                    n_groups=inf.n_groups, group_rows=list(inf.group_rows)[:inf.n_groups],
                    kernel_size=inf.kernel_size, taps=inf.taps, n_in=inf.n_in,
                    strided=bool(inf.strided), out_extent=tuple(inf.out_extent))

    def export(self, pairs: bool = True, perm: bool = True) -> dict:
        """Copy nbr, mask, tap offsets (and the mask-tile row orders [G, N], the
        pair lists) to numpy (host)."""
        import numpy as np
        info = self.info()
        n, p, taps = info["n"], info["pairs"], info["taps"]
        out = dict(nbr=np.empty((n, taps), np.int32),
                   mask=np.empty(n if taps == 27 else (n, 4), np.uint32),
                   tap_off=np.empty(taps + 1, np.int64))
        if perm:
            out["perm"] = np.empty((max(info["n_groups"], 1), n), np.int32)
            out["group_rows"] = np.asarray(info["group_rows"], np.int64)
        if pairs:
            out["pair_in"] = np.empty(p, np.int32)
            out["pair_out"] = np.empty(p, np.int32)

        def ptr(key):
            a = out.get(key)
            return ctypes.c_void_p(a.ctypes.data) if a is not None and a.size else None
        _check(lib().smc_map_export(self._h, ptr("nbr"), ptr("mask"), ptr("perm"),
                                    ptr("pair_in"), ptr("pair_out"), ptr("tap_off")))
        return out

    def forward(self, x, w: PackedWeights, relu: bool = False, out=None, out_f32: bool = False,
                algo: str = "pairs", stream=None):
        """x: bf16 [N, C_in] CUDA tensor -> bf16 [N, C_out] (float32 with out_f32).

        algo: "pairs" (per-tap pair lists: each row is its centre product plus
        its partial-product slab rows; one kernel with the slab in LDS for
        3x3x3 maps and C_in, C_out <= 64 (C_in a multiple of 8), else two kernels with the
        slab in device memory), "pairs_slab" (always the two-kernel form) or
        "mask_tiles" (output-stationary tiles of mask-sorted rows)."""
        if algo not in ALGOS:
            raise ValueError(f"algo must be one of {ALGOS}")
        import torch
        _need(x, torch.bfloat16, "x", 2)
        if x.shape[0] != self.n_in:
            raise ValueError(f"x has {x.shape[0]} rows, the map has {self.n_in} inputs")
        if x.shape[1] != w.c_in:
            raise ValueError(f"x has {x.shape[1]} channels, weights expect {w.c_in}")
        if w.kernel_size != self.kernel_size:
            raise ValueError(f"weights are {w.kernel_size}^3, the map is {self.kernel_size}^3")
        odt = torch.float32 if out_f32 else torch.bfloat16
        if out is None:
            out = torch.empty((self.n, w.c_out), dtype=odt, device=x.device)
        else:
            _need(out, odt, "out", 2)
            if tuple(out.shape) != (self.n, w.c_out):
                raise ValueError("out has the wrong shape")
        _check(lib().smc_conv_forward(self._h, ctypes.c_void_p(x.data_ptr()), w.c_in,
                                      ctypes.c_void_p(w.buf.data_ptr()), w.c_out,
                                      ctypes.c_void_p(out.data_ptr()),
                                      (SMC_FWD_RELU if relu else 0)
                                      | (SMC_FWD_OUT_F32 if out_f32 else 0)
                                      | (SMC_FWD_MASK_TILES if algo == "mask_tiles" else 0)
                                      | (SMC_FWD_SLAB_IN_MEMORY if algo == "pairs_slab" else 0),
                                      _stream(stream)))
        return out


def subm_conv3d(coords, x, w, spatial_shape=None, relu: bool = False, route: str = "auto"):
    """One layer from raw inputs: builds a map (kernel size from w: 27 or 125
    taps), packs w, runs the layer."""
    wp = pack_weights(w)
    m = KernelMap().build(coords, spatial_shape=spatial_shape, route=route,
                          kernel_size=wp.kernel_size)
    return m.forward(x, wp, relu=relu)


def probe_mfma_bf16(iters: int, stream=None) -> float:
    """Enqueue the MFMA-only probe kernel on the stream; returns the flops it
    executes (the caller times it)."""
    import torch
    L = lib()
    n_cu = torch.cuda.get_device_properties(torch.cuda.current_device()).multi_processor_count
    nbytes = L.smc_probe_mfma_out_bytes(n_cu)
    out = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda")
    flops = ctypes.c_double()
    _check(L.smc_probe_mfma_bf16(int(iters), ctypes.c_void_p(out.data_ptr()), nbytes,
                                 ctypes.byref(flops), _stream(stream)))
    probe_mfma_bf16._keep = out          # alive until the stream has run the kernel
    return flops.value


def probe_copy(dst, src, stream=None):
    """dst[:] = src[:] (CUDA tensors of equal byte size) by the library's copy probe."""
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != nbytes:
        raise ValueError("dst and src differ in size")
    _check(lib().smc_probe_copy(ctypes.c_void_p(dst.data_ptr()), ctypes.c_void_p(src.data_ptr()),
                                nbytes, _stream(stream)))
