"""The C-ABI library loads and exports every symbol its header declares.

Runs without a GPU: the calls made here only validate arguments or report
static information, none launches a kernel.
"""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "smconv.h")

smc = pytest.importorskip("submanifold_sparse_convolution_amd")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(smc_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(smc.library_path()):
        pytest.fail("libsmconv.so is not built (run __graft_entry__.build())")
    return smc.lib()


def test_header_declares_the_binding_symbols():
    assert declared_functions() == sorted(smc.EXPORTED_SYMBOLS)


def test_every_declared_symbol_is_exported(L):
    nm = subprocess.run(["nm", "-D", "--defined-only", smc.library_path()],
                        capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\b[Tt]\s+(smc_[a-z0-9_]+)$", nm, flags=re.M))
    for name in declared_functions():
        assert name in exported, name
        assert getattr(L, name) is not None


def test_static_calls(L):
    assert L.smc_version() >= 100
    assert L.smc_status_string(0) == b"ok"
    assert L.smc_status_string(2) == b"duplicate coordinates"
    assert L.smc_status_string(999) == b"unknown status"
    # packed weights: K^3 taps x ceil(co/16) x ceil(ci/32) x 64 lanes x 16 bytes
    # (column blocks padded to the wave tile), and for K = 3 with c_in, c_out
    # <= 64 (c_in a multiple of 8) a second copy in 32-column tiles for the
    # one-kernel forward, unless the first already has 2 column blocks per tile;
    # for c_in <= 128 and c_out > 64 a second copy in 64-column tiles for the
    # off-centre kernel
    assert L.smc_weight_packed_bytes(3, 128, 128) == 2 * 27 * 8 * 4 * 64 * 16
    assert L.smc_weight_packed_bytes(3, 64, 64) == 2 * 27 * 4 * 2 * 64 * 16
    assert L.smc_weight_packed_bytes(3, 64, 128) == 2 * 27 * 8 * 2 * 64 * 16
    assert L.smc_weight_packed_bytes(3, 32, 96) == 27 * 8 * 64 * 16 + 27 * 2 * 4 * 64 * 16
    assert L.smc_weight_packed_bytes(3, 40, 72) == 27 * 8 * 2 * 64 * 16 + 27 * 2 * 2 * 4 * 64 * 16
    assert L.smc_weight_packed_bytes(3, 16, 32) == 27 * 2 * 1 * 64 * 16
    assert L.smc_weight_packed_bytes(3, 136, 128) == 27 * 8 * 5 * 64 * 16
    assert L.smc_weight_packed_bytes(3, 1, 1) == 27 * 1 * 1 * 64 * 16
    assert L.smc_weight_packed_bytes(5, 64, 32) == 125 * 2 * 2 * 64 * 16
    assert L.smc_weight_packed_bytes(3, 0, 5) == 0
    assert L.smc_weight_packed_bytes(4, 16, 16) == 0


def test_argument_errors_without_gpu(L):
    h = ctypes.c_void_p()
    assert L.smc_map_create(ctypes.byref(h)) == 0
    # kernel_size 4 -> unsupported; 5 without pair lists -> unsupported; ncols 2 -> arg;
    # n < 0 -> arg; no GPU work happens
    assert L.smc_map_build(h, None, 0, 4, None, 0, 4, 0, 0, None) == 8
    assert L.smc_map_build(h, None, 0, 4, None, 0, 5, 0, 2, None) == 8
    assert L.smc_map_build(h, None, 0, 2, None, 0, 3, 0, 0, None) == 1
    assert L.smc_map_build(h, None, -1, 4, None, 0, 3, 0, 0, None) == 1
    assert L.smc_map_build(h, None, 0, 4, None, 0, 3, 7, 0, None) == 1
    assert b"route" in L.smc_last_error()
    assert L.smc_map_build(None, None, 0, 4, None, 0, 3, 0, 0, None) == 1
    info = smc.MapInfo()
    assert L.smc_map_info(h, ctypes.byref(info)) == 7          # never built
    assert L.smc_map_sync(h) == 7
    assert L.smc_conv_forward(h, None, 16, None, 16, None, 0, None) == 7
    assert L.smc_weight_pack(None, 3, 16, 16, None, None) == 1
    assert L.smc_map_destroy(h) == 0
    assert L.smc_map_destroy(None) == 0
    # the allocator pair: both set or both NULL
    free_only = ctypes.CFUNCTYPE(None, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p)(
        lambda ctx, p, s: None)
    assert L.smc_set_allocator(None, ctypes.cast(free_only, ctypes.c_void_p), None) == 1
    assert b"both" in L.smc_last_error()
    assert L.smc_set_allocator(None, None, None) == 0


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    import importlib
    mod = importlib.import_module("submanifold_sparse_convolution_amd")
    monkeypatch.setattr(mod, "_LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(mod, "_lib", None)
    with pytest.raises(RuntimeError, match="not built"):
        mod.lib()


def test_host_code_under_asan_and_ubsan(tmp_path):
    """The library's host code (the C ABI source) built with AddressSanitizer
    and UndefinedBehaviorSanitizer (host pass only; the kernels are the
    regular objects) and driven by a C program through every argument-error
    path of the header: no sanitizer report, every status as documented."""
    build = os.path.join(ROOT, "_build")
    objs = sorted(f for f in os.listdir(build) if f.endswith(".o")) if os.path.isdir(build) else []
    if "smconv_api.o" not in objs:
        pytest.fail("the library objects are not built (run __graft_entry__.build())")
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    clang = "/opt/rocm/llvm/bin/clang"
    inc = ["-I", os.path.join(ROOT, "include")]
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined"]
    api_o = str(tmp_path / "smconv_api.o")
    lib = str(tmp_path / "libsmconv_asan.so")
    src = os.path.join(ROOT, "submanifold_sparse_convolution_amd", "csrc", "smconv_api.hip")
    subprocess.run([hipcc, "-O1", "-g", "-std=c++17", "-fPIC", "--offload-arch=gfx950",
                    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", *san, *inc,
                    "-c", src, "-o", api_o], check=True, capture_output=True)
    others = [os.path.join(build, f) for f in objs if f != "smconv_api.o"]
    subprocess.run([hipcc, "-shared", "-fPIC", "--offload-arch=gfx950", *san, api_o, *others,
                    "-o", lib], check=True, capture_output=True)
    exe = str(tmp_path / "abi_host_check")
    subprocess.run([clang, "-O1", "-g", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=undefined", *inc,
                    os.path.join(ROOT, "tests", "abi_host_check.c"), lib,
                    "-Wl,-rpath," + str(tmp_path), "-o", exe], check=True, capture_output=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", HIP_VISIBLE_DEVICES="")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "abi host check ok" in r.stdout
