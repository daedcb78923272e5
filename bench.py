#!/usr/bin/env python3
"""Benchmark: microseconds per submanifold 3x3x3 layer including the kernel
map, effective TFLOP/s on useful MACs, and the roofline of the dominant
kernel, on the five seeded synthetic voxel sets.

One step = one pass of the whole hot path over one voxel set already
resident in HBM: build the kernel map from raw coordinates (route, neighbour
search with masks, compaction into per-tap pair lists) and run the layer(s)
(gather -> MFMA -> slab -> centre-tap GEMM with the bf16 finalize). Weights
are packed once before the timed region (a packed weight is reused by every
forward); the packing time is reported on its own.

The headline (the JSON line's "value") is the Stage set: 91,000 voxels,
C = 128, six layers with independent weights sharing one map built every
step, ReLU between layers; value = (map + 6 layers) / 6 microseconds per
layer. Beside it, "configs" holds every set (tiny, lidar, deep, wide,
stage) with its own timing, roofline, cold and warm map builds and the CPU
oracle timed on the host cores (map and compute apart). "strided" holds the
downsampling layers, "peaks_measured" an MFMA-only loop and a device copy,
"wide_sorted_route" the Wide set with the sorted mapper forced (the auto route
maps its 3.06e9-cell grid densely when 13 GB fit the dense-grid budget).

Timing: W warm-up steps, then a timed region of exactly K steps between
device synchronisations, repeated three times; ms_per_step is the median
region's wall clock per step.

Prints ONE JSON line. --gpus above 1 exits: the library runs on one GPU.

Kernel durations come from a second pass with the library's stage timers:
every kernel records one stop event (without the system fence) on the
library's stream and is charged the interval from the previous kernel's stop
to its own, so the kernels' times add up to the step and a single-kernel
stage's average is that kernel's average interval.

Algorithmic bytes of a launch are the compulsory ones only: every input
that comes from outside the layer and every output it leaves, each once.
Intermediates of the method (the grid, keys, sort passes, the slab, row
bases) count zero.
  k_gemm_centre     2 N C_in (x) + 2 C_in C_out (centre weights) + 2 N C_out (y)
  k_gemm_nc         2 (T-1) C_in C_out (off-centre weights) + 8 (P - N) (pair lists)
  k_gemm_rows       2 N C_in + 2 T C_in C_out + 8 (P - N) + 2 N C_out (the two above in one)
  (the *_big kernels of wide inputs: as k_gemm_nc / k_gemm_centre)
  k_dense_scatter / k_make_keys   16 N (coordinates)
  k_lookup_compact  16 N (coordinates) + 4 N (masks) + 8 P (pair lists) [+ 4 T N table]
  k_compact         4 N (masks) + 8 P (pair lists)
  k_sorted_lookup / k_dense_lookup   4 N masks [+ 4 T N table]
  k_conv_masktile   2 N C_in + 2 T C_in C_out + 2 N C_out (+ 8 N C_out per extra group pass)
  strided layers (M output rows): k_gemm_nc 2 N C_in + 2 T C_in C_out + 8 P (every tap),
                    k_slab_sum 2 M C_out, k_lookup_compact (dense route: the M query
                    points' lookup inside the compaction) 16 M + 4 M + 8 P
  sort passes, k_weight_pack (outside the step), fills: 0
A stage of several kernels (a strided map's neighbour stage: the input grid or
sorted keys, the output cells through a bitmap of the output grid or, above
2^30 cells, a sort of candidate keys, and on the sorted route the query
lookup) is listed with its
kernels and time but has no byte model and is never the roofline's kernel;
"output_cells_route" says which output route a strided build took.

  --summarize-pmc FETCH_DIR WRITE_DIR   turn two `rocprofv3 --pmc FETCH_SIZE`
      / `--pmc WRITE_SIZE` runs of this script (with --copy-probe-mb) into
      profiles/traffic_<workload>_<algo>.json (with --strided-layer:
      traffic_<workload>_strided.json, runs that time the stride-2 layer), which
      later runs read for the roofline's "traffic" (null when a kernel source
      changed since).
  --summarize-mfma PMC_DIR BENCH_OUT   turn one `rocprofv3 --pmc
      SQ_INSTS_VALU_MFMA_MOPS_BF16 SQ_VALU_MFMA_BUSY_CYCLES` run of this script
      (its stdout saved in BENCH_OUT) into profiles/mfma_<workload>_<algo>.json:
      executed vs useful MFMA flops and the MFMA busy share of the GEMM kernels.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "µs per subm-conv layer incl. map + effective TFLOP/s (useful MACs) vs peak"
PEAK_BF16_TFLOPS = 2500.0       # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0           # MI355X HBM3E
RIDGE = PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)   # flop per byte
CSRC = os.path.join(ROOT, "submanifold_sparse_convolution_amd", "csrc")
CONFIG_NAMES = ("tiny", "lidar", "deep", "wide", "stage")
HEADLINE = "stage"

# stage timer index -> name (include/smconv.h SMC_STAGE_*)
STAGES = ("map", "neighbours", "mask_sort", "compact", "gemm", "centre")
# the sources that define each kernel (the digest of a traffic record)
KERNEL_SOURCES = {
    "k_compact": ("compact_kernels.hip",), "k_mask_hist": ("compact_kernels.hip",),
    "k_lookup_compact": ("compact_kernels.hip",), "k_compact5": ("compact_kernels.hip",),
    "k_dense_lookup5": ("map_kernels.hip",), "k_dense_lookup": ("map_kernels.hip",),
    "k_dense_scatter": ("map_kernels.hip",), "k_make_keys": ("map_kernels.hip",),
    "k_sorted_lookup": ("map_kernels.hip",),
    "k_gemm_nc": ("gemm_kernels.hip", "gemm_common.h"),
    "k_gemm_centre": ("gemm_kernels.hip", "gemm_common.h"),
    "k_gemm_nc_big": ("gemm_kernels.hip", "gemm_common.h"),
    "k_gemm_centre_big": ("gemm_kernels.hip", "gemm_common.h"),
    "k_gemm_rows": ("rows_kernels.hip", "gemm_common.h"),
    "k_slab_sum": ("gemm_kernels.hip", "gemm_common.h"),
    "k_conv_masktile": ("masktile_kernels.hip", "gemm_common.h"),
    "k_os_pass": ("radix_sort.hip",),
}


def dev_bf16(bits):
    import numpy as np
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


# --------------------------------------------------------------------------
# byte and flop models
# --------------------------------------------------------------------------

def kernel_model(kernel, n, p, c_in, c_out, taps=27, table=False, n_out=None, groups=1):
    """Compulsory bytes and useful flops of one launch of `kernel` (module
    docstring). n input rows, p pairs, n_out output rows (strided layers,
    whose off-centre GEMM runs every tap and reads the inputs once)."""
    m = n if n_out is None else n_out
    if n_out is not None and kernel in ("k_gemm_nc", "k_gemm_nc_big"):
        return 2 * n * c_in + 2 * taps * c_in * c_out + 8 * p, 2.0 * p * c_in * c_out
    if kernel == "k_slab_sum":
        return 2 * m * c_out, 0.0
    p_nc = p - n
    t4 = 4 * taps * m if table else 0
    if kernel in ("k_gemm_centre", "k_gemm_centre_big"):
        return 2 * n * c_in + 2 * c_in * c_out + 2 * n * c_out, 2.0 * n * c_in * c_out
    if kernel in ("k_gemm_nc", "k_gemm_nc_big"):
        return 2 * (taps - 1) * c_in * c_out + 8 * p_nc, 2.0 * p_nc * c_in * c_out
    if kernel == "k_gemm_rows":
        return (2 * n * c_in + 2 * taps * c_in * c_out + 8 * p_nc + 2 * n * c_out,
                2.0 * p * c_in * c_out)
    if kernel == "k_conv_masktile":
        extra = 8 * m * c_out * (groups - 1)
        return (2 * n * c_in + 2 * taps * c_in * c_out + 2 * m * c_out + extra,
                2.0 * p * c_in * c_out)
    if kernel in ("k_dense_scatter", "k_make_keys"):
        return 16 * n, 0.0
    if kernel == "k_lookup_compact":
        return 16 * m + 4 * m + 8 * p + t4, 0.0
    if kernel in ("k_compact", "k_compact5"):
        return (4 if taps == 27 else 16) * n + 8 * p, 0.0
    if kernel in ("k_sorted_lookup", "k_dense_lookup", "k_dense_lookup5", "k_query_lookup"):
        return (4 if taps == 27 else 16) * m + t4, 0.0
    return 0, 0.0


def map_bytes(n, p, taps=27, table=False, perm=False):
    """Compulsory bytes of a whole map build: coordinates in; masks, pair
    lists (and the neighbour table / mask order when kept) out."""
    return 16 * n + (4 if taps == 27 else 16) * n + 8 * p + (4 * taps * n if table else 0) + \
        (4 * n if perm else 0)


def layer_bytes(n, p, c_in, c_out, taps=27):
    """Compulsory bytes of one layer's GEMM: x, all weights, pair lists, y."""
    return 2 * n * c_in + 2 * taps * c_in * c_out + 8 * p + 2 * n * c_out


# --------------------------------------------------------------------------
# one workload on the GPU
# --------------------------------------------------------------------------

TIMED_REGIONS = 3

ORDERS = {"plain": 0, "calibrated": 1, "grouped": 3}   # mask-tile row order -> offset groups
CALIBRATION_SEED_OFFSET = 1000


def calibrate(w, n_groups):
    """Bit order and groups chosen on a held-out voxel set: the same generator
    and sizes with another seed (the calibration frame), never the timed set."""
    import dataclasses

    import torch

    import submanifold_sparse_convolution_amd as smc
    import synth

    wc = dataclasses.replace(w, seed=w.seed + CALIBRATION_SEED_OFFSET)
    cal = smc.KernelMap().build(torch.from_numpy(synth.make_coords(wc)).cuda(),
                                spatial_shape=wc.grid, batch_size=1, pairs=False)
    t0 = time.perf_counter()
    bo, go = cal.calibrate(n_groups)
    secs = time.perf_counter() - t0
    cal.close()
    return bo, go, secs


def tile_work_ratio(mask, perm, group_rows, group_masks):
    """Executed tap-rows of the mask tiles / useful tap-rows (pairs), from an
    exported map: per group, 64-row tiles of its order, each costing its rows
    times the taps of the group present in any of them."""
    import numpy as np

    def popc(a):
        a = a.astype(np.uint32)
        c = np.zeros(a.shape, np.int64)
        for b in range(27):
            c += ((a >> np.uint32(b)) & np.uint32(1)).astype(np.int64)
        return c
    mask = mask.astype(np.uint32)
    useful = int(popc(mask).sum())
    executed = 0
    for g, gm in enumerate(group_masks):
        sub = mask[perm[g, :group_rows[g]]] & np.uint32(gm)
        nt = (len(sub) + 63) // 64
        if nt == 0:
            continue
        pad = np.zeros(nt * 64 - len(sub), np.uint32)
        u = np.bitwise_or.reduce(np.concatenate([sub, pad]).reshape(nt, 64), axis=1)
        r = np.full(nt, 64)
        r[-1] = len(sub) - (nt - 1) * 64
        executed += int((popc(u) * r).sum())
    return executed / useful if useful else 1.0


BIG_MIN_C, BIG_MAX_C = 129, 576     # C_in of the weight-resident wide GEMM kernels


def rows_form(algo, kernel_size, c_in, c_out=None, strided=False):
    """True where the pair-list forward runs as the one-kernel row-range GEMM."""
    return (algo == "pairs" and kernel_size == 3 and c_in <= 64 and c_out <= 64 and c_in % 8 == 0
            and not strided)


OUT_BITMAP_CELLS = 1 << 30      # strided output grids up to this many cells use the bitmap


def strided_output_kernels(out_cells, route="sorted"):
    """The kernels that find a strided map's output cells: a bitmap of the output
    grid (mark, then count, scan and write; on the dense route the input scatter
    marks the bits; a bitmap of at most 2 chunks of 1,024 words per CU in one
    look-back pass) or, for a larger grid, a radix sort of 8 candidate keys per
    input (candidates, sort passes, unique count, scan, unique write)."""
    if out_cells <= OUT_BITMAP_CELLS:
        mark = () if route == "dense" else ("k_stride_mark",)
        if (out_cells + 31) // 32 <= 2 * 256 * 1024:
            return mark + ("k_bits_emit",)
        return mark + ("k_bits_count", "k_scan_counts", "k_bits_write")
    return ("k_stride_candidates", "k_os_pass", "k_unique_count", "k_scan_counts",
            "k_unique_write")


def stage_kernels(stage, algo, route, kernel_size=3, strided=False, c_in=128, out_cells=0):
    """The kernels one execution of a stage launches (pair path unless stated);
    out_cells: a strided map's output grid cells (batch x extents)."""
    big = BIG_MIN_C <= c_in <= BIG_MAX_C and c_in % 8 == 0
    if stage == "gemm":
        if algo == "mask_tiles":
            return ("k_conv_masktile",)
        if rows_form(algo, kernel_size, c_in, c_in):
            return ("k_gemm_rows",)
        return ("k_gemm_nc_big",) if big else ("k_gemm_nc",)
    if stage == "centre":
        if strided:
            return ("k_slab_sum",)
        return ("k_gemm_centre_big",) if big else ("k_gemm_centre",)
    if stage == "mask_sort":
        return ("k_mask_hist", "k_os_pass")
    # dense route, pair lists: the lookup runs inside the compaction (for a strided
    # map, of its query points)
    fused = route == "dense" and algo != "mask_tiles" and kernel_size == 3
    if stage == "neighbours":
        if strided:
            inputs = ("k_dense_scatter",) if route == "dense" else ("k_make_keys", "k_os_pass",
                                                                    "k_key_dups")
            look = () if fused else ("k_dense_lookup" if route == "dense" else "k_query_lookup",)
            return inputs + strided_output_kernels(out_cells, route) + look
        if route == "sorted":
            return ("k_make_keys", "k_os_pass", "k_sorted_lookup")
        if fused:
            return ("k_dense_scatter",)
        return ("k_dense_scatter", "k_dense_lookup5" if kernel_size == 5 else "k_dense_lookup")
    if stage == "compact":
        if fused:
            return ("k_lookup_compact",)
        return ("k_compact5",) if kernel_size == 5 else ("k_compact",)
    return ()


def run_workload(name, steps, warmup, sync_build=False, algo="pairs", copy_probe_mb=0,
                 order="plain", kernel_size=3, frames=1, strided=False, cold=False,
                 route="auto"):
    import torch

    import submanifold_sparse_convolution_amd as smc
    import synth

    w = synth.workload(name)
    coords = synth.make_coords(w) if frames == 1 else synth.batched_coords(w, frames)
    n_rows = len(coords)
    taps = kernel_size ** 3
    c = w.channels
    coords_d = torch.from_numpy(coords).cuda()
    x_d = dev_bf16(synth.features(n_rows, c, w.seed))
    w_ds = [dev_bf16(synth.weights(c, c, w.seed, layer, taps)) for layer in range(w.layers)]
    cal = None
    cold_us = None
    build_kw = dict(spatial_shape=w.grid, batch_size=frames, pairs=(algo != "mask_tiles"),
                    sort=(algo == "mask_tiles"), kernel_size=kernel_size, route=route)
    if cold and not strided:
        # the first build on a fresh handle: its buffers are allocated, the
        # dense route's occupancy bitmap zero-filled once (host clock around
        # a synchronous build). A tiny build on another handle first, so the
        # library's code is loaded on the device before the clock starts.
        wm = smc.KernelMap().build(torch.zeros((1, 4), dtype=torch.int32, device="cuda"),
                                   spatial_shape=(1, 1, 1), batch_size=1)
        wm.close()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        mc = smc.KernelMap().build(coords_d, **build_kw)
        torch.cuda.synchronize()
        cold_us = (time.perf_counter() - t0) * 1e6
        mc.close()
    m = smc.KernelMap()
    if algo == "mask_tiles" and order != "plain":
        bo, go, secs = calibrate(w, ORDERS[order])
        m.set_order(bo, go)
        cal = dict(bit_order=bo, group_of=go, seconds=round(secs, 3),
                   seed=w.seed + CALIBRATION_SEED_OFFSET)
    if copy_probe_mb:
        # a plain device copy of known size: the reference for the PMC byte counters
        a = torch.empty(copy_probe_mb << 20, dtype=torch.uint8, device="cuda")
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        smc.probe_copy(b, a)
        torch.cuda.synchronize()
        del a, b
    # weight packing, once per weight (timed on its own)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    packed = [smc.pack_weights(wd) for wd in w_ds]
    torch.cuda.synchronize()
    ev0.record()
    for _ in range(10):
        for wd, pk in zip(w_ds, packed):
            smc.pack_weights(wd, out=pk)
    ev1.record()
    torch.cuda.synchronize()
    pack_us = ev0.elapsed_time(ev1) * 1e3 / (10 * w.layers)

    if strided:
        # a downsampling layer: the output rows are new cells (one layer)
        m.build_strided(coords_d, spatial_shape=w.grid, batch_size=frames, route=route,
                        pairs=algo != "mask_tiles", sort=algo == "mask_tiles")
        ys = [torch.empty((m.n, c), dtype=torch.bfloat16, device="cuda") for _ in range(2)]
    else:
        ys = [torch.empty((n_rows, c), dtype=torch.bfloat16, device="cuda") for _ in range(2)]

    def step():
        if strided:
            m.build_strided(coords_d, spatial_shape=w.grid, batch_size=frames, sync=sync_build,
                            route=route, pairs=algo != "mask_tiles",
                            sort=algo == "mask_tiles")
            return m.forward(x_d, packed[0], out=ys[0], algo=algo)
        m.build(coords_d, sync=sync_build, **build_kw)
        h = x_d
        for layer in range(w.layers):
            h = m.forward(h, packed[layer], relu=layer + 1 < w.layers, out=ys[layer & 1],
                          algo=algo)
        return h

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    m.sync()
    # timed regions: K steps between device synchronisations, TIMED_REGIONS times;
    # the median region (wall clock) is reported, so that one stall of the host
    # does not decide the figure
    regions = []
    for _ in range(TIMED_REGIONS):
        torch.cuda.synchronize()
        ev0.record()
        t0 = time.perf_counter()
        for _ in range(steps):
            step()
        ev1.record()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        m.sync()                              # the builds' device-side checks passed
        regions.append(((t1 - t0) * 1e3 / steps, ev0.elapsed_time(ev1) / steps))
    regions.sort()
    wall_ms, gpu_ms = regions[len(regions) // 2]

    # second pass with per-kernel HIP events (stream-ordered, on the library's stream)
    m.timing(True)
    for _ in range(steps):
        step()
    stages = m.timing_read(reset=True)
    m.timing(False)
    info = m.info()
    work_ratio = None
    if algo == "mask_tiles" and not strided:
        ex = m.export(pairs=False)
        go = cal["group_of"] if cal else [0] * 27
        gms = [sum(1 << t for t in range(27) if go[t] == g) for g in range(info["n_groups"])]
        work_ratio = tile_work_ratio(ex["mask"], ex["perm"], ex["group_rows"], gms)
    m.close()

    pairs = info["pairs"]
    layers = 1 if strided else w.layers
    per_layer_us = wall_ms * 1e3 / layers
    flops_layer = 2.0 * pairs * c * c
    # per execution, and executions per step
    stage_us = {k: (v[0] * 1e3 / v[1] if v[1] else 0.0) for k, v in stages.items()}
    stage_per_step = {k: (v[1] / steps if steps else 0.0) for k, v in stages.items()}
    # warm build: the build's own event bracket (first to last kernel, the
    # handle's grids already resident)
    warm_us = None if strided else stage_us.get("map")
    return dict(workload=w, coords=coords, info=info, pairs=pairs, ms_per_step=wall_ms,
                gpu_ms_per_step=gpu_ms, per_layer_us=per_layer_us, pack_us=pack_us,
                tflops_effective=flops_layer * layers / (wall_ms * 1e-3) / 1e12,
                stage_us=stage_us, stage_per_step=stage_per_step, algo=algo, order=order,
                calibration=cal, tile_work_ratio=work_ratio, kernel_size=kernel_size,
                frames=frames, n=n_rows, strided=strided, n_out=info["n"], layers=layers,
                map_cold_us=cold_us, map_warm_us=warm_us, steps=steps)


# --------------------------------------------------------------------------
# roofline
# --------------------------------------------------------------------------

def source_digest(kernel):
    files = KERNEL_SOURCES.get(kernel)
    if files is None:
        return None
    h = hashlib.sha256()
    for f in files:
        path = os.path.join(CSRC, f)
        if os.path.exists(path):
            with open(path, "rb") as fh:
                h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_for(workload, algo, kernel):
    """Calibrated HBM bytes per launch of `kernel`, from the committed PMC record,
    or None (no record, or the kernel's source changed since it was taken)."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}_{algo}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    k = rec.get("kernels", {}).get(kernel)
    if not k or k.get("source_digest") != source_digest(kernel):
        return None
    return round(k["bytes_per_launch"])


def stage_rows(r):
    """Per stage: kernels, us per execution, executions per step, and for a
    single-kernel stage its compulsory bytes and flops."""
    info = r["info"]
    route = info["route"]
    c = r["workload"].channels
    taps = r["kernel_size"] ** 3
    out = {}
    for st in STAGES[1:]:
        us = r["stage_us"].get(st, 0.0)
        if us <= 0.0:
            continue
        ks = stage_kernels(st, r["algo"], route, r["kernel_size"], r["strided"], c,
                           out_cells=r["frames"] * math.prod(info["out_extent"]))
        row = dict(kernels=list(ks), us=us, per_step=r["stage_per_step"].get(st, 0.0))
        if len(ks) == 1:
            groups = info["n_groups"] if r["algo"] == "mask_tiles" else 1
            # the neighbour table is written for mask tiles and by a strided map's
            # sorted-route query lookup; fused dense builds keep none
            by, fl = kernel_model(ks[0], r["n"], r["pairs"], c, c, taps,
                                  table=r["algo"] == "mask_tiles"
                                  or (r["strided"] and route != "dense"),
                                  n_out=r["n_out"] if r["strided"] else None, groups=groups)
            row.update(bytes=by, flops=fl)
        out[st] = row
    return out


def roofline(r):
    """The dominant kernel (largest time per step among single-kernel stages)
    and its roofline on compulsory bytes (or useful flops)."""
    rows = {k: v for k, v in stage_rows(r).items() if "bytes" in v}
    if not rows:
        return None
    st = max(rows, key=lambda s: rows[s]["us"] * rows[s]["per_step"])
    mo = rows[st]
    kernel = mo["kernels"][0]
    intensity = mo["flops"] / mo["bytes"] if mo["bytes"] else 0.0
    mfma = intensity > RIDGE
    us = mo["us"]
    gbs = mo["bytes"] / (us * 1e-6) / 1e9
    tfl = mo["flops"] / (us * 1e-6) / 1e12
    out = {"kernel": kernel, "stage": st, "bound": "mfma" if mfma else "hbm",
           "achieved": round(tfl if mfma else gbs, 3 if mfma else 1),
           "peak": PEAK_BF16_TFLOPS if mfma else PEAK_HBM_GBS,
           "unit": "TFLOP/s" if mfma else "GB/s"}
    out["frac"] = round(out["achieved"] / out["peak"], 5)
    plain = r["kernel_size"] == 3 and r["frames"] == 1 and r["order"] == "plain"
    rec = "strided" if r["strided"] else r["algo"]    # counter records: pair path, stride-2 layer
    out["traffic"] = (traffic_for(r["workload"].name, rec, kernel)
                      if plain and (r["algo"] == "pairs" or not r["strided"]) else None)
    out["avg_us"] = round(us, 3)
    out["launches_per_step"] = round(mo["per_step"], 3)
    out["algorithmic_bytes"] = mo["bytes"]
    out["flops_useful"] = mo["flops"]
    out["hbm_frac"] = round(gbs / PEAK_HBM_GBS, 5)
    out["mfma_frac_useful"] = round(tfl / PEAK_BF16_TFLOPS, 5)
    return out


def summary(r):
    """The figures of one run: time per layer, throughput, stages, roofline."""
    info = r["info"]
    w = r["workload"]
    c = w.channels
    n, p = r["n"], r["pairs"]
    taps = r["kernel_size"] ** 3
    out = {
        "workload": w.name, "n": n, "pairs": p, "pairs_per_voxel": round(p / n, 4) if n else 0,
        "route": info["route"], "key_bits": info["key_bits"], "c_in": c, "c_out": c,
        "layers": r["layers"], "us_per_layer": round(r["per_layer_us"], 2),
        "ms_per_step": round(r["ms_per_step"], 4),
        "gpu_ms_per_step_events": round(r["gpu_ms_per_step"], 4),
        "tflops_effective": round(r["tflops_effective"], 3),
        "frac_bf16_peak": round(r["tflops_effective"] / PEAK_BF16_TFLOPS, 5),
        "weight_pack_us": round(r["pack_us"], 2),
        "stages": {k: {kk: (round(vv, 3) if isinstance(vv, float) else vv) for kk, vv in v.items()}
                   for k, v in stage_rows(r).items()},
        "map_us_events": round(r["stage_us"].get("map", 0.0), 2),
        "roofline": roofline(r),
    }
    if not r["strided"]:
        step_bytes = map_bytes(n, p, taps) + r["layers"] * layer_bytes(n, p, c, c, taps)
        out["step_compulsory_bytes"] = step_bytes
        out["step_hbm_frac"] = round(step_bytes / (r["ms_per_step"] * 1e-3) / 1e9 / PEAK_HBM_GBS, 5)
    else:
        out["n_out"] = r["n_out"]
        cells = r["frames"] * math.prod(info["out_extent"])
        out["output_cells_route"] = "bitmap" if cells <= OUT_BITMAP_CELLS else "candidate_sort"
    if r["map_cold_us"] is not None:
        out["map_cold_us"] = round(r["map_cold_us"], 1)
        out["map_cold_note"] = ("first build on a fresh handle, host clock around a synchronous "
                                "build: buffer allocation and the occupancy-bitmap zero fill "
                                "(dense route) included")
    if r["map_warm_us"] is not None:
        out["map_warm_us"] = round(r["map_warm_us"], 2)
    if info["route"] == "dense":
        out["dense_grid_cells"] = info["grid_cells"]
    if r["tile_work_ratio"] is not None:
        out["tile_work_ratio"] = round(r["tile_work_ratio"], 4)
    return out


# --------------------------------------------------------------------------
# CPU oracle and measured peaks
# --------------------------------------------------------------------------

def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        blas = [i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"]
        return max(blas) if blas else 1
    except Exception:
        return os.cpu_count() or 1


def cpu_baseline(name, budget_s=8.0, reps=3):
    """The CPU oracle, as it stands, on the same workload: its map (dict
    lookups, mask sort, pair lists) and one layer's compute (per-tap float64
    matmuls, bf16 rounding) timed apart, median of up to `reps` runs within
    about budget_s seconds each. Per layer = map / layers + compute."""
    import synth
    from oracle import smconv_oracle as so
    w = synth.workload(name)
    coords = synth.make_coords(w)
    xb = synth.features(w.n, w.channels, w.seed)
    wb = synth.weights(w.channels, w.channels, w.seed)
    x = so.bf16_bits_to_f64(xb)
    wf = so.bf16_bits_to_f64(wb)
    map_t, comp_t = [], []
    t_start = time.perf_counter()
    while len(map_t) < reps:
        t0 = time.perf_counter()
        nbr, mask = so.build_kernel_map(coords)
        so.mask_sort(mask)
        pin, pout, toff = so.compact_pairs(nbr, mask)
        map_t.append(time.perf_counter() - t0)
        if time.perf_counter() - t_start > budget_s:
            break
    t_start = time.perf_counter()
    while len(comp_t) < reps:
        t0 = time.perf_counter()
        acc = so.conv_accumulate(x, wf, pin, pout, toff, x.shape[0])
        so.round_to_bf16(acc)
        comp_t.append(time.perf_counter() - t0)
        if time.perf_counter() - t_start > budget_s:
            break
    mp, cp = statistics.median(map_t), statistics.median(comp_t)
    cores = blas_threads()
    return {"value": round((mp / w.layers + cp) * 1e6, 1), "unit": "us/layer", "cores": cores,
            "kind": "oracle", "map_us": round(mp * 1e6, 1), "compute_us_per_layer": round(cp * 1e6, 1),
            "sample": (f"{name}: {len(map_t)} map build(s) (dict lookups, mask sort, pair lists; "
                       f"single-threaded Python) and {len(comp_t)} layer computation(s) "
                       f"(per-tap float64 matmuls on {cores} BLAS threads, bf16 rounding), "
                       f"medians; per layer = map / {w.layers} + one layer"),
            "host_cpus": os.cpu_count()}


def measured_peaks():
    """An MFMA-only loop and a device copy on this GPU, next to the spec peaks."""
    import torch

    import submanifold_sparse_convolution_amd as smc
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    out = {}
    smc.probe_mfma_bf16(1000)                           # warm-up
    torch.cuda.synchronize()
    ev0.record()
    flops = smc.probe_mfma_bf16(200000)
    ev1.record()
    torch.cuda.synchronize()
    tf = flops / (ev0.elapsed_time(ev1) * 1e-3) / 1e12
    out["mfma_bf16_tflops"] = round(tf, 1)
    out["mfma_frac_of_spec"] = round(tf / PEAK_BF16_TFLOPS, 4)
    nbytes = 1 << 30
    a = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    a.fill_(1)
    smc.probe_copy(b, a)
    torch.cuda.synchronize()
    reps = 10
    ev0.record()
    for _ in range(reps):
        smc.probe_copy(b, a)
    ev1.record()
    torch.cuda.synchronize()
    gbs = 2.0 * nbytes * reps / (ev0.elapsed_time(ev1) * 1e-3) / 1e9
    out["copy_gbs"] = round(gbs, 1)
    b.copy_(a)
    torch.cuda.synchronize()
    ev0.record()
    for _ in range(reps):
        b.copy_(a)
    ev1.record()
    torch.cuda.synchronize()
    gbs_t = 2.0 * nbytes * reps / (ev0.elapsed_time(ev1) * 1e-3) / 1e9
    out["torch_copy_gbs"] = round(gbs_t, 1)
    out["copy_frac_of_spec"] = round(max(gbs, gbs_t) / PEAK_HBM_GBS, 4)
    out["note"] = ("k_probe_mfma: 8 waves per CU, 8 independent v_mfma_f32_16x16x32_bf16 chains "
                   "each; k_probe_copy and torch's copy_: 1 GiB device-to-device, read + write "
                   "bytes counted; copy_frac_of_spec takes the faster")
    del a, b
    return out


# --------------------------------------------------------------------------
# rocprofv3 summaries (run on the CPU)
# --------------------------------------------------------------------------

def _short(k):
    import re
    k = k.replace("(anonymous namespace)::", "").replace("void ", "").replace("smc::", "")
    return re.sub(r"\(.*", "", k).split("<")[0].strip()


def _pmc_rows(d, counter):
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {d}")
    rows = []
    for fn in files:
        with open(fn) as f:
            for row in csv.DictReader(f):
                if row.get("Counter_Name") == counter:
                    rows.append((row["Kernel_Name"], float(row["Counter_Value"])))
    return rows


MFMA_COUNTERS = ("SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_VALU_MFMA_BUSY_CYCLES")
N_SIMD = 256 * 4                 # MI355X: 256 CUs of 4 SIMDs
CLOCK_HZ = 2.4e9                 # MI355X peak engine clock


def summarize_mfma(pmc_dir, workload, algo, bench_out):
    """Per-dispatch MFMA counters of the GEMM kernels from one `rocprofv3 --pmc
    SQ_INSTS_VALU_MFMA_MOPS_BF16 SQ_VALU_MFMA_BUSY_CYCLES` run of this script:
    executed bf16 MFMA flops (MOPS x 512) next to the useful flops of the same
    launch (2 x pairs x C_in x C_out over the pairs that launch covers; n,
    pairs and C from the JSON line the profiled run printed, in bench_out),
    and the MFMA busy share of all SIMD cycles over the dispatch's own
    (profiled) duration."""
    line = None
    with open(bench_out) as f:
        for ln in f:
            if ln.startswith('{"metric"'):
                line = json.loads(ln)
    if line is None:
        raise SystemExit(f"no bench JSON line in {bench_out}")
    cfg = line["config"]
    n, p, c = cfg["n"], cfg["pairs"], cfg["c_in"]
    useful = {"k_gemm_nc": 2.0 * (p - n) * c * c, "k_gemm_centre": 2.0 * n * c * c,
              "k_conv_masktile": 2.0 * p * c * c}
    useful["k_gemm_nc_big"], useful["k_gemm_centre_big"] = useful["k_gemm_nc"], useful["k_gemm_centre"]
    useful["k_gemm_rows"] = 2.0 * p * c * c
    files = glob.glob(os.path.join(pmc_dir, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {pmc_dir}")
    per = {}                       # kernel -> dispatch -> {counter: value, "ns": duration}
    for fn in files:
        with open(fn) as f:
            for row in csv.DictReader(f):
                k = _short(row["Kernel_Name"])
                if k not in useful or row["Counter_Name"] not in MFMA_COUNTERS:
                    continue
                d = per.setdefault(k, {}).setdefault(row["Dispatch_Id"], {})
                d[row["Counter_Name"]] = float(row["Counter_Value"])
                d["ns"] = float(row["End_Timestamp"]) - float(row["Start_Timestamp"])
    out = {"workload": workload, "algo": algo, "n": n, "pairs": p, "c": c,
           "clock_hz": CLOCK_HZ, "simds": N_SIMD, "kernels": {}}
    for k, ds in sorted(per.items()):
        mops = statistics.mean(d.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0.0) for d in ds.values())
        busy = statistics.mean(d.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) for d in ds.values())
        ns = statistics.mean(d["ns"] for d in ds.values())
        executed = mops * 512.0
        out["kernels"][k] = {
            "dispatches": len(ds), "mfma_flops_executed": executed, "flops_useful": useful[k],
            "useful_over_executed": useful[k] / executed if executed else None,
            "mfma_busy_cycles": busy, "profiled_ns": ns,
            "mfma_busy_frac": busy / (ns * 1e-9 * CLOCK_HZ * N_SIMD) if ns else None,
            "useful_tflops_profiled": useful[k] / (ns * 1e-9) / 1e12 if ns else None,
            "source_digest": source_digest(k)}
    path = os.path.join(ROOT, "profiles", f"mfma_{workload}_{algo}.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print(f"wrote {path}")
    for k, v in out["kernels"].items():
        print(f"{k}: executed {v['mfma_flops_executed']:.4g} flop, useful {v['flops_useful']:.4g} "
              f"({v['useful_over_executed']:.3f}); MFMA busy {v['mfma_busy_frac']:.4f} of the "
              f"SIMD cycles over {v['profiled_ns'] / 1e3:.2f} us (profiled)")


def summarize_trace(trace_dir, title, command, out_md):
    """A rocprofv3 --kernel-trace run (run_kernel_trace.csv under trace_dir)
    as a markdown table: per kernel and grid size, dispatches and durations
    (us). The grid tells the voxel sets apart in a run that times several."""
    files = glob.glob(os.path.join(trace_dir, "**", "*kernel_trace.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no kernel_trace.csv under {trace_dir}")
    groups = {}
    for fn in files:
        with open(fn) as f:
            for row in csv.DictReader(f):
                k = _short(row["Kernel_Name"])
                grid = row.get("Grid_Size_X") or row.get("Grid_Size") or ""
                if row.get("Grid_Size_Y") not in (None, "", "1"):
                    grid = f"{grid}x{row['Grid_Size_Y']}"
                ns = float(row["End_Timestamp"]) - float(row["Start_Timestamp"])
                groups.setdefault((k, grid), []).append(ns / 1e3)
    total = sum(sum(v) for v in groups.values())
    lines = [f"# Kernel trace: {title}", "",
             "Command (from the repository root; rocprofv3 writes its CSV files under the "
             "given directory):", "", "```", command, "```", "",
             "Per kernel and grid size (work-items in x, x blocks in y), durations in microseconds:",
             "", "| kernel | grid | calls | avg | min | max | share |",
             "|---|---|---|---|---|---|---|"]
    for (k, grid), v in sorted(groups.items(), key=lambda kv: -sum(kv[1])):
        lines.append(f"| `{k}` | {grid} | {len(v)} | {statistics.mean(v):.2f} | {min(v):.2f} | "
                     f"{max(v):.2f} | {100 * sum(v) / total:.1f} % |")
    with open(out_md, "w") as f:
        f.write("\n".join(lines) + "\n")
    print(f"wrote {out_md}")


def summarize_pmc(fetch_dir, write_dir, workload, algo, copy_mb):
    """Per-dispatch FETCH_SIZE / WRITE_SIZE (KiB) of every kernel, scaled by what the
    same counters read for a plain device copy (k_probe_copy) of copy_mb MiB."""
    out = {"workload": workload, "algo": algo, "copy_probe_mib": copy_mb, "kernels": {}}
    per = {}
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        vals = {}
        for k, v in _pmc_rows(d, counter):
            vals.setdefault(_short(k), []).append(v)
        per[counter] = vals
    if "k_probe_copy" not in per["FETCH_SIZE"]:
        raise SystemExit("no k_probe_copy dispatch found for the calibration")
    cname = "k_probe_copy"
    kib = copy_mb * 1024.0
    f_copy = max(per["FETCH_SIZE"][cname])
    w_copy = max(per["WRITE_SIZE"].get(cname, [0.0]))
    out["copy_kernel"] = cname
    out["copy_fetch_kib"] = f_copy
    out["copy_write_kib"] = w_copy
    out["fetch_scale"] = kib / f_copy if f_copy else None
    out["write_scale"] = kib / w_copy if w_copy else None
    for k in sorted(set(per["FETCH_SIZE"]) | set(per["WRITE_SIZE"])):
        if not k.startswith("k_") or k.startswith("k_probe"):
            continue
        fv = per["FETCH_SIZE"].get(k, [])
        wv = per["WRITE_SIZE"].get(k, [])
        f_avg = statistics.mean(fv) if fv else 0.0
        w_avg = statistics.mean(wv) if wv else 0.0
        fb = f_avg * 1024.0 * (out["fetch_scale"] or 1.0)
        wb = w_avg * 1024.0 * (out["write_scale"] or 1.0)
        out["kernels"][k] = {"dispatches": len(fv), "fetch_kib_raw": f_avg, "write_kib_raw": w_avg,
                             "fetch_bytes": fb, "write_bytes": wb,
                             "bytes_per_launch": fb + wb, "source_digest": source_digest(k)}
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}_{algo}.json")
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print(f"wrote {path}")
    for k, v in out["kernels"].items():
        print(f"  {k:22s} fetch {v['fetch_bytes'] / 1e6:9.3f} MB  write {v['write_bytes'] / 1e6:9.3f} MB"
              f"  ({v['dispatches']} dispatches)")


# --------------------------------------------------------------------------
# main
# --------------------------------------------------------------------------

def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=HEADLINE, choices=list(CONFIG_NAMES))
    ap.add_argument("--algo", default="pairs", choices=["pairs", "pairs_slab", "mask_tiles"],
                    help="forward algorithm of the headline line")
    ap.add_argument("--order", default="plain", choices=list(ORDERS),
                    help="mask-tile row order: plain mask value, calibrated bit order, or "
                         "calibrated order with 3 offset groups (calibrated on another seed)")
    ap.add_argument("--sync-build", action="store_true",
                    help="wait for the map's device-side checks inside every step")
    ap.add_argument("--configs", default=",".join(CONFIG_NAMES),
                    help="comma-separated sets timed beside the headline ('none': only it)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=6.0,
                    help="seconds per oracle part (map, compute) and set")
    ap.add_argument("--no-strided", action="store_true")
    ap.add_argument("--strided-layer", action="store_true",
                    help="time the set's stride-2 layer as the main line (profiling runs; "
                         "its counter summaries go to profiles/traffic_<set>_strided.json)")
    ap.add_argument("--no-peaks", action="store_true")
    ap.add_argument("--other-algo", action="store_true",
                    help="also time the mask-tile forward (three row orders) on the headline set")
    ap.add_argument("--copy-probe-mb", type=int, default=0,
                    help="run one plain device copy of this many MiB first (PMC calibration)")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"))
    ap.add_argument("--summarize-mfma", nargs=2, metavar=("PMC_DIR", "BENCH_OUT"),
                    help="summarise a rocprofv3 --pmc run of the MFMA counters and the "
                         "JSON line that run printed")
    ap.add_argument("--summarize-trace", nargs=4, metavar=("TRACE_DIR", "TITLE", "COMMAND", "OUT_MD"),
                    help="summarise a rocprofv3 --kernel-trace run into a markdown table")
    ap.add_argument("--report", default="",
                    help="also run the mask-tile orders, 5x5x5 kernels and batched frames of "
                         "every set and write their figures to this JSON file")
    args = ap.parse_args()

    if args.summarize_trace:
        summarize_trace(*args.summarize_trace)
        return
    if args.summarize_mfma:
        summarize_mfma(args.summarize_mfma[0], args.workload, args.algo, args.summarize_mfma[1])
        return
    if args.summarize_pmc:
        summarize_pmc(args.summarize_pmc[0], args.summarize_pmc[1], args.workload,
                      "strided" if args.strided_layer else args.algo,
                      args.copy_probe_mb or 256)
        return

    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (the library "
              "has no multi-GPU path)", file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    configs = [] if args.configs == "none" else [c for c in args.configs.split(",") if c]
    for cname in configs:
        if cname not in CONFIG_NAMES:
            raise SystemExit(f"unknown set {cname}")

    r = run_workload(args.workload, args.steps, args.warmup, args.sync_build, args.algo,
                     args.copy_probe_mb, args.order, cold=not args.strided_layer,
                     strided=args.strided_layer)
    w, info = r["workload"], r["info"]
    c = w.channels
    s = summary(r)
    line = {
        "metric": METRIC,
        "value": round(r["per_layer_us"], 2),
        "unit": "us/layer",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "timed_regions": TIMED_REGIONS,
        "ms_per_step": round(r["ms_per_step"], 4),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": f"{w.name}: {w.n} voxels, grid {w.grid[0]}x{w.grid[1]}x{w.grid[2]}, "
                        f"C_in=C_out={c}, "
                        + ("one stride-2 layer" if args.strided_layer
                           else f"{w.layers} layer(s) sharing one map") + f", seed {w.seed}",
            "n": w.n, "pairs": r["pairs"], "pairs_per_voxel": round(r["pairs"] / w.n, 4),
            "route": info["route"], "c_in": c, "c_out": c, "layers": r["layers"],
            "map_built_every_step": True, "build_mode": "sync" if args.sync_build else "async",
            "algo": args.algo, "value_is": "(map + all layers) / layers, microseconds",
            **({"order": args.order} if args.algo == "mask_tiles" else {}),
        },
        "tflops_effective": s["tflops_effective"],
        "frac_bf16_peak": s["frac_bf16_peak"],
        "gpu_ms_per_step_events": s["gpu_ms_per_step_events"],
        "stages": s["stages"],
        "weight_pack_us": s["weight_pack_us"],
        "map_cold_us": s.get("map_cold_us"),
        "map_warm_us": s.get("map_warm_us"),
        "step_hbm_frac": s.get("step_hbm_frac"),
        "roofline": s["roofline"],
    }
    if r["tile_work_ratio"] is not None:
        line["tile_work_ratio"] = round(r["tile_work_ratio"], 4)
    if not args.no_peaks:
        line["peaks_measured"] = measured_peaks()
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(args.workload, args.cpu_budget)
    if configs:
        entries = []
        for cname in configs:
            if cname == args.workload and args.algo == "pairs" and args.order == "plain":
                e = dict(s)
            else:
                rr = run_workload(cname, args.steps, args.warmup, args.sync_build, cold=True)
                e = summary(rr)
            if not args.no_cpu_baseline:
                e["cpu_baseline"] = (line["cpu_baseline"] if cname == args.workload
                                     and "cpu_baseline" in line
                                     else cpu_baseline(cname, args.cpu_budget))
            entries.append(e)
        line["configs"] = entries
        if "wide" in configs:
            # the sorted mapper (packed keys, radix sort, plane searches) on the Wide
            # scene, which the auto route now maps densely where memory allows
            rr = run_workload("wide", args.steps, args.warmup, args.sync_build, route="sorted")
            e = summary(rr)
            line["wide_sorted_route"] = {k: e[k] for k in ("route", "key_bits", "us_per_layer",
                                                           "map_us_events", "stages")}
    if not args.no_strided:
        # downsampling layers (kernel 3, stride 2) on the same sets: new output cells,
        # pair-list forward over them; map built every step
        line["strided"] = []
        for cname in ("lidar", "deep", "wide", "stage"):
            rr = run_workload(cname, max(10, args.steps // 2), args.warmup, strided=True)
            e = summary(rr)
            line["strided"].append({k: e[k] for k in ("workload", "n", "n_out", "pairs", "route",
                                                      "output_cells_route", "us_per_layer",
                                                      "tflops_effective", "stages", "roofline")})
    if args.other_algo:
        line["other_algo"] = []
        for order2 in ORDERS:
            r2 = run_workload(args.workload, args.steps, args.warmup, args.sync_build,
                              "mask_tiles", order=order2)
            e = summary(r2)
            line["other_algo"].append({"algo": "mask_tiles", "order": order2,
                                       "us_per_layer": e["us_per_layer"],
                                       "tflops_effective": e["tflops_effective"],
                                       "tile_work_ratio": e.get("tile_work_ratio"),
                                       "stages": e["stages"]})
    if args.report:
        rep = {}
        runs = []
        for name in CONFIG_NAMES:
            runs += [(name, "mask_tiles", o, 3, 1) for o in ORDERS]
        runs += [("lidar", "pairs", "plain", 5, 1), ("deep", "pairs", "plain", 5, 1),
                 ("wide", "pairs", "plain", 5, 1), ("lidar", "pairs", "plain", 3, 4),
                 ("lidar", "pairs", "plain", 5, 4)]
        for name, algo, order, ks, frames in runs:
            rr = run_workload(name, max(20, args.steps // 2), args.warmup, algo=algo,
                              order=order, kernel_size=ks, frames=frames)
            key = (f"{name}/{algo}" + ("" if order == "plain" else f"/{order}")
                   + ("" if ks == 3 else f"/k{ks}") + ("" if frames == 1 else f"/b{frames}"))
            rep[key] = summary(rr)
            rep[key].update(kernel_size=ks, frames=frames, calibration=rr["calibration"])
        with open(args.report, "w") as f:
            json.dump(rep, f, indent=1)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
