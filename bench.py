#!/usr/bin/env python3
"""Benchmark: microseconds per submanifold 3x3x3 layer including the kernel
map, effective TFLOP/s on useful MACs, and the roofline of the dominant
kernel.

One step = one pass of the whole hot path over one seeded synthetic voxel
set already resident in HBM: build the kernel map from raw coordinates
(route, neighbour search with masks, compaction into per-tap pair lists --
or the mask sort for the mask-tile algorithm) and run the layer(s) (gather
-> MFMA -> slab -> centre-tap GEMM with the bf16 finalize). Weights are
packed once before the timed region (a packed weight is reused for every
forward) and the packing time is reported on its own.

Prints ONE JSON line. --gpus above 1 exits: this build measures one GPU.

Per-stage times come from a second pass with the library's stage timers:
every kernel launched in a stage carries its own HIP start/stop events
(stamped by the kernel's dispatch), so a single-kernel stage's average is
that kernel's average duration, as rocprofv3's kernel trace reports it.

  --summarize-pmc FETCH_DIR WRITE_DIR   turn two `rocprofv3 --pmc FETCH_SIZE`
      / `--pmc WRITE_SIZE` runs of this script (with --copy-probe-mb) into
      profiles/traffic_<workload>_<algo>.json, which later runs read for the
      roofline's "traffic" (null when a kernel source changed since).
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

# stage -> the kernels it launches (dense route; the sorted route's neighbour
# stage is k_make_keys + k_key_hist + k_os_pass + k_sorted_lookup)
STAGE_KERNELS = {
    "neighbours": ("k_dense_scatter", "k_dense_lookup"),
    "mask_sort": ("k_mask_hist", "k_os_pass"),
    "compact": ("k_compact",),
    "gemm": ("k_gemm_nc",),
    "centre": ("k_gemm_centre",),
}
# dense route with pair lists: the lookup is fused into the compaction kernel
STAGE_KERNELS_FUSED = {
    "neighbours": ("k_dense_scatter",),
    "compact": ("k_lookup_compact",),
    "gemm": ("k_gemm_nc",),
    "centre": ("k_gemm_centre",),
}
MASK_TILE_GEMM = ("k_conv_masktile",)
KERNEL_SOURCES = {
    "k_compact": "compact_kernels.hip", "k_mask_hist": "compact_kernels.hip",
    "k_lookup_compact": "compact_kernels.hip", "k_compact5": "compact_kernels.hip",
    "k_dense_lookup5": "map_kernels.hip",
    "k_gemm_nc": "gemm_kernels.hip", "k_gemm_centre": "gemm_kernels.hip",
    "k_conv_masktile": "masktile_kernels.hip", "k_dense_scatter": "map_kernels.hip",
    "k_dense_lookup": "map_kernels.hip", "k_os_pass": "radix_sort.hip",
}


def dev_bf16(bits):
    import numpy as np
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def stage_model(stage, algo, route, n, p, c_in, c_out, taps=27):
    """Algorithmic (compulsory) bytes and useful flops of one stage execution.

    Each input is counted once and each output once; reads of random grid cells
    and gathered rows count their payload only. taps: 27 (3x3x3) or 125 (5x5x5);
    the fused lookup + compaction kernel exists for 27 taps only.
    """
    p_nc = p - n
    fused = route == "dense" and algo == "pairs" and taps == 27
    t4 = 4 * taps                                  # bytes of one neighbour-table row
    if stage == "neighbours":
        if fused:
            # scatter: coords in, grid cell + the row's cell record out; the previous
            # build's cells read and put back (same count, taken as n)
            return 16 * n + 4 * n + 4 * n + 4 * n + 4 * n, 0
        mw = 4 if taps == 27 else 16              # mask bytes per row
        if route == "dense":
            # scatter as above; lookup: coords + taps cells in, nbr + mask out
            return 16 * n + 16 * n + (16 * n + t4 * n) + (t4 * n + mw * n), 0
        # sorted: coords -> keys, key sort passes, K^2 searches per row (8-byte keys)
        k2 = 9 if taps == 27 else 25
        return 16 * n + 8 * n + 5 * 2 * 12 * n + k2 * 8 * n + (t4 + mw) * n, 0
    if stage == "mask_sort":
        return 4 * n + 3 * 2 * 8 * n, 0
    if stage == "compact":
        if fused:
            # coords + 27 cells in; nbr, mask, pair lists (in, out, slot), rowbase out
            return 16 * n + 108 * n + 108 * n + 4 * n + 12 * p + 4 * n, 0
        return (4 if taps == 27 else 16) * n + t4 * n + 12 * p + 4 * n, 0
    if stage == "gemm" and algo == "pairs":
        return ((2 * c_in + 8 + 4 * c_out) * p_nc + 2 * (taps - 1) * c_in * c_out,
                2.0 * p_nc * c_in * c_out)
    if stage == "gemm":          # mask tiles: x once, all weights, nbr/mask/perm, y once
        return (2 * c_in * n + 2 * 27 * c_in * c_out + 116 * n + 2 * c_out * n,
                2.0 * p * c_in * c_out)
    if stage == "centre":
        return (2 * c_in * n + 2 * c_in * c_out + 8 * n + 4 * c_out * p_nc + 2 * c_out * n,
                2.0 * n * c_in * c_out)
    return 0, 0


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


def run_workload(name, steps, warmup, sync_build=False, algo="pairs", copy_probe_mb=0,
                 order="plain", kernel_size=3, frames=1, strided=False):
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
    m = smc.KernelMap()
    cal = None
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
        b.copy_(a)
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
        m.build_strided(coords_d, spatial_shape=w.grid, batch_size=frames)
        ys = [torch.empty((m.n, c), dtype=torch.bfloat16, device="cuda") for _ in range(2)]
    else:
        ys = [torch.empty((n_rows, c), dtype=torch.bfloat16, device="cuda") for _ in range(2)]

    def step():
        if strided:
            m.build_strided(coords_d, spatial_shape=w.grid, batch_size=frames, sync=sync_build)
            return m.forward(x_d, packed[0], out=ys[0], algo="mask_tiles")
        m.build(coords_d, spatial_shape=w.grid, batch_size=frames, sync=sync_build,
                pairs=(algo == "pairs"), sort=(algo == "mask_tiles"), kernel_size=kernel_size)
        h = x_d
        for layer in range(w.layers):
            h = m.forward(h, packed[layer], relu=layer + 1 < w.layers, out=ys[layer & 1],
                          algo=algo)
        return h

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    m.sync()
    # timed region: K steps between device synchronisations
    ev0.record()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    ev1.record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    m.sync()                                  # the builds' device-side checks passed
    wall_ms = (t1 - t0) * 1e3 / steps
    gpu_ms = ev0.elapsed_time(ev1) / steps

    # second pass with per-kernel HIP events (stream-ordered, on the library's stream)
    m.timing(True)
    for _ in range(steps):
        step()
    stages = m.timing_read(reset=True)
    m.timing(False)
    info = m.info()
    work_ratio = None
    if algo == "mask_tiles":
        ex = m.export(pairs=False)
        go = cal["group_of"] if cal else [0] * 27
        gms = [sum(1 << t for t in range(27) if go[t] == g) for g in range(info["n_groups"])]
        work_ratio = tile_work_ratio(ex["mask"], ex["perm"], ex["group_rows"], gms)
    m.close()

    pairs = info["pairs"]
    layers = 1 if strided else w.layers
    per_layer_us = wall_ms * 1e3 / layers
    flops_layer = 2.0 * pairs * c * c
    stage_us = {k: (v[0] * 1e3 / v[1] if v[1] else 0.0) for k, v in stages.items()}
    # per execution; forward stages run once per layer
    model = {}
    for st in ("neighbours", "mask_sort", "compact", "gemm", "centre"):
        if stage_us.get(st, 0.0) <= 0.0:
            continue
        if strided:
            by, fl = strided_model(st, info["route"], n_rows, info["n"], pairs, c, c)
        else:
            by, fl = stage_model(st, algo, info["route"], n_rows, pairs, c, c, taps)
        if st == "gemm" and algo == "mask_tiles" and info["n_groups"] > 1:
            # float32 partial sums: written by each early pass and read once after
            by += 8 * c * sum(info["group_rows"][:-1])
        us = stage_us[st]
        model[st] = dict(us=us, bytes=by, flops=fl, gbs=by / (us * 1e-6) / 1e9,
                         tflops=fl / (us * 1e-6) / 1e12 if fl else 0.0)
    return dict(workload=w, coords=coords, info=info, pairs=pairs, ms_per_step=wall_ms,
                gpu_ms_per_step=gpu_ms, per_layer_us=per_layer_us, pack_us=pack_us,
                tflops_effective=flops_layer * layers / (wall_ms * 1e-3) / 1e12,
                stage_us=stage_us, model=model, algo=algo, order=order, calibration=cal,
                tile_work_ratio=work_ratio, kernel_size=kernel_size, frames=frames, n=n_rows,
                strided=strided, n_out=info["n"])


def source_digest(kernel):
    f = KERNEL_SOURCES.get(kernel)
    if f is None:
        return None
    h = hashlib.sha256()
    for path in sorted([os.path.join(CSRC, f), os.path.join(CSRC, "gemm_common.h"),
                        os.path.join(CSRC, "smc_internal.h")]):
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


def strided_model(stage, route, n, m, p, c_in, c_out):
    """Algorithmic bytes and useful flops of a strided layer's stages (n inputs,
    m outputs, p input-output pairs): candidates 8 keys per input, their sort
    (4 passes of key + value), unique, the 27-tap lookup of every output, the
    mask sort of the outputs and the mask-tile GEMM."""
    if stage == "neighbours":
        cand = 16 * n + 64 * n + 4 * 2 * 12 * 8 * n + 64 * n + 32 * m
        look = 16 * m + 108 * m + 4 * m + (108 * m if route == "dense" else 9 * 8 * m)
        return cand + look + (16 * n if route == "dense" else 16 * n + 8 * n + 5 * 2 * 12 * n), 0
    if stage == "mask_sort":
        return 4 * m + 3 * 2 * 8 * m, 0
    if stage == "gemm":
        return (2 * c_in * n + 2 * 27 * c_in * c_out + 116 * m + 2 * c_out * m,
                2.0 * p * c_in * c_out)
    return 0, 0


def stage_kernels(stage, algo, route, kernel_size=3):
    """The kernels one execution of a stage launches."""
    if stage == "gemm" and algo == "mask_tiles":
        return MASK_TILE_GEMM
    fused = route == "dense" and algo == "pairs" and kernel_size == 3
    if stage == "neighbours":
        if route == "sorted":
            return ("k_make_keys", "k_key_hist", "k_os_pass", "k_sorted_lookup")
        if fused:
            return ("k_dense_scatter",)
        return ("k_dense_scatter", "k_dense_lookup5" if kernel_size == 5 else "k_dense_lookup")
    if stage == "compact":
        if fused:
            return ("k_lookup_compact",)
        return ("k_compact5",) if kernel_size == 5 else ("k_compact",)
    return STAGE_KERNELS[stage]


def roofline(r):
    """The dominant stage (largest kernel time) and its roofline."""
    model = r["model"]
    if not model:
        return None
    st = max(model, key=lambda s: model[s]["us"])
    mo = model[st]
    kernels = stage_kernels(st, r["algo"], r["info"]["route"], r.get("kernel_size", 3))
    if r.get("strided") and st == "neighbours":
        kernels = ("k_dense_scatter" if r["info"]["route"] == "dense" else "k_make_keys",
                   "k_stride_candidates", "k_key_hist", "k_os_pass", "k_unique_count",
                   "k_scan_counts", "k_unique_write",
                   "k_dense_lookup" if r["info"]["route"] == "dense" else "k_query_lookup")
    kernel = kernels[0] if len(kernels) == 1 else "+".join(kernels)
    intensity = mo["flops"] / mo["bytes"] if mo["bytes"] else 0.0
    mfma = intensity > RIDGE
    out = {"kernel": kernel, "stage": st,
           "bound": "mfma" if mfma else "hbm",
           "achieved": round(mo["tflops"] if mfma else mo["gbs"], 3 if mfma else 1),
           "peak": PEAK_BF16_TFLOPS if mfma else PEAK_HBM_GBS,
           "unit": "TFLOP/s" if mfma else "GB/s"}
    out["frac"] = round(out["achieved"] / out["peak"], 5)
    plain = r.get("kernel_size", 3) == 3 and r.get("frames", 1) == 1 and r.get("order") == "plain"
    out["traffic"] = (traffic_for(r["workload"].name, r["algo"], kernel)
                      if len(kernels) == 1 and plain else None)
    out["avg_us"] = round(mo["us"], 3)
    out["algorithmic_bytes"] = mo["bytes"]
    out["flops_useful"] = mo["flops"]
    out["mfma_frac_useful"] = round(mo["tflops"] / PEAK_BF16_TFLOPS, 5)
    return out


def cpu_baseline(name, budget_s=12.0):
    """The CPU oracle (untouched) on the same workload, repeated for ~budget_s."""
    import synth
    from oracle import smconv_oracle as so
    try:
        from threadpoolctl import threadpool_info
        blas = [i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"]
        cores = max(blas) if blas else 1
    except Exception:
        cores = os.cpu_count() or 1
    w = synth.workload(name)
    coords = synth.make_coords(w)
    xb = synth.features(w.n, w.channels, w.seed)
    wb = synth.weights(w.channels, w.channels, w.seed)
    times = []
    t_start = time.perf_counter()
    while True:
        t0 = time.perf_counter()
        so.subm_conv(coords, xb, wb)
        times.append(time.perf_counter() - t0)
        if time.perf_counter() - t_start > budget_s or len(times) >= 20:
            break
    med = statistics.median(times)
    return {"value": med * 1e6, "unit": "us/layer", "cores": cores, "kind": "oracle",
            "sample": f"{len(times)} full {name} layers (map from a dict, float64 per-tap matmuls),"
                      f" median; the map part is single-threaded Python, the matmuls use "
                      f"{cores} BLAS threads"}


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
    (profiled) duration. Runs on the CPU."""
    import re

    def short(k):
        k = k.replace("(anonymous namespace)::", "").replace("void ", "").replace("smc::", "")
        return re.sub(r"\(.*", "", k).split("<")[0].strip()

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
    files = glob.glob(os.path.join(pmc_dir, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {pmc_dir}")
    per = {}                       # kernel -> dispatch -> {counter: value, "ns": duration}
    for fn in files:
        with open(fn) as f:
            for row in csv.DictReader(f):
                k = short(row["Kernel_Name"])
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
            "mfma_busy_frac": busy / (ns * 1e-9 * CLOCK_HZ * N_SIMD) if ns else None}
    path = os.path.join(ROOT, "profiles", f"mfma_{workload}_{algo}.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print(f"wrote {path}")
    for k, v in out["kernels"].items():
        print(f"{k}: executed {v['mfma_flops_executed']:.4g} flop, useful {v['flops_useful']:.4g} "
              f"({v['useful_over_executed']:.3f}); MFMA busy {v['mfma_busy_frac']:.4f} of the "
              f"SIMD cycles over {v['profiled_ns'] / 1e3:.2f} us (profiled)")


def summarize_pmc(fetch_dir, write_dir, workload, algo, copy_mb):
    """Per-dispatch FETCH_SIZE / WRITE_SIZE (KiB) of every kernel, scaled by what the
    same counters read for a plain device copy of copy_mb MiB."""
    import re

    def short(k):
        k = k.replace("(anonymous namespace)::", "").replace("void ", "").replace("smc::", "")
        return re.sub(r"\(.*", "", k).split("<")[0].strip()

    out = {"workload": workload, "algo": algo, "copy_probe_mib": copy_mb, "kernels": {}}
    per = {}
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        vals = {}
        for k, v in _pmc_rows(d, counter):
            vals.setdefault(short(k), []).append(v)
        per[counter] = vals
    copy_names = [k for k in per["FETCH_SIZE"] if "copyBuffer" in k or "elementwise" in k.lower()]
    if not copy_names:
        raise SystemExit("no copy kernel found for the calibration")
    cname = max(copy_names, key=lambda k: max(per["FETCH_SIZE"][k]))
    kib = copy_mb * 1024.0
    f_copy = max(per["FETCH_SIZE"][cname])
    w_copy = max(per["WRITE_SIZE"].get(cname, [0.0]))
    out["copy_kernel"] = cname
    out["copy_fetch_kib"] = f_copy
    out["copy_write_kib"] = w_copy
    out["fetch_scale"] = kib / f_copy if f_copy else None
    out["write_scale"] = kib / w_copy if w_copy else None
    for k in sorted(set(per["FETCH_SIZE"]) | set(per["WRITE_SIZE"])):
        if not k.startswith("k_"):
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


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="lidar",
                    choices=["tiny", "lidar", "deep", "wide", "stage"])
    ap.add_argument("--algo", default="pairs", choices=["pairs", "mask_tiles"],
                    help="forward algorithm of the headline line (the other is reported too)")
    ap.add_argument("--order", default="plain", choices=list(ORDERS),
                    help="mask-tile row order: plain mask value, calibrated bit order, or "
                         "calibrated order with 3 offset groups (calibrated on another seed)")
    ap.add_argument("--sync-build", action="store_true",
                    help="wait for the map's device-side checks inside every step")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-other-algo", action="store_true")
    ap.add_argument("--copy-probe-mb", type=int, default=0,
                    help="run one plain device copy of this many MiB first (PMC calibration)")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"))
    ap.add_argument("--summarize-mfma", nargs=2, metavar=("PMC_DIR", "BENCH_OUT"),
                    help="summarise a rocprofv3 --pmc run of the MFMA counters and the "
                         "JSON line that run printed")
    ap.add_argument("--report", default="",
                    help="also run every workload and write their figures to this JSON file")
    args = ap.parse_args()

    if args.summarize_mfma:
        summarize_mfma(args.summarize_mfma[0], args.workload, args.algo, args.summarize_mfma[1])
        return
    if args.summarize_pmc:
        summarize_pmc(args.summarize_pmc[0], args.summarize_pmc[1], args.workload, args.algo,
                      args.copy_probe_mb or 256)
        return

    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported by this build "
              "(no multi-GPU path: every box here has one GPU)", file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)

    r = run_workload(args.workload, args.steps, args.warmup, args.sync_build, args.algo,
                     args.copy_probe_mb, args.order)
    w, info = r["workload"], r["info"]
    c = w.channels
    line = {
        "metric": METRIC,
        "value": round(r["per_layer_us"], 2),
        "unit": "us/layer",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["ms_per_step"], 4),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": f"{w.name}: {w.n} voxels, grid {w.grid[0]}x{w.grid[1]}x{w.grid[2]}, "
                        f"C_in=C_out={c}, {w.layers} layer(s), seed {w.seed}",
            "n": w.n, "pairs": r["pairs"], "pairs_per_voxel": round(r["pairs"] / w.n, 4),
            "route": info["route"], "c_in": c, "c_out": c, "layers": w.layers,
            "map_built_every_step": True, "build_mode": "sync" if args.sync_build else "async",
            "algo": args.algo,
            **({"order": args.order} if args.algo == "mask_tiles" else {}),
        },
        "tflops_effective": round(r["tflops_effective"], 3),
        "frac_bf16_peak": round(r["tflops_effective"] / PEAK_BF16_TFLOPS, 5),
        "gpu_ms_per_step_events": round(r["gpu_ms_per_step"], 4),
        "stage_us": {k: round(v, 2) for k, v in r["stage_us"].items()},
        "stages": {k: {"us": round(v["us"], 2), "GB/s": round(v["gbs"], 1),
                       "hbm_frac": round(v["gbs"] / PEAK_HBM_GBS, 4),
                       "TFLOP/s": round(v["tflops"], 2)} for k, v in r["model"].items()},
        "weight_pack_us": round(r["pack_us"], 2),
        "roofline": roofline(r),
    }
    if r["tile_work_ratio"] is not None:
        line["tile_work_ratio"] = round(r["tile_work_ratio"], 4)
    if not args.no_other_algo:
        # the other forward algorithm, and the mask-tile row orders
        variants = [("pairs", "plain")] if args.algo == "mask_tiles" else []
        variants += [("mask_tiles", o) for o in ORDERS
                     if not (args.algo == "mask_tiles" and o == args.order)]
        line["other_algo"] = []
        for algo2, order2 in variants:
            r2 = run_workload(args.workload, args.steps, args.warmup, args.sync_build, algo2,
                              order=order2)
            e = {"algo": algo2, "us_per_layer": round(r2["per_layer_us"], 2),
                 "tflops_effective": round(r2["tflops_effective"], 3),
                 "stage_us": {k: round(v, 2) for k, v in r2["stage_us"].items()}}
            if algo2 == "mask_tiles":
                e["order"] = order2
                e["tile_work_ratio"] = round(r2["tile_work_ratio"], 4)
            line["other_algo"].append(e)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(args.workload)
    if args.report:
        rep = {}
        runs = []
        for name in ("tiny", "lidar", "deep", "wide", "stage"):
            runs += [(name, "pairs", "plain", 3, 1)]
            runs += [(name, "mask_tiles", o, 3, 1) for o in ORDERS]
        # 5x5x5 kernels, and several frames as batches of one map
        runs += [("lidar", "pairs", "plain", 5, 1), ("deep", "pairs", "plain", 5, 1),
                 ("wide", "pairs", "plain", 5, 1), ("lidar", "pairs", "plain", 3, 4),
                 ("lidar", "pairs", "plain", 5, 4)]
        runs = [r + (False,) for r in runs]
        # strided (downsampling) layers, mask tiles
        runs += [(nm, "mask_tiles", "plain", 3, 1, True) for nm in ("lidar", "deep", "wide", "stage")]
        for name, algo, order, ks, frames, strided in runs:
            rr = run_workload(name, max(20, args.steps // 2), args.warmup, algo=algo,
                              order=order, kernel_size=ks, frames=frames, strided=strided)
            key = (f"{name}/{algo}" + ("" if order == "plain" else f"/{order}")
                   + ("" if ks == 3 else f"/k{ks}") + ("" if frames == 1 else f"/b{frames}")
                   + ("/strided" if strided else ""))
            rep[key] = {k: rr[k] for k in ("pairs", "ms_per_step", "per_layer_us", "pack_us",
                                           "tflops_effective", "stage_us", "model",
                                           "tile_work_ratio", "calibration", "kernel_size",
                                           "frames", "n", "n_out", "strided")}
            rep[key]["route"] = rr["info"]["route"]
            rep[key]["roofline"] = roofline(rr)
        with open(args.report, "w") as f:
            json.dump(rep, f, indent=1)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
