"""Seeded synthetic voxel sets, features and weights.

This module only draws inputs. It holds none of the convolution's arithmetic:
no neighbour search, no mask, no pair list, no accumulation. Both the CPU
oracle's tests and the GPU path's tests and benchmark take their inputs from
here, so the two sides see identical data.

Workloads (stand-ins for the public LiDAR / indoor captures the pages measure
on, which are not available here):

* ``tiny``   2,048 distinct cells drawn uniformly from a 24^3 grid, C=16.
* ``lidar``  ~32,000 voxels on a 1440x1440x41 grid from the ground+box
             generator below, C=128.
* ``deep``   ~15,000 voxels on 360x360x11, C=512.
* ``wide``   ~95,000 voxels over 2095x2095x695 (a grid too large for a dense
             presence table), C=128.
* ``stage``  ~91,000 voxels on 1440x1440x41, C=128, six layers sharing one map.

Values are bf16. They are drawn as float32 and rounded to bf16 with torch's
own float32 -> bfloat16 conversion (round to nearest even); they are handed
out as raw uint16 bit patterns so that every consumer decodes them itself.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

__all__ = [
    "Workload", "WORKLOADS", "workload", "make_coords", "tiny_coords",
    "ground_box_coords", "bf16_bits_from_f32", "features", "weights",
    "int_features", "int_weights", "box_coords", "isolated_coords", "batched_coords",
]


@dataclass(frozen=True)
class Workload:
    name: str
    n: int                      # target number of active voxels
    grid: tuple                 # (X, Y, Z) extent of the coordinate grid
    channels: int               # C_in = C_out
    seed: int
    layers: int = 1             # >1: a stage of layers sharing one kernel map
    kind: str = "ground_box"    # or "uniform"
    notes: str = field(default="", compare=False)


WORKLOADS = {
    "tiny": Workload("tiny", 2048, (24, 24, 24), 16, 1, kind="uniform"),
    "lidar": Workload("lidar", 32000, (1440, 1440, 41), 128, 2),
    "deep": Workload("deep", 15000, (360, 360, 11), 512, 3),
    "wide": Workload("wide", 95000, (2095, 2095, 695), 128, 4),
    "stage": Workload("stage", 91000, (1440, 1440, 41), 128, 5, layers=6),
}


def workload(name: str) -> Workload:
    return WORKLOADS[name]


# --------------------------------------------------------------------------
# coordinates
# --------------------------------------------------------------------------

def _with_batch(xyz: np.ndarray, batch: int = 0) -> np.ndarray:
    out = np.empty((xyz.shape[0], 4), dtype=np.int32)
    out[:, 0] = batch
    out[:, 1:] = xyz
    return out


def tiny_coords(seed: int = 1, n: int = 2048, side: int = 24) -> np.ndarray:
    """``n`` distinct cells drawn without replacement from a side^3 grid.

    Returns int32 [n, 4] rows (b, x, y, z) with b = 0, in draw order.
    """
    rng = np.random.default_rng(seed)
    lin = rng.choice(side ** 3, size=n, replace=False)
    x, y, z = np.unravel_index(lin, (side, side, side))
    return _with_batch(np.stack([x, y, z], axis=1).astype(np.int32))


def _box_surface_lin(x0, y0, z0, wx, wy, h, grid):
    X, Y, Z = grid
    xs = np.arange(x0, x0 + wx)
    ys = np.arange(y0, y0 + wy)
    zs = np.arange(z0, z0 + h)
    gx, gy, gz = np.meshgrid(xs, ys, zs, indexing="ij")
    on_face = ((gx == x0) | (gx == x0 + wx - 1) | (gy == y0) | (gy == y0 + wy - 1)
               | (gz == z0) | (gz == z0 + h - 1))
    gx, gy, gz = gx[on_face], gy[on_face], gz[on_face]
    return (gx.astype(np.int64) * Y + gy) * Z + gz


def ground_box_coords(n: int, grid, seed: int, n_boxes: int = 200) -> np.ndarray:
    """Ground slab plus box surfaces, the outdoor-scan stand-in.

    1. round(0.7 n) ground voxels: x, y uniform over the grid, z in {0, 1};
       a candidate is kept with probability 1 / (1 + r / 200), r being its
       distance in cells from the grid centre ((X-1)/2, (Y-1)/2). Distinct
       cells are kept in draw order until there are enough.
    2. ``n_boxes`` axis-aligned boxes: widths U{4..40} in x and y, height
       U{4..20} clipped to Z, lower corner uniform so the box fits the grid.
    3. The cells on at least one face of some box, minus the ground cells,
       sorted by linear index; n - round(0.7 n) of them are drawn without
       replacement.
    4. All rows are shuffled, so input order carries no spatial order.

    Returns int32 [n, 4] rows (b, x, y, z) with b = 0.
    """
    X, Y, Z = grid
    rng = np.random.default_rng(seed)
    n_ground = int(round(0.7 * n))
    cx, cy = (X - 1) / 2.0, (Y - 1) / 2.0

    chosen: list = []
    seen: set = set()
    while len(chosen) < n_ground:
        m = max(4 * (n_ground - len(chosen)), 1024)
        x = rng.integers(0, X, size=m)
        y = rng.integers(0, Y, size=m)
        z = rng.integers(0, min(2, Z), size=m)
        r = np.sqrt((x - cx) ** 2 + (y - cy) ** 2)
        keep = rng.random(m) < 1.0 / (1.0 + r / 200.0)
        lin = (x[keep].astype(np.int64) * Y + y[keep]) * Z + z[keep]
        for v in lin.tolist():
            if v not in seen:
                seen.add(v)
                chosen.append(v)
                if len(chosen) == n_ground:
                    break
    ground = np.asarray(chosen, dtype=np.int64)

    surf = []
    for _ in range(n_boxes):
        wx = int(rng.integers(4, 41))
        wy = int(rng.integers(4, 41))
        h = min(int(rng.integers(4, 21)), Z)
        x0 = int(rng.integers(0, X - wx + 1))
        y0 = int(rng.integers(0, Y - wy + 1))
        z0 = int(rng.integers(0, Z - h + 1))
        surf.append(_box_surface_lin(x0, y0, z0, wx, wy, h, grid))
    surf = np.unique(np.concatenate(surf))
    surf = np.setdiff1d(surf, ground, assume_unique=True)
    n_box = n - n_ground
    if n_box > surf.size:
        raise ValueError(f"box surfaces hold {surf.size} cells, {n_box} requested")
    box = rng.choice(surf, size=n_box, replace=False)

    lin = np.concatenate([ground, box])
    lin = lin[rng.permutation(lin.size)]
    x, rem = np.divmod(lin, Y * Z)
    y, z = np.divmod(rem, Z)
    return _with_batch(np.stack([x, y, z], axis=1).astype(np.int32))


def make_coords(w: Workload) -> np.ndarray:
    if w.kind == "uniform":
        return tiny_coords(w.seed, w.n, w.grid[0])
    return ground_box_coords(w.n, w.grid, w.seed)


def box_coords(a: int, b: int, c: int, origin=(0, 0, 0), batch: int = 0,
               seed: int | None = None) -> np.ndarray:
    """Every cell of an a x b x c box (optionally shuffled)."""
    g = np.stack(np.meshgrid(np.arange(a), np.arange(b), np.arange(c),
                             indexing="ij"), axis=-1).reshape(-1, 3)
    g = g + np.asarray(origin)
    if seed is not None:
        g = g[np.random.default_rng(seed).permutation(len(g))]
    return _with_batch(g.astype(np.int32), batch)


def isolated_coords(n: int, spacing: int = 2, seed: int = 0) -> np.ndarray:
    """n voxels on a lattice of pitch ``spacing`` >= 2 (no two are adjacent)."""
    side = int(np.ceil(n ** (1 / 3))) + 1
    rng = np.random.default_rng(seed)
    lin = rng.choice(side ** 3, size=n, replace=False)
    x, y, z = np.unravel_index(lin, (side, side, side))
    return _with_batch((np.stack([x, y, z], axis=1) * spacing).astype(np.int32))


# --------------------------------------------------------------------------
# values
# --------------------------------------------------------------------------

def bf16_bits_from_f32(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 with torch's conversion; uint16 bits."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def features(n: int, c: int, seed: int) -> np.ndarray:
    """bf16 bits of N(0, 1) draws, shape [n, c]."""
    rng = np.random.default_rng(seed + 1000)
    return bf16_bits_from_f32(rng.standard_normal((n, c), dtype=np.float32))


def weights(c_in: int, c_out: int, seed: int, layer: int = 0, taps: int = 27) -> np.ndarray:
    """bf16 bits of N(0, 1) / sqrt(taps c_in) draws, shape [taps, c_in, c_out]
    (27 taps for a 3x3x3 kernel, 125 for 5x5x5)."""
    rng = np.random.default_rng(seed + 2000 + layer)
    w = rng.standard_normal((taps, c_in, c_out), dtype=np.float32)
    return bf16_bits_from_f32(w / np.float32(np.sqrt(float(taps) * c_in)))


def batched_coords(w: "Workload", frames: int) -> np.ndarray:
    """``frames`` independent voxel sets of workload w (seeds seed, seed + 1,
    ...), stacked as batches b = 0 .. frames - 1 and shuffled together."""
    parts = []
    for b in range(frames):
        c = make_coords(Workload(w.name, w.n, w.grid, w.channels, w.seed + b, w.layers, w.kind))
        c[:, 0] = b
        parts.append(c)
    out = np.concatenate(parts)
    return out[np.random.default_rng(w.seed + 7000).permutation(len(out))]


def int_features(n: int, c: int, seed: int, lo: int = -3, hi: int = 3) -> np.ndarray:
    """Small integers (exact in bf16), bf16 bits, shape [n, c]."""
    rng = np.random.default_rng(seed + 3000)
    return bf16_bits_from_f32(rng.integers(lo, hi + 1, size=(n, c)).astype(np.float32))


def int_weights(c_in: int, c_out: int, seed: int, layer: int = 0,
                lo: int = -2, hi: int = 2) -> np.ndarray:
    rng = np.random.default_rng(seed + 4000 + layer)
    return bf16_bits_from_f32(
        rng.integers(lo, hi + 1, size=(27, c_in, c_out)).astype(np.float32))
