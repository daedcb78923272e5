"""CPU oracle for submanifold sparse 3x3x3 convolution.

TEST INFRASTRUCTURE. Only the test suite, the smoke check and the
benchmark's CPU-baseline leg import this module. The GPU library never calls
it, never links it, and shares no code, table or helper with it.

Sources (the pages this follows):

* [P1] "[Kernel] Add submanifold sparse 3D convolution (bf16 implicit GEMM,
  gfx950)", FlyDSL pull request #942 -- sections "Summary", "Design, and the measurements behind it", "Test plan",
  and its commit messages.
* [P5] "Sparse convolution in FP32", DriveRT project page -- sections
  "The starting point", "Neighbour masks and sorted rows", "Calibrated bit
  order", "Offset-group partitioning".

What is computed ([P5] "The starting point"; [P1] Summary): for every
active voxel p of the set S (the output set is S itself),

    Y[p, co] = sum over the 27 offsets d with p + d in S of
               sum over ci of X[p + d, ci] * W[k(d), ci, co]

and the same with the 125 offsets of a 5 x 5 x 5 kernel ([P1] "Test plan"
lists kernel sizes 3 and 5).

Readings fixed here where the pages are silent:

* offset order: k(d) = 9 (dx + 1) + 3 (dy + 1) + (dz + 1), x slowest; the
  centre is k = 13. The same k indexes the mask bit and W's first axis. For
  K = 5 the same rule with offsets -2..2: k = 25 (dx + 2) + 5 (dy + 2) +
  (dz + 2), centre 62; the 125-bit mask is kept as four 32-bit words.
* sign: output p reads input p + d (cross-correlation).
* W layout: [K^3, C_in, C_out].
* coordinates: rows (b, x, y, z) for [N, 4]; (x, y, z) with b = 0 for [N, 3];
  neighbours never cross batches.
* duplicate coordinates are a caller error (raised here).
* mask sort: ascending plain mask value, ties by ascending row.
* calibrated bit order and offset groups: see ``group_row_orders`` and
  ``calibrate_order`` (a greedy search; the pages do not say how the order
  or the groups are chosen).
* strided layer: stride 2, padding (K-1)/2, outputs ordered by (b, x, y, z);
  see ``build_strided_map``.
* pair lists: tap-major, and within a tap in ascending output row (the
  order inside a tap does not change the sum; [P1]'s compaction lists each
  tap's rows in the order it scans them).
* rounding to bf16: round to nearest, ties to even.

Accumulation is float64 by default (the products of two bf16 values are
exact in float64, so the only error is the float64 summation, far below the
float32 accumulator the GPU uses); ``acc_dtype=np.float32`` gives the
float32 per-offset accumulation the pages describe.

Pins for every function live in tests/test_oracle_pins.py (brute-force
neighbour enumeration, closed-form pair counts on full boxes, masked dense
convolution via numpy shifted slices and via torch.nn.functional.conv3d,
integer-exact and one-hot cases, hand-derived worked examples, and bf16
rounding against torch's conversion). No function here is unpinned.
"""
from __future__ import annotations

import numpy as np

TAPS = 27
CENTRE = 13
KERNEL_SIZES = (3, 5)


def taps_of(kernel_size: int) -> int:
    """Offsets of a K x K x K kernel (27 or 125)."""
    if kernel_size not in KERNEL_SIZES:
        raise ValueError("kernel_size must be 3 or 5")
    return kernel_size ** 3


def centre_of(kernel_size: int) -> int:
    """Tap of the zero offset: the middle of the K^3 taps (13 or 62)."""
    return (taps_of(kernel_size) - 1) // 2


class DuplicateCoordinate(ValueError):
    pass


def tap_offsets(kernel_size: int = 3) -> list:
    """The K^3 offsets d in tap order k = K^2 (dx+r) + K (dy+r) + (dz+r),
    r = (K-1)/2 (for K = 3: k = 9(dx+1) + 3(dy+1) + (dz+1))."""
    taps_of(kernel_size)
    r = (kernel_size - 1) // 2
    offs = []
    for dx in range(-r, r + 1):
        for dy in range(-r, r + 1):
            for dz in range(-r, r + 1):
                offs.append((dx, dy, dz))
    return offs


# --------------------------------------------------------------------------
# bf16 helpers ([P1] "Design, and the measurements behind it": features and
# weights are stored as bf16)
# --------------------------------------------------------------------------

def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Decode bf16 bit patterns: a bf16 is the top half of a float32."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round real values to the nearest bf16 value, ties to even.

    bf16 keeps 8 significant bits. Write x = m * 2**e with 0.5 <= |m| < 1;
    the bf16 grid spacing around x is 2**(e - 8), never finer than the
    subnormal spacing 2**-133. Dividing by the spacing is exact, and
    numpy's round() rounds halves to even, which is the rule wanted.
    Values are returned as float64 (every bf16 is exact there).
    """
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)
    spacing = np.ldexp(1.0, np.maximum(e - 8, -133))
    r = np.round(x / spacing) * spacing
    big = np.abs(r) > 3.3895313892515355e38     # above the largest bf16
    r = np.where(big, np.copysign(np.inf, x), r)
    return np.where(np.isfinite(x), r, x)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """bf16 bit patterns of ``round_to_bf16(x)``."""
    r = round_to_bf16(x).astype(np.float32)     # exact: bf16 values fit float32
    return (r.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


# --------------------------------------------------------------------------
# kernel map ([P5] "Neighbour masks and sorted rows"; [P1] "Summary", "Design, and the measurements behind it")
# --------------------------------------------------------------------------

def _rows_bxyz(coords: np.ndarray) -> np.ndarray:
    c = np.asarray(coords)
    if c.ndim != 2 or c.shape[1] not in (3, 4):
        raise ValueError("coords must be [N, 3] or [N, 4]")
    if c.shape[1] == 3:
        c = np.concatenate([np.zeros((c.shape[0], 1), c.dtype), c], axis=1)
    return c.astype(np.int64)


def build_kernel_map(coords: np.ndarray, kernel_size: int = 3):
    """Neighbour table and neighbour masks from a hash map.

    A dictionary maps each (b, x, y, z) to its row. For row i and tap k,
    nbr[i, k] is the row at c_i + d_k, or -1 when that cell is inactive, and
    bit k of row i's mask is set exactly when the neighbour exists. This is
    the table plus mask that the map builder of [P5] "Neighbour masks and
    sorted rows" emits; the centre column is always the row itself. K = 5
    ([P1] "Test plan": kernel sizes 3 and 5) gives 125 taps.

    Returns (nbr int32 [N, K^3], mask): mask is uint32 [N] for K = 3 (27
    bits) and uint32 [N, 4] for K = 5 (bit k in word k // 32, bit k % 32).
    """
    kv = taps_of(kernel_size)
    c = _rows_bxyz(coords)
    n = c.shape[0]
    table = {}
    for i in range(n):
        key = tuple(c[i].tolist())
        if key in table:
            raise DuplicateCoordinate(f"rows {table[key]} and {i} share {key}")
        table[key] = i
    offs = tap_offsets(kernel_size)
    nbr = np.full((n, kv), -1, dtype=np.int32)
    words = (kv + 31) // 32
    mask = np.zeros((n, words), dtype=np.uint32)
    for i in range(n):
        b, x, y, z = c[i].tolist()
        m = 0
        for k, (dx, dy, dz) in enumerate(offs):
            j = table.get((b, x + dx, y + dy, z + dz))
            if j is not None:
                nbr[i, k] = j
                m |= 1 << k
        for q in range(words):
            mask[i, q] = (m >> (32 * q)) & 0xFFFFFFFF
    return nbr, (mask[:, 0].copy() if kernel_size == 3 else mask)


def mask_sort(mask: np.ndarray) -> np.ndarray:
    """Rows ordered by neighbour mask ([P5] "Neighbour masks and sorted rows").

    The page sorts rows by mask so that rows with equal masks sit together;
    ties are broken by ascending row here so that the order is unique.
    Returns perm int32 [N]: perm[s] is the row at sorted position s.
    """
    m = [int(v) for v in np.asarray(mask).tolist()]
    order = sorted(range(len(m)), key=lambda r: (m[r], r))
    return np.asarray(order, dtype=np.int32)


# --------------------------------------------------------------------------
# mask-tile row orders ([P5] "Calibrated bit order", "Offset-group
# partitioning"; "Neighbour masks and sorted rows")
# --------------------------------------------------------------------------

def _check_order(bit_order, group_of):
    order = list(range(TAPS - 1, -1, -1)) if bit_order is None else [int(t) for t in bit_order]
    if sorted(order) != list(range(TAPS)):
        raise ValueError("bit_order must list each of the 27 taps once")
    groups = [0] * TAPS if group_of is None else [int(g) for g in group_of]
    if len(groups) != TAPS or min(groups) < 0:
        raise ValueError("group_of must give a group index >= 0 for each tap")
    n_groups = max(groups) + 1
    if sorted(set(groups)) != list(range(n_groups)):
        raise ValueError("group indices must be 0 .. G-1 with no gap")
    if groups[CENTRE] != n_groups - 1:
        raise ValueError("the centre tap must be in the last group")
    return order, groups, n_groups


def group_row_orders(mask: np.ndarray, bit_order=None, group_of=None):
    """Row order of every offset group for the mask-tile GEMM.

    [P5] "Calibrated bit order": rows are sorted by their mask with its bits
    taken in a chosen order (``bit_order`` lists the taps from most to least
    significant; None is the plain mask value, tap 26 first).
    [P5] "Offset-group partitioning": the taps are split into groups
    (``group_of[k]`` is tap k's group) and each group has its own row order,
    under the mask restricted to the group's taps. Reading fixed here: group
    g lists the rows with at least one tap in the group, by (restricted mask
    in bit order, row); the rows with none follow, by row. The centre tap
    must be in the last group, so the last group holds every row (the page's
    last launch spans every row).

    Returns (orders, counts): orders is int32 [G, N] (row ids), counts[g]
    the number of rows of group g that have a tap in it.
    """
    order, groups, n_groups = _check_order(bit_order, group_of)
    m = [int(v) for v in np.asarray(mask).tolist()]
    n = len(m)
    out = np.zeros((n_groups, n), dtype=np.int32)
    counts = []
    for g in range(n_groups):
        taps = [t for t in order if groups[t] == g]          # most significant first
        keys = []
        for r in range(n):
            bits = tuple((m[r] >> t) & 1 for t in taps)
            keys.append((0 if any(bits) else 1, bits, r))
        keys.sort()
        out[g] = [k[2] for k in keys]
        counts.append(sum(1 for k in keys if k[0] == 0))
    return out, np.asarray(counts, dtype=np.int64)


def tile_work(mask: np.ndarray, rows, count: int, taps=None, tile: int = 64) -> int:
    """Tap-rows a mask-tile pass executes ([P5] "Neighbour masks and sorted
    rows": a tile evaluates the union of its rows' offsets for every row).

    The first ``count`` entries of ``rows`` are cut into consecutive tiles of
    ``tile`` rows; each tile costs its row count times the number of taps
    (of ``taps``, default all 27) present in at least one of its rows.
    """
    allowed = set(range(TAPS)) if taps is None else {int(t) for t in taps}
    m = [int(v) for v in np.asarray(mask).tolist()]
    work = 0
    for s in range(0, int(count), tile):
        part = [int(r) for r in rows[s:min(s + tile, int(count))]]
        union = {t for r in part for t in allowed if (m[r] >> t) & 1}
        work += len(part) * len(union)
    return work


def calibrate_order(mask: np.ndarray, n_groups: int = 1, tile: int = 64):
    """A bit order and offset groups chosen on a calibration map.

    The pages calibrate a permutation of the 27 bits offline ([P5]
    "Calibrated bit order") and split the offsets into a few groups ([P5]
    "Offset-group partitioning") without saying how either is chosen. The
    reading fixed here is a greedy search on the executed work of the mask
    tiles (``tile_work`` of the one-group order):

    1. Start from the 26 off-centre taps by ascending count of rows that
       have them (ties: lower tap first); the centre, present in every row,
       is always least significant.
    2. For each position from the most significant down, try every
       remaining tap there, the others following in their current order,
       and keep the one with the least work (ties: the earlier candidate).
    3. Groups: the off-centre taps, in the chosen order, are cut into
       ``n_groups`` consecutive runs, run g holding positions
       floor(26 g / G) .. floor(26 (g+1) / G) - 1; the centre joins the last.

    Returns (bit_order list[27], group_of list[27]).
    """
    if not 1 <= n_groups <= 26:
        raise ValueError("n_groups must be in 1 .. 26")
    m = np.asarray(mask, dtype=np.uint32)
    counts = [int(((m >> np.uint32(t)) & 1).sum()) for t in range(TAPS)]
    remaining = sorted((t for t in range(TAPS) if t != CENTRE), key=lambda t: (counts[t], t))
    chosen: list = []
    n = len(m)

    def work_of(order):
        orders, cnt = group_row_orders(m, order, None)
        return tile_work(m, orders[0], cnt[0], None, tile)

    while remaining:
        best_t, best_w = None, None
        for t in remaining:
            cand = chosen + [t] + [r for r in remaining if r != t] + [CENTRE]
            w = work_of(cand) if n else 0
            if best_w is None or w < best_w:
                best_t, best_w = t, w
        chosen.append(best_t)
        remaining.remove(best_t)
    order = chosen + [CENTRE]
    group_of = [0] * TAPS
    for g in range(n_groups):
        for pos in range((26 * g) // n_groups, (26 * (g + 1)) // n_groups):
            group_of[chosen[pos]] = g
    group_of[CENTRE] = n_groups - 1
    return order, group_of


def mask_bit(mask: np.ndarray, k: int) -> np.ndarray:
    """Bit k of every row's mask (uint32 [N] or words [N, W]) as a bool array."""
    m = np.asarray(mask, dtype=np.uint32)
    if m.ndim == 1:
        return ((m >> np.uint32(k)) & np.uint32(1)) == 1
    return ((m[:, k // 32] >> np.uint32(k % 32)) & np.uint32(1)) == 1


def compact_pairs(nbr: np.ndarray, mask: np.ndarray):
    """Per-tap pair lists holding only the neighbours that exist.

    [P1] "Design, and the measurements behind it" (compaction): only valid (input, output) pairs are listed,
    grouped by tap so that a run of pairs shares one weight slab; the centre
    tap is listed like the others ([P1] commit d4161ef, "The centre tap is
    compacted along with the rest"). Within a tap, pairs follow ascending
    output row. The tap count is nbr's width (27 or 125).

    Returns (pair_in int32 [P], pair_out int32 [P], tap_off int64 [taps+1]);
    the pairs of tap k are [tap_off[k], tap_off[k+1]).
    """
    nbr = np.asarray(nbr)
    ins, outs, off = [], [], [0]
    for k in range(nbr.shape[1]):
        rows = np.nonzero(mask_bit(mask, k))[0]
        ins.append(nbr[rows, k].astype(np.int32))
        outs.append(rows.astype(np.int32))
        off.append(off[-1] + rows.size)
    return (np.concatenate(ins) if ins else np.zeros(0, np.int32),
            np.concatenate(outs) if outs else np.zeros(0, np.int32),
            np.asarray(off, dtype=np.int64))


# --------------------------------------------------------------------------
# strided (downsampling) convolution ([P5] "Calibrated bit order": the
# strided kernels change the coordinate set; "One kernel family, configured
# per stage": conv1 to conv4 of the backbone)
# --------------------------------------------------------------------------

def strided_out_shape(spatial_shape, kernel_size: int = 3, stride: int = 2, padding=None):
    """Output grid extent per axis: floor((X + 2p - K) / s) + 1 (p = (K-1)/2 by default)."""
    if padding is None:
        padding = (kernel_size - 1) // 2
    return tuple((int(e) + 2 * padding - kernel_size) // stride + 1 for e in spatial_shape)


def build_strided_map(coords, spatial_shape, kernel_size: int = 3, stride: int = 2,
                      padding=None):
    """Output cells and kernel map of a strided sparse convolution.

    The pages do not define the strided layer beyond its changing the
    coordinate set. Reading fixed here (the usual downsampling layer): output
    cell o of a batch exists when some active input c of that batch equals
    s o - p + d for a tap d in [0, K)^3, with o inside the output grid
    (``strided_out_shape``); output rows are ordered by (b, x, y, z). Tap k =
    K^2 dx + K dy + dz, the submanifold numbering with offsets shifted by r;
    nbr[o, k] is the row of input s o - p + d_k, or -1; bit k of mask[o] is set
    when it exists. Input coordinates must lie in [0, spatial_shape).

    The default padding is p = (K - 1) / 2 (1 for K = 3, 2 for K = 5), so the
    taps of output o are the cells s o + d' with d' in [-r, r]^3.

    Returns (out_coords int32 [M, 4], out_shape, nbr int32 [M, K^3],
    mask uint32 [M] (K = 3) or [M, 4] words (K = 5)).
    """
    kv = taps_of(kernel_size)
    if padding is None:
        padding = (kernel_size - 1) // 2
    c = _rows_bxyz(coords)
    shape = tuple(int(e) for e in spatial_shape)
    oshape = strided_out_shape(shape, kernel_size, stride, padding)
    table = {}
    for i in range(c.shape[0]):
        key = tuple(c[i].tolist())
        if key in table:
            raise DuplicateCoordinate(f"rows {table[key]} and {i} share {key}")
        if any(not 0 <= key[1 + a] < shape[a] for a in range(3)) or key[0] < 0:
            raise ValueError(f"row {i} = {key} outside the grid {shape}")
        table[key] = i
    taps = [(dx, dy, dz) for dx in range(kernel_size) for dy in range(kernel_size)
            for dz in range(kernel_size)]
    outs = set()
    for (b, x, y, z) in table:
        for d in taps:
            t = (x + padding - d[0], y + padding - d[1], z + padding - d[2])
            if all(v % stride == 0 and 0 <= v // stride < oshape[a] for a, v in enumerate(t)):
                outs.add((b, t[0] // stride, t[1] // stride, t[2] // stride))
    out = sorted(outs)
    m = len(out)
    nbr = np.full((m, kv), -1, dtype=np.int32)
    words = (kv + 31) // 32
    mask = np.zeros((m, words), dtype=np.uint32)
    for o, (b, ox, oy, oz) in enumerate(out):
        bits = 0
        for k, d in enumerate(taps):
            j = table.get((b, stride * ox - padding + d[0], stride * oy - padding + d[1],
                           stride * oz - padding + d[2]))
            if j is not None:
                nbr[o, k] = j
                bits |= 1 << k
        for q in range(words):
            mask[o, q] = (bits >> (32 * q)) & 0xFFFFFFFF
    oc = np.asarray(out, dtype=np.int32).reshape(m, 4)
    return oc, oshape, nbr, (mask[:, 0].copy() if kernel_size == 3 else mask)


def strided_conv(coords, spatial_shape, x_bits, w_bits, relu: bool = False,
                 acc_dtype=np.float64):
    """One strided layer: Y[o] = sum over taps k with nbr[o, k] >= 0 of
    X[nbr[o, k]] @ W[k] (the same per-tap accumulation as the submanifold
    layer, over the strided map). Returns a dict with the map, the
    accumulator and the bf16 output (ReLU after rounding when ``relu``)."""
    k_size = {27: 3, 125: 5}[np.asarray(w_bits).shape[0]]
    oc, oshape, nbr, mask = build_strided_map(coords, spatial_shape, k_size)
    pin, pout, toff = compact_pairs(nbr, mask)
    x = bf16_bits_to_f64(x_bits)
    w = bf16_bits_to_f64(w_bits)
    acc = conv_accumulate(x, w, pin, pout, toff, oc.shape[0], acc_dtype)
    y = round_to_bf16(acc)
    if relu:
        y = np.maximum(y, 0.0)
    return dict(out_coords=oc, out_shape=oshape, nbr=nbr, mask=mask,
                perm=mask_sort(mask) if k_size == 3 else None, pair_in=pin, pair_out=pout,
                tap_off=toff, acc=acc, y=y, y_bits=bf16_bits(y))


# --------------------------------------------------------------------------
# compute ([P5] "The starting point"; [P1] "Design, and the measurements behind it", commit d4161ef)
# --------------------------------------------------------------------------

def conv_accumulate(x: np.ndarray, w: np.ndarray, pair_in, pair_out, tap_off,
                    n_out: int, acc_dtype=np.float64) -> np.ndarray:
    """Per-offset gather -> matmul -> scatter-add into an accumulator.

    For each tap k, the gathered input rows X[pair_in] times W[k] are added
    to rows pair_out of the accumulator. An output row appears at most once
    per tap, so the indexed add never collides. x: [N_in, C_in] values,
    w: [taps, C_in, C_out] values (both real-valued arrays).
    """
    x = np.asarray(x, dtype=acc_dtype)
    w = np.asarray(w, dtype=acc_dtype)
    acc = np.zeros((n_out, w.shape[2]), dtype=acc_dtype)
    for k in range(w.shape[0]):
        a, b = int(tap_off[k]), int(tap_off[k + 1])
        if a == b:
            continue
        acc[pair_out[a:b]] += x[pair_in[a:b]] @ w[k]
    return acc


def conv_rows(x: np.ndarray, w: np.ndarray, nbr: np.ndarray, rows) -> np.ndarray:
    """The defining sum, evaluated row by row for the listed output rows.

    Y[i] = sum over taps k with nbr[i, k] >= 0 of X[nbr[i, k]] @ W[k],
    in float64. Used to check single rows of large problems.
    """
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    out = np.zeros((len(rows), w.shape[2]), dtype=np.float64)
    for t, i in enumerate(rows):
        for k in range(nbr.shape[1]):
            j = int(nbr[i, k])
            if j >= 0:
                out[t] += x[j] @ w[k]
    return out


def subm_conv(coords, x_bits, w_bits, relu: bool = False, acc_dtype=np.float64):
    """One submanifold K x K x K layer from raw inputs (K from w's first axis:
    27 taps for K = 3, 125 for K = 5).

    coords int [N, 3|4]; x_bits, w_bits bf16 bit patterns. Returns a dict
    with the map (nbr, mask, perm for K = 3, pair lists), the accumulator and
    the output as bf16 bits (ReLU after rounding when ``relu``).
    """
    k_size = {27: 3, 125: 5}[np.asarray(w_bits).shape[0]]
    nbr, mask = build_kernel_map(coords, k_size)
    perm = mask_sort(mask) if k_size == 3 else None
    pin, pout, toff = compact_pairs(nbr, mask)
    x = bf16_bits_to_f64(x_bits)
    w = bf16_bits_to_f64(w_bits)
    acc = conv_accumulate(x, w, pin, pout, toff, x.shape[0], acc_dtype)
    y = round_to_bf16(acc)
    if relu:
        y = np.maximum(y, 0.0)
    return dict(nbr=nbr, mask=mask, perm=perm, pair_in=pin, pair_out=pout,
                tap_off=toff, acc=acc, y=y, y_bits=bf16_bits(y))


def stage(coords, x_bits, w_bits_list, acc_dtype=np.float64):
    """Consecutive layers sharing one kernel map, ReLU between layers.

    The map is built once and reused by every layer ([P1] Performance,
    the 6-layer stage sharing one map). The ReLU is applied to the bf16
    output of every layer but the last, to every row ([P5] "Offset-group
    partitioning": the rectification must span every row).
    Returns the list of per-layer outputs (float64 bf16 values).
    """
    nbr, mask = build_kernel_map(coords)
    perm = mask_sort(mask)
    pin, pout, toff = compact_pairs(nbr, mask)
    h = bf16_bits_to_f64(x_bits)
    outs = []
    for li, wb in enumerate(w_bits_list):
        acc = conv_accumulate(h, bf16_bits_to_f64(wb), pin, pout, toff,
                              h.shape[0], acc_dtype)
        y = round_to_bf16(acc)
        if li + 1 < len(w_bits_list):
            y = np.maximum(y, 0.0)
        outs.append(y)
        h = y
    return outs
