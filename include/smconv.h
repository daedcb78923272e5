/*
 * smconv.h -- C ABI of the submanifold sparse 3x3x3 convolution library
 * for AMD Instinct MI355X (gfx950).
 *
 * What the library computes ("Sparse convolution in FP32", DriveRT, section
 * "The starting point"; "[Kernel] Add submanifold sparse 3D convolution
 * (bf16 implicit GEMM, gfx950)", FlyDSL PR #942, Summary): for each active
 * voxel p of the input set S, whose output set is S itself,
 *
 *     Y[p, co] = sum over offsets d in {-1,0,1}^3 with p + d in S of
 *                sum over ci of X[p + d, ci] * W[k(d), ci, co],
 *
 * with k(d) = 9 (dx+1) + 3 (dy+1) + (dz+1) (x slowest; the centre is 13).
 * Raw int32 voxel coordinates go in, the kernel map is built internally and
 * can be reused by every layer that shares the coordinates (PR #942,
 * commit 706a0bf, which keys the map cache on the coordinates; here the
 * reuse is an explicit handle), features and weights are bf16 and the
 * accumulation is float32 (PR #942, section "Design, and the measurements behind it").
 *
 * Conventions for every call:
 *  - Every call returns an int status (smc_status); 0 is success. No C++
 *    exception crosses this interface. smc_last_error() gives a message for
 *    the last failing call of the calling thread.
 *  - "device pointer" means memory the HIP runtime can read from the GPU
 *    the library was first used on (e.g. a torch CUDA tensor's data_ptr);
 *    "host pointer" means ordinary CPU memory.
 *  - "stream" is a hipStream_t passed as void* (NULL = the null stream).
 *    All GPU work is enqueued on that stream; the caller keeps every input
 *    alive and unmodified until the stream has run the work.
 *  - The caller owns every buffer it passes. The library keeps no caller
 *    pointer after a call returns (except in work already enqueued).
 *  - A map handle owns its own device buffers, allocated when a build or
 *    forward needs more room than it has (grow-only) and freed by
 *    smc_map_destroy: with hipMalloc/hipFree, or with the caller's allocator
 *    (smc_set_allocator). A handle is not thread-safe; all builds and
 *    forwards that use one handle must be issued on one stream, or the
 *    caller must order them.
 *  - bf16 tensors are passed as uint16_t bit patterns.
 */
#ifndef SMCONV_H
#define SMCONV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct smc_map smc_map;

typedef enum smc_status {
    SMC_OK = 0,
    SMC_ERR_ARG = 1,          /* a bad argument (null pointer, n < 0, C < 1, ...) */
    SMC_ERR_DUPLICATE = 2,    /* two rows share one (b, x, y, z): a caller error */
    SMC_ERR_RANGE = 3,        /* a coordinate outside [0, spatial_shape) or b outside [0, batch) */
    SMC_ERR_KEY_OVERFLOW = 4, /* the packed sorted-route key needs more than 64 bits */
    SMC_ERR_ALLOC = 5,        /* hipMalloc / hipHostMalloc failed */
    SMC_ERR_HIP = 6,          /* a HIP runtime call or a kernel launch failed */
    SMC_ERR_STATE = 7,        /* the map is not built, or was built with an error */
    SMC_ERR_UNSUPPORTED = 8,  /* a valid request this version does not implement (kernel_size != 3) */
    SMC_ERR_GRID = 9          /* the dense route was forced on a grid of 2^36 cells or more */
} smc_status;

/* Map routes ("[Kernel] Add submanifold sparse 3D convolution", section
 * "Design, and the measurements behind it": two mappers chosen by
 * bounding-box volume). */
enum {
    SMC_ROUTE_AUTO = 0,   /* dense presence grid when its 4.25 bytes a cell (int32 ids,
                             two occupancy bitmaps) fit 1/16 of the device's memory,
                             at most 16 GiB, and (if the handle must allocate it)
                             half the memory free at the build; sorted packed keys
                             otherwise */
    SMC_ROUTE_DENSE = 1,  /* force the dense presence grid */
    SMC_ROUTE_SORTED = 2  /* force the sorted packed-key mapper */
};

/* smc_map_build flags */
enum {
    SMC_BUILD_ASYNC = 1,    /* do not wait for the device-side checks; call smc_map_sync() later */
    SMC_BUILD_NO_PAIRS = 2, /* skip the per-tap pair lists: the pair-list forward and the
                               pair exports are then refused */
    SMC_BUILD_NO_SORT = 4,  /* skip the mask-sorted row order: SMC_FWD_MASK_TILES forwards
                               and the perm export are then refused */
    SMC_BUILD_TABLE = 8     /* keep the [n, K^3] neighbour table in device memory. Only the
                               dense-route 3x3x3 build with pair lists and without the mask
                               order leaves it out otherwise (its fused lookup and compaction
                               write the pair lists straight from the lookups); every other
                               build keeps it, because its later steps read it */
};

/* smc_conv_forward flags */
enum {
    SMC_FWD_RELU = 1,       /* apply max(y, 0) to the (rounded) output */
    SMC_FWD_OUT_F32 = 2,    /* write the float32 accumulator itself: y is float [n, c_out] */
    SMC_FWD_MASK_TILES = 4, /* output-stationary mask-tile algorithm (see smc_conv_forward) */
    SMC_FWD_SLAB_IN_MEMORY = 8 /* pair lists: always the two-kernel form with the slab in device
                                  memory, also where the row-range kernel would run */
};

typedef struct smc_map_info_s {
    int64_t n;              /* active voxels (rows) */
    int32_t route;          /* SMC_ROUTE_DENSE or SMC_ROUTE_SORTED */
    int32_t key_bits;       /* sorted route: bits of the packed coordinate key; dense: 0 */
    int32_t origin[3];      /* grid origin (x, y, z) the coordinates are taken relative to */
    int32_t extent[3];      /* grid extent (X, Y, Z) */
    int32_t batch;          /* number of batches B */
    int32_t tile_m;         /* pairs per GEMM tile */
    int64_t grid_cells;     /* dense route: cells of the padded presence grid (in whole
                               8 x 8 x 16 bricks when Z + 2 r >= 256); sorted: 0 */
    int64_t pairs;          /* P: valid (input, output) pairs including the centre tap */
    int64_t pairs_padded;   /* sum over taps of tap_count rounded up to tile_m (0 without pairs) */
    int64_t n_tiles;        /* pairs_padded / tile_m: GEMM tiles of all taps (0 without pairs) */
    int64_t tap_count[125]; /* pairs per tap (the first `taps` entries) */
    int32_t status;         /* smc_status of the build's device-side checks */
    int32_t n_groups;       /* offset groups of the mask-tile row orders (0: map not sorted) */
    int64_t group_rows[4];  /* rows with a tap of each group (the last group: every row) */
    int32_t kernel_size;    /* K: 3 or 5 */
    int32_t taps;           /* K^3: 27 or 125 */
    int64_t n_in;           /* input rows (= n except for a strided map) */
    int32_t strided;        /* 1 for a map from smc_map_build_strided */
    int32_t out_extent[3];  /* output grid extent (strided: floor((X + 2 - 3) / 2) + 1) */
} smc_map_info_t;

/*
 * Device allocator for every buffer a map handle takes from now on, for the
 * whole process: alloc(ctx, bytes, stream) returns a device pointer on the
 * current device, aligned to 256 bytes, usable on `stream` (the hipStream_t of
 * the call that needs it, as void*; NULL: the null stream), or NULL on failure
 * (the call then returns SMC_ERR_ALLOC; a pointer not aligned to 256 bytes is
 * given back and the call returns SMC_ERR_ALLOC too); free(ctx, ptr, stream)
 * gives it back. A caller with
 * its own pool (e.g. torch's caching allocator, bound from Python) keeps all
 * device memory in that pool this way. Both NULL restores hipMalloc/hipFree.
 * A buffer is always freed by the allocator that made it, even after the
 * allocator changed. The functions are called from the library's calls
 * (build, forward, destroy) on the calling thread, never from a GPU
 * callback; they must not call back into the library. Returns SMC_ERR_ARG
 * when only one of the two is NULL.
 */
typedef void* (*smc_alloc_fn)(void* ctx, size_t bytes, void* stream);
typedef void (*smc_free_fn)(void* ctx, void* ptr, void* stream);
int smc_set_allocator(smc_alloc_fn alloc, smc_free_fn free_fn, void* ctx);

/* Create an empty map handle. *out receives it. No device memory is taken yet. */
int smc_map_create(smc_map** out);

/* Free the handle and every device buffer it owns. Waits for the handle's
 * outstanding work first. NULL is accepted and ignored. */
int smc_map_destroy(smc_map* map);

/*
 * Build the kernel map of a voxel set: neighbour table, 27-bit neighbour
 * masks, mask-sorted row order (unless SMC_BUILD_NO_SORT) and per-tap pair
 * lists (unless SMC_BUILD_NO_PAIRS).
 *
 * Steps (all on the GPU): bounding box -> route by grid volume ("[Kernel]
 * Add submanifold sparse 3D convolution", section "Design, and the measurements behind it",
 * the mapper table) ->
 *   dense route:  presence grid scatter, 27 lookups per row;
 *   sorted route: packed keys with packed(q + d) = packed(q) + packed(d),
 *                 radix sort, 9 binary searches per row (the Z-Delta mapper, same section);
 * -> neighbour table + masks ("Sparse convolution in FP32", "Neighbour masks
 * and sorted rows") -> radix sort of rows by mask -> per-tap counts, scan
 * and pair write, ascending output row within a tap ("[Kernel] ...", same
 * section; commits 6ee20cd and f9cb4f1), which also numbers
 * every row's off-centre pairs for the pair-list forward.
 *
 * coords        device pointer, int32 [n, ncols], row-major. ncols = 4: rows
 *               (b, x, y, z); ncols = 3: rows (x, y, z) with b = 0.
 * n             rows, n >= 0 (n = 0 builds an empty map).
 * spatial_shape host pointer to int32 [3] (X, Y, Z), or NULL. Given: every
 *               coordinate must satisfy 0 <= c < shape (else SMC_ERR_RANGE) and the
 *               grid is [0, shape). NULL: the grid is the coordinates' bounding
 *               box, which costs one device->host read inside this call.
 * batch_size    number of batches B (b in [0, B)); <= 0 derives it (one read).
 * kernel_size   3 or 5 (else SMC_ERR_UNSUPPORTED): 27 or 125 taps, tap
 *               k = K^2 (dx+r) + K (dy+r) + (dz+r) for offsets -r..r, r = (K-1)/2
 *               ("[Kernel] Add submanifold sparse 3D convolution", "Test plan":
 *               kernel sizes 3 and 5). A 5x5x5 map always has pair lists
 *               (SMC_BUILD_NO_PAIRS is refused) and never a mask order (the
 *               mask-tile algorithm is 3x3x3 only; SMC_BUILD_NO_SORT is implied).
 * route         SMC_ROUTE_*.
 * flags         SMC_BUILD_* bits or 0. Without SMC_BUILD_ASYNC the call waits for the
 *               device-side checks and returns SMC_ERR_DUPLICATE / SMC_ERR_RANGE
 *               when they fail. With it the call returns after enqueueing, and
 *               does not wait for an earlier asynchronous build either: the
 *               checks of every build since the last wait are reported by the
 *               next smc_map_sync(), synchronous build, smc_map_info or export
 *               (a build that fails on the host before enqueueing, or an empty
 *               one, discards the earlier map with its unread checks). A map
 *               whose checks failed is in-bounds but meaningless and is refused
 *               by smc_conv_forward once the failure has been read.
 * The dense route keeps its presence grid (4 bytes per padded cell) in the
 * handle between builds and leaves it cleared, so only the first build on
 * a handle pays for filling it.
 * A build without the neighbour table in memory (see SMC_BUILD_TABLE) still
 * exports it: smc_map_export fills it on the host from the pair lists, which
 * hold every (input row, output row, tap) of the map.
 */
int smc_map_build(smc_map* map, const int32_t* coords, int64_t n, int ncols,
                  const int32_t* spatial_shape, int batch_size, int kernel_size,
                  int route, unsigned flags, void* stream);

/*
 * Strided (downsampling) map: kernel 3, stride 2, padding 1 ("Sparse
 * convolution in FP32" (DriveRT), section "Calibrated bit order": the
 * strided layers change the coordinate set and run as mask-sorted tiles).
 * Output cell o (per batch) exists when an input c = 2 o - 1 + d, d in
 * [0, 3)^3, is active; its 27 taps are the cells 2 o + d' (d' in [-1, 1]^3,
 * the submanifold tap numbering), so nbr[o][k] is the input row at
 * 2 o + d_k or -1. Output rows are ordered by (b, x, y, z); their
 * coordinates come from smc_map_export_out_coords. Unless SMC_BUILD_NO_PAIRS,
 * the map carries per-tap pair lists over its output rows in which the
 * centre tap (the input at 2 o, present or not) is a tap like the others;
 * unless SMC_BUILD_NO_SORT, the plain mask order of its output rows.
 * smc_conv_forward (x: n_in input rows, y: n output rows) then runs the
 * pair lists (every tap's products to the slab, each output row the sum of
 * its slab rows in order) or, with SMC_FWD_MASK_TILES or without pair lists,
 * the mask-tile algorithm.
 * Arguments as smc_map_build; coordinates count from 0: with spatial_shape
 * NULL the grid is [0, max + 1) per axis, and a negative coordinate is
 * SMC_ERR_RANGE. kernel_size must be 3 and stride 2 (else
 * SMC_ERR_UNSUPPORTED); n <= 2^24. The output count n (the caller needs it to
 * size y) reaches the host once: with the mask order (no SMC_BUILD_NO_SORT)
 * it is read back inside the call; a pair-list build without it (and with
 * 8 n_in <= 2^23) sizes the lookup and the compaction by the bound 8 n_in,
 * which read the count on the device, and the count is read on first use
 * (smc_map_rows, smc_map_info, the forward), so the call waits for nothing. With SMC_BUILD_ASYNC the
 * kernels after the count are only enqueued in either case.
 * Steps: the input grid or sorted input keys as for smc_map_build; the output
 * cells, through a bitmap of the output grid (count per block, scan, write
 * in (b, x, y, z) order) or, above 2^30 output cells, by sorting every
 * input's (at most 8) candidate output keys and keeping the distinct ones;
 * the 27-tap lookup around each query point; the pair lists and/or the mask
 * sort.
 */
int smc_map_build_strided(smc_map* map, const int32_t* coords, int64_t n, int ncols,
                          const int32_t* spatial_shape, int batch_size, int kernel_size,
                          int stride, int route, unsigned flags, void* stream);

/* Output coordinates of a strided map: host int32 [n, 4] rows (b, x, y, z) in
 * output-grid cells, in output-row order. SMC_ERR_STATE for other maps. */
int smc_map_export_out_coords(smc_map* map, int32_t* out_coords);

/* Wait for the map's last build and return the status of its device-side
 * checks (SMC_OK, SMC_ERR_DUPLICATE, SMC_ERR_RANGE). */
int smc_map_sync(smc_map* map);

/* Wait for the last build and describe the map. info: host pointer. */
int smc_map_info(smc_map* map, smc_map_info_t* info);

/* Output and input rows of the last build (host pointers, either may be
 * NULL), without waiting for the build: the only wait is, after a strided
 * pair-list build, for its output count (an event right after the output
 * cells; the lookup and compaction go on behind it). For callers that size y
 * right after an asynchronous build. */
int smc_map_rows(smc_map* map, int64_t* n, int64_t* n_in);

/*
 * Copy the map to host memory for inspection (parity tests). Each pointer is
 * a host pointer or NULL (skipped):
 *   nbr      int32 [n, taps]  row of c_i + d_k, or -1
 *   mask     uint32 [n] (K = 3) or [n, 4] (K = 5: bit k in word k / 32)
 *                           bit k set iff nbr[i, k] >= 0
 *   perm     int32 [G, n]   G = info.n_groups row orders (needs a sorted map). With
 *                           the plain order (G = 1): rows by ascending (mask, row).
 *                           Otherwise group g lists its group_rows[g] rows that have
 *                           a tap of the group, by (mask restricted to the group,
 *                           bits in the set order, row), then the other rows by row.
 *   pair_in  int32 [pairs]  tap-major, ascending output row within a tap
 *   pair_out int32 [pairs]
 *   tap_off  int64 [taps+1] pairs of tap k are [tap_off[k], tap_off[k+1])
 * Waits for the device. SMC_ERR_STATE if perm is asked of a map built with
 * SMC_BUILD_NO_SORT, or pair_in / pair_out of one built with SMC_BUILD_NO_PAIRS.
 */
int smc_map_export(smc_map* map, int32_t* nbr, uint32_t* mask, int32_t* perm,
                   int32_t* pair_in, int32_t* pair_out, int64_t* tap_off);

/*
 * Bit order and offset groups of the mask sort of later builds ("Sparse
 * convolution in FP32" (DriveRT), sections "Calibrated bit order" and
 * "Offset-group partitioning"). The order a tile meets its rows in decides
 * how many taps its union holds: rows are sorted by their mask with the
 * bits in the order given, and with several groups every group has its own
 * row order under the mask restricted to the group's taps, and
 * SMC_FWD_MASK_TILES runs one pass per group.
 * bit_order  host int32 [27]: the taps from most to least significant, or
 *            NULL for 26, 25, ..., 0 (the plain mask value).
 * group_of   host int32 [27]: group 0..G-1 of each tap (G <= 4, no empty
 *            group, the centre tap 13 in group G-1 so that the last pass
 *            holds every row), or NULL for one group.
 * Takes effect at the next smc_map_build (a built map keeps its order).
 * SMC_ERR_ARG on an invalid order or grouping; the previous one then stays.
 */
int smc_map_set_order(smc_map* map, const int32_t* bit_order, const int32_t* group_of);

/*
 * Choose a bit order and n_groups offset groups (1..4) on a built map, as
 * the calibration frame of the section "Calibrated bit order". The pages do
 * not say how; here a greedy search minimises the tap-rows that 64-row mask
 * tiles of the one-group order execute: from the off-centre taps by
 * ascending count (ties: lower tap), each position from the most
 * significant down takes the remaining tap with the least work (ties: the
 * earlier one), the others following in their current order; the centre
 * tap is always last. The off-centre taps, in that order, are then cut into
 * n_groups runs (run g: positions floor(26 g / G) .. floor(26 (g+1) / G) - 1)
 * and the centre joins the last. Host-side planning: it reads the masks
 * back once and runs 351 sorts of n keys on the CPU (about a second at
 * n = 100k); it is meant to run once per workload, not per layer.
 * bit_order, group_of: host int32 [27] outputs, ready for smc_map_set_order.
 */
int smc_map_calibrate(smc_map* map, int n_groups, int32_t* bit_order, int32_t* group_of);

/* Bytes of the packed weight buffer for a K x K x K kernel (K = 3 or 5) and
 * c_in x c_out (both >= 1); 0 for an invalid request. Where the one-kernel
 * pair-list forward runs (K = 3, c_in and c_out <= 64, c_in a multiple of 8) the buffer
 * also holds that kernel's column tiles, packed after the others; for c_in <= 128
 * and c_out > 64, the off-centre GEMM's 64-column tiles likewise. */
size_t smc_weight_packed_bytes(int kernel_size, int c_in, int c_out);

/*
 * Pack weights for the GEMM ("[Kernel] Add submanifold sparse 3D
 * convolution", section "Design, and the measurements behind it": weights
 * packed so that a wave reads fully used cache lines). w: device pointer, bf16
 * [K^3, c_in, c_out] row-major (W[k][ci][co]). out: device pointer of
 * smc_weight_packed_bytes(K, c_in, c_out) bytes, 16-byte aligned. Channels are
 * zero-padded internally, so any c >= 1 works. Pack once per weight tensor and
 * reuse the result for every forward; the forward takes weights packed for
 * the map's kernel size (the caller's duty: a raw pointer carries no size).
 */
int smc_weight_pack(const uint16_t* w, int kernel_size, int c_in, int c_out, void* out,
                    void* stream);

/*
 * One submanifold convolution layer over a built map. Two algorithms:
 *  - default, per-tap pair lists ("[Kernel] Add submanifold sparse 3D
 *    convolution", section "Design, and the measurements behind it" and
 *    commit d4161ef: gather -> mfma_f32_16x16x32_bf16 with float32
 *    accumulate -> scatter): each non-centre pair's float32 product row goes
 *    to a partial-product slab (one row per pair, a row's pairs
 *    consecutive), the centre tap (every row with itself) runs as a dense
 *    GEMM, and each output row is its centre product plus its slab rows in
 *    order. On a 3 x 3 x 3 map with c_in, c_out <= 64 (c_in a multiple of 8), one
 *    kernel does all of it over 256-row chunks with the chunk's slab rows in
 *    LDS; otherwise (or with SMC_FWD_SLAB_IN_MEMORY) two kernels pass the
 *    slab through device memory. Both forms give the same bits. Needs a map
 *    built without SMC_BUILD_NO_PAIRS;
 *  - SMC_FWD_MASK_TILES ("Sparse convolution in FP32", "Neighbour masks and
 *    sorted rows"): tiles of mask-sorted rows run the union of their masks'
 *    taps and keep every tap's sum in registers; with one offset group, one
 *    kernel and nothing in memory but the output. With G groups
 *    (smc_map_set_order), one pass per group over that group's rows; the
 *    first G-1 leave float32 partial sums in the handle (4 n c_out bytes,
 *    grow-only) and the last, which holds every row, adds them and writes y
 *    ("Offset-group partitioning"). Needs a map built without
 *    SMC_BUILD_NO_SORT.
 * Neither uses atomics: the output is the same on every run.
 * x       device pointer, bf16 [n, c_in] row-major (rows in coordinate order).
 * wpacked device pointer from smc_weight_pack(map kernel size, c_in, c_out).
 * y       device pointer, 16-byte aligned, bf16 [n, c_out] (float [n, c_out] with
 *         SMC_FWD_OUT_F32); every row is written.
 * flags   SMC_FWD_RELU | SMC_FWD_OUT_F32 | SMC_FWD_SLAB_IN_MEMORY, or 0. Without
 *         SMC_FWD_OUT_F32 the output is the float32 accumulator rounded to bf16
 *         (to nearest, ties to even).
 * The two-kernel form's slab lives in the handle (grow-only, 4 c_out bytes
 * per off-centre pair). The host reads no pair count: the GEMM reads them on
 * the device, and the slab is sized for 26 pairs per row when the build's
 * counts have not been read (asynchronous builds) and that bound is under
 * 4 GiB; otherwise the call waits for the build and sizes it exactly.
 * Refuses (SMC_ERR_STATE) a map whose synchronous build failed or a map
 * that was never built.
 */
int smc_conv_forward(smc_map* map, const uint16_t* x, int c_in, const void* wpacked,
                     int c_out, void* y, unsigned flags, void* stream);

/*
 * smc_conv_forward without any allocation, for callers that cannot allocate
 * device memory during the call: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc. Same arguments, flags, algorithms,
 * kernels and results as smc_conv_forward on the same map. The pair-list
 * slab (4 c_out bytes per off-centre pair), or the float32 partial sums of a
 * grouped mask-tile forward (4 n c_out bytes), lives in a fixed device array
 * of 32 MiB that the library holds on every GPU it runs on until the process
 * ends (its address is looked up when a map is first built on that GPU);
 * larger needs return SMC_ERR_UNSUPPORTED before any work is enqueued. When
 * the map's build has not been waited for and 26 pairs per row could exceed
 * the array, the call waits for the build's counts first (one host read).
 * The array is shared by every call on that GPU and keeps the last call's
 * contents; nothing in it needs to start at zero. Calls that overlap on one
 * GPU (other streams, other threads, other handles) race on it: the caller
 * must order them. Stage timers do not run in this call. SMC_ERR_HIP if the
 * array's device address could not be looked up on the map's GPU.
 */
int smc_conv_forward_noalloc(smc_map* map, const uint16_t* x, int c_in, const void* wpacked,
                             int c_out, void* y, unsigned flags, void* stream);

/* Stage timers. Stages of a build and of a forward, for measurement. */
enum {
    SMC_STAGE_MAP = 0,         /* the whole smc_map_build enqueue (all steps below it) */
    SMC_STAGE_NEIGHBOURS = 1,  /* route-specific neighbour search: table + masks */
    SMC_STAGE_MASK_SORT = 2,   /* radix sort of rows by mask */
    SMC_STAGE_COMPACT = 3,     /* pair count, scan and write */
    SMC_STAGE_GEMM = 4,        /* pair lists: GEMM of every tap but the centre; mask tiles: all */
    SMC_STAGE_CENTRE = 5,      /* pair lists: centre-tap GEMM fused with the slab sum and output */
    SMC_STAGE_COUNT = 6
};

/*
 * Turn per-stage timing on or off for one handle. While on, every kernel the
 * handle launches carries one stop event, stamped by the kernel's own
 * dispatch (hipExtLaunchKernel) when it ends, and a kernel's time is the
 * interval from the previous timed kernel's stop (or from a start marker
 * before the first kernel after timing was turned on) to its own: on a stream
 * that the GPU runs back to back, the kernel's duration plus the dispatch gap
 * before it, so the stage times of a sequence add up to its elapsed time. All
 * timed work of a handle must go to one stream. A stage's time is the sum of
 * its kernels'; SMC_STAGE_MAP is the sum over every kernel of the build. Off
 * by default.
 */
int smc_timing_enable(smc_map* map, int on);

/*
 * Wait for the timed work and add up its stage times. ms and calls are host
 * arrays of SMC_STAGE_COUNT entries (either may be NULL): milliseconds of GPU
 * time and number of timed executions per stage since the last reset.
 * reset != 0 clears the totals after reading.
 */
int smc_timing_read(smc_map* map, double* ms, int64_t* calls, int reset);

/*
 * Attainable-peak probes (measurement only; they compute nothing of the
 * convolution). The spec peaks used as roofline denominators are 2.5 PFLOP/s
 * dense bf16 MFMA and 8 TB/s HBM; these give what the part reaches here.
 *
 * smc_probe_mfma_bf16: enqueues one kernel of 8 waves per compute unit (2 per SIMD),
 * each running iters rounds of 8 independent v_mfma_f32_16x16x32_bf16 on
 * register operands (iters rounded up to a multiple of 16). out is a device buffer of out_bytes bytes, at least
 * smc_probe_mfma_out_bytes(compute units of the current device) (one float
 * per thread is written). *flops (host, may be NULL) receives the flops the
 * kernel executes. The caller times it on the stream. SMC_ERR_ARG for
 * iters < 1, out NULL or out_bytes too small.
 *
 * smc_probe_copy: dst[0, bytes) = src[0, bytes) by a grid-stride kernel of
 * 16-byte loads and stores; device pointers, 16-byte aligned, bytes a
 * multiple of 16, the ranges must not overlap (SMC_ERR_ARG otherwise).
 */
size_t smc_probe_mfma_out_bytes(int n_cu);
int smc_probe_mfma_bf16(int64_t iters, float* out, size_t out_bytes, double* flops,
                        void* stream);
int smc_probe_copy(void* dst, const void* src, size_t bytes, void* stream);

/*
 * Test hook for the error path of the device-side waits. While on, the
 * dense-route 3x3x3 compaction of this handle's builds waits for a look-back
 * epoch that no block publishes, with a limit of 64 polls per thread instead
 * of 2^22, so every wait runs out almost at once: the kernel still ends
 * normally, its results are invalid (in bounds), and the build reports
 * SMC_ERR_HIP ("a look-back wait ... ran out") like a real timeout. on = 0
 * restores normal builds. For tests only; no result of a build made with it
 * on is meaningful.
 */
int smc_test_force_lookback_timeout(smc_map* map, int on);

/* Static text for a status code. */
const char* smc_status_string(int status);

/* Message for the calling thread's last failing call ("" if none). */
const char* smc_last_error(void);

/* Library version, major*10000 + minor*100 + patch. */
int smc_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SMCONV_H */
