// Internal declarations shared by the library's HIP sources (not installed).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace smc {

constexpr int kTaps = 27;           // 3 x 3 x 3 kernel (the mask-tile path, the fused lookup)
constexpr int kCentre = 13;
constexpr int kMaxTaps = 125;       // 5 x 5 x 5 kernel
constexpr int kMaxMaskWords = 4;    // 32-bit words of a 125-bit mask
constexpr int kTileM = 64;          // granularity of the per-tap pair counts reported as padded
constexpr int kCapAlign = 256;      // each tap's run of the pair arrays: n rounded up to this
                                    // (a multiple of every GEMM tile height)
constexpr int kBlock = 256;         // threads per block for the map kernels
constexpr int kMaxSplit = 1024;     // splitter table entries of the sorted route's searches

// Per-kernel timing. While a stage timer of the API is active, take() hands
// out a stop event for every kernel launched, and the launch carries it
// (hipExtLaunchKernel: the event is stamped by the kernel's own dispatch when
// the kernel ends).
struct KernelTimer {
    void* ctx = nullptr;
    bool (*take)(void* ctx, hipEvent_t* stop) = nullptr;
};
extern thread_local KernelTimer g_ktimer;

// Every kernel of the library is launched through here.
template <typename... P, typename... A>
inline void launch(void (*kern)(P...), dim3 grid, dim3 block, size_t lds, hipStream_t s,
                   A... args) {
    static_assert(sizeof...(P) == sizeof...(A), "argument count");
    hipEvent_t b = nullptr;
    if (g_ktimer.take && !g_ktimer.take(g_ktimer.ctx, &b)) b = nullptr;
    hipExtLaunchKernelGGL(kern, grid, block, (uint32_t)lds, s, nullptr, b, 0u,
                          static_cast<P>(args)...);
}

// bits of the device status word
enum : uint32_t { kStDuplicate = 1u, kStRange = 2u, kStSortStall = 4u };

// Small device-side record written by the map kernels and read back once.
struct MapState {
    uint32_t status;        // kSt* bits
    int32_t bbox[8];        // min x, y, z, max x, y, z, min b, max b
    int32_t totals[4];      // pairs, pairs padded per tap to the tile, tiles, slab rows
    int32_t tap_off[kMaxTaps + 1];  // start of each tap's pair run (k cap; tap_off[taps] = taps cap)
    int32_t tap_count[kMaxTaps];    // pairs per tap (written by the compaction)
    int32_t tap_tot[kTaps];         // pairs per tap, accumulated by the mask histogram (K = 3)
    int32_t group_rows[4];  // rows with a tap in each offset group (mask-tile row orders)
    int32_t n_out;          // strided map: output rows
};

constexpr int kMaxGroups = 4;

// Significance order of the mask bits and offset groups of the mask-tile row
// orders. Tap t is bit pos[t] of group grp[t]'s key; group g of a row has key
// = its group-g taps placed at those bits. plain: one group, pos[t] = t (the
// key is the mask itself).
struct MaskOrder {
    int32_t n_groups = 1;
    int32_t group_bits = 27;  // bits of a group key: the largest group's tap count
    int32_t plain = 1;
    uint8_t pos[27];
    uint8_t grp[27];
};

// Digit plan of a radix sort: passes x bits (bits in 8..11).
struct SortPlan {
    int passes = 1;
    int bits = 8;
};

// Look-back table and ticket counter shared by the single-pass kernels of
// one map (sort passes, compaction), plus the host-side epoch counter.
struct SortWork {
    uint64_t* look = nullptr;
    uint32_t* ticket = nullptr;
    uint32_t epoch = 0;
    // many-tile sorts (reduce, then scan): per-(digit, tile) counts and the
    // scan's per-segment sums, sized by sort_scan_ints(n) (nullptr: onesweep only)
    uint32_t* cnt = nullptr;
    int64_t cnt_ints = 0;
    // test hook (smc_test_force_lookback_timeout): the dense route's fused
    // compaction waits for an epoch no block publishes, 64 spins at most
    bool force_timeout = false;
};

constexpr int kMaskBits = 27;
constexpr int kHistMaskInts = 3 * 1024;       // mask sort: up to 3 passes x 10 bits
constexpr int kHistKeyInts = 6 * 2048;        // key sort: up to 6 passes x 11 bits
constexpr int kHistInts = kHistMaskInts + kHistKeyInts;

// Where voxels live. Coordinates are taken relative to origin; a voxel is in
// range when 0 <= rel < ext and 0 <= b < batch.
struct Geom {
    int32_t origin[3];
    int32_t ext[3];
    int32_t batch;
    int32_t ncols;
    int32_t ksize;          // kernel size K (3 or 5)
    int32_t pad;            // r = (K - 1) / 2: padding cells per side (grid) / key offset
    // strides of the grid padded by r cells on every side (the sorted route's
    // keys are its linear cell indices)
    int64_t sz_y;           // (Z + 2r)
    int64_t sz_x;           // (Y + 2r) (Z + 2r)
    int64_t sz_b;           // (X + 2r) (Y + 2r) (Z + 2r)
    // the dense route's bricks (brick_cell), when brick is set: strides in bricks
    int64_t bs_y;           // ceil((Z + 2r) / 16)
    int64_t bs_x;           // ceil((Y + 2r) / 8) bs_y
    int64_t bs_b;           // ceil((X + 2r) / 8) bs_x
    int32_t brick;          // dense route: 1 = bricked cells, 0 = linear (sz_*)
};

// Dense-route layouts. Linear: cell b sz_b + xp sz_x + yp sz_y + zp of the
// padded grid. Bricked (for tall grids, Z + 2r >= kBrickMinZ): bricks of
// 8 x 8 x 16 (x, y, z) cells in (b, x, y, z) order, the cells of a brick in
// (x, y, z) order. A brick's occupancy bits fill one 128-byte line (each
// (x, y) column's 16 bits a half word) and its row ids one 4 KiB page, so a
// row's 3 x 3 x 3 neighbourhood mostly reads one line of bits and one page of
// ids, where the linear order gives every (dx, dy) column a line of its own
// once Z + 2r is in the hundreds. On short grids the brick arithmetic costs
// more than it saves (measured, 1440 x 1440 x 41: fused lookup 20.6 -> 23.4 us;
// 2095 x 2095 x 695: 28.5 -> 23.6 us). Grid cells: bs_b x batch x 1024.
constexpr int kBrickMinZ = 256;
__host__ __device__ inline int64_t brick_cell(const Geom& g, int b, int64_t xp, int64_t yp,
                                              int64_t zp) {
    return ((b * g.bs_b + (xp >> 3) * g.bs_x + (yp >> 3) * g.bs_y + (zp >> 4)) << 10) |
           ((xp & 7) << 7) | ((yp & 7) << 4) | (zp & 15);
}

template <bool BRICK>
__device__ inline int64_t grid_cell(const Geom& g, int b, int64_t xp, int64_t yp, int64_t zp) {
    if (BRICK) return brick_cell(g, b, xp, yp, zp);
    return b * g.sz_b + xp * g.sz_x + yp * g.sz_y + zp;
}

// The record (and sort histograms) the next build will use: the first kernel
// of a build clears it, so no build needs a clearing launch of its own.
// st == nullptr: nothing to clear.
struct NextRecord {
    MapState* st = nullptr;
    uint32_t* hist = nullptr;
    int hist_ints = 0;
    uint32_t* sticky = nullptr;   // the record's status bits are ORed in here before it is cleared
};

// Cells of the previous dense build, to put back to empty in the other bitmap
// (occupancy bitmaps are double-buffered: a build sets bits in one while its
// first kernel clears the words the previous build set in the other one).
struct PrevCells {
    const int32_t* cells = nullptr;   // bitmap word of each row's cell in that build (-1: none)
    int64_t n = 0;
    uint32_t* bits = nullptr;         // occupancy bits of that build's grid
};

// Occupancy bits of the len (<= 5) cells (xp, yp, zp .. zp + len - 1) of the
// padded grid, all inside it (bit j = cell zp + j). Linear: a 64-bit window
// (the bit array has a word of slack past the last cell's). Bricked: the
// column's bits in its brick, and in the next brick along z when the run
// crosses into it.
template <bool BRICK>
__device__ inline uint32_t column_bits(const uint32_t* __restrict__ bits, const Geom& g, int b,
                                       int64_t xp, int64_t yp, int64_t zp, int len) {
    if (!BRICK) {
        const int64_t c0 = grid_cell<false>(g, b, xp, yp, zp);
        const uint64_t two = (uint64_t)bits[c0 >> 5] | ((uint64_t)bits[(c0 >> 5) + 1] << 32);
        return (uint32_t)(two >> (c0 & 31)) & ((1u << len) - 1u);
    }
    const int64_t c = brick_cell(g, b, xp, yp, zp);
    const int lo = (int)(zp & 15);
    uint32_t v = (bits[c >> 5] >> (c & 31)) & ((1u << (16 - lo)) - 1u);
    if (lo + len > 16) {
        const int64_t c2 = (c | 1023) + 1 + (c & 0x3F0);   // z = 0 of the next brick
        v |= ((bits[c2 >> 5] >> (c2 & 31)) & 0xFFFFu) << (16 - lo);
    }
    return v & ((1u << len) - 1u);
}

// ---- map kernels (map_kernels.hip) ----
// (sticky: as in NextRecord; nullptr for a record that holds no build yet)
hipError_t launch_state_init(MapState* st, uint32_t* hist, int hist_ints, uint32_t* sticky,
                             hipStream_t s);
hipError_t launch_bbox(const int32_t* coords, int64_t n, int ncols, MapState* st, hipStream_t s);
hipError_t launch_fill_i32(int32_t* p, int64_t n, int32_t v, hipStream_t s);
// Dense route: an int32 grid of row ids plus one occupancy bit per cell. A
// cell's row id is only read when its bit is set, so the int32 grid needs no
// initial fill and no reset; the bits of a build are cleared (whole words)
// by the next build that uses the other grid. bits has 2 words of padding.
// obits, sg (strided builds whose output cells go through a bitmap): each row
// also sets the bits of the output cells it feeds (stride_mark), in the same
// pass.
struct StrideGeom;
hipError_t launch_dense_scatter(const int32_t* coords, int64_t n, const Geom& g, int32_t* grid,
                                uint32_t* bits, int32_t* cells, MapState* st,
                                const NextRecord& next, const PrevCells& prev, hipStream_t s,
                                uint32_t* obits = nullptr, const StrideGeom* sg = nullptr);
hipError_t launch_clear_cells(const PrevCells& prev, hipStream_t s);
// nbr [n, K^3]; mask [n] (K = 3) or [n, 4] words (K = 5): g.ksize decides.
hipError_t launch_dense_lookup(const int32_t* coords, int64_t n, const Geom& g, const int32_t* grid,
                               const uint32_t* bits, int32_t* nbr, uint32_t* mask, hipStream_t s);
// Keys of the sorted route, and the digit histograms of every pass of `plan`
// added into hist (which must start at zero).
hipError_t launch_make_keys(const int32_t* coords, int64_t n, const Geom& g, bool wide, void* keys,
                            MapState* st, const NextRecord& next, const SortPlan& plan,
                            uint32_t* hist, hipStream_t s);
// split: the key sort's splitter table (keys i << split_shift), which every
// block reads into LDS for the top levels of its searches.
hipError_t launch_sorted_lookup(const void* keys, const uint32_t* vals, int64_t n, const Geom& g,
                                bool wide, const void* split, int split_shift, int32_t* nbr,
                                uint32_t* mask, MapState* st, hipStream_t s);
// Smallest shift with ceil(n / 2^shift) <= kMaxSplit.
inline int split_shift_for(int64_t n) {
    int sh = 0;
    while (((n + ((int64_t)1 << sh) - 1) >> sh) > kMaxSplit) ++sh;
    return sh;
}

// ---- strided maps (strided_kernels.hip) ----
// Output grid of a strided layer and the packing of its cells into 64-bit
// keys (b | x | y | z, z lowest); sentinel = 1 << (key bits), above every key.
struct StrideGeom {
    int32_t oext[3];
    int32_t wb, wx, wy, wz;
    int32_t stride, pad, ksize;
    int32_t origin[3];      // input coordinate of output cell 0's grid origin (0)
    uint64_t sentinel;
};
int64_t unique_blocks(int64_t n_c);

// Output cells along one axis fed by input coordinate v: o = (v + pad - d) / s
// for taps d with the division exact and o inside [0, oext).
__device__ inline int axis_cands(int v, int oext, const StrideGeom& sg, int& o0, int& o1) {
    int cnt = 0;
#pragma unroll
    for (int d = 0; d < 3; ++d) {
        const int t = v + sg.pad - d;
        const bool ok = t >= 0 && t % sg.stride == 0 && t / sg.stride < oext;
        if (ok) {
            if (cnt == 0) o0 = t / sg.stride;
            else o1 = t / sg.stride;
            ++cnt;
        }
    }
    return cnt;                                   // at most 2 for K = 3, stride 2
}

// Bit of output cell (b, x, y, z) in the output-grid bitmap ((b, x, y, z) order).
__device__ inline int64_t out_bit(const StrideGeom& sg, int b, int x, int y, int z) {
    return (((int64_t)b * sg.oext[0] + x) * sg.oext[1] + y) * sg.oext[2] + z;
}

// Set the bits of the (at most 8) output cells that input cell (b, x, y, z),
// relative to the grid origin and inside it, feeds. The z candidates are
// neighbours (z0 = z1 + 1): their bits go out together, one atomic per
// (x, y) unless they straddle a word.
__device__ inline void stride_mark(const StrideGeom& sg, int b, int x, int y, int z,
                                   uint32_t* __restrict__ obits) {
    int x0 = 0, x1 = 0, y0 = 0, y1 = 0, z0 = 0, z1 = 0;
    const int nx = axis_cands(x, sg.oext[0], sg, x0, x1);
    const int ny = axis_cands(y, sg.oext[1], sg, y0, y1);
    const int nz = axis_cands(z, sg.oext[2], sg, z0, z1);
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int e = 0; e < 2; ++e)
            if (a < nx && e < ny) {
                const int64_t L = out_bit(sg, b, a ? x1 : x0, e ? y1 : y0, nz == 2 ? z1 : z0);
                const int lo = (int)(L & 31);
                uint32_t bits = 1u << lo;
                if (nz == 2) {
                    if (lo != 31) bits |= 2u << lo;
                    else atomicOr(&obits[(L >> 5) + 1], 1u);
                }
                atomicOr(&obits[L >> 5], bits);
            }
}
// Output cells through a bitmap of the output grid (words of it, zero on entry
// and left zero): coords -> output coords [M, 4] and query points [M, 4] in
// (b, x, y, z) order, st->n_out = M; counts: out_bitmap_blocks(words) words of
// scratch; bitmaps of at most 2 n_cu chunks go through one look-back pass over
// ws.look (at least out_bitmap_blocks(words) entries).
constexpr int64_t kOutBitmapWords = (int64_t)1 << 25;   // 128 MiB: larger grids sort candidates
int64_t out_bitmap_words(const StrideGeom& sg, int batch);
int64_t out_bitmap_blocks(int64_t words);
// marked: the bits are set already (by the dense scatter of the same rows).
hipError_t launch_stride_bitmap(const int32_t* coords, int64_t n, const Geom& g,
                                const StrideGeom& sg, uint32_t* obits, int64_t words,
                                uint32_t* counts, int32_t* ocoords, int32_t* qcoords,
                                MapState* st, SortWork& ws, int n_cu, hipStream_t s,
                                bool marked = false);
// The next look-back epoch of ws (never 0), for a kernel that tags entries with it.
uint32_t take_epoch(SortWork& ws);
// coords [n, ncols] -> 8 candidate output keys per row (sentinels where fewer)
hipError_t launch_stride_candidates(const int32_t* coords, int64_t n, const Geom& g,
                                    const StrideGeom& sg, uint64_t* keys, MapState* st,
                                    hipStream_t s);
// sorted candidate keys -> output coords [M, 4], query points [M, 4] (input
// coordinates), st->n_out = M; counts: unique_blocks(n_c) words of scratch
hipError_t launch_unique(const uint64_t* keys, int64_t n_c, const StrideGeom& sg,
                         uint32_t* counts, int32_t* ocoords, int32_t* qcoords, MapState* st,
                         hipStream_t s);
// sorted keys with an equal neighbour: the duplicate-coordinate status bit
hipError_t launch_key_dups(const void* keys, bool wide, int64_t n, MapState* st, hipStream_t s);
// sorted route: the 27 taps around each query point from the sorted input keys
// m_dev (optional): a device row count read by the kernel; the rows are then
// min(m, *m_dev) (m the bound the grid was sized by).
hipError_t launch_query_lookup(const void* keys, const uint32_t* vals, int64_t n_in, const Geom& g,
                               bool wide, const int32_t* qcoords, int64_t m, int32_t* nbr,
                               uint32_t* mask, hipStream_t s, const int32_t* m_dev = nullptr);

// ---- radix sort (radix_sort.hip) ----
// Stable LSD sort of (key, value) pairs on the low passes*bits key bits, one
// kernel per pass. keys_in is only read; if vals_in is null the values are
// the input indices. hist holds the global digit counts of every pass
// ([passes][1 << bits], e.g. from launch_key_hist). *keys_out / *vals_out
// receive the scratch buffers that hold the result.
SortPlan sort_plan(int key_bits, int max_bits = 11);
SortPlan key_sort_plan(int key_bits, int64_t n);
int64_t sort_tiles(int64_t n);
size_t sort_look_bytes(int64_t n);
// u32 words a many-tile sort of n keys needs in SortWork::cnt (0: onesweep)
int64_t sort_scan_ints(int64_t n);
hipError_t launch_key_hist(const void* keys, bool wide, int64_t n, const SortPlan& plan,
                           uint32_t* hist, hipStream_t s);
hipError_t radix_sort_u32(const uint32_t* keys_in, const uint32_t* vals_in, int64_t n,
                          const SortPlan& plan, const uint32_t* hist, uint32_t* kbuf0,
                          uint32_t* kbuf1, uint32_t* vbuf0, uint32_t* vbuf1, SortWork& ws,
                          uint32_t* status, const uint32_t** keys_out, const uint32_t** vals_out,
                          hipStream_t s, void* split = nullptr, int split_shift = 0);
hipError_t radix_sort_u64(const uint64_t* keys_in, const uint32_t* vals_in, int64_t n,
                          const SortPlan& plan, const uint32_t* hist, uint64_t* kbuf0,
                          uint64_t* kbuf1, uint32_t* vbuf0, uint32_t* vbuf1, SortWork& ws,
                          uint32_t* status, const uint64_t** keys_out, const uint32_t** vals_out,
                          hipStream_t s, void* split = nullptr, int split_shift = 0);
// split (optional): the sort's last pass also writes split[i] = sorted key
// i << split_shift, for every i with i << split_shift < n (a splitter table
// for two-level searches of the sorted keys).


// ---- compaction (compact_kernels.hip) ----
// Digit histograms of the mask sort and pairs per tap, in one read of the
// masks. A plain order sorts the masks themselves (keys == nullptr). Otherwise
// every row gets one key per group, keys[g n + row] = (g << (B + 1)) | (the
// group key, or 1 << B if the row has no tap of the group), which one sort
// of G n items orders group by group (B = ord.group_bits); group_rows[g]
// counts the rows with a tap of group g.
int mask_sort_bits(const MaskOrder& ord);
hipError_t launch_mask_hist(const uint32_t* mask, int64_t n, const SortPlan& plan,
                            const MaskOrder& ord, uint32_t* keys, uint32_t* hist, int32_t* tap_tot,
                            int32_t* group_rows, hipStream_t s);
int64_t compact_chunks(int64_t n);
size_t compact_look_bytes(int64_t n);
size_t compact_look_bytes_k(int64_t n, int ksize);
// Pairs of tap k go to [k cap, k cap + tap_count[k]) in ascending output row;
// pair_slot numbers the off-centre pairs row by row (rowbase[i] = first slab
// row of output row i; rowbase[n] = all off-centre pairs). ksize 3 or 5
// (mask words and tap count follow it). For ksize 3, chunk_pre ([chunks + 1]
// x (kTaps + 1)) receives each 256-row chunk's starts: row c, column k < kTaps
// = pairs of tap k in chunks before c, column kTaps = slab rows before c (row
// c = chunks: the totals). ksize 5 leaves it alone.
// dense_centre false (3 x 3 x 3 only): the centre tap is a tap like the others
// (strided maps), with slab rows of its own and pair_in from the table.
hipError_t launch_compact(const uint32_t* mask, const int32_t* nbr, int64_t n, int ksize,
                          int64_t cap, int tile_m, MapState* st, int32_t* pair_in,
                          int32_t* pair_out, int32_t* pair_slot, int32_t* rowbase,
                          int32_t* chunk_pre, SortWork& ws, uint32_t* status, hipStream_t s,
                          bool dense_centre = true, const int32_t* n_dev = nullptr);
// Dense route: neighbour lookup and compaction in one kernel (also writes nbr
// and mask).
// sparse_centre: coords are a strided map's query points (the centre a tap
// like the others); n_dev: a device row count, n its bound (see launch_compact).
hipError_t launch_lookup_compact(const int32_t* coords, int64_t n, const Geom& g,
                                 const int32_t* grid, const uint32_t* bits, int32_t* nbr,
                                 uint32_t* mask, int64_t cap,
                                 int tile_m, MapState* st, int32_t* pair_in, int32_t* pair_out,
                                 int32_t* pair_slot, int32_t* rowbase, int32_t* chunk_pre,
                                 SortWork& ws, uint32_t* status, hipStream_t s,
                                 bool sparse_centre = false, const int32_t* n_dev = nullptr);

// ---- GEMM (gemm_kernels.hip) ----
// taps: 27 or 125 (the packed weights hold that many taps).
size_t packed_weight_bytes(int taps, int c_in, int c_out);
hipError_t launch_weight_pack(const uint16_t* w, int taps, int c_in, int c_out, void* out,
                              hipStream_t s);
// n: input rows (bounds the gathered rows). skip_centre: the centre tap runs
// as a dense GEMM of its own (k_gemm_centre); false for strided maps, whose
// centre tap is sparse like the others.
// y, out_f32, relu: the output of pairs marked as their row's only one
// (pair_slot -2 - row, strided maps), written here instead of a slab row.
hipError_t launch_gemm_nc(const uint16_t* x, int c_in, const void* wpacked, int c_out, int taps,
                          const int32_t* pair_in, const int32_t* pair_slot, const MapState* st,
                          int64_t cap, int64_t n, int n_cu, float* part, hipStream_t s,
                          bool skip_centre = true, void* y = nullptr, bool out_f32 = false,
                          bool relu = false);
// Output rows of a strided map: y[i] = the sum of slab rows rowbase[i] ..
// rowbase[i+1] - 1 in order (bf16 rounded or float, optional ReLU), m rows;
// rows without slab rows (one pair: written by the GEMM) are left alone.
hipError_t launch_slab_sum(const float* part, const int32_t* rowbase, int64_t m, int c_out,
                           void* y, bool out_f32, bool relu, int n_cu, hipStream_t s);
// rowbase: [n + 1], row i's slab rows are rowbase[i] .. rowbase[i+1] - 1.
hipError_t launch_gemm_centre(const uint16_t* x, int c_in, const void* wpacked, int c_out,
                              int taps, const int32_t* rowbase, int64_t n, const float* part,
                              void* y, bool out_f32, bool relu, int n_cu, hipStream_t s);
// Row-range GEMM (rows_kernels.hip): the whole pair-list layer in one kernel
// for 3 x 3 x 3 maps and c_in, c_out <= 64 (c_in a multiple of 8), the
// partial-product slab kept in LDS. Its weights are a second packing after the
// first (rows_weight_offset). Wider layers keep the two-kernel form: with a
// wave's resident weights for 96 or 128 input channels a block walks its
// chunks latency-bound (measured on the 91k-row set at 128 channels: 62 us
// against 29 us for the two kernels with 16 waves of 128 registers, 66 us
// with 8 waves of 256 and the next chunk's loads issued ahead; at 64
// channels 19 us against 23 us).
constexpr int kRowsMaxC = 64;
inline bool rows_eligible(int taps, int c_in, int c_out) {
    return taps == 27 && c_in <= kRowsMaxC && c_out <= kRowsMaxC && (c_in & 7) == 0;
}
size_t rows_weight_offset(int taps, int c_in, int c_out);   // 0: the first packing serves
size_t rows_weight_bytes(int taps, int c_in, int c_out);    // bytes of the second packing (or 0)
int rows_pack_nbw(int c_out);                               // its column blocks per tile
hipError_t launch_gemm_rows(const uint16_t* x, int c_in, const void* wpacked, int c_out,
                            const int32_t* pair_in, const int32_t* pair_slot,
                            const int32_t* chunk_pre, const int32_t* rowbase, const MapState* st,
                            int64_t cap, int64_t n, void* y, bool out_f32, bool relu, int n_cu,
                            hipStream_t s);

// ---- mask-tile GEMM (masktile_kernels.hip) ----
// One pass over the rows of one offset group: taps gm of the rows listed at
// perm (entries are item indices, row = entry - goff). rows: device count of
// listed rows, or nullptr for all n. Rows with a tap in prev (earlier groups)
// add their float32 partial sums; the last pass writes y, the others write
// the float32 partial sums.
struct GroupPass {
    uint32_t gm = 0x7FFFFFFu;
    uint32_t prev = 0;
    bool last = true;
    const uint32_t* perm = nullptr;
    int64_t goff = 0;
    const int32_t* rows = nullptr;
    float* partial = nullptr;
    bool centre_self = true;    // the centre tap reads the output row itself (submanifold);
                                // false: it is gathered through the table like every tap
    int64_t n_in = 0;           // input rows (0: the same as the n output rows)
};
hipError_t launch_conv_masktile(const uint16_t* x, int c_in, const void* wpacked, int c_out,
                                const int32_t* nbr, const uint32_t* mask, const GroupPass& gp,
                                int64_t n, const uint16_t* zrow, void* y, bool out_f32, bool relu,
                                hipStream_t s);

}  // namespace smc
