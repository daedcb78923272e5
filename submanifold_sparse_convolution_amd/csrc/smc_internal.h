// Internal declarations shared by the library's HIP sources (not installed).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace smc {

constexpr int kTaps = 27;
constexpr int kCentre = 13;
constexpr int kTileM = 64;          // pairs per GEMM tile (4 waves x 16 rows)
constexpr int kBlock = 256;         // threads per block for the map kernels
constexpr int kChunk = 256;         // sorted rows per compaction chunk

// bits of the device status word
enum : uint32_t { kStDuplicate = 1u, kStRange = 2u };

// Small device-side record written by the map kernels and read back once.
struct MapState {
    uint32_t status;        // kSt* bits
    int32_t bbox[8];        // min x, y, z, max x, y, z, min b, max b
    int32_t totals[4];      // pairs, pairs_padded, n_tiles, unused
    int32_t tap_off[28];    // padded start of each tap's pair run (tap_off[27] = pairs_padded)
    int32_t tap_count[27];  // unpadded pairs per tap
};

// Where voxels live. Coordinates are taken relative to origin; a voxel is in
// range when 0 <= rel < ext and 0 <= b < batch.
struct Geom {
    int32_t origin[3];
    int32_t ext[3];
    int32_t batch;
    int32_t ncols;
    // dense route: strides of the grid padded by one cell on every side
    int64_t sz_y;           // (Z + 2)
    int64_t sz_x;           // (Y + 2) (Z + 2)
    int64_t sz_b;           // (X + 2) (Y + 2) (Z + 2)
    // sorted route: bit widths of the packed key fields (z lowest)
    int32_t wz, wy, wx, wb;
};

// ---- map kernels (map_kernels.hip) ----
hipError_t launch_state_init(MapState* st, hipStream_t s);
hipError_t launch_bbox(const int32_t* coords, int64_t n, int ncols, MapState* st, hipStream_t s);
hipError_t launch_fill_i32(int32_t* p, int64_t n, int32_t v, hipStream_t s);
hipError_t launch_dense_scatter(const int32_t* coords, int64_t n, const Geom& g, int32_t* grid,
                                MapState* st, hipStream_t s);
hipError_t launch_dense_lookup(const int32_t* coords, int64_t n, const Geom& g, const int32_t* grid,
                               int32_t* nbr, uint32_t* mask, hipStream_t s);
hipError_t launch_dense_clear(const int32_t* coords, int64_t n, const Geom& g, int32_t* grid,
                              hipStream_t s);
hipError_t launch_make_keys(const int32_t* coords, int64_t n, const Geom& g, bool wide, void* keys,
                            MapState* st, hipStream_t s);
hipError_t launch_sorted_lookup(const void* keys, const uint32_t* vals, int64_t n, const Geom& g,
                                bool wide, int32_t* nbr, uint32_t* mask, MapState* st,
                                hipStream_t s);

// ---- radix sort (radix_sort.hip) ----
// Stable LSD sort of (key, value) pairs on the low key_bits bits of the keys.
// keys_in is only read. If vals_in is null the values are the input indices.
// Returns in *keys_out / *vals_out which scratch buffer holds the result.
size_t radix_counts_elems(int64_t n);
hipError_t radix_sort_u32(const uint32_t* keys_in, const uint32_t* vals_in, int64_t n, int key_bits,
                          uint32_t* kbuf0, uint32_t* kbuf1, uint32_t* vbuf0, uint32_t* vbuf1,
                          uint32_t* counts, const uint32_t** keys_out, const uint32_t** vals_out,
                          hipStream_t s);
hipError_t radix_sort_u64(const uint64_t* keys_in, const uint32_t* vals_in, int64_t n, int key_bits,
                          uint64_t* kbuf0, uint64_t* kbuf1, uint32_t* vbuf0, uint32_t* vbuf1,
                          uint32_t* counts, const uint64_t** keys_out, const uint32_t** vals_out,
                          hipStream_t s);

// ---- compaction (compact_kernels.hip) ----
hipError_t launch_pair_count(const uint32_t* perm, const uint32_t* mask, int64_t n,
                             int32_t* counts, hipStream_t s);
hipError_t launch_pair_scan(int32_t* counts, int64_t n, int tile_m, MapState* st,
                            int32_t* pair_in, int32_t* pair_out, int32_t* tile_tap,
                            hipStream_t s);
hipError_t launch_pair_write(const uint32_t* perm, const uint32_t* mask, const int32_t* nbr,
                             int64_t n, const int32_t* chunk_off, int32_t* pair_in,
                             int32_t* pair_out, hipStream_t s);

// ---- GEMM (gemm_kernels.hip) ----
size_t packed_weight_bytes(int c_in, int c_out);
hipError_t launch_weight_pack(const uint16_t* w, int c_in, int c_out, void* out, hipStream_t s);
hipError_t launch_fill_f32(float* p, int64_t n, hipStream_t s);
hipError_t launch_gemm(const uint16_t* x, int c_in, const void* wpacked, int c_out,
                       const int32_t* pair_in, const int32_t* pair_out, const int32_t* tile_tap,
                       const MapState* st, int64_t max_tiles, int n_cu, float* acc,
                       hipStream_t s);
hipError_t launch_finalize(float* acc, void* y, bool out_f32, int64_t count, bool relu,
                           hipStream_t s);

}  // namespace smc
