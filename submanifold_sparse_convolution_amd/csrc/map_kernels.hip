// Kernel-map construction: bounding box, the dense presence-grid route and
// the sorted packed-key route. Both routes emit the same neighbour table
// nbr[n][27] (row of c_i + d_k, or -1) and 27-bit masks (bit k set iff the
// neighbour exists), as described in "Sparse convolution in FP32" (DriveRT),
// "Neighbour masks and sorted rows". The two routes and their trade-off
// (O(volume) grid vs. one sort plus binary searches, flat in volume) follow
// "[Kernel] Add submanifold sparse 3D convolution (bf16 implicit GEMM,
// gfx950)", section "Design, and the measurements behind it", the mapper table.
#include "smc_internal.h"

#include <cstddef>

#include <climits>

namespace smc {
namespace {

__device__ inline bool load_rel(const int32_t* __restrict__ coords, int64_t i, const Geom& g,
                                int& b, int& x, int& y, int& z) {
    const int32_t* c = coords + i * g.ncols;
    if (g.ncols == 4) {
        b = c[0];
        c += 1;
    } else {
        b = 0;
    }
    x = c[0] - g.origin[0];
    y = c[1] - g.origin[1];
    z = c[2] - g.origin[2];
    return (unsigned)b < (unsigned)g.batch && (unsigned)x < (unsigned)g.ext[0] &&
           (unsigned)y < (unsigned)g.ext[1] && (unsigned)z < (unsigned)g.ext[2];
}

// linear cell of a voxel in the grid padded by r cells on every side: the
// sorted route's key
__device__ inline int64_t dense_cell(const Geom& g, int b, int x, int y, int z) {
    return b * g.sz_b + (int64_t)(x + g.pad) * g.sz_x + (int64_t)(y + g.pad) * g.sz_y + (z + g.pad);
}

// Puts a build record in its starting state (bounding box empty, everything
// else zero) and clears its sort histograms; grid-strided over all threads.
// The status bits the record holds (an earlier build's device checks, maybe
// never read by the host) are first ORed into *sticky, which the host reads
// and clears when it next waits for the handle's builds.
__device__ inline void clear_record(MapState* st, uint32_t* hist, int hist_ints, uint32_t* sticky) {
    const int64_t t0 = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
    const int64_t nt = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = t0; i < hist_ints; i += nt) hist[i] = 0;
    constexpr int kWords = (int)(sizeof(MapState) / 4);
    constexpr int kBox = (int)(offsetof(MapState, bbox) / 4);
    static_assert(offsetof(MapState, status) == 0, "status is word 0");
    uint32_t* wv = reinterpret_cast<uint32_t*>(st);
    if (t0 == 0 && sticky) {
        const uint32_t old = wv[0];
        if (old) atomicOr(sticky, old);
    }
    for (int64_t i = t0; i < kWords; i += nt) {
        const int b = (int)i - kBox;
        wv[i] = (b >= 0 && b < 8) ? (uint32_t)((b < 3 || b == 6) ? INT_MAX : INT_MIN) : 0u;
    }
}

__global__ __launch_bounds__(kBlock) void k_state_init(MapState* st, uint32_t* hist, int hist_ints,
                                                       uint32_t* sticky) {
    clear_record(st, hist, hist_ints, sticky);
}

__device__ inline int wave_min(int v) {
    for (int o = 32; o > 0; o >>= 1) v = min(v, __shfl_xor(v, o));
    return v;
}
__device__ inline int wave_max(int v) {
    for (int o = 32; o > 0; o >>= 1) v = max(v, __shfl_xor(v, o));
    return v;
}

__global__ __launch_bounds__(kBlock) void k_bbox(const int32_t* __restrict__ coords, int64_t n,
                                                 int ncols, MapState* st) {
    int lo[4] = {INT_MAX, INT_MAX, INT_MAX, INT_MAX};
    int hi[4] = {INT_MIN, INT_MIN, INT_MIN, INT_MIN};
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x) {
        const int32_t* c = coords + i * ncols;
        int b = ncols == 4 ? c[0] : 0;
        const int32_t* p = c + (ncols == 4 ? 1 : 0);
        for (int d = 0; d < 3; ++d) {
            lo[d] = min(lo[d], p[d]);
            hi[d] = max(hi[d], p[d]);
        }
        lo[3] = min(lo[3], b);
        hi[3] = max(hi[3], b);
    }
    __shared__ int s_lo[kBlock / 64][4], s_hi[kBlock / 64][4];
    const int w = threadIdx.x >> 6;
    for (int d = 0; d < 4; ++d) {
        lo[d] = wave_min(lo[d]);
        hi[d] = wave_max(hi[d]);
        if ((threadIdx.x & 63) == 0) {
            s_lo[w][d] = lo[d];
            s_hi[w][d] = hi[d];
        }
    }
    __syncthreads();
    if (threadIdx.x < 4) {
        const int d = threadIdx.x;
        int a = s_lo[0][d], b = s_hi[0][d];
        for (int v = 1; v < kBlock / 64; ++v) {
            a = min(a, s_lo[v][d]);
            b = max(b, s_hi[v][d]);
        }
        atomicMin(&st->bbox[d == 3 ? 6 : d], a);
        atomicMax(&st->bbox[d == 3 ? 7 : 3 + d], b);
    }
}

__global__ __launch_bounds__(kBlock) void k_fill_i32(int32_t* p, int64_t n, int32_t v) {
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x)
        p[i] = v;
}

// One thread per row: set the row's occupancy bit (its previous value
// flags a second row at the same coordinates), store the row id in the int32
// grid and record the cell's bitmap word in cells. Thread i first clears the
// bitmap word recorded for row i of the previous dense build (other bitmap),
// so the launch covers max(n, prev.n) threads. (Measured: a non-returning
// atomic here, with the duplicate check moved to the lookup's read of each
// row's own cell, was slower: LiDAR build + layer 35.3 -> 35.7 us.)
// obits (a strided build's output-cell bitmap): the row also marks the output
// cells it feeds.
__global__ __launch_bounds__(kBlock) void k_dense_scatter(const int32_t* __restrict__ coords,
                                                          int64_t n, Geom g,
                                                          int32_t* __restrict__ grid,
                                                          uint32_t* __restrict__ bits,
                                                          int32_t* __restrict__ cells,
                                                          MapState* st, NextRecord next,
                                                          PrevCells prev,
                                                          uint32_t* __restrict__ obits,
                                                          StrideGeom sg) {
    if (next.st) clear_record(next.st, next.hist, next.hist_ints, next.sticky);
    const int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
    if (i < prev.n) {
        const int32_t c = prev.cells[i];
        if (c >= 0) prev.bits[c] = 0u;
    }
    if (i >= n) return;
    int b, x, y, z;
    if (!load_rel(coords, i, g, b, x, y, z)) {
        atomicOr(&st->status, kStRange);
        cells[i] = -1;
        return;
    }
    const int64_t cell = g.brick ? grid_cell<true>(g, b, x + g.pad, y + g.pad, z + g.pad)
                                 : grid_cell<false>(g, b, x + g.pad, y + g.pad, z + g.pad);
    cells[i] = (int32_t)(cell >> 5);             // its bitmap word (grids below 2^36 cells)
    const uint32_t bit = 1u << (cell & 31);
    const uint32_t old = atomicOr(&bits[cell >> 5], bit);
    if (old & bit) atomicOr(&st->status, kStDuplicate);
    grid[cell] = (int32_t)i;
    if (obits) stride_mark(sg, b, x, y, z, obits);
}

// Only the cleanup part of k_dense_scatter (a build that writes no grid).
__global__ __launch_bounds__(kBlock) void k_clear_cells(PrevCells prev) {
    const int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
    if (i < prev.n) {
        const int32_t c = prev.cells[i];
        if (c >= 0) prev.bits[c] = 0u;
    }
}

// 16 lanes per row (9 active), lane c for the (dx, dy) column c = 3 (dx + 1) +
// (dy + 1). The column's occupancy bits of z - 1 .. z + 1 give its 3 taps
// 3c .. 3c + 2, and only occupied cells read the grid. The lane writes those 3
// neighbour entries (a row's 27 are contiguous); the row's mask is ORed
// together from the lanes' 3-bit patterns.
template <bool BRICK>
__global__ __launch_bounds__(kBlock) void k_dense_lookup(const int32_t* __restrict__ coords,
                                                         int64_t n, Geom g,
                                                         const int32_t* __restrict__ grid,
                                                         const uint32_t* __restrict__ bits,
                                                         int32_t* __restrict__ nbr,
                                                         uint32_t* __restrict__ mask) {
    constexpr int kCols = 9;
    const int64_t t = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
    const int64_t row = t >> 4;
    const int c = (int)(t & 15);
    uint32_t pat = 0;
    if (row < n && c < kCols) {
        int v[3] = {-1, -1, -1};
        int b, x, y, z;
        if (load_rel(coords, row, g, b, x, y, z)) {
            const int64_t xp = x + g.pad + c / 3 - 1, yp = y + g.pad + c % 3 - 1;
            const int64_t zp = z + g.pad - 1;
            pat = column_bits<BRICK>(bits, g, b, xp, yp, zp, 3);
#pragma unroll
            for (int j = 0; j < 3; ++j)
                if ((pat >> j) & 1u) v[j] = grid[grid_cell<BRICK>(g, b, xp, yp, zp + j)];
        }
        int32_t* dst = nbr + row * kTaps + 3 * c;
#pragma unroll
        for (int j = 0; j < 3; ++j) dst[j] = v[j];
    }
    uint32_t m = pat << (3 * (c < kCols ? c : 0));
#pragma unroll
    for (int o = 8; o > 0; o >>= 1) m |= __shfl_xor(m, o, 16);
    if (row < n && c == 0) mask[row] = m;
}

// 5 x 5 x 5 kernel: 32 lanes per row (25 active), lane c for the (dx, dy)
// column c = 5 (dx + 2) + (dy + 2). The column's occupancy bits of z - 2 ..
// z + 2 give its 5 taps 5c .. 5c + 4, and only occupied cells read the
// grid. The lane writes those 5 neighbour entries (a row's 125 are
// contiguous); the row's 4 mask words are ORed together from the lanes'
// 5-bit patterns.
template <bool BRICK>
__global__ __launch_bounds__(kBlock) void k_dense_lookup5(const int32_t* __restrict__ coords,
                                                          int64_t n, Geom g,
                                                          const int32_t* __restrict__ grid,
                                                          const uint32_t* __restrict__ bits,
                                                          int32_t* __restrict__ nbr,
                                                          uint32_t* __restrict__ mask) {
    constexpr int kT = 125, kCols = 25;
    const int64_t t = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
    const int64_t row = t >> 5;
    const int c = (int)(t & 31);
    uint32_t pat = 0;
    if (row < n && c < kCols) {
        int v[5] = {-1, -1, -1, -1, -1};
        int b, x, y, z;
        if (load_rel(coords, row, g, b, x, y, z)) {
            const int64_t xp = x + g.pad + c / 5 - 2, yp = y + g.pad + c % 5 - 2;
            const int64_t zp = z + g.pad - 2;
            pat = column_bits<BRICK>(bits, g, b, xp, yp, zp, 5);
#pragma unroll
            for (int j = 0; j < 5; ++j)
                if ((pat >> j) & 1u) v[j] = grid[grid_cell<BRICK>(g, b, xp, yp, zp + j)];
        }
        int32_t* dst = nbr + row * kT + 5 * c;
#pragma unroll
        for (int j = 0; j < 5; ++j) dst[j] = v[j];
    }
    // mask word q: the patterns' bits 5c + j that fall in [32 q, 32 q + 32)
    uint32_t w[kMaxMaskWords];
#pragma unroll
    for (int q = 0; q < kMaxMaskWords; ++q) {
        const int sh = 5 * c - 32 * q;
        w[q] = sh >= 32 || sh <= -5 ? 0u : sh >= 0 ? pat << sh : pat >> -sh;
#pragma unroll
        for (int o = 16; o > 0; o >>= 1) w[q] |= __shfl_xor(w[q], o, 32);
    }
    if (row < n && c < kMaxMaskWords)
        mask[row * kMaxMaskWords + c] = c == 0 ? w[0] : c == 1 ? w[1] : c == 2 ? w[2] : w[3];
}

// Key of a voxel: its cell in the grid padded by r cells on every side,
// b (X + 2r)(Y + 2r)(Z + 2r) + (x + r)(Y + 2r)(Z + 2r) + (y + r)(Z + 2r) + z + r,
// i.e. (b, x, y, z) packed with mixed radices instead of power-of-two bit
// fields: the same order, and since the padding keeps every neighbour inside
// its field, key(q + d) = key(q) + key offset of d (the packed(q + d) =
// packed(q) + packed(d) property of the Z-Delta mapper), in fewer bits.
// 8 keys per thread (2048 per block). The same pass also counts every sort
// pass's digits (block counts in LDS, then one global add per non-zero bin),
// so the sort needs no histogram read of its own. (Spatial keys spread over
// the bins, so the LDS atomics rarely collide.)
constexpr int kKeyItems = 8;
template <typename K>
__global__ __launch_bounds__(kBlock) void k_make_keys(const int32_t* __restrict__ coords,
                                                      int64_t n, Geom g, K* __restrict__ keys,
                                                      MapState* st, NextRecord next, int bits,
                                                      int passes, uint32_t* __restrict__ hist) {
    extern __shared__ uint32_t s_h[];             // passes << bits digit counters
    if (next.st) clear_record(next.st, next.hist, next.hist_ints, next.sticky);
    const int bins = 1 << bits;
    for (int i = threadIdx.x; i < passes * bins; i += kBlock) s_h[i] = 0;
    __syncthreads();
    const int64_t base = (int64_t)blockIdx.x * kBlock * kKeyItems;
    for (int it = 0; it < kKeyItems; ++it) {
        const int64_t i = base + it * kBlock + threadIdx.x;
        if (i >= n) break;
        int b, x, y, z;
        K key;
        if (load_rel(coords, i, g, b, x, y, z)) {
            key = (K)dense_cell(g, b, x, y, z);
        } else {
            atomicOr(&st->status, kStRange);
            key = ~(K)0;
        }
        keys[i] = key;
        for (int p = 0; p < passes; ++p)
            atomicAdd(&s_h[p * bins + ((uint32_t)(key >> (p * bits)) & (bins - 1))], 1u);
    }
    __syncthreads();
    for (int i = threadIdx.x; i < passes * bins; i += kBlock)
        if (s_h[i]) atomicAdd(&hist[i], s_h[i]);
}

template <typename K>
__device__ inline int64_t lower_bound(const K* __restrict__ keys, int64_t n, K t) {
    int64_t lo = 0, len = n;
    while (len > 0) {
        int64_t half = len >> 1;
        if (keys[lo + half] < t) {
            lo += half + 1;
            len -= half + 1;
        } else {
            len = half;
        }
    }
    return lo;
}

// lower_bound of t in the sorted keys, in two levels: first over the
// splitter table in LDS (s_split[i] = keys[i << sh], ns entries), then over
// the one run of 2^sh keys that can hold the answer (keys of run i - 1 are
// below t when splitter i - 1 is, and splitter i is not).
template <typename K>
__device__ inline int64_t lower_bound_split(const K* __restrict__ keys, int64_t n, K t,
                                            const K* s_split, int ns, int sh) {
    int lo = 0, len = ns;
    while (len > 0) {
        const int half = len >> 1;
        if (s_split[lo + half] < t) {
            lo += half + 1;
            len -= half + 1;
        } else {
            len = half;
        }
    }
    if (lo == 0) return 0;                        // keys[0] >= t
    const int64_t a = ((int64_t)(lo - 1) << sh) + 1;
    const int64_t b = lo < ns ? (int64_t)lo << sh : n;
    return a + lower_bound(keys + a, b - a, t);
}

// Lanes per sorted key: one per dx plane (3 for K = 3, 5 for K = 5), rounded
// up to a power of two. The K^2 taps of a plane (dy, dz in -r .. r) have keys
// in [lo, hi] = key(x + dx, y - r, z - r) .. key(x + dx, y + r, z + r), and
// so sit in one run of the sorted keys: one search for lo, then a walk
// forward to hi, each key's offset from lo giving its (dy, dz) (keys between
// the columns, other z of the same (x, y), are skipped). On sparse sets a
// run holds a few keys, so a row takes K searches instead of K^2. A run of
// more than kWalk keys (a dense slab) falls back to one search per (dx, dy)
// column and K compares.
template <typename K, int KS>
__global__ __launch_bounds__(kBlock) void k_sorted_lookup(const K* __restrict__ keys,
                                                          const uint32_t* __restrict__ vals,
                                                          int64_t n, Geom g,
                                                          const K* __restrict__ split, int sh,
                                                          int32_t* __restrict__ nbr,
                                                          uint32_t* __restrict__ mask,
                                                          MapState* st) {
    constexpr int R = (KS - 1) / 2, KV = KS * KS * KS, PL = KS * KS;
    constexpr int LANES = KS == 3 ? 4 : 8;
    constexpr int MW = (KV + 31) / 32;
    constexpr int kWalk = 4 * KS;
    __shared__ K s_split[kMaxSplit];
    const int ns = (int)((n + ((int64_t)1 << sh) - 1) >> sh);
    for (int i = threadIdx.x; i < ns; i += blockDim.x) s_split[i] = split[i];
    __syncthreads();
    const int64_t t = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
    const int64_t s = t / LANES;
    const int c = (int)(t % LANES);
    uint32_t bits[MW];
#pragma unroll
    for (int q = 0; q < MW; ++q) bits[q] = 0;
    if (s < n && c < KS) {
        const K q = keys[s];
        // vals is a permutation of [0, n); the clamps only matter if a sort wait stalled
        const int row = (int)min(vals[s], (uint32_t)(n - 1));
        const int dx = c - R;
        const K lo = q + (K)(dx * g.sz_x - R * g.sz_y - R);
        const K hi = q + (K)(dx * g.sz_x + R * g.sz_y + R);
        int32_t* out = nbr + (int64_t)row * KV + PL * c;    // the plane's K^2 entries
#pragma unroll
        for (int e = 0; e < PL; ++e) out[e] = -1;
        if (dx == 0 && s + 1 < n && keys[s + 1] == q) atomicOr(&st->status, kStDuplicate);
        int64_t j = lower_bound_split(keys, n, lo, s_split, ns, sh);
        int walked = 0;
        for (; j < n && walked < kWalk; ++j, ++walked) {
            const K kj = keys[j];
            if (kj > hi) break;
            const K off = kj - lo;                    // <= 2r (Z + 2r) + 2r
            int dy = 0;
#pragma unroll
            for (int i = 1; i < KS; ++i) dy += off >= (K)(i * g.sz_y) ? 1 : 0;
            const K dz = off - (K)(dy * g.sz_y);
            if (dz < (K)KS) {
                const int kk = PL * c + KS * dy + (int)dz;
                out[KS * dy + dz] = (int)min(vals[j], (uint32_t)(n - 1));
#pragma unroll
                for (int w = 0; w < MW; ++w) bits[w] |= (kk >> 5) == w ? 1u << (kk & 31) : 0u;
            }
        }
        if (walked == kWalk && j < n && keys[j] <= hi) {
            // a dense run: the plane's columns one by one (entries rewritten in order)
#pragma unroll
            for (int w = 0; w < MW; ++w) {
                const int first = 32 * w - PL * c;  // this plane's taps in word w
                uint32_t keep = 0xFFFFFFFFu;
                for (int e = 0; e < PL; ++e)
                    if (e - first >= 0 && e - first < 32) keep &= ~(1u << (e - first));
                bits[w] &= keep;
            }
            for (int dy = 0; dy < KS; ++dy) {
                const K first = lo + (K)(dy * g.sz_y);
                int64_t jc = lower_bound_split(keys, n, first, s_split, ns, sh);
#pragma unroll
                for (int dz = 0; dz < KS; ++dz) {
                    int hit = -1;
                    if (jc < n && keys[jc] == first + (K)dz) {
                        hit = (int)min(vals[jc], (uint32_t)(n - 1));
                        ++jc;
                    }
                    const int kk = PL * c + KS * dy + dz;
                    out[KS * dy + dz] = hit;
                    if (hit >= 0) {
#pragma unroll
                        for (int w = 0; w < MW; ++w) bits[w] |= (kk >> 5) == w ? 1u << (kk & 31) : 0u;
                    }
                }
            }
        }
    }
#pragma unroll
    for (int w = 0; w < MW; ++w)
#pragma unroll
        for (int o = LANES / 2; o > 0; o >>= 1) bits[w] |= __shfl_xor(bits[w], o, LANES);
    if (s < n && c == 0) {
        const int64_t r = min(vals[s], (uint32_t)(n - 1));
        if (KS == 3) {
            mask[r] = bits[0];
        } else {
#pragma unroll
            for (int w = 0; w < MW; ++w) mask[r * kMaxMaskWords + w] = bits[w];
        }
    }
}

inline unsigned blocks_for(int64_t threads) {
    int64_t b = (threads + kBlock - 1) / kBlock;
    return (unsigned)(b < 1 ? 1 : b);
}

}  // namespace

hipError_t launch_state_init(MapState* st, uint32_t* hist, int hist_ints, uint32_t* sticky,
                             hipStream_t s) {
    unsigned blocks = (unsigned)((hist_ints + kBlock - 1) / kBlock);
    if (blocks < 1) blocks = 1;
    if (blocks > 64) blocks = 64;
    launch(k_state_init, blocks, kBlock, 0, s, st, hist, hist_ints, sticky);
    return hipGetLastError();
}

hipError_t launch_bbox(const int32_t* coords, int64_t n, int ncols, MapState* st, hipStream_t s) {
    unsigned blocks = (unsigned)((n + 8 * kBlock - 1) / (8 * kBlock));
    if (blocks < 1) blocks = 1;
    if (blocks > 256) blocks = 256;
    launch(k_bbox, blocks, kBlock, 0, s, coords, n, ncols, st);
    return hipGetLastError();
}

hipError_t launch_fill_i32(int32_t* p, int64_t n, int32_t v, hipStream_t s) {
    if (n <= 0) return hipSuccess;
    unsigned blocks = blocks_for(n);
    if (blocks > 65536) blocks = 65536;
    launch(k_fill_i32, blocks, kBlock, 0, s, p, n, v);
    return hipGetLastError();
}

hipError_t launch_dense_scatter(const int32_t* coords, int64_t n, const Geom& g, int32_t* grid,
                                uint32_t* bits, int32_t* cells, MapState* st,
                                const NextRecord& next, const PrevCells& prev, hipStream_t s,
                                uint32_t* obits, const StrideGeom* sg) {
    if (obits && !sg) return hipErrorInvalidValue;
    launch(k_dense_scatter, blocks_for(n > prev.n ? n : prev.n), kBlock, 0, s, coords, n, g, grid,
           bits, cells, st, next, prev, obits, obits ? *sg : StrideGeom{});
    return hipGetLastError();
}

hipError_t launch_clear_cells(const PrevCells& prev, hipStream_t s) {
    if (prev.n <= 0) return hipSuccess;
    launch(k_clear_cells, blocks_for(prev.n), kBlock, 0, s, prev);
    return hipGetLastError();
}

hipError_t launch_dense_lookup(const int32_t* coords, int64_t n, const Geom& g, const int32_t* grid,
                               const uint32_t* bits, int32_t* nbr, uint32_t* mask, hipStream_t s) {
    if (g.ksize == 5) {
        if (g.brick)
            launch(k_dense_lookup5<true>, blocks_for(n * 32), kBlock, 0, s, coords, n, g, grid,
                   bits, nbr, mask);
        else
            launch(k_dense_lookup5<false>, blocks_for(n * 32), kBlock, 0, s, coords, n, g, grid,
                   bits, nbr, mask);
    } else if (g.brick) {
        launch(k_dense_lookup<true>, blocks_for(n * 16), kBlock, 0, s, coords, n, g, grid, bits,
               nbr, mask);
    } else {
        launch(k_dense_lookup<false>, blocks_for(n * 16), kBlock, 0, s, coords, n, g, grid, bits,
               nbr, mask);
    }
    return hipGetLastError();
}

hipError_t launch_make_keys(const int32_t* coords, int64_t n, const Geom& g, bool wide, void* keys,
                            MapState* st, const NextRecord& next, const SortPlan& plan,
                            uint32_t* hist, hipStream_t s) {
    const unsigned blocks = blocks_for((n + kKeyItems - 1) / kKeyItems);
    const size_t lds = (size_t)plan.passes * (1u << plan.bits) * 4;
    if (wide)
        launch(k_make_keys<uint64_t>, blocks, kBlock, lds, s, coords, n, g, (uint64_t*)keys, st,
               next, plan.bits, plan.passes, hist);
    else
        launch(k_make_keys<uint32_t>, blocks, kBlock, lds, s, coords, n, g, (uint32_t*)keys, st,
               next, plan.bits, plan.passes, hist);
    return hipGetLastError();
}

hipError_t launch_sorted_lookup(const void* keys, const uint32_t* vals, int64_t n, const Geom& g,
                                bool wide, const void* split, int split_shift, int32_t* nbr,
                                uint32_t* mask, MapState* st, hipStream_t s) {
    if (((n + ((int64_t)1 << split_shift) - 1) >> split_shift) > kMaxSplit) return hipErrorInvalidValue;
    if (g.ksize == 5) {
        if (wide)
            launch(k_sorted_lookup<uint64_t, 5>, blocks_for(n * 8), kBlock, 0, s,
                   (const uint64_t*)keys, vals, n, g, (const uint64_t*)split, split_shift, nbr,
                   mask, st);
        else
            launch(k_sorted_lookup<uint32_t, 5>, blocks_for(n * 8), kBlock, 0, s,
                   (const uint32_t*)keys, vals, n, g, (const uint32_t*)split, split_shift, nbr,
                   mask, st);
    } else if (wide) {
        launch(k_sorted_lookup<uint64_t, 3>, blocks_for(n * 4), kBlock, 0, s,
               (const uint64_t*)keys, vals, n, g, (const uint64_t*)split, split_shift, nbr, mask,
               st);
    } else {
        launch(k_sorted_lookup<uint32_t, 3>, blocks_for(n * 4), kBlock, 0, s,
               (const uint32_t*)keys, vals, n, g, (const uint32_t*)split, split_shift, nbr, mask,
               st);
    }
    return hipGetLastError();
}

}  // namespace smc
