// Kernel map of a strided (downsampling) sparse convolution.
//
// "Sparse convolution in FP32" (DriveRT), section "Calibrated bit order":
// the strided layers change the coordinate set, and their kernels are the
// same mask-sorted tiles as the submanifold ones. The layer taken here is the
// usual downsampling one: kernel K = 3, stride 2, padding 1. Output cell o
// exists when an input c = 2 o - 1 + d (d in [0, 3)^3) is active; its taps are
// the 27 cells around the query point q = 2 o, numbered like the submanifold
// taps. Output rows are ordered by (b, x, y, z).
//
// Output cells, two routes chosen by the size of the output grid:
//  * at most 2^30 cells (kOutBitmapWords words of one bit per cell, in
//    (b, x, y, z) order): every input sets the bits of the (at most 8) output
//    cells it feeds; per-block popcounts of the bitmap words are scanned once;
//    each block writes its set bits' cells in bit order, so in (b, x, y, z)
//    order, and clears its words again. The bitmap is zeroed when it is
//    allocated and is all zero between builds;
//  * larger grids: every input emits those cells as packed 64-bit keys; one
//    radix sort orders them; a count / scan / write pass keeps the first of
//    each run.
// Both write the output coordinates and the query points. The neighbour
// lookup around the query points then reuses the dense grid, or searches the
// sorted input keys (k_query_lookup, one search per dx plane as in the Z-Delta
// mapper).
#include "lookback.h"
#include "smc_internal.h"

namespace smc {
namespace {

constexpr int kUThreads = 256;
constexpr int kUItems = 4;
constexpr int kUTile = kUThreads * kUItems;     // sorted candidates per unique block

__device__ inline uint64_t pack_out(const StrideGeom& sg, int b, int x, int y, int z) {
    uint64_t k = (uint64_t)b;
    k = (k << sg.wx) | (uint64_t)x;
    k = (k << sg.wy) | (uint64_t)y;
    k = (k << sg.wz) | (uint64_t)z;
    return k;
}

// Eight key slots per input row: the output cells it feeds, then the sentinel
// (above every key: it sorts last and is dropped).
__global__ __launch_bounds__(kBlock) void k_stride_candidates(const int32_t* __restrict__ coords,
                                                              int64_t n, Geom g, StrideGeom sg,
                                                              uint64_t* __restrict__ keys,
                                                              MapState* st) {
    const int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
    if (i >= n) return;
    const int32_t* c = coords + i * g.ncols;
    const int b = g.ncols == 4 ? c[0] : 0;
    const int32_t* p = c + (g.ncols == 4 ? 1 : 0);
    const int x = p[0] - g.origin[0], y = p[1] - g.origin[1], z = p[2] - g.origin[2];
    const bool in = (unsigned)b < (unsigned)g.batch && (unsigned)x < (unsigned)g.ext[0] &&
                    (unsigned)y < (unsigned)g.ext[1] && (unsigned)z < (unsigned)g.ext[2];
    uint64_t* out = keys + i * 8;
    int written = 0;
    if (in) {
        int x0 = 0, x1 = 0, y0 = 0, y1 = 0, z0 = 0, z1 = 0;
        const int nx = axis_cands(x, sg.oext[0], sg, x0, x1);
        const int ny = axis_cands(y, sg.oext[1], sg, y0, y1);
        const int nz = axis_cands(z, sg.oext[2], sg, z0, z1);
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
            for (int e = 0; e < 2; ++e)
#pragma unroll
                for (int f = 0; f < 2; ++f)
                    if (a < nx && e < ny && f < nz)
                        out[written++] = pack_out(sg, b, a ? x1 : x0, e ? y1 : y0, f ? z1 : z0);
    } else {
        atomicOr(&st->status, kStRange);
    }
    for (int j = written; j < 8; ++j) out[j] = sg.sentinel;
}

// first of a run of equal keys (and not the sentinel)
__device__ inline bool run_head(const uint64_t* __restrict__ keys, int64_t i, uint64_t sentinel) {
    const uint64_t k = keys[i];
    return k < sentinel && (i == 0 || keys[i - 1] != k);
}

__device__ inline uint32_t block_sum(uint32_t v, uint32_t* s_w) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    if (lane == 0) s_w[w] = v;
    __syncthreads();
    uint32_t t = 0;
    for (int q = 0; q < (int)(blockDim.x >> 6); ++q) t += s_w[q];
    return t;
}

__global__ __launch_bounds__(kUThreads) void k_unique_count(const uint64_t* __restrict__ keys,
                                                            int64_t n_c, uint64_t sentinel,
                                                            uint32_t* __restrict__ counts) {
    __shared__ uint32_t s_w[kUThreads / 64];
    const int64_t base = (int64_t)blockIdx.x * kUTile;
    uint32_t c = 0;
#pragma unroll
    for (int j = 0; j < kUItems; ++j) {
        const int64_t i = base + (int64_t)threadIdx.x * kUItems + j;
        if (i < n_c && run_head(keys, i, sentinel)) ++c;
    }
    const uint32_t t = block_sum(c, s_w);
    if (threadIdx.x == 0) counts[blockIdx.x] = t;
}

// Exclusive scan of the per-block counts in place (one block); the total is the
// number of output rows. Thread t takes the contiguous segment
// [t per, (t + 1) per), its loads 16 at a time in flight: its sum, one block
// scan of the 1,024 sums, then the segment's prefixes. (A pass per 1,024
// counts, three barriers each, took 14 us for 11,665 counts.)
__global__ __launch_bounds__(1024) void k_scan_counts(uint32_t* __restrict__ counts, int64_t nb,
                                                      MapState* st) {
    constexpr int kB = 16;
    __shared__ uint32_t s_w[16];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int64_t per = (nb + 1023) / 1024;
    const int64_t i0 = (int64_t)threadIdx.x * per;
    const int64_t i1 = i0 + per < nb ? i0 + per : nb;
    uint32_t sum = 0;
    for (int64_t b0 = i0; b0 < i1; b0 += kB) {
        uint32_t v[kB];
#pragma unroll
        for (int j = 0; j < kB; ++j) v[j] = b0 + j < i1 ? counts[b0 + j] : 0u;
#pragma unroll
        for (int j = 0; j < kB; ++j) sum += v[j];
    }
    uint32_t inc = sum;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const uint32_t t = __shfl_up(inc, o);
        if (lane >= o) inc += t;
    }
    if (lane == 63) s_w[w] = inc;
    __syncthreads();
    uint32_t before = 0;
    for (int q = 0; q < w; ++q) before += s_w[q];
    uint32_t run = before + inc - sum;
    for (int64_t b0 = i0; b0 < i1; b0 += kB) {
        uint32_t v[kB];
#pragma unroll
        for (int j = 0; j < kB; ++j) v[j] = b0 + j < i1 ? counts[b0 + j] : 0u;
#pragma unroll
        for (int j = 0; j < kB; ++j)
            if (b0 + j < i1) {
                counts[b0 + j] = run;
                run += v[j];
            }
    }
    if (threadIdx.x == 1023) st->n_out = (int32_t)(before + inc);
}

// Each run head goes to output row offs[block] + (heads before it in the
// block): its coordinates (b, x, y, z) and query point (b, s x - pad + r, ...)
// in input coordinates.
__global__ __launch_bounds__(kUThreads) void k_unique_write(
    const uint64_t* __restrict__ keys, int64_t n_c, StrideGeom sg,
    const uint32_t* __restrict__ offs, int32_t* __restrict__ ocoords,
    int32_t* __restrict__ qcoords) {
    __shared__ uint32_t s_w[kUThreads / 64];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int64_t base = (int64_t)blockIdx.x * kUTile + (int64_t)threadIdx.x * kUItems;
    bool h[kUItems];
    uint32_t c = 0;
#pragma unroll
    for (int j = 0; j < kUItems; ++j) {
        h[j] = base + j < n_c && run_head(keys, base + j, sg.sentinel);
        c += h[j] ? 1u : 0u;
    }
    uint32_t inc = c;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const uint32_t t = __shfl_up(inc, o);
        if (lane >= o) inc += t;
    }
    if (lane == 63) s_w[w] = inc;
    __syncthreads();
    uint32_t pos = offs[blockIdx.x] + inc - c;
    for (int q = 0; q < w; ++q) pos += s_w[q];
    const uint64_t mz = (1ull << sg.wz) - 1, my = (1ull << sg.wy) - 1, mx = (1ull << sg.wx) - 1;
    const int r = (sg.ksize - 1) / 2;
#pragma unroll
    for (int j = 0; j < kUItems; ++j) {
        if (!h[j]) continue;
        const uint64_t k = keys[base + j];
        const int z = (int)(k & mz), y = (int)((k >> sg.wz) & my),
                  x = (int)((k >> (sg.wz + sg.wy)) & mx), b = (int)(k >> (sg.wz + sg.wy + sg.wx));
        reinterpret_cast<int4*>(ocoords)[pos] = make_int4(b, x, y, z);
        reinterpret_cast<int4*>(qcoords)[pos] =
            make_int4(b, sg.stride * x - sg.pad + r + sg.origin[0],
                      sg.stride * y - sg.pad + r + sg.origin[1],
                      sg.stride * z - sg.pad + r + sg.origin[2]);
        ++pos;
    }
}

// ---- output cells through a bitmap of the output grid (small output grids) ----
// Bit L = ((b OX + x) OY + y) OZ + z: the same (b, x, y, z) order as the packed
// keys, so reading the set bits in order lists the output cells sorted and
// without repeats, with no candidate sort.
constexpr int kBWords = 4;                        // bitmap words per thread
constexpr int kBTile = kUThreads * kBWords;       // words per count / write block

__global__ __launch_bounds__(kBlock) void k_stride_mark(const int32_t* __restrict__ coords,
                                                        int64_t n, Geom g, StrideGeom sg,
                                                        uint32_t* __restrict__ obits,
                                                        MapState* st) {
    const int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
    if (i >= n) return;
    const int32_t* c = coords + i * g.ncols;
    const int b = g.ncols == 4 ? c[0] : 0;
    const int32_t* p = c + (g.ncols == 4 ? 1 : 0);
    const int x = p[0] - g.origin[0], y = p[1] - g.origin[1], z = p[2] - g.origin[2];
    const bool in = (unsigned)b < (unsigned)g.batch && (unsigned)x < (unsigned)g.ext[0] &&
                    (unsigned)y < (unsigned)g.ext[1] && (unsigned)z < (unsigned)g.ext[2];
    if (!in) {
        atomicOr(&st->status, kStRange);
        return;
    }
    stride_mark(sg, b, x, y, z, obits);
}

__global__ __launch_bounds__(kUThreads) void k_bits_count(const uint32_t* __restrict__ obits,
                                                          int64_t words,
                                                          uint32_t* __restrict__ counts) {
    __shared__ uint32_t s_w[kUThreads / 64];
    const int64_t base = (int64_t)blockIdx.x * kBTile + (int64_t)threadIdx.x * kBWords;
    uint32_t c = 0;
#pragma unroll
    for (int j = 0; j < kBWords; ++j)
        if (base + j < words) c += (uint32_t)__popc(obits[base + j]);
    const uint32_t t = block_sum(c, s_w);
    if (threadIdx.x == 0) counts[blockIdx.x] = t;
}

// The set bits of each block's words go to output rows offs[block] + (set bits
// before them in the block), as k_unique_write does for run heads; each word is
// cleared once read, so the bitmap is empty again for the next build.
__global__ __launch_bounds__(kUThreads) void k_bits_write(uint32_t* __restrict__ obits,
                                                          int64_t words, StrideGeom sg,
                                                          const uint32_t* __restrict__ offs,
                                                          int32_t* __restrict__ ocoords,
                                                          int32_t* __restrict__ qcoords) {
    __shared__ uint32_t s_w[kUThreads / 64];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int64_t base = (int64_t)blockIdx.x * kBTile + (int64_t)threadIdx.x * kBWords;
    uint32_t v[kBWords];
    uint32_t c = 0;
#pragma unroll
    for (int j = 0; j < kBWords; ++j) {
        v[j] = base + j < words ? obits[base + j] : 0u;
        c += (uint32_t)__popc(v[j]);
    }
    uint32_t inc = c;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const uint32_t t = __shfl_up(inc, o);
        if (lane >= o) inc += t;
    }
    if (lane == 63) s_w[w] = inc;
    __syncthreads();
    uint32_t pos = offs[blockIdx.x] + inc - c;
    for (int q = 0; q < w; ++q) pos += s_w[q];
    const int r = (sg.ksize - 1) / 2;
    // (the bitmap route covers fewer than 2^32 cells: 32-bit cell arithmetic)
    const uint32_t ez = (uint32_t)sg.oext[2], ey = (uint32_t)sg.oext[1], ex = (uint32_t)sg.oext[0];
#pragma unroll
    for (int j = 0; j < kBWords; ++j) {
        if (base + j >= words) break;
        if (v[j]) obits[base + j] = 0u;
        for (uint32_t bits = v[j]; bits; bits &= bits - 1) {
            uint32_t L = ((uint32_t)(base + j) << 5) + (uint32_t)__builtin_ctz(bits);
            const int z = (int)(L % ez);
            L /= ez;
            const int y = (int)(L % ey);
            L /= ey;
            const int x = (int)(L % ex);
            const int b = (int)(L / ex);
            reinterpret_cast<int4*>(ocoords)[pos] = make_int4(b, x, y, z);
            reinterpret_cast<int4*>(qcoords)[pos] =
                make_int4(b, sg.stride * x - sg.pad + r + sg.origin[0],
                          sg.stride * y - sg.pad + r + sg.origin[1],
                          sg.stride * z - sg.pad + r + sg.origin[2]);
            ++pos;
        }
    }
}

// The same in one pass, for bitmaps of at most 2 chunks per CU (512 on this
// GPU): block b takes chunk b (far fewer blocks than the device holds at once,
// so every block is resident and a block only waits for running blocks),
// counts its set bits, publishes the count, adds the counts of every earlier
// chunk by decoupled look-back (the whole block reads 1,024 predecessors per
// round trip), then writes its set bits as above. The last block stores the
// total as the output count. One launch instead of three (strided layers: 6
// chunks 118.6 -> 115.2 us, 333 chunks 134.3 -> 133.2 and 74.9 -> 74.3 us).
// Larger bitmaps keep the three passes: a block per chunk with tickets from
// one counter serialised on its atomics (60 -> 180 us for 11,665 chunks).
__global__ __launch_bounds__(kUThreads) void k_bits_emit(uint32_t* __restrict__ obits,
                                                         int64_t words, StrideGeom sg,
                                                         uint64_t* __restrict__ look,
                                                         uint32_t epoch,
                                                         int32_t* __restrict__ ocoords,
                                                         int32_t* __restrict__ qcoords,
                                                         MapState* __restrict__ st) {
    __shared__ uint32_t s_w[kUThreads / 64];
    __shared__ uint32_t s_tot, s_pre[1], s_done[1];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int64_t bid = blockIdx.x;
    const int64_t base = bid * kBTile + (int64_t)threadIdx.x * kBWords;
    uint32_t v[kBWords];
    uint32_t c = 0;
#pragma unroll
    for (int j = 0; j < kBWords; ++j) {
        v[j] = base + j < words ? obits[base + j] : 0u;
        c += (uint32_t)__popc(v[j]);
    }
    uint32_t inc = c;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const uint32_t t = __shfl_up(inc, o);
        if (lane >= o) inc += t;
    }
    if (lane == 63) s_w[w] = inc;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t tot = 0;
        for (int q = 0; q < kUThreads / 64; ++q) tot += s_w[q];
        s_tot = tot;
        __hip_atomic_store(&look[bid], lb_pack(epoch & 0x3FFFFFFFu, bid == 0 ? kIncl : kAgg, tot),
                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    block_lookback<1, 4, kUThreads>(look, bid - 1, epoch, &st->status, s_pre, s_done);
    const uint32_t pre = s_pre[0];
    if (threadIdx.x == 0) {
        if (bid > 0)
            __hip_atomic_store(&look[bid], lb_pack(epoch & 0x3FFFFFFFu, kIncl, pre + s_tot),
                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (bid == (int64_t)gridDim.x - 1) st->n_out = (int32_t)(pre + s_tot);
    }
    uint32_t pos = pre + inc - c;
    for (int q = 0; q < w; ++q) pos += s_w[q];
    const int r = (sg.ksize - 1) / 2;
    // (the bitmap route covers fewer than 2^32 cells: 32-bit cell arithmetic)
    const uint32_t ez = (uint32_t)sg.oext[2], ey = (uint32_t)sg.oext[1], ex = (uint32_t)sg.oext[0];
#pragma unroll
    for (int j = 0; j < kBWords; ++j) {
        if (base + j >= words) break;
        if (v[j]) obits[base + j] = 0u;
        for (uint32_t bits = v[j]; bits; bits &= bits - 1) {
            uint32_t L = ((uint32_t)(base + j) << 5) + (uint32_t)__builtin_ctz(bits);
            const int z = (int)(L % ez);
            L /= ez;
            const int y = (int)(L % ey);
            L /= ey;
            const int x = (int)(L % ex);
            const int b = (int)(L / ex);
            reinterpret_cast<int4*>(ocoords)[pos] = make_int4(b, x, y, z);
            reinterpret_cast<int4*>(qcoords)[pos] =
                make_int4(b, sg.stride * x - sg.pad + r + sg.origin[0],
                          sg.stride * y - sg.pad + r + sg.origin[1],
                          sg.stride * z - sg.pad + r + sg.origin[2]);
            ++pos;
        }
    }
}

template <typename K>
__device__ inline int64_t lower_bound_k(const K* __restrict__ keys, int64_t n, K t) {
    int64_t lo = 0, len = n;
    while (len > 0) {
        const int64_t half = len >> 1;
        if (keys[lo + half] < t) {
            lo += half + 1;
            len -= half + 1;
        } else {
            len = half;
        }
    }
    return lo;
}

// Sorted route: the 27 taps around each query point, searched in the sorted
// input keys with 4 lanes per query, one per dx plane: the plane's 9 taps
// have keys in one run [key(x + dx, y - 1, z - 1), key(x + dx, y + 1, z + 1)],
// found by one lower_bound and walked, each key's offset giving its (dy, dz).
// A run of more than 12 keys falls back to a search per (dx, dy) column.
template <typename K>
__global__ __launch_bounds__(kBlock) void k_query_lookup(const K* __restrict__ keys,
                                                         const uint32_t* __restrict__ vals,
                                                         int64_t n_in, Geom g,
                                                         const int32_t* __restrict__ qcoords,
                                                         int64_t m, int32_t* __restrict__ nbr,
                                                         uint32_t* __restrict__ mask,
                                                         const int32_t* __restrict__ m_dev) {
    constexpr int kWalk = 12;
    if (m_dev && *m_dev < m) m = *m_dev;          // rows counted on the device (grid: a bound)
    const int64_t t = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
    const int64_t o = t >> 2;
    const int c = (int)(t & 3);
    uint32_t bits = 0;
    if (o < m && c < 3) {
        const int32_t* q = qcoords + o * 4;
        // the input's key of the query point: its cell in the padded input grid
        const K key = (K)(q[0] * g.sz_b + (int64_t)(q[1] - g.origin[0] + g.pad) * g.sz_x +
                          (int64_t)(q[2] - g.origin[1] + g.pad) * g.sz_y +
                          (q[3] - g.origin[2] + g.pad));
        const int dx = c - 1;
        const K lo = key + (K)(dx * g.sz_x - g.sz_y - 1);
        const K hi = key + (K)(dx * g.sz_x + g.sz_y + 1);
        int32_t* out = nbr + o * kTaps + 9 * c;           // the plane's 9 entries
#pragma unroll
        for (int e = 0; e < 9; ++e) out[e] = -1;
        int64_t j = lower_bound_k(keys, n_in, lo);
        int walked = 0;
        for (; j < n_in && walked < kWalk; ++j, ++walked) {
            const K kj = keys[j];
            if (kj > hi) break;
            const K off = kj - lo;
            const int dy = (off >= (K)g.sz_y ? 1 : 0) + (off >= (K)(2 * g.sz_y) ? 1 : 0);
            const K dz = off - (K)(dy * g.sz_y);
            if (dz < (K)3) {
                out[3 * dy + dz] = (int)min(vals[j], (uint32_t)(n_in - 1));
                bits |= 1u << (9 * c + 3 * dy + (int)dz);
            }
        }
        if (walked == kWalk && j < n_in && keys[j] <= hi) {   // a dense run: column by column
            bits = 0;
            for (int dy = 0; dy < 3; ++dy) {
                const K first = lo + (K)(dy * g.sz_y);
                int64_t jc = lower_bound_k(keys, n_in, first);
#pragma unroll
                for (int dz = 0; dz < 3; ++dz) {
                    int hit = -1;
                    if (jc < n_in && keys[jc] == first + (K)dz) {
                        hit = (int)min(vals[jc], (uint32_t)(n_in - 1));
                        ++jc;
                    }
                    out[3 * dy + dz] = hit;
                    if (hit >= 0) bits |= 1u << (9 * c + 3 * dy + dz);
                }
            }
        }
    }
    bits |= __shfl_xor(bits, 2, 4);
    bits |= __shfl_xor(bits, 1, 4);
    if (o < m && c == 0) mask[o] = bits;
}

// Two rows with one key: duplicate coordinates (sorted route of a strided map).
template <typename K>
__global__ __launch_bounds__(kBlock) void k_key_dups(const K* __restrict__ keys, int64_t n,
                                                     MapState* st) {
    const int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
    if (i + 1 < n && keys[i] == keys[i + 1]) atomicOr(&st->status, kStDuplicate);
}

inline unsigned blocks_of(int64_t threads, int per) {
    const int64_t b = (threads + per - 1) / per;
    return (unsigned)(b < 1 ? 1 : b);
}

}  // namespace

int64_t unique_blocks(int64_t n_c) { return (n_c + kUTile - 1) / kUTile; }

hipError_t launch_stride_candidates(const int32_t* coords, int64_t n, const Geom& g,
                                    const StrideGeom& sg, uint64_t* keys, MapState* st,
                                    hipStream_t s) {
    if (n <= 0) return hipSuccess;
    launch(k_stride_candidates, blocks_of(n, kBlock), kBlock, 0, s, coords, n, g, sg, keys, st);
    return hipGetLastError();
}

hipError_t launch_unique(const uint64_t* keys, int64_t n_c, const StrideGeom& sg,
                         uint32_t* counts, int32_t* ocoords, int32_t* qcoords, MapState* st,
                         hipStream_t s) {
    if (n_c <= 0) return hipSuccess;
    const int64_t nb = unique_blocks(n_c);
    launch(k_unique_count, (unsigned)nb, kUThreads, 0, s, keys, n_c, sg.sentinel, counts);
    launch(k_scan_counts, 1u, 1024, 0, s, counts, nb, st);
    launch(k_unique_write, (unsigned)nb, kUThreads, 0, s, keys, n_c, sg, (const uint32_t*)counts,
           ocoords, qcoords);
    return hipGetLastError();
}

int64_t out_bitmap_words(const StrideGeom& sg, int batch) {
    return ((int64_t)batch * sg.oext[0] * sg.oext[1] * sg.oext[2] + 31) / 32;
}

int64_t out_bitmap_blocks(int64_t words) { return (words + kBTile - 1) / kBTile; }

hipError_t launch_stride_bitmap(const int32_t* coords, int64_t n, const Geom& g,
                                const StrideGeom& sg, uint32_t* obits, int64_t words,
                                uint32_t* counts, int32_t* ocoords, int32_t* qcoords,
                                MapState* st, SortWork& ws, int n_cu, hipStream_t s, bool marked) {
    if (n <= 0 || words <= 0) return hipSuccess;
    const int64_t nb = out_bitmap_blocks(words);
    if (!marked)
        launch(k_stride_mark, blocks_of(n, kBlock), kBlock, 0, s, coords, n, g, sg, obits, st);
    if (nb <= 2 * (int64_t)n_cu) {
        launch(k_bits_emit, (unsigned)nb, kUThreads, 0, s, obits, words, sg, ws.look,
               take_epoch(ws), ocoords, qcoords, st);
        return hipGetLastError();
    }
    launch(k_bits_count, (unsigned)nb, kUThreads, 0, s, (const uint32_t*)obits, words, counts);
    launch(k_scan_counts, 1u, 1024, 0, s, counts, nb, st);
    launch(k_bits_write, (unsigned)nb, kUThreads, 0, s, obits, words, sg, (const uint32_t*)counts,
           ocoords, qcoords);
    return hipGetLastError();
}

hipError_t launch_query_lookup(const void* keys, const uint32_t* vals, int64_t n_in, const Geom& g,
                               bool wide, const int32_t* qcoords, int64_t m, int32_t* nbr,
                               uint32_t* mask, hipStream_t s, const int32_t* m_dev) {
    if (m <= 0) return hipSuccess;
    if (wide)
        launch(k_query_lookup<uint64_t>, blocks_of(m * 4, kBlock), kBlock, 0, s,
               (const uint64_t*)keys, vals, n_in, g, qcoords, m, nbr, mask, m_dev);
    else
        launch(k_query_lookup<uint32_t>, blocks_of(m * 4, kBlock), kBlock, 0, s,
               (const uint32_t*)keys, vals, n_in, g, qcoords, m, nbr, mask, m_dev);
    return hipGetLastError();
}

hipError_t launch_key_dups(const void* keys, bool wide, int64_t n, MapState* st, hipStream_t s) {
    if (n <= 1) return hipSuccess;
    if (wide)
        launch(k_key_dups<uint64_t>, blocks_of(n, kBlock), kBlock, 0, s, (const uint64_t*)keys, n, st);
    else
        launch(k_key_dups<uint32_t>, blocks_of(n, kBlock), kBlock, 0, s, (const uint32_t*)keys, n, st);
    return hipGetLastError();
}

}  // namespace smc
