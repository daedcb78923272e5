// Compaction of the neighbour table into per-tap pair lists.
//
// Only existing (input, output) pairs are listed, grouped by tap so that a
// GEMM tile shares one weight slab, and each tap's run is padded to a
// multiple of the tile height ("[Kernel] Add submanifold sparse 3D
// convolution (bf16 implicit GEMM, gfx950)", Design "Compaction"). Within a
// tap, pairs follow the mask-sorted row order ("Sparse convolution in FP32",
// "Neighbour masks and sorted rows"). That pull request counts per (tap,
// tile), scans the small count table and then writes, keeping the totals on
// the device (commits "move pair compaction from torch onto three fx
// kernels", "scan the pair counts on the device"). Here the per-tap totals
// come for free from the mask histogram pass, and the count/scan/write
// become one kernel: each chunk of sorted rows finds the pairs of earlier
// chunks by decoupled look-back (same ticket + epoch scheme as the sort).
#include "smc_internal.h"

namespace smc {
namespace {

constexpr int kHThreads = 256;
constexpr int kHItems = 4;
constexpr int kHTile = kHThreads * kHItems;       // rows per histogram block
constexpr int kCThreads = 256;
constexpr int kCWaves = kCThreads / 64;
constexpr int kCItems = 4;
constexpr int kCChunk = kCThreads * kCItems;      // sorted rows per compaction block
constexpr uint32_t kSpinLimit = 1u << 22;
constexpr uint64_t kAgg = 1, kIncl = 2;

__device__ inline uint64_t lb_pack(uint32_t epoch, uint64_t state, uint32_t count) {
    return ((uint64_t)epoch << 34) | (state << 32) | count;
}

// Sum of column d of the look-back table over blocks pb, pb-1, ... back to
// the first inclusive entry (8 loads per round trip).
__device__ inline uint32_t lookback8(uint64_t* look, int stride, int d, int64_t pb,
                                     uint32_t epoch, uint32_t* status) {
    const uint32_t ep = epoch & 0x3FFFFFFFu;
    uint32_t prefix = 0;
    uint32_t spins = 0;
    while (pb >= 0) {
        uint64_t e[8];
#pragma unroll
        for (int j = 0; j < 8; ++j)
            e[j] = pb - j >= 0 ? __hip_atomic_load(&look[(pb - j) * stride + d], __ATOMIC_RELAXED,
                                                   __HIP_MEMORY_SCOPE_AGENT)
                               : 0;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            if (pb - j < 0) return prefix;
            while ((uint32_t)(e[j] >> 34) != ep) {
                if (++spins > kSpinLimit) {
                    atomicOr(status, kStSortStall);
                    return prefix;
                }
                __builtin_amdgcn_s_sleep(1);
                e[j] = __hip_atomic_load(&look[(pb - j) * stride + d], __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT);
            }
            prefix += (uint32_t)e[j];
            if (((e[j] >> 32) & 3u) == kIncl) return prefix;
        }
        pb -= 8;
    }
    return prefix;
}

// One read of the masks: digit histograms of every mask-sort pass, pairs per
// tap (mask column sums), and -- on the dense route -- the grid cells of the
// rows put back to empty (the lookups that needed them have finished).
__global__ __launch_bounds__(kHThreads) void k_mask_hist(const uint32_t* __restrict__ mask,
                                                         int64_t n, int bits, int passes,
                                                         uint32_t* __restrict__ hist,
                                                         int32_t* __restrict__ tap_tot,
                                                         const int32_t* __restrict__ coords,
                                                         Geom g, int32_t* __restrict__ grid) {
    extern __shared__ uint32_t s_h[];             // passes << bits, then 27 tap counters
    const int bins = 1 << bits;
    uint32_t* s_tap = s_h + passes * bins;
    for (int i = threadIdx.x; i < passes * bins + kTaps; i += kHThreads) s_h[i] = 0;
    __syncthreads();
    const int lane = threadIdx.x & 63;
    int64_t base = (int64_t)blockIdx.x * kHTile;
    uint32_t tap_acc = 0;                          // lane k < 27 keeps tap k's wave count
    uint32_t mv[kHItems];
#pragma unroll
    for (int i = 0; i < kHItems; ++i) {
        int64_t idx = base + i * kHThreads + threadIdx.x;
        const uint32_t v = mask[idx < n ? idx : n - 1];
        mv[i] = idx < n ? v : 0u;
    }
#pragma unroll
    for (int i = 0; i < kHItems; ++i) {
        int64_t idx = base + i * kHThreads + threadIdx.x;
        const uint32_t m = mv[i];
        if (idx < n) {
            for (int p = 0; p < passes; ++p)
                atomicAdd(&s_h[p * bins + ((m >> (p * bits)) & (bins - 1))], 1u);
            if (grid) {
                const int32_t* c = coords + idx * g.ncols;
                int b = g.ncols == 4 ? c[0] : 0;
                const int32_t* q = c + (g.ncols == 4 ? 1 : 0);
                int x = q[0] - g.origin[0], y = q[1] - g.origin[1], z = q[2] - g.origin[2];
                if ((unsigned)b < (unsigned)g.batch && (unsigned)x < (unsigned)g.ext[0] &&
                    (unsigned)y < (unsigned)g.ext[1] && (unsigned)z < (unsigned)g.ext[2])
                    grid[b * g.sz_b + (int64_t)(x + 1) * g.sz_x + (int64_t)(y + 1) * g.sz_y +
                         (z + 1)] = -1;
            }
        }
#pragma unroll
        for (int k = 0; k < kTaps; ++k) {
            uint32_t c = (uint32_t)__popcll(__ballot((m >> k) & 1u));
            if (lane == k) tap_acc += c;
        }
    }
    if (lane < kTaps && tap_acc) atomicAdd(&s_tap[lane], tap_acc);
    __syncthreads();
    for (int i = threadIdx.x; i < passes * bins; i += kHThreads)
        if (s_h[i]) atomicAdd(&hist[i], s_h[i]);
    if (threadIdx.x < kTaps && s_tap[threadIdx.x]) atomicAdd(&tap_tot[threadIdx.x], (int32_t)s_tap[threadIdx.x]);
}

// Rows [bid*kCChunk, +kCChunk) of the mask-sorted order. Wave w owns a
// contiguous quarter; for each tap the block counts its rows with that bit,
// finds the count of earlier chunks by look-back, and writes its pairs.
__global__ __launch_bounds__(kCThreads) void k_compact(
    const uint32_t* __restrict__ perm, const uint32_t* __restrict__ mask,
    const int32_t* __restrict__ nbr, int64_t n, const int32_t* __restrict__ tap_tot, int tile_m,
    MapState* st, int32_t* __restrict__ pair_in, int32_t* __restrict__ pair_out,
    int32_t* __restrict__ tile_tap, uint64_t* __restrict__ look, uint32_t* ticket,
    uint32_t epoch, uint32_t* status) {
    __shared__ uint32_t s_bid;
    __shared__ int32_t s_off[kTaps + 1];          // padded tap starts
    __shared__ int32_t s_tot[kTaps];
    __shared__ uint32_t s_wc[kCWaves][kTaps];     // per-wave counts, then offsets in the chunk
    __shared__ uint32_t s_pre[kTaps];             // pairs of this tap in earlier chunks
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    if (tid == 0) {
        s_bid = atomicAdd(ticket, 1u);
        int32_t off = 0;
        for (int k = 0; k < kTaps; ++k) {
            int32_t t = tap_tot[k];
            s_tot[k] = t;
            s_off[k] = off;
            off += (t + tile_m - 1) / tile_m * tile_m;
        }
        s_off[kTaps] = off;
    }
    __syncthreads();
    const uint32_t bid = s_bid;
    const int64_t base = (int64_t)bid * kCChunk + (int64_t)w * (kCChunk / kCWaves);
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));

    uint32_t row[kCItems], m[kCItems];
#pragma unroll
    for (int i = 0; i < kCItems; ++i) {
        int64_t s = base + i * 64 + lane;
        row[i] = min(perm[s < n ? s : n - 1], (uint32_t)(n - 1));   // clamp: see the sort
    }
#pragma unroll
    for (int i = 0; i < kCItems; ++i) {
        int64_t s = base + i * 64 + lane;
        const uint32_t mv = mask[row[i]];
        m[i] = s < n ? mv : 0u;
    }
    // per-wave count of each tap (lane k accumulates tap k)
    uint32_t cnt = 0;
#pragma unroll
    for (int k = 0; k < kTaps; ++k) {
        uint32_t c = 0;
#pragma unroll
        for (int i = 0; i < kCItems; ++i) c += (uint32_t)__popcll(__ballot((m[i] >> k) & 1u));
        if (lane == k) cnt = c;
    }
    if (lane < kTaps) s_wc[w][lane] = cnt;
    __syncthreads();
    if (tid < kTaps) {
        const int k = tid;
        uint32_t run = 0;
#pragma unroll
        for (int v = 0; v < kCWaves; ++v) {
            uint32_t c = s_wc[v][k];
            s_wc[v][k] = run;
            run += c;
        }
        __hip_atomic_store(&look[(int64_t)bid * kTaps + k],
                           lb_pack(epoch, bid == 0 ? kIncl : kAgg, run), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
        uint32_t prefix = 0;
        if (bid > 0) {
            prefix = lookback8(look, kTaps, k, (int64_t)bid - 1, epoch, status);
            __hip_atomic_store(&look[(int64_t)bid * kTaps + k], lb_pack(epoch, kIncl, prefix + run),
                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        s_pre[k] = prefix;
    }
    __syncthreads();
    // write pairs: neighbour ids of 9 taps x 4 rows loaded together, then stored
#pragma unroll
    for (int k0 = 0; k0 < kTaps; k0 += 9) {
        int32_t nv[9][kCItems];
#pragma unroll
        for (int kk = 0; kk < 9; ++kk)
#pragma unroll
            for (int i = 0; i < kCItems; ++i) nv[kk][i] = nbr[(int64_t)row[i] * kTaps + k0 + kk];
#pragma unroll
        for (int kk = 0; kk < 9; ++kk) {
            const int k = k0 + kk;
            const int64_t start = (int64_t)s_off[k] + s_pre[k] + s_wc[w][k];
            const int64_t lim = (int64_t)s_off[k] + s_tot[k];
            uint32_t run = 0;
#pragma unroll
            for (int i = 0; i < kCItems; ++i) {
                uint64_t b = __ballot((m[i] >> k) & 1u);
                if ((m[i] >> k) & 1u) {
                    int64_t pos = start + run + (uint32_t)__popcll(b & below);
                    if (pos < lim) {               // false only after a stalled wait
                        pair_in[pos] = nv[kk][i];
                        pair_out[pos] = (int32_t)row[i];
                    }
                }
                run += (uint32_t)__popcll(b);
            }
        }
    }
    // pads, totals, tile taps
    const int32_t padded = s_off[kTaps];
    const int32_t n_tiles = padded / tile_m;
    if (bid == 0) {
        for (int k = 0; k < kTaps; ++k)
            for (int p = s_off[k] + s_tot[k] + tid; p < s_off[k + 1]; p += kCThreads) {
                pair_in[p] = -1;
                pair_out[p] = -1;
            }
        if (tid == 0) {
            int32_t p = 0;
            for (int k = 0; k < kTaps; ++k) p += s_tot[k];
            st->totals[0] = p;
            st->totals[1] = padded;
            st->totals[2] = n_tiles;
        }
        if (tid < kTaps) {
            st->tap_count[tid] = s_tot[tid];
            st->tap_off[tid] = s_off[tid];
        }
        if (tid == 0) st->tap_off[kTaps] = padded;
    }
    for (int64_t t = (int64_t)bid * kCThreads + tid; t < n_tiles; t += (int64_t)gridDim.x * kCThreads) {
        const int32_t p = (int32_t)t * tile_m;
        int k = 0;
        while (k + 1 < kTaps && s_off[k + 1] <= p) ++k;
        tile_tap[t] = k;
    }
    if (bid == gridDim.x - 1 && tid == 0) atomicExch(ticket, 0u);
}

}  // namespace

hipError_t launch_mask_hist(const uint32_t* mask, int64_t n, const SortPlan& plan, uint32_t* hist,
                            int32_t* tap_tot, const int32_t* coords, const Geom& g,
                            int32_t* grid, hipStream_t s) {
    unsigned blocks = (unsigned)((n + kHTile - 1) / kHTile);
    size_t lds = ((size_t)plan.passes * (1u << plan.bits) + kTaps) * 4;
    k_mask_hist<<<blocks, kHThreads, lds, s>>>(mask, n, plan.bits, plan.passes, hist, tap_tot,
                                               coords, g, grid);
    return hipGetLastError();
}

int64_t compact_chunks(int64_t n) { return (n + kCChunk - 1) / kCChunk; }

hipError_t launch_compact(const uint32_t* perm, const uint32_t* mask, const int32_t* nbr, int64_t n,
                          const int32_t* tap_tot, int tile_m, MapState* st, int32_t* pair_in,
                          int32_t* pair_out, int32_t* tile_tap, SortWork& ws, uint32_t* status,
                          hipStream_t s) {
    uint32_t epoch = ++ws.epoch & 0x3FFFFFFFu;
    if (epoch == 0) epoch = ++ws.epoch & 0x3FFFFFFFu;
    unsigned blocks = (unsigned)compact_chunks(n);
    k_compact<<<blocks, kCThreads, 0, s>>>(perm, mask, nbr, n, tap_tot, tile_m, st, pair_in,
                                           pair_out, tile_tap, ws.look, ws.ticket, epoch, status);
    return hipGetLastError();
}

}  // namespace smc
