// Compaction of the neighbour table into per-tap pair lists.
//
// Only existing (input, output) pairs are listed, grouped by tap so that a GEMM tile shares one
// weight slab ("[Kernel] Add submanifold sparse 3D convolution (bf16 implicit GEMM, gfx950)",
// section "Design, and the measurements behind it"); within a tap the pairs follow ascending
// output row. That pull request counts per (tap, tile), scans the small count table and then
// writes, keeping the totals on the device (commits 6ee20cd and f9cb4f1). Here count, scan and
// write are one kernel: each chunk of rows finds the pairs of earlier chunks by decoupled
// look-back (same ticket + epoch scheme as the sort), and every tap owns a fixed run of the
// pair arrays (cap entries, cap = n rounded up to the tile height), so no chunk needs the other
// taps' totals first.
//
// The same pass numbers the off-centre pairs of every output row
// consecutively (row order, then tap order): pair_slot[p] is the row of a
// float32 partial-product slab where the GEMM of the non-centre taps stores
// the pair's product, and rowbase[i] is the first slab row of output row i.
// The centre-tap GEMM then sums each row's slab rows in its epilogue: no
// atomics and no accumulator to clear.
#include "smc_internal.h"

namespace smc {
namespace {

constexpr int kHThreads = 256;
constexpr int kHItems = 4;
constexpr int kHTile = kHThreads * kHItems;       // rows per histogram block
constexpr int kCThreads = 256;
constexpr int kCWaves = kCThreads / 64;
constexpr int kCChunk = kCThreads;                // rows per compaction block (one per thread)
constexpr int kCNbrVec = kCChunk * kTaps / 4;     // 16-byte words of the chunk's neighbour rows
constexpr int kCNbrPer = (kCNbrVec + kCThreads - 1) / kCThreads;
constexpr uint32_t kSpinLimit = 1u << 22;
constexpr uint64_t kAgg = 1, kIncl = 2;

__device__ inline uint64_t lb_pack(uint32_t epoch, uint64_t state, uint32_t count) {
    return ((uint64_t)epoch << 34) | (state << 32) | count;
}

// Sum of column d of the look-back table over blocks pb, pb-1, ... back to
// the first inclusive entry (W loads per round trip).
template <int W>
__device__ inline uint32_t lookback(uint64_t* look, int stride, int d, int64_t pb, uint32_t epoch,
                                    uint32_t* status) {
    const uint32_t ep = epoch & 0x3FFFFFFFu;
    uint32_t prefix = 0;
    uint32_t spins = 0;
    while (pb >= 0) {
        uint64_t e[W];
#pragma unroll
        for (int j = 0; j < W; ++j)
            e[j] = pb - j >= 0 ? __hip_atomic_load(&look[(pb - j) * stride + d], __ATOMIC_RELAXED,
                                                   __HIP_MEMORY_SCOPE_AGENT)
                               : 0;
#pragma unroll
        for (int j = 0; j < W; ++j) {
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
        pb -= W;
    }
    return prefix;
}

// Prefix of column k (k < NC) over blocks pb, pb-1, ..., read by the whole
// block: thread t < 9 NC covers column t % NC and every 9th predecessor
// starting at pb - t / NC, W of them per round trip (72 predecessors per
// column per round). A round finds, per column, the nearest entry that
// holds an inclusive prefix (LDS minimum of the distance), and sums the
// entries up to and including it; columns without one go on to the next
// round. Every thread of the block must call this. The result is in
// s_sum[k] on return.
template <int NC, int W>
__device__ void block_lookback(uint64_t* look, int64_t pb, uint32_t epoch, uint32_t* status,
                               uint32_t* s_sum, uint32_t* s_near, uint32_t* s_done) {
    constexpr int kLanes = 9;                     // threads per column
    const int tid = threadIdx.x;
    const int k = tid % NC, j0 = tid / NC;
    const bool active = tid < kLanes * NC;
    const uint32_t ep = epoch & 0x3FFFFFFFu;
    if (tid < NC) {
        s_sum[tid] = 0;
        s_done[tid] = pb < 0 ? 1u : 0u;
    }
    __syncthreads();
    uint32_t spins = 0;
    for (int64_t top = pb; top >= 0; top -= kLanes * W) {
        if (tid < NC) s_near[tid] = 0xFFFFFFFFu;
        __syncthreads();
        const bool go = active && !s_done[k];
        uint64_t e[W];
        uint32_t near = 0xFFFFFFFFu;
#pragma unroll
        for (int j = 0; j < W; ++j) {
            const int64_t idx = top - j0 - (int64_t)j * kLanes;
            e[j] = 0;
            if (go && idx >= 0)
                e[j] = __hip_atomic_load(&look[idx * NC + k], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
#pragma unroll
        for (int j = 0; j < W; ++j) {
            const int64_t idx = top - j0 - (int64_t)j * kLanes;
            if (!go || idx < 0) continue;
            while ((uint32_t)(e[j] >> 34) != ep) {
                if (++spins > kSpinLimit) {
                    atomicOr(status, kStSortStall);
                    e[j] = 0;
                    break;
                }
                __builtin_amdgcn_s_sleep(1);
                e[j] = __hip_atomic_load(&look[idx * NC + k], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
            if (((e[j] >> 32) & 3u) == kIncl) near = min(near, (uint32_t)(top - idx));
        }
        if (go && near != 0xFFFFFFFFu) atomicMin(&s_near[k], near);
        __syncthreads();
        const uint32_t lim = go ? s_near[k] : 0u;
        uint32_t part = 0;
#pragma unroll
        for (int j = 0; j < W; ++j) {
            const int64_t idx = top - j0 - (int64_t)j * kLanes;
            if (go && idx >= 0 && (uint32_t)(top - idx) <= lim) part += (uint32_t)e[j];
        }
        if (part) atomicAdd(&s_sum[k], part);
        __syncthreads();
        if (tid < NC && !s_done[tid] && (s_near[tid] != 0xFFFFFFFFu || top - kLanes * W < 0))
            s_done[tid] = 1u;
        __syncthreads();
        bool all = true;
        for (int q = 0; q < NC; ++q) all = all && s_done[q];
        if (all) break;
    }
}

// One read of the masks: digit histograms of every mask-sort pass, pairs per
// tap (mask column sums), and -- on the dense route, when no compaction
// follows (grid not null) -- the grid cells of the rows put back to empty
// (the lookups that needed them have finished).
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

// Rows [bid*kCChunk, +kCChunk) in row order, one per thread. For each tap
// (and for the slab rows, column kTaps) the block counts its rows, finds the
// count of earlier chunks by look-back and writes its pairs. The chunk's
// neighbour rows (contiguous in the table) are read once, coalesced, into
// LDS at the start; the chunk's pairs are first listed in LDS as (row, tap)
// entries in output order, then written out with consecutive threads on
// consecutive pair positions. The last chunk publishes the totals.
__global__ __launch_bounds__(kCThreads) void k_compact(
    const uint32_t* __restrict__ mask, const int32_t* __restrict__ nbr, int64_t n, int64_t cap,
    int tile_m, MapState* st, int32_t* __restrict__ pair_in, int32_t* __restrict__ pair_out,
    int32_t* __restrict__ pair_slot, int32_t* __restrict__ rowbase, uint64_t* __restrict__ look,
    uint32_t* ticket, uint32_t epoch, uint32_t* status, const int32_t* __restrict__ coords, Geom g,
    int32_t* __restrict__ grid) {
    constexpr int kCols = kTaps + 1;
    __shared__ uint32_t s_bid;
    __shared__ uint32_t s_wc[kCWaves][kCols];     // per-wave counts, then offsets in the chunk
    __shared__ uint32_t s_pre[kCols];             // counts of earlier chunks
    __shared__ uint32_t s_loc[kCols];             // chunk-local start of each tap's pairs
    __shared__ uint32_t s_tot[kCols];             // the chunk's own counts
    __shared__ uint32_t s_near[kCols], s_done[kCols];   // look-back scratch
    __shared__ int4 s_nb4[kCNbrVec];              // the chunk's neighbour rows [kCChunk][kTaps]
    __shared__ uint16_t s_list[kCChunk * kTaps];  // (row | tap << 8) in output order
    __shared__ uint32_t s_m[kCChunk], s_rb[kCChunk];
    const int32_t* s_nb = reinterpret_cast<const int32_t*>(s_nb4);
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    if (tid == 0) s_bid = atomicAdd(ticket, 1u);
    __syncthreads();
    const uint32_t bid = s_bid;
    const int64_t base0 = (int64_t)bid * kCChunk;
    const int64_t row = base0 + tid;
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));

    // loads: mask, neighbour rows (whole 16-byte words; the table is padded so the last
    // word of the last row is readable), coordinates for the grid cleanup
    const uint32_t mv = mask[row < n ? row : n - 1];
    int4 nv4[kCNbrPer];
    {
        const int4* src = reinterpret_cast<const int4*>(nbr + base0 * kTaps);
        const int64_t q_last = (n * kTaps + 3) / 4 - 1 - base0 * kTaps / 4;   // last readable word
#pragma unroll
        for (int j = 0; j < kCNbrPer; ++j) {
            const int64_t q = tid + j * kCThreads;
            nv4[j] = src[q < q_last ? q : q_last];
        }
    }
    int4 cq = make_int4(0, 0, 0, 0);              // (b, x, y, z) of the row
    if (grid) {
        const int32_t* c = coords + min(row, n - 1) * g.ncols;
        cq = g.ncols == 4 ? make_int4(c[0], c[1], c[2], c[3]) : make_int4(0, c[0], c[1], c[2]);
    }
    const uint32_t m = row < n ? mv : 0u;
    const uint32_t deg = m ? (uint32_t)__popc(m & ~(1u << kCentre)) : 0u;
    // per-wave count of each tap (lane k keeps tap k) and of slab rows (lane kTaps)
    uint32_t cnt = 0;
#pragma unroll
    for (int k = 0; k < kTaps; ++k) {
        const uint32_t c = (uint32_t)__popcll(__ballot((m >> k) & 1u));
        if (lane == k) cnt = c;
    }
    uint32_t incl = deg;                          // inclusive wave scan of the slab rows
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const uint32_t t = __shfl_up(incl, o, 64);
        if (lane >= o) incl += t;
    }
    const uint32_t wave_slab = __shfl(incl, 63, 64);
    if (lane < kTaps) s_wc[w][lane] = cnt;
    if (lane == kTaps) s_wc[w][kTaps] = wave_slab;
    s_m[tid] = m;
#pragma unroll
    for (int j = 0; j < kCNbrPer; ++j) {
        const int q = tid + j * kCThreads;
        if (q < kCNbrVec) s_nb4[q] = nv4[j];
    }
    __syncthreads();
    if (tid < kCols) {
        const int k = tid;
        uint32_t run = 0;
#pragma unroll
        for (int v = 0; v < kCWaves; ++v) {
            uint32_t c = s_wc[v][k];
            s_wc[v][k] = run;
            run += c;
        }
        s_tot[k] = run;                           // the chunk's own count, for now
        __hip_atomic_store(&look[(int64_t)bid * kCols + k],
                           lb_pack(epoch, bid == 0 ? kIncl : kAgg, run), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    }
    block_lookback<kCols, 8>(look, (int64_t)bid - 1, epoch, status, s_pre, s_near, s_done);
    if (tid < kCols) {
        const int k = tid;
        const uint32_t run = s_tot[k];
        const uint32_t prefix = s_pre[k];
        if (bid > 0)
            __hip_atomic_store(&look[(int64_t)bid * kCols + k], lb_pack(epoch, kIncl, prefix + run),
                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (bid == gridDim.x - 1) {
            // the last chunk: prefix + run is the total of column k
            const uint32_t tot = prefix + run;
            if (k < kTaps) {
                st->tap_count[k] = (int32_t)tot;
                st->tap_off[k] = (int32_t)(k * cap);
            } else {
                st->totals[3] = (int32_t)tot;             // slab rows = off-centre pairs
                st->tap_off[kTaps] = (int32_t)(kTaps * cap);
            }
        }
    }
    __syncthreads();
    if (tid == 0) {                               // chunk-local tap starts, totals
        uint32_t loc = 0;
        int32_t p = 0, padded = 0;
        for (int k = 0; k < kTaps; ++k) {
            s_loc[k] = loc;
            loc += s_tot[k];
            const int32_t c = (int32_t)(s_pre[k] + s_tot[k]);
            p += c;
            padded += (c + tile_m - 1) / tile_m * tile_m;
        }
        s_loc[kTaps] = loc;
        if (bid == gridDim.x - 1) {
            st->totals[0] = p;
            st->totals[1] = padded;
            st->totals[2] = padded / tile_m;
        }
    }
    // first slab row of the row
    const uint32_t rb = s_pre[kTaps] + s_wc[w][kTaps] + incl - deg;
    if (row < n) rowbase[row] = (int32_t)rb;
    s_rb[tid] = rb;
    __syncthreads();
    // list the chunk's pairs in output order: tap-major, rows ascending
#pragma unroll
    for (int k = 0; k < kTaps; ++k) {
        const uint64_t b = __ballot((m >> k) & 1u);
        if ((m >> k) & 1u)
            s_list[s_loc[k] + s_wc[w][k] + (uint32_t)__popcll(b & below)] =
                (uint16_t)(tid | (k << 8));
    }
    __syncthreads();
    // write them out: entry p of tap k goes to k cap + (pairs of k in earlier chunks) + its rank
    const int total = (int)s_loc[kTaps];
    for (int p = tid; p < total; p += kCThreads) {
        const uint32_t e = s_list[p];
        const int lr = (int)(e & 0xFFu), k = (int)(e >> 8);
        const int64_t pos = (int64_t)k * cap + s_pre[k] + (p - (int)s_loc[k]);
        if (pos >= (int64_t)k * cap + cap) continue;          // only after a stalled wait
        const uint32_t mr = s_m[lr];
        pair_in[pos] = k == kCentre ? (int32_t)(base0 + lr) : s_nb[lr * kTaps + k];
        pair_out[pos] = (int32_t)(base0 + lr);
        pair_slot[pos] = k == kCentre
                             ? -1
                             : (int32_t)(s_rb[lr] + __popc(mr & ((1u << k) - 1u) & ~(1u << kCentre)));
    }
    // dense route: the grid cell of this row goes back to empty (every lookup has finished)
    if (grid) {
        const int b = cq.x;
        const int x = cq.y - g.origin[0], y = cq.z - g.origin[1], z = cq.w - g.origin[2];
        if (row < n && (unsigned)b < (unsigned)g.batch && (unsigned)x < (unsigned)g.ext[0] &&
            (unsigned)y < (unsigned)g.ext[1] && (unsigned)z < (unsigned)g.ext[2])
            grid[b * g.sz_b + (int64_t)(x + 1) * g.sz_x + (int64_t)(y + 1) * g.sz_y + (z + 1)] = -1;
    }
    if (bid == gridDim.x - 1 && tid == 0) atomicExch(ticket, 0u);
}

}  // namespace

hipError_t launch_mask_hist(const uint32_t* mask, int64_t n, const SortPlan& plan, uint32_t* hist,
                            int32_t* tap_tot, const int32_t* coords, const Geom& g,
                            int32_t* grid, hipStream_t s) {
    unsigned blocks = (unsigned)((n + kHTile - 1) / kHTile);
    size_t lds = ((size_t)plan.passes * (1u << plan.bits) + kTaps) * 4;
    launch(k_mask_hist, blocks, kHThreads, lds, s, mask, n, plan.bits, plan.passes, hist, tap_tot,
                                               coords, g, grid);
    return hipGetLastError();
}

int64_t compact_chunks(int64_t n) { return (n + kCChunk - 1) / kCChunk; }

size_t compact_look_bytes(int64_t n) { return (size_t)compact_chunks(n) * (kTaps + 1) * 8; }

hipError_t launch_compact(const uint32_t* mask, const int32_t* nbr, int64_t n, int64_t cap,
                          int tile_m, MapState* st, int32_t* pair_in, int32_t* pair_out,
                          int32_t* pair_slot, int32_t* rowbase, SortWork& ws, uint32_t* status,
                          const int32_t* coords, const Geom& g, int32_t* grid, hipStream_t s) {
    uint32_t epoch = ++ws.epoch & 0x3FFFFFFFu;
    if (epoch == 0) epoch = ++ws.epoch & 0x3FFFFFFFu;
    unsigned blocks = (unsigned)compact_chunks(n);
    launch(k_compact, blocks, kCThreads, 0, s, mask, nbr, n, cap, tile_m, st, pair_in, pair_out,
                                           pair_slot, rowbase, ws.look, ws.ticket, epoch, status,
                                           coords, g, grid);
    return hipGetLastError();
}

}  // namespace smc
