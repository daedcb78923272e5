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
constexpr int kCItems = 2;
constexpr int kCChunk = kCThreads * kCItems;      // rows per compaction block
constexpr int kCNbrVec = kCChunk * kTaps / 4;     // 16-byte words of the chunk's neighbour rows
constexpr int kCNbrPer = (kCNbrVec + kCThreads - 1) / kCThreads;
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

// Rows [bid*kCChunk, +kCChunk) in row order. Wave w owns a contiguous
// quarter; for each tap (and for the slab rows, column kTaps) the block
// counts its rows, finds the count of earlier chunks by look-back, and
// writes its pairs. The chunk's neighbour rows (contiguous in the table) are
// read once, coalesced, into LDS at the start, so the pair writes read LDS
// only. The last chunk publishes the totals.
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
    __shared__ uint32_t s_tot[kCols];             // totals (last chunk only)
    __shared__ int4 s_nb4[kCNbrVec];              // the chunk's neighbour rows [kCChunk][kTaps]
    const int32_t* s_nb = reinterpret_cast<const int32_t*>(s_nb4);
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    if (tid == 0) s_bid = atomicAdd(ticket, 1u);
    __syncthreads();
    const uint32_t bid = s_bid;
    const int64_t base0 = (int64_t)bid * kCChunk;
    const int64_t base = base0 + (int64_t)w * (kCChunk / kCWaves);
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));

    // loads: masks, neighbour rows (whole 16-byte words; the table is padded so the last
    // word of the last row is readable), coordinates for the grid cleanup
    uint32_t m[kCItems], deg[kCItems];
#pragma unroll
    for (int i = 0; i < kCItems; ++i) {
        const int64_t r = base + i * 64 + lane;
        const uint32_t mv = mask[r < n ? r : n - 1];
        m[i] = r < n ? mv : 0u;
    }
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
    int4 cq[kCItems];                             // (b, x, y, z) of the rows
    if (grid) {
#pragma unroll
        for (int i = 0; i < kCItems; ++i) {
            const int32_t* c = coords + min(base + i * 64 + lane, n - 1) * g.ncols;
            cq[i] = g.ncols == 4 ? make_int4(c[0], c[1], c[2], c[3]) : make_int4(0, c[0], c[1], c[2]);
        }
    }
#pragma unroll
    for (int i = 0; i < kCItems; ++i) deg[i] = m[i] ? (uint32_t)__popc(m[i] & ~(1u << kCentre)) : 0u;
    // per-wave count of each tap (lane k accumulates tap k) and of slab rows (lane kTaps)
    uint32_t cnt = 0;
#pragma unroll
    for (int k = 0; k < kTaps; ++k) {
        uint32_t c = 0;
#pragma unroll
        for (int i = 0; i < kCItems; ++i) c += (uint32_t)__popcll(__ballot((m[i] >> k) & 1u));
        if (lane == k) cnt = c;
    }
    // inclusive wave scans of the slab rows per item
    uint32_t incl[kCItems], item_tot[kCItems];
#pragma unroll
    for (int i = 0; i < kCItems; ++i) {
        uint32_t v = deg[i];
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const uint32_t t = __shfl_up(v, o, 64);
            if (lane >= o) v += t;
        }
        incl[i] = v;
        item_tot[i] = __shfl(v, 63, 64);
    }
    uint32_t wave_slab = 0;
#pragma unroll
    for (int i = 0; i < kCItems; ++i) wave_slab += item_tot[i];
    if (lane < kTaps) s_wc[w][lane] = cnt;
    if (lane == kTaps) s_wc[w][kTaps] = wave_slab;
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
        __hip_atomic_store(&look[(int64_t)bid * kCols + k],
                           lb_pack(epoch, bid == 0 ? kIncl : kAgg, run), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
        uint32_t prefix = 0;
        if (bid > 0) {
            prefix = lookback8(look, kCols, k, (int64_t)bid - 1, epoch, status);
            __hip_atomic_store(&look[(int64_t)bid * kCols + k], lb_pack(epoch, kIncl, prefix + run),
                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        s_pre[k] = prefix;
        if (bid == gridDim.x - 1) {
            // the last chunk: prefix + run is the total of column k
            const uint32_t tot = prefix + run;
            s_tot[k] = tot;
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
    if (bid == gridDim.x - 1 && tid == 0) {
        int32_t p = 0, padded = 0;
        for (int k = 0; k < kTaps; ++k) {
            const int32_t c = (int32_t)s_tot[k];
            p += c;
            padded += (c + tile_m - 1) / tile_m * tile_m;
        }
        st->totals[0] = p;
        st->totals[1] = padded;
        st->totals[2] = padded / tile_m;
    }
    // first slab row of every row
    uint32_t rb[kCItems];
    {
        uint32_t off = s_pre[kTaps] + s_wc[w][kTaps];
#pragma unroll
        for (int i = 0; i < kCItems; ++i) {
            rb[i] = off + incl[i] - deg[i];
            off += item_tot[i];
            const int64_t r = base + i * 64 + lane;
            if (r < n) rowbase[r] = (int32_t)rb[i];
        }
    }
    // pairs, tap by tap (the centre's input row is the row itself)
#pragma unroll
    for (int k = 0; k < kTaps; ++k) {
        const int64_t start = (int64_t)k * cap + s_pre[k] + s_wc[w][k];
        const int64_t lim = (int64_t)k * cap + cap;
        const uint32_t lower = (1u << k) - 1u;
        uint32_t run = 0;
#pragma unroll
        for (int i = 0; i < kCItems; ++i) {
            const uint64_t b = __ballot((m[i] >> k) & 1u);
            const int lr = w * (kCChunk / kCWaves) + i * 64 + lane;   // row within the chunk
            if ((m[i] >> k) & 1u) {
                const int64_t pos = start + run + (uint32_t)__popcll(b & below);
                if (pos < lim) {                   // false only after a stalled wait
                    pair_in[pos] = k == kCentre ? (int32_t)(base0 + lr) : s_nb[lr * kTaps + k];
                    pair_out[pos] = (int32_t)(base0 + lr);
                    pair_slot[pos] = k == kCentre
                                         ? -1
                                         : (int32_t)(rb[i] + __popc(m[i] & lower & ~(1u << kCentre)));
                }
            }
            run += (uint32_t)__popcll(b);
        }
    }
    // dense route: the grid cells of these rows go back to empty (every lookup has finished)
    if (grid) {
#pragma unroll
        for (int i = 0; i < kCItems; ++i) {
            const int64_t r = base + i * 64 + lane;
            const int b = cq[i].x;
            const int x = cq[i].y - g.origin[0], y = cq[i].z - g.origin[1], z = cq[i].w - g.origin[2];
            if (r < n && (unsigned)b < (unsigned)g.batch && (unsigned)x < (unsigned)g.ext[0] &&
                (unsigned)y < (unsigned)g.ext[1] && (unsigned)z < (unsigned)g.ext[2])
                grid[b * g.sz_b + (int64_t)(x + 1) * g.sz_x + (int64_t)(y + 1) * g.sz_y + (z + 1)] = -1;
        }
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
