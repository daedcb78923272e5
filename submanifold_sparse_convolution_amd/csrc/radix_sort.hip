// Stable LSD radix sort of (key, value) pairs: one kernel per digit pass.
//
// Used twice in the map build: on packed voxel keys in the sorted route
// (the sort the Z-Delta mapper needs; "[Kernel] Add submanifold sparse 3D
// convolution (bf16 implicit GEMM, gfx950)", section "Design, and the
// measurements behind it") and on neighbour masks to group rows with equal
// masks ("Sparse convolution in FP32", "Neighbour masks and sorted rows": a
// GPU radix sort orders the rows by mask).
//
// Design for small inputs (10^4 - 10^5 keys), where each kernel launch is a
// large share of the cost:
//  * the global digit histograms of every pass are counted in one read of
//    the keys, by the kernel that produces them (mask lookup, key packing)
//    or by k_key_hist;
//  * each pass is a single kernel: a block ranks its tile stably (each wave
//    owns a contiguous quarter of the tile and keeps per-digit running
//    counts in LDS, so no block barrier per item), publishes its digit
//    counts, adds up the counts of every tile before it (at most 64 tiles:
//    one or two round trips, all loads in flight; a chain of inclusive
//    prefixes, as in decoupled look-back, cost one round trip per few tiles:
//    Wide key sort 11.8 us per pass), then scatters.
// Sorts of many tiles take another route per pass (reduce, then scan): with
// thousands of digit columns a block would read through every earlier tile's
// counts (a look-back pass over 8 x 10^5 keys measured about 100 us). There, one kernel counts
// each tile's digits into a digit-major table, a two-level scan turns the
// table into global start positions, and a third kernel ranks and scatters
// exactly like the onesweep pass. No block waits for another.
// Wait safety: when the grid does not fit on the device at once, block
// indices are taken from a ticket counter in launch order, so a block only
// ever waits for blocks that already hold a ticket, i.e. are running. Each
// wait is also bounded; a wait that runs out flags the status word and the
// block carries on with in-bounds (wrong) output. Count entries carry an
// epoch, so stale entries from earlier passes are never taken for ready ones
// and the table needs no clearing.
#include "smc_internal.h"

namespace smc {
namespace {

constexpr int kOsThreads = 256;
constexpr int kOsWaves = kOsThreads / 64;
constexpr int kOsItems = 8;                     // keys per thread
constexpr int kOsTile = kOsThreads * kOsItems;  // 2048 keys per block
constexpr uint32_t kSpinLimit = 1u << 22;

__device__ inline uint64_t ld_acquire(const uint64_t* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline void st_release(uint64_t* p, uint64_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Tile counts, two digits per look-back entry: entry (tile, q) of thread t
// holds the tile's counts of digits t DPT + 2q and t DPT + 2q + 1 (16 bits
// each: a tile has at most 2048 keys) under the pass's epoch.
__device__ inline uint64_t agg_pack(uint32_t epoch, uint32_t c0, uint32_t c1) {
    return ((uint64_t)epoch << 34) | ((uint64_t)c1 << 16) | c0;
}

// prefix[j] = the count of digit d0 + j (d0 = t DPT) over tiles 0 .. tiles - 1,
// read from every one of those tiles' entries. A tile publishes its counts
// before it waits on anything, so with all tiles running these reads take one
// or two round trips, where a chain of inclusive prefixes would take one per
// few tiles.
template <int DPT>
__device__ inline void prefix_all(const uint64_t* look, int t, int64_t tiles, uint32_t epoch,
                                  uint32_t* status, uint32_t (&prefix)[DPT]) {
    constexpr int NW = (DPT + 1) / 2;
    constexpr int B = 32 / NW;                    // tiles per batch of loads
    const uint32_t ep = epoch & 0x3FFFFFFFu;
#pragma unroll
    for (int j = 0; j < DPT; ++j) prefix[j] = 0;
    uint32_t spins = 0;
    for (int64_t p0 = 0; p0 < tiles; p0 += B) {
        // (clamped, not branched: each branch around a load made the compiler wait for
        // the load before it, so the loads went out one or two at a time)
        uint64_t e[B][NW];
#pragma unroll
        for (int i = 0; i < B; ++i) {
            const int64_t pi = p0 + i < tiles ? p0 + i : tiles - 1;
#pragma unroll
            for (int q = 0; q < NW; ++q) e[i][q] = ld_acquire(&look[(pi * NW + q) * kOsThreads + t]);
        }
#pragma unroll
        for (int i = 0; i < B; ++i) {
            if (p0 + i >= tiles) break;
#pragma unroll
            for (int q = 0; q < NW; ++q) {
                while ((uint32_t)(e[i][q] >> 34) != ep) {
                    if (++spins > kSpinLimit) {
                        atomicOr(status, kStSortStall);
                        e[i][q] = 0;                       // give up: counts 0
                        break;
                    }
                    __builtin_amdgcn_s_sleep(1);
                    e[i][q] = ld_acquire(&look[((p0 + i) * NW + q) * kOsThreads + t]);
                }
                prefix[2 * q] += (uint32_t)e[i][q] & 0xFFFFu;
                if (2 * q + 1 < DPT) prefix[2 * q + 1] += (uint32_t)(e[i][q] >> 16) & 0xFFFFu;
            }
        }
    }
}

template <typename K, int BITS>
__global__ __launch_bounds__(kOsThreads) void k_os_pass(
    const K* __restrict__ kin, const uint32_t* __restrict__ vin, K* __restrict__ kout,
    uint32_t* __restrict__ vout, int64_t n, int shift, const uint32_t* __restrict__ hist,
    uint64_t* __restrict__ look, uint32_t* ticket, bool by_index, uint32_t epoch,
    uint32_t* status, K* __restrict__ split, int split_shift) {
    constexpr int BINS = 1 << BITS;
    constexpr int DPT = BINS / kOsThreads;      // digits per thread
    __shared__ uint32_t s_bid;
    __shared__ uint32_t s_wcnt[kOsWaves][BINS]; // per-wave counts, then per-wave offsets
    __shared__ uint32_t s_base[BINS];           // global start of this tile's run of each digit
    __shared__ uint32_t s_part[kOsThreads];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;

    // tile of this block: the block index when the grid fits on the device at
    // once (every block then runs whatever the dispatch order), else a ticket
    // taken on arrival, so every tile a block waits on is already running
    if (tid == 0 && !by_index) s_bid = atomicAdd(ticket, 1u);
#pragma unroll
    for (int j = 0; j < DPT; ++j)
#pragma unroll
        for (int v = 0; v < kOsWaves; ++v) s_wcnt[v][tid * DPT + j] = 0;
    __syncthreads();
    const uint32_t bid = by_index ? blockIdx.x : s_bid;
    const int64_t base = (int64_t)bid * kOsTile + (int64_t)w * (kOsTile / kOsWaves);
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));

    // stable rank within the wave's contiguous run
    K key[kOsItems];
    uint32_t val[kOsItems], rank[kOsItems], dig[kOsItems];
#pragma unroll
    for (int i = 0; i < kOsItems; ++i) {               // all loads in flight together
        int64_t idx = base + i * 64 + lane;
        const int64_t ic = idx < n ? idx : n - 1;          // clamped: loads never branch
        key[i] = kin[ic];
        val[i] = vin ? vin[ic] : (uint32_t)idx;
    }
#pragma unroll
    for (int i = 0; i < kOsItems; ++i) {
        int64_t idx = base + i * 64 + lane;
        bool valid = idx < n;
        uint32_t d = (uint32_t)(key[i] >> shift) & (BINS - 1);
        dig[i] = valid ? d : 0xFFFFFFFFu;
        uint64_t peers = __ballot(valid);
#pragma unroll
        for (int b = 0; b < BITS; ++b) {
            uint64_t bb = __ballot((d >> b) & 1u);
            peers &= ((d >> b) & 1u) ? bb : ~bb;
        }
        uint32_t before = valid ? s_wcnt[w][d] : 0u;
        rank[i] = before + (uint32_t)__popcll(peers & below);
        if (valid && (peers & below) == 0) s_wcnt[w][d] = before + (uint32_t)__popcll(peers);
        __builtin_amdgcn_wave_barrier();
    }
    __syncthreads();

    // per digit: wave offsets inside the tile, tile count (published)
    constexpr int NW = (DPT + 1) / 2;
    uint32_t tile_cnt[2 * NW];
#pragma unroll
    for (int j = 0; j < DPT; ++j) {
        int d = tid * DPT + j;
        uint32_t run = 0;
#pragma unroll
        for (int v = 0; v < kOsWaves; ++v) {
            uint32_t c = s_wcnt[v][d];
            s_wcnt[v][d] = run;
            run += c;
        }
        tile_cnt[j] = run;
    }
    if (DPT & 1) tile_cnt[DPT] = 0;
#pragma unroll
    for (int q = 0; q < NW; ++q)
        st_release(&look[((int64_t)bid * NW + q) * kOsThreads + tid],
                   agg_pack(epoch, tile_cnt[2 * q], tile_cnt[2 * q + 1]));

    // global start of each digit: exclusive scan of the pass histogram
    uint32_t hsum = 0, hv[DPT];
#pragma unroll
    for (int j = 0; j < DPT; ++j) {
        hv[j] = hist[tid * DPT + j];
        hsum += hv[j];
    }
    {
        uint32_t inc = hsum;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            uint32_t y = __shfl_up(inc, o);
            if (lane >= o) inc += y;
        }
        if (lane == 63) s_part[w] = inc;
        __syncthreads();
        uint32_t off = inc - hsum;
        for (int v = 0; v < w; ++v) off += s_part[v];
#pragma unroll
        for (int j = 0; j < DPT; ++j) {
            s_base[tid * DPT + j] = off;
            off += hv[j];
        }
    }

    // keys of each digit in the tiles before this one
    if (bid > 0) {
        uint32_t prefix[DPT];
        prefix_all<DPT>(look, tid, (int64_t)bid, epoch, status, prefix);
#pragma unroll
        for (int j = 0; j < DPT; ++j) s_base[tid * DPT + j] += prefix[j];
    }
    __syncthreads();

    // scatter
#pragma unroll
    for (int i = 0; i < kOsItems; ++i) {
        uint32_t d = dig[i];
        if (d == 0xFFFFFFFFu) continue;
        int64_t pos = (int64_t)s_base[d] + s_wcnt[w][d] + rank[i];
        if (pos >= n) pos = n - 1;               // only reachable after a stalled wait
        kout[pos] = key[i];
        vout[pos] = val[i];
        if (split && (pos & (((int64_t)1 << split_shift) - 1)) == 0) split[pos >> split_shift] = key[i];
    }
    if (!by_index && bid == gridDim.x - 1 && tid == 0) atomicExch(ticket, 0u);   // all tickets taken
}

constexpr int kManyTiles = 64;                  // above this many tiles: reduce, then scan
constexpr int kScanSeg = 4096;                  // scan segment (1024 threads x 4)

// Stable rank of this thread's kOsItems keys inside its wave's contiguous
// quarter of the tile, the wave's per-digit counts in s_wcnt (shared by the
// onesweep and the scatter kernels).
template <typename K, int BITS>
__device__ __forceinline__ void rank_tile(const K* __restrict__ kin, const uint32_t* __restrict__ vin,
                                          int64_t n, int shift, int64_t base, K (&key)[kOsItems],
                                          uint32_t (&val)[kOsItems], uint32_t (&rank)[kOsItems],
                                          uint32_t (&dig)[kOsItems],
                                          uint32_t (*s_wcnt)[1 << BITS]) {
    constexpr int BINS = 1 << BITS;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
#pragma unroll
    for (int i = 0; i < kOsItems; ++i) {
        const int64_t idx = base + i * 64 + lane;
        const int64_t ic = idx < n ? idx : n - 1;
        key[i] = kin[ic];
        val[i] = vin ? vin[ic] : (uint32_t)idx;
    }
#pragma unroll
    for (int i = 0; i < kOsItems; ++i) {
        const int64_t idx = base + i * 64 + lane;
        const bool valid = idx < n;
        const uint32_t d = (uint32_t)(key[i] >> shift) & (BINS - 1);
        dig[i] = valid ? d : 0xFFFFFFFFu;
        uint64_t peers = __ballot(valid);
#pragma unroll
        for (int b = 0; b < BITS; ++b) {
            const uint64_t bb = __ballot((d >> b) & 1u);
            peers &= ((d >> b) & 1u) ? bb : ~bb;
        }
        const uint32_t before = valid ? s_wcnt[w][d] : 0u;
        rank[i] = before + (uint32_t)__popcll(peers & below);
        if (valid && (peers & below) == 0) s_wcnt[w][d] = before + (uint32_t)__popcll(peers);
        __builtin_amdgcn_wave_barrier();
    }
}

// Reduce: digit counts of tile blockIdx.x into cnt[d * tiles + tile].
template <typename K, int BITS>
__global__ __launch_bounds__(kOsThreads) void k_rs_count(const K* __restrict__ kin, int64_t n,
                                                         int shift, uint32_t* __restrict__ cnt,
                                                         int64_t tiles) {
    constexpr int BINS = 1 << BITS;
    __shared__ uint32_t s_h[BINS];
    for (int d = threadIdx.x; d < BINS; d += kOsThreads) s_h[d] = 0;
    __syncthreads();
    const int64_t base = (int64_t)blockIdx.x * kOsTile;
#pragma unroll
    for (int i = 0; i < kOsItems; ++i) {
        const int64_t idx = base + i * kOsThreads + threadIdx.x;
        if (idx < n) atomicAdd(&s_h[(uint32_t)(kin[idx] >> shift) & (BINS - 1)], 1u);
    }
    __syncthreads();
    for (int d = threadIdx.x; d < BINS; d += kOsThreads) cnt[(int64_t)d * tiles + blockIdx.x] = s_h[d];
}

// Exclusive scan of segments of kScanSeg words in place; seg[blockIdx.x] = the
// segment's total.
__global__ __launch_bounds__(1024) void k_scan_segments(uint32_t* __restrict__ a, int64_t len,
                                                        uint32_t* __restrict__ seg) {
    __shared__ uint32_t s_w[16];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int64_t base = (int64_t)blockIdx.x * kScanSeg + (int64_t)threadIdx.x * 4;
    uint32_t v[4], t = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        v[j] = base + j < len ? a[base + j] : 0u;
        t += v[j];
    }
    uint32_t inc = t;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const uint32_t u = __shfl_up(inc, o);
        if (lane >= o) inc += u;
    }
    if (lane == 63) s_w[w] = inc;
    __syncthreads();
    uint32_t run = inc - t;
    for (int q = 0; q < w; ++q) run += s_w[q];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        if (base + j < len) a[base + j] = run;
        run += v[j];
    }
    if (threadIdx.x == 1023) seg[blockIdx.x] = run;
}

// Exclusive scan of the segment totals in place (one block, any length).
__global__ __launch_bounds__(1024) void k_scan_top(uint32_t* __restrict__ a, int64_t len) {
    __shared__ uint32_t s_w[16];
    __shared__ uint32_t s_carry;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    if (threadIdx.x == 0) s_carry = 0;
    __syncthreads();
    for (int64_t c0 = 0; c0 < len; c0 += 1024) {
        const int64_t i = c0 + threadIdx.x;
        const uint32_t v = i < len ? a[i] : 0u;
        uint32_t inc = v;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const uint32_t u = __shfl_up(inc, o);
            if (lane >= o) inc += u;
        }
        if (lane == 63) s_w[w] = inc;
        __syncthreads();
        uint32_t before = s_carry;
        for (int q = 0; q < w; ++q) before += s_w[q];
        if (i < len) a[i] = before + inc - v;
        __syncthreads();
        if (threadIdx.x == 1023) s_carry = before + inc;
        __syncthreads();
    }
}

// Scatter: rank the tile as the onesweep pass does; each digit's run of the
// tile starts at the scanned count table entry (plus its segment's prefix).
template <typename K, int BITS>
__global__ __launch_bounds__(kOsThreads) void k_rs_scatter(
    const K* __restrict__ kin, const uint32_t* __restrict__ vin, K* __restrict__ kout,
    uint32_t* __restrict__ vout, int64_t n, int shift, const uint32_t* __restrict__ cnt,
    const uint32_t* __restrict__ seg, int64_t tiles, K* __restrict__ split, int split_shift) {
    constexpr int BINS = 1 << BITS;
    constexpr int DPT = BINS / kOsThreads;
    __shared__ uint32_t s_wcnt[kOsWaves][BINS];
    __shared__ uint32_t s_base[BINS];
    const int tid = threadIdx.x, w = tid >> 6;
#pragma unroll
    for (int j = 0; j < DPT; ++j)
#pragma unroll
        for (int v = 0; v < kOsWaves; ++v) s_wcnt[v][tid * DPT + j] = 0;
    __syncthreads();
    const int64_t bid = blockIdx.x;
    const int64_t base = bid * kOsTile + (int64_t)w * (kOsTile / kOsWaves);
    K key[kOsItems];
    uint32_t val[kOsItems], rank[kOsItems], dig[kOsItems];
    rank_tile<K, BITS>(kin, vin, n, shift, base, key, val, rank, dig, s_wcnt);
    __syncthreads();
#pragma unroll
    for (int j = 0; j < DPT; ++j) {
        const int d = tid * DPT + j;
        uint32_t run = 0;
#pragma unroll
        for (int v = 0; v < kOsWaves; ++v) {
            const uint32_t c = s_wcnt[v][d];
            s_wcnt[v][d] = run;
            run += c;
        }
        const int64_t e = (int64_t)d * tiles + bid;
        s_base[d] = cnt[e] + seg[e / kScanSeg];
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kOsItems; ++i) {
        const uint32_t d = dig[i];
        if (d == 0xFFFFFFFFu) continue;
        int64_t pos = (int64_t)s_base[d] + s_wcnt[w][d] + rank[i];
        if (pos >= n) pos = n - 1;
        kout[pos] = key[i];
        vout[pos] = val[i];
        if (split && (pos & (((int64_t)1 << split_shift) - 1)) == 0) split[pos >> split_shift] = key[i];
    }
}

template <typename K, int BITS>
hipError_t launch_rs_pass(const K* kin, const uint32_t* vin, K* kout, uint32_t* vout, int64_t n,
                          int shift, uint32_t* cnt, K* split, int split_shift, hipStream_t s) {
    const int64_t tiles = (n + kOsTile - 1) / kOsTile;
    const int64_t len = tiles * (1 << BITS);
    const int64_t nseg = (len + kScanSeg - 1) / kScanSeg;
    uint32_t* seg = cnt + len;
    launch(k_rs_count<K, BITS>, (unsigned)tiles, kOsThreads, 0, s, kin, n, shift, cnt, tiles);
    launch(k_scan_segments, (unsigned)nseg, 1024, 0, s, cnt, len, seg);
    launch(k_scan_top, 1u, 1024, 0, s, seg, nseg);
    launch(k_rs_scatter<K, BITS>, (unsigned)tiles, kOsThreads, 0, s, kin, vin, kout, vout, n, shift,
           (const uint32_t*)cnt, (const uint32_t*)seg, tiles, split, split_shift);
    return hipGetLastError();
}

// Global digit histograms of every pass in one read of the keys.
template <typename K>
__global__ __launch_bounds__(kOsThreads) void k_key_hist(const K* __restrict__ keys, int64_t n,
                                                         int bits, int passes,
                                                         uint32_t* __restrict__ hist) {
    extern __shared__ uint32_t s_h[];            // passes << bits counters
    const int bins = 1 << bits;
    for (int i = threadIdx.x; i < passes * bins; i += kOsThreads) s_h[i] = 0;
    __syncthreads();
    int64_t base = (int64_t)blockIdx.x * kOsTile;
    for (int i = 0; i < kOsItems; ++i) {
        int64_t idx = base + i * kOsThreads + threadIdx.x;
        if (idx < n) {
            K k = keys[idx];
            for (int p = 0; p < passes; ++p)
                atomicAdd(&s_h[p * bins + ((uint32_t)(k >> (p * bits)) & (bins - 1))], 1u);
        }
    }
    __syncthreads();
    for (int i = threadIdx.x; i < passes * bins; i += kOsThreads)
        if (s_h[i]) atomicAdd(&hist[i], s_h[i]);
}

// Whether `blocks` blocks of k_os_pass<K, BITS> fit on the current device at
// once (occupancy per CU times CUs, queried once per instance and device).
template <typename K, int BITS>
bool pass_fits(unsigned blocks) {
    constexpr int kDevs = 64;
    static int64_t cap[kDevs] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kDevs) return false;
    if (cap[dev] == 0) {
        int per_cu = 0, n_cu = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k_os_pass<K, BITS>, kOsThreads,
                                                         0) != hipSuccess ||
            hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
            return false;
        cap[dev] = (int64_t)per_cu * n_cu > 0 ? (int64_t)per_cu * n_cu : -1;
    }
    return (int64_t)blocks <= cap[dev];
}

template <typename K, int BITS>
hipError_t launch_pass(const K* kin, const uint32_t* vin, K* kout, uint32_t* vout, int64_t n,
                       int shift, const uint32_t* hist, uint64_t* look, uint32_t* ticket,
                       uint32_t epoch, uint32_t* status, K* split, int split_shift, hipStream_t s) {
    unsigned blocks = (unsigned)((n + kOsTile - 1) / kOsTile);
    const bool by_index = pass_fits<K, BITS>(blocks);
    launch(k_os_pass<K, BITS>, blocks, kOsThreads, 0, s, kin, vin, kout, vout, n, shift, hist, look,
           ticket, by_index, epoch, status, split, split_shift);
    return hipGetLastError();
}

template <typename K>
hipError_t sort_impl(const K* keys_in, const uint32_t* vals_in, int64_t n, const SortPlan& plan,
                     const uint32_t* hist, K* kbuf0, K* kbuf1, uint32_t* vbuf0, uint32_t* vbuf1,
                     SortWork& ws, uint32_t* status, const K** keys_out,
                     const uint32_t** vals_out, K* split, int split_shift, hipStream_t s) {
    const K* kcur = keys_in;
    const uint32_t* vcur = vals_in;
    K* kdst[2] = {kbuf0, kbuf1};
    uint32_t* vdst[2] = {vbuf0, vbuf1};
    const int bins = 1 << plan.bits;
    for (int p = 0; p < plan.passes; ++p) {
        uint32_t epoch = ++ws.epoch & 0x3FFFFFFFu;
        if (epoch == 0) epoch = ++ws.epoch & 0x3FFFFFFFu;
        const uint32_t* h = hist + (size_t)p * bins;
        hipError_t e;
        const int64_t tiles = (n + kOsTile - 1) / kOsTile;
        K* sp = p == plan.passes - 1 ? split : nullptr;           // the last pass lists splitters
        if (tiles > kManyTiles && ws.cnt && ws.cnt_ints >= sort_scan_ints(n)) {
            switch (plan.bits) {
                case 8: e = launch_rs_pass<K, 8>(kcur, vcur, kdst[p & 1], vdst[p & 1], n, p * 8, ws.cnt, sp, split_shift, s); break;
                case 9: e = launch_rs_pass<K, 9>(kcur, vcur, kdst[p & 1], vdst[p & 1], n, p * 9, ws.cnt, sp, split_shift, s); break;
                case 10: e = launch_rs_pass<K, 10>(kcur, vcur, kdst[p & 1], vdst[p & 1], n, p * 10, ws.cnt, sp, split_shift, s); break;
                default: e = launch_rs_pass<K, 11>(kcur, vcur, kdst[p & 1], vdst[p & 1], n, p * 11, ws.cnt, sp, split_shift, s); break;
            }
            if (e != hipSuccess) return e;
            kcur = kdst[p & 1];
            vcur = vdst[p & 1];
            continue;
        }
        switch (plan.bits) {
            case 8: e = launch_pass<K, 8>(kcur, vcur, kdst[p & 1], vdst[p & 1], n, p * 8, h, ws.look, ws.ticket, epoch, status, sp, split_shift, s); break;
            case 9: e = launch_pass<K, 9>(kcur, vcur, kdst[p & 1], vdst[p & 1], n, p * 9, h, ws.look, ws.ticket, epoch, status, sp, split_shift, s); break;
            case 10: e = launch_pass<K, 10>(kcur, vcur, kdst[p & 1], vdst[p & 1], n, p * 10, h, ws.look, ws.ticket, epoch, status, sp, split_shift, s); break;
            default: e = launch_pass<K, 11>(kcur, vcur, kdst[p & 1], vdst[p & 1], n, p * 11, h, ws.look, ws.ticket, epoch, status, sp, split_shift, s); break;
        }
        if (e != hipSuccess) return e;
        kcur = kdst[p & 1];
        vcur = vdst[p & 1];
    }
    *keys_out = kcur;
    *vals_out = vcur;
    return hipSuccess;
}

}  // namespace

SortPlan sort_plan(int key_bits, int max_bits) {
    SortPlan p;
    if (key_bits < 1) key_bits = 1;
    p.passes = (key_bits + max_bits - 1) / max_bits;
    int b = (key_bits + p.passes - 1) / p.passes;
    p.bits = b < 8 ? 8 : b;
    return p;
}

// Coordinate keys: at most 9-bit digits while the passes are single kernels
// (a thread reads 2^bits / 512 count entries per earlier tile, so wider
// digits cost more reads per pass than the pass they save), 11 otherwise.
SortPlan key_sort_plan(int key_bits, int64_t n) {
    return sort_plan(key_bits, sort_tiles(n) <= kManyTiles ? 9 : 11);
}

int64_t sort_tiles(int64_t n) { return (n + kOsTile - 1) / kOsTile; }

int64_t sort_scan_ints(int64_t n) {
    const int64_t tiles = sort_tiles(n);
    if (tiles <= kManyTiles) return 0;
    const int64_t len = tiles * 2048;              // the widest digit (11 bits)
    return len + (len + kScanSeg - 1) / kScanSeg;
}

size_t sort_look_bytes(int64_t n) {
    int64_t t = sort_tiles(n);
    return (size_t)(t < 1 ? 1 : t) * 2048 * sizeof(uint64_t);
}

hipError_t launch_key_hist(const void* keys, bool wide, int64_t n, const SortPlan& plan,
                           uint32_t* hist, hipStream_t s) {
    unsigned blocks = (unsigned)((n + kOsTile - 1) / kOsTile);
    size_t lds = (size_t)plan.passes * (1u << plan.bits) * 4;
    if (wide)
        launch(k_key_hist<uint64_t>, blocks, kOsThreads, lds, s, (const uint64_t*)keys, n, plan.bits,
                                                             plan.passes, hist);
    else
        launch(k_key_hist<uint32_t>, blocks, kOsThreads, lds, s, (const uint32_t*)keys, n, plan.bits,
                                                             plan.passes, hist);
    return hipGetLastError();
}

hipError_t radix_sort_u32(const uint32_t* keys_in, const uint32_t* vals_in, int64_t n,
                          const SortPlan& plan, const uint32_t* hist, uint32_t* kbuf0,
                          uint32_t* kbuf1, uint32_t* vbuf0, uint32_t* vbuf1, SortWork& ws,
                          uint32_t* status, const uint32_t** keys_out, const uint32_t** vals_out,
                          hipStream_t s, void* split, int split_shift) {
    return sort_impl<uint32_t>(keys_in, vals_in, n, plan, hist, kbuf0, kbuf1, vbuf0, vbuf1, ws,
                               status, keys_out, vals_out, (uint32_t*)split, split_shift, s);
}

hipError_t radix_sort_u64(const uint64_t* keys_in, const uint32_t* vals_in, int64_t n,
                          const SortPlan& plan, const uint32_t* hist, uint64_t* kbuf0,
                          uint64_t* kbuf1, uint32_t* vbuf0, uint32_t* vbuf1, SortWork& ws,
                          uint32_t* status, const uint64_t** keys_out, const uint32_t** vals_out,
                          hipStream_t s, void* split, int split_shift) {
    return sort_impl<uint64_t>(keys_in, vals_in, n, plan, hist, kbuf0, kbuf1, vbuf0, vbuf1, ws,
                               status, keys_out, vals_out, (uint64_t*)split, split_shift, s);
}

}  // namespace smc
