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
#include <atomic>

#include "lookback.h"
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
// Exclusive prefix over the wave's lanes of a value below 2^B, from one
// ballot per bit plane: the count of lower lanes with bit b set, times 2^b.
// The wave total comes back in *total.
template <int B>
__device__ __forceinline__ uint32_t wave_excl_scan(uint32_t v, uint32_t* total) {
    uint32_t excl = 0, tot = 0;
#pragma unroll
    for (int b = 0; b < B; ++b) {
        const uint64_t m = __ballot((v >> b) & 1u);
        excl += __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                          __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u)) << b;
        tot += (uint32_t)__popcll(m) << b;
    }
    *total = tot;
    return excl;
}

// OR of v over the wave's lanes (the same value in every lane).
__device__ __forceinline__ uint32_t wave_or(uint32_t v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v |= __shfl_xor(v, o, 64);
    return (uint32_t)__builtin_amdgcn_readfirstlane((int)v);   // uniform: kept in a scalar register
}

// Count of lower lanes of the wave whose bit is set in m.
__device__ __forceinline__ uint32_t lanes_below(uint64_t m) {
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// One read of the masks: digit histograms of every mask-sort pass and pairs
// per tap (mask column sums). With a calibrated order or offset groups
// ("Sparse convolution in FP32" (DriveRT), sections "Calibrated bit order" and
// "Offset-group partitioning") the sort keys are not the masks: each row gets
// one key per group, its group taps moved to their bits in that group's key,
// the group index above them and, for a row without a tap of the group, a
// bit that sends it behind every row that has one. The keys are written out
// here and histogrammed instead, and rows with a tap per group are counted.
__global__ __launch_bounds__(kHThreads) void k_mask_hist(const uint32_t* __restrict__ mask,
                                                         int64_t n, int bits, int passes,
                                                         MaskOrder ord, uint32_t* __restrict__ keys,
                                                         uint32_t* __restrict__ hist,
                                                         int32_t* __restrict__ tap_tot,
                                                         int32_t* __restrict__ group_rows) {
    extern __shared__ uint32_t s_h[];             // passes << bits, 27 tap and 4 group counters
    const int bins = 1 << bits;
    uint32_t* s_tap = s_h + passes * bins;
    uint32_t* s_grp = s_tap + kTaps;
    for (int i = threadIdx.x; i < passes * bins + kTaps + kMaxGroups; i += kHThreads) s_h[i] = 0;
    __syncthreads();
    const int lane = threadIdx.x & 63;
    const int G = ord.n_groups, B = ord.group_bits;
    const int gshift = G > 1 ? B + 1 : 0;
    int64_t base = (int64_t)blockIdx.x * kHTile;
    uint32_t tap_acc = 0;                          // lane k < 27 keeps tap k's wave count
    uint32_t grp_acc = 0;                          // lane g < G keeps group g's wave count
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
        if (ord.plain) {
            if (idx < n) {
                for (int p = 0; p < passes; ++p)
                    atomicAdd(&s_h[p * bins + ((m >> (p * bits)) & (bins - 1))], 1u);
            }
        } else {
            uint32_t kg[kMaxGroups] = {0u, 0u, 0u, 0u};
#pragma unroll
            for (int t = 0; t < kTaps; ++t) {
                const uint32_t b = ((m >> t) & 1u) << ord.pos[t];
#pragma unroll
                for (int g = 0; g < kMaxGroups; ++g) kg[g] |= ord.grp[t] == g ? b : 0u;
            }
#pragma unroll
            for (int g = 0; g < kMaxGroups; ++g) {
                if (g >= G) break;
                const uint32_t key = ((uint32_t)g << gshift) | (kg[g] ? kg[g] : 1u << B);
                if (idx < n) {
                    keys[g * n + idx] = key;
                    for (int p = 0; p < passes; ++p)
                        atomicAdd(&s_h[p * bins + ((key >> (p * bits)) & (bins - 1))], 1u);
                }
                const uint32_t c = (uint32_t)__popcll(__ballot(idx < n && kg[g] != 0u));
                if (lane == g) grp_acc += c;
            }
        }
#pragma unroll
        for (int k = 0; k < kTaps; ++k) {
            uint32_t c = (uint32_t)__popcll(__ballot((m >> k) & 1u));
            if (lane == k) tap_acc += c;
        }
    }
    if (lane < kTaps && tap_acc) atomicAdd(&s_tap[lane], tap_acc);
    if (lane < kMaxGroups && grp_acc) atomicAdd(&s_grp[lane], grp_acc);
    __syncthreads();
    for (int i = threadIdx.x; i < passes * bins; i += kHThreads)
        if (s_h[i]) atomicAdd(&hist[i], s_h[i]);
    if (threadIdx.x < kTaps && s_tap[threadIdx.x]) atomicAdd(&tap_tot[threadIdx.x], (int32_t)s_tap[threadIdx.x]);
    if (threadIdx.x < kMaxGroups && s_grp[threadIdx.x])
        atomicAdd(&group_rows[threadIdx.x], (int32_t)s_grp[threadIdx.x]);
}

// Chunk of this block. A chunk waits only on lower chunks. When the whole
// grid fits on the device at once (by_index), every block gets dispatched
// whatever the order, so the chunk is the block index; otherwise a ticket
// taken on arrival orders the chunks by dispatch, so every chunk a block waits
// on belongs to a block that is already running. The ticket is reset by the
// last chunk's block.
__device__ __forceinline__ uint32_t chunk_of_block(bool by_index, uint32_t* ticket,
                                                   uint32_t* s_slot) {
    if (by_index) return blockIdx.x;
    if (threadIdx.x == 0) *s_slot = atomicAdd(ticket, 1u);
    __syncthreads();
    return *s_slot;
}

// LDS of one compaction chunk.
struct CompactLds {
    uint32_t bid;
    uint32_t wc[kCWaves][kTaps + 1];              // per-wave counts, then offsets in the chunk
    uint32_t pre[kTaps + 1];                      // counts of earlier chunks
    uint32_t loc[kTaps + 1];                      // chunk-local start of each tap's pairs
    uint32_t tot[kTaps + 1];                      // the chunk's own counts
    uint32_t done[kTaps + 1];                     // look-back scratch
    int32_t nb[kCChunk * kTaps];                  // the chunk's neighbour rows
    uint16_t list[kCChunk * kTaps];               // (row | tap << 8) in output order
    uint32_t m[kCChunk], rb[kCChunk];
};

// Everything of a chunk after its masks are known (m: this thread's row;
// L.nb filled): per-tap counts, look-back over earlier chunks, the chunk's
// pairs listed in LDS as (row, tap) entries in output order, then written out
// with consecutive threads on consecutive pair positions. The last chunk
// publishes the totals. chunk_pre[bid][k] receives the pairs of tap k (k <
// kTaps) and the slab rows (k = kTaps) in earlier chunks. dense_centre: the
// centre tap pairs every row with itself and gets no slab rows (submanifold
// maps); otherwise it is a tap like the others (strided maps), and the only
// pair of a row gets pair_slot -2 - row instead of a slab row: its product is
// the row's output. With nbr_out, the chunk's neighbour rows are stored
// there (coalesced) between publishing the counts and the look-back, where
// the block would otherwise wait. Starts and ends with all threads in step.
__device__ __forceinline__ void compact_chunk(CompactLds& L, uint32_t m, uint32_t bid, uint32_t last, int64_t n,
                                              int64_t cap, int tile_m, MapState* st,
                                              int32_t* __restrict__ pair_in,
                                              int32_t* __restrict__ pair_out,
                                              int32_t* __restrict__ pair_slot,
                                              int32_t* __restrict__ rowbase,
                                              int32_t* __restrict__ chunk_pre,
                                              uint64_t* __restrict__ look, uint32_t epoch,
                                              uint32_t* status, int32_t* __restrict__ nbr_out,
                                              bool dense_centre = true,
                                              uint32_t spin_limit = kSpinLimit,
                                              uint32_t wait_xor = 0u) {
    constexpr int kCols = kTaps + 1;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int64_t base0 = (int64_t)bid * kCChunk;
    const int64_t row = base0 + tid;
    // slab rows of the row: its off-centre pairs, or with a sparse centre (a
    // strided map, whose output o need not be an input) every pair of a row
    // with two or more; a row with one pair has none (the GEMM writes its
    // output directly)
    const uint32_t slab_taps = dense_centre ? ~(1u << kCentre) : ~0u;
    const uint32_t pop = (uint32_t)__popc(m & slab_taps);
    const uint32_t deg = dense_centre || pop > 1u ? pop : 0u;
    // per-wave count of each tap (lane k keeps tap k) and of slab rows (lane kTaps),
    // over the taps some row of the wave has (the wave's OR of masks)
    const uint32_t uni = wave_or(m);
    uint32_t cnt = 0;
    for (uint32_t u = uni; u; u &= u - 1) {
        const int k = __builtin_ctz(u);
        const uint32_t c = (uint32_t)__popcll(__ballot((m >> k) & 1u));
        if (lane == k) cnt = c;
    }
    uint32_t wave_slab;                           // slab rows of the wave's earlier rows
    const uint32_t excl = wave_excl_scan<5>(deg, &wave_slab);
    if (lane < kTaps) L.wc[w][lane] = cnt;
    if (lane == kTaps) L.wc[w][kTaps] = wave_slab;
    L.m[tid] = m;
    __syncthreads();
    if (tid < kCols) {
        const int k = tid;
        uint32_t run = 0;
#pragma unroll
        for (int v = 0; v < kCWaves; ++v) {
            uint32_t c = L.wc[v][k];
            L.wc[v][k] = run;
            run += c;
        }
        L.tot[k] = run;
        __hip_atomic_store(&look[(int64_t)bid * kCols + k],
                           lb_pack(epoch, bid == 0 ? kIncl : kAgg, run), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    }
    if (nbr_out) {                                // neighbour rows out, coalesced
        const int4* nb4 = reinterpret_cast<const int4*>(L.nb);
        int4* dst = reinterpret_cast<int4*>(nbr_out + base0 * kTaps);
        const int64_t q_end = ((n - base0) * kTaps + 3) / 4;      // words holding rows < n
        int4 t4[kCNbrPer];                        // all LDS reads first, then the stores
#pragma unroll
        for (int j = 0; j < kCNbrPer; ++j) {
            const int q = tid + j * kCThreads;
            t4[j] = nb4[q < kCNbrVec ? q : 0];
        }
#pragma unroll
        for (int j = 0; j < kCNbrPer; ++j) {
            const int q = tid + j * kCThreads;
            if (q < kCNbrVec && q < q_end) dst[q] = t4[j];
        }
    }
    block_lookback<kCols, 16, 9>(look, (int64_t)bid - 1, epoch, status, L.pre, L.done, spin_limit,
                                 wait_xor);
    if (tid < kCols) {
        const int k = tid;
        const uint32_t run = L.tot[k];
        const uint32_t prefix = L.pre[k];
        // per-chunk starts of every tap's pairs and of the slab rows (the last
        // chunk also writes the totals as row last + 1), for row-range GEMMs
        chunk_pre[(int64_t)bid * kCols + k] = (int32_t)prefix;
        if (bid == last) chunk_pre[(int64_t)(bid + 1) * kCols + k] = (int32_t)(prefix + run);
        if (bid > 0)
            __hip_atomic_store(&look[(int64_t)bid * kCols + k], lb_pack(epoch, kIncl, prefix + run),
                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (bid == last) {
            // the last chunk: prefix + run is the total of column k
            const uint32_t tot = prefix + run;
            if (k < kTaps) {
                st->tap_count[k] = (int32_t)tot;
                st->tap_off[k] = (int32_t)(k * cap);
            } else {
                st->totals[3] = (int32_t)tot;             // slab rows = off-centre pairs
                st->tap_off[kTaps] = (int32_t)(kTaps * cap);
                rowbase[n] = (int32_t)tot;                // end of the last row's run
            }
        }
    }
    __syncthreads();
    if (tid < 64) {                               // wave 0, lane k: tap k's chunk-local start
        const int k = tid;
        const uint32_t t = k < kTaps ? L.tot[k] : 0u;             // at most kCChunk
        uint32_t all;
        const uint32_t loc = wave_excl_scan<9>(t, &all);
        if (k <= kTaps) L.loc[k] = loc;                           // lane kTaps: the chunk's pairs
        if (bid == last) {               // the last chunk: pairs and padded tiles
            int32_t c = k < kTaps ? (int32_t)(L.pre[k] + t) : 0;
            int32_t padded = (c + tile_m - 1) / tile_m * tile_m;
#pragma unroll
            for (int o = 32; o > 0; o >>= 1) {
                c += __shfl_xor(c, o, 64);
                padded += __shfl_xor(padded, o, 64);
            }
            if (k == 0) {
                st->totals[0] = c;
                st->totals[1] = padded;
                st->totals[2] = padded / tile_m;
            }
        }
    }
    // first slab row of the row
    const uint32_t rb = L.pre[kTaps] + L.wc[w][kTaps] + excl;
    if (row < n) rowbase[row] = (int32_t)rb;
    L.rb[tid] = rb;
    __syncthreads();
    // list the chunk's pairs in output order: tap-major, rows ascending. Lane k
    // holds the wave's first list slot of tap k; the loop reads it with readlane.
    const uint32_t first = lane < kTaps ? L.loc[lane] + L.wc[w][lane] : 0u;
    for (uint32_t u = uni; u; u &= u - 1) {
        const int k = __builtin_ctz(u);
        const uint64_t b = __ballot((m >> k) & 1u);
        const uint32_t f = (uint32_t)__builtin_amdgcn_readlane((int)first, k);
        if ((m >> k) & 1u) L.list[f + lanes_below(b)] = (uint16_t)(tid | (k << 8));
    }
    __syncthreads();
    // write them out: entry p of tap k goes to k cap + (pairs of k in earlier chunks) + its rank
    const int total = (int)L.loc[kTaps];
    for (int p = tid; p < total; p += kCThreads) {
        const uint32_t e = L.list[p];
        const int lr = (int)(e & 0xFFu), k = (int)(e >> 8);
        const int64_t pos = (int64_t)k * cap + L.pre[k] + (p - (int)L.loc[k]);
        if (pos >= (int64_t)k * cap + cap) continue;          // only after a stalled wait
        const uint32_t mr = L.m[lr];
        const bool self = dense_centre && k == kCentre;
        const bool direct = !dense_centre && __popc(mr) == 1;    // the row's only pair
        pair_in[pos] = self ? (int32_t)(base0 + lr) : L.nb[lr * kTaps + k];
        pair_out[pos] = (int32_t)(base0 + lr);
        pair_slot[pos] = self     ? -1
                         : direct ? -2 - (int32_t)(base0 + lr)
                                  : (int32_t)(L.rb[lr] + __popc(mr & ((1u << k) - 1u) & slab_taps));
    }
}

// Compaction of a neighbour table in memory (sorted route): rows
// [bid*kCChunk, +kCChunk) in row order, one per thread. The chunk's
// neighbour rows (contiguous in the table) are read once, coalesced, into
// LDS.
// One chunk of k_compact: rows [bid kCChunk, +kCChunk) of n, last = the last
// chunk's index.
__device__ __forceinline__ void compact_table_chunk(
    CompactLds& L, uint32_t bid, uint32_t last, const uint32_t* __restrict__ mask,
    const int32_t* __restrict__ nbr, int64_t n, int64_t cap, int tile_m, MapState* st,
    int32_t* __restrict__ pair_in, int32_t* __restrict__ pair_out, int32_t* __restrict__ pair_slot,
    int32_t* __restrict__ rowbase, int32_t* __restrict__ chunk_pre, uint64_t* __restrict__ look,
    uint32_t epoch, uint32_t* status, bool dense_centre) {
    const int tid = threadIdx.x;
    const int64_t base0 = (int64_t)bid * kCChunk;
    const int64_t row = base0 + tid;
    // mask, neighbour rows (whole 16-byte words; the table is padded so the last word
    // of the last row is readable)
    const uint32_t mv = n > 0 ? mask[row < n ? row : n - 1] : 0u;
    int4 nv4[kCNbrPer];
    {
        const int4* src = reinterpret_cast<const int4*>(nbr + base0 * kTaps);
        int64_t q_last = (n * kTaps + 3) / 4 - 1 - base0 * kTaps / 4;         // last readable word
        if (q_last < 0) q_last = 0;               // no rows: the table's first word (allocated)
#pragma unroll
        for (int j = 0; j < kCNbrPer; ++j) {
            const int64_t q = tid + j * kCThreads;
            nv4[j] = src[q < q_last ? q : q_last];
        }
    }
    int4* nb4 = reinterpret_cast<int4*>(L.nb);
#pragma unroll
    for (int j = 0; j < kCNbrPer; ++j) {
        const int q = tid + j * kCThreads;
        if (q < kCNbrVec) nb4[q] = nv4[j];
    }
    compact_chunk(L, row < n ? mv : 0u, bid, last, n, cap, tile_m, st, pair_in, pair_out, pair_slot,
                  rowbase, chunk_pre, look, epoch, status, nullptr, dense_centre);
}

// Compaction of a neighbour table in memory: one chunk per block. With n_dev
// (a device row count; n is then only its bound, 8 inputs a row for a strided
// map) the grid is at most the resident blocks and block b takes chunks b,
// b + gridDim.x, ... up to the count's last chunk. A chunk's look-back waits
// only on lower chunks, each held by a resident block that waits only on
// lower ones again, so every wait ends; no ticket is taken (a ticket per
// block, 800 to 1000 atomics on one word, cost 10 us).
__global__ __launch_bounds__(kCThreads) void k_compact(
    const uint32_t* __restrict__ mask, const int32_t* __restrict__ nbr, int64_t n, int64_t cap,
    int tile_m, MapState* st, int32_t* __restrict__ pair_in, int32_t* __restrict__ pair_out,
    int32_t* __restrict__ pair_slot, int32_t* __restrict__ rowbase, int32_t* __restrict__ chunk_pre,
    uint64_t* __restrict__ look, uint32_t* ticket, bool by_index, uint32_t epoch, uint32_t* status,
    bool dense_centre, const int32_t* __restrict__ n_dev) {
    __shared__ CompactLds L;
    if (n_dev) {
        const int64_t nd = *n_dev;
        if (nd < n) n = nd > 0 ? nd : 0;
        const uint32_t last = n > 0 ? (uint32_t)((n + kCChunk - 1) / kCChunk - 1) : 0u;
        for (uint32_t bid = blockIdx.x; bid <= last; bid += gridDim.x) {
            compact_table_chunk(L, bid, last, mask, nbr, n, cap, tile_m, st, pair_in, pair_out,
                                pair_slot, rowbase, chunk_pre, look, epoch, status, dense_centre);
            __syncthreads();                      // the chunk's LDS reads done before the next
        }
        return;
    }
    const uint32_t bid = chunk_of_block(by_index, ticket, &L.bid);
    compact_table_chunk(L, bid, gridDim.x - 1, mask, nbr, n, cap, tile_m, st, pair_in, pair_out,
                        pair_slot, rowbase, chunk_pre, look, epoch, status, dense_centre);
    if (!by_index && bid == gridDim.x - 1 && threadIdx.x == 0) atomicExch(ticket, 0u);
}

// Lookup and compaction in one kernel: each thread looks up its row's 27
// neighbour rows (the lookup policy), writes them to LDS and its mask,
// then the chunk is compacted (which also stores the chunk's neighbour rows to
// the table, coalesced).
//
// Dense route: each row's 27 cells as 9 (dx, dy) columns of 3 consecutive
// cells (z fastest): first their occupancy bits, then the row ids of the
// occupied ones. SPARSE: the rows are a strided map's query points (input
// coordinates of 2 o), whose centre cell is looked up like the other taps (the
// input at 2 o may be absent).
template <bool SPARSE, bool BRICK>
struct DenseLookup {
    static constexpr bool kDenseCentre = !SPARSE;
    const int32_t* coords;
    Geom g;
    const int32_t* grid;
    const uint32_t* bits;
    __device__ __forceinline__ void operator()(int64_t row, int64_t n, int32_t (&v)[kTaps]) const {
        const int64_t rc = row < n ? row : (n > 0 ? n - 1 : 0);
        const int32_t* c = coords + rc * g.ncols;
        const int b = g.ncols == 4 ? c[0] : 0;
        const int32_t* q = c + (g.ncols == 4 ? 1 : 0);
        const int x = q[0] - g.origin[0], y = q[1] - g.origin[1], z = q[2] - g.origin[2];
        const bool ok = row < n && (unsigned)b < (unsigned)g.batch &&
                        (unsigned)x < (unsigned)g.ext[0] && (unsigned)y < (unsigned)g.ext[1] &&
                        (unsigned)z < (unsigned)g.ext[2];
        // the row's cell in the padded grid (g.pad cells of padding a side), z
        // one lower: its 3x3x3 neighbourhood is (xp - 1 .. xp + 1, yp - 1 ..
        // yp + 1, zp .. zp + 2). Rows out of range (and rows past n) read the
        // neighbourhood of padded cell (1, 1, 1) of batch 0 instead, which lies
        // inside the grid; their values are unused.
        const int bb = ok ? b : 0;
        const int64_t xp = ok ? x + g.pad : 1, yp = ok ? y + g.pad : 1;
        const int64_t zp = ok ? z + g.pad - 1 : 0;
        // occupancy of the 9 (dx, dy) columns (3 bits each) ...
        uint32_t cb[9];
#pragma unroll
        for (int dx = 0; dx < 3; ++dx)
#pragma unroll
            for (int dy = 0; dy < 3; ++dy)
                cb[3 * dx + dy] = column_bits<BRICK>(bits, g, bb, xp + dx - 1, yp + dy - 1, zp, 3);
        // ... then row ids of the occupied cells only. Every tap issues its load; an
        // empty one reads cell 0 (one line, cached for the whole launch), so no load
        // is conditional.
#pragma unroll
        for (int dx = 0; dx < 3; ++dx)
#pragma unroll
            for (int dy = 0; dy < 3; ++dy)
#pragma unroll
                for (int dz = 0; dz < 3; ++dz) {
                    const int k = 9 * dx + 3 * dy + dz;
                    if (!SPARSE && k == kCentre) continue;
                    const bool on = (cb[3 * dx + dy] >> dz) & 1u;
                    const int64_t cc = grid_cell<BRICK>(g, bb, xp + dx - 1, yp + dy - 1, zp + dz);
                    v[k] = grid[on ? cc : 0];
                    v[k] = on ? v[k] : -1;
                }
        if (!SPARSE) v[kCentre] = (int32_t)row;
#pragma unroll
        for (int k = 0; k < kTaps; ++k) v[k] = ok ? v[k] : -1;
    }
};

// One chunk: rows [bid kCChunk, +kCChunk) of n, last = the last chunk's index.
template <class LOOKUP>
__device__ __forceinline__ void lookup_compact_chunk(
    CompactLds& L, uint32_t bid, uint32_t last, const LOOKUP& lk, int64_t n,
    int32_t* __restrict__ nbr, uint32_t* __restrict__ mask, int64_t cap, int tile_m, MapState* st,
    int32_t* __restrict__ pair_in, int32_t* __restrict__ pair_out, int32_t* __restrict__ pair_slot,
    int32_t* __restrict__ rowbase, int32_t* __restrict__ chunk_pre, uint64_t* __restrict__ look,
    uint32_t epoch, uint32_t* status, uint32_t spin_limit, uint32_t wait_xor) {
    const int tid = threadIdx.x;
    const int64_t row = (int64_t)bid * kCChunk + tid;
    int32_t v[kTaps];
    lk(row, n, v);
    uint32_t m = 0;
#pragma unroll
    for (int k = 0; k < kTaps; ++k) {
        m |= (v[k] >= 0 ? 1u : 0u) << k;
        L.nb[tid * kTaps + k] = v[k];
    }
    if (row < n) mask[row] = m;
    __syncthreads();
    compact_chunk(L, m, bid, last, n, cap, tile_m, st, pair_in, pair_out, pair_slot, rowbase,
                  chunk_pre, look, epoch, status, nbr, LOOKUP::kDenseCentre, spin_limit, wait_xor);
}

// One chunk per block; with n_dev (a device row count, n only its bound) the
// grid is at most the resident blocks, each taking chunks blockIdx.x,
// + gridDim.x, ... up to the count's last chunk (as k_compact).
template <class LOOKUP>
__global__ __launch_bounds__(kCThreads) void k_lookup_compact(
    LOOKUP lk, int64_t n, int32_t* __restrict__ nbr, uint32_t* __restrict__ mask, int64_t cap,
    int tile_m, MapState* st, int32_t* __restrict__ pair_in, int32_t* __restrict__ pair_out,
    int32_t* __restrict__ pair_slot, int32_t* __restrict__ rowbase,
    int32_t* __restrict__ chunk_pre, uint64_t* __restrict__ look, uint32_t* ticket, bool by_index,
    uint32_t epoch, uint32_t* status, uint32_t spin_limit, uint32_t wait_xor,
    const int32_t* __restrict__ n_dev) {
    __shared__ CompactLds L;
    if (n_dev) {
        const int64_t nd = *n_dev;
        if (nd < n) n = nd > 0 ? nd : 0;
        const uint32_t last = n > 0 ? (uint32_t)((n + kCChunk - 1) / kCChunk - 1) : 0u;
        for (uint32_t bid = blockIdx.x; bid <= last; bid += gridDim.x) {
            lookup_compact_chunk(L, bid, last, lk, n, nbr, mask, cap, tile_m, st, pair_in,
                                 pair_out, pair_slot, rowbase, chunk_pre, look, epoch, status,
                                 spin_limit, wait_xor);
            __syncthreads();                      // the chunk's LDS reads done before the next
        }
        return;
    }
    const uint32_t bid = chunk_of_block(by_index, ticket, &L.bid);
    lookup_compact_chunk(L, bid, gridDim.x - 1, lk, n, nbr, mask, cap, tile_m, st, pair_in,
                         pair_out, pair_slot, rowbase, chunk_pre, look, epoch, status, spin_limit,
                         wait_xor);
    if (!by_index && bid == gridDim.x - 1 && threadIdx.x == 0) atomicExch(ticket, 0u);
}

// Compaction for the 5 x 5 x 5 kernel: 125 taps, masks of 4 words, 256-row
// chunks in row order, a block look-back over 126 columns (125 taps + slab
// rows, 2 lanes per column). Same outputs and layout as the 3 x 3 x 3
// compaction.
constexpr int kK5Taps = 125, kK5Centre = 62, kK5Cols = kK5Taps + 1;

// Index of the r-th set bit (r < popcount) of m.
__device__ __forceinline__ int select_bit(uint64_t m, uint32_t r) {
    int pos = 0;
#pragma unroll
    for (int w = 32; w > 0; w >>= 1) {
        const uint32_t c = (uint32_t)__popcll(m & ((1ull << w) - 1));
        if (r >= c) {
            r -= c;
            m >>= w;
            pos += w;
        }
    }
    return pos;
}

// K = 5 compaction, one 256-row chunk per block (a row per thread). Each wave
// transposes its 64 masks through LDS so that lane j holds taps j and 64 + j: the
// rows with the tap (a 64-bit lane set) and their count. After the column
// look-back the wave lists its pairs in (tap, row) order, 64 at a time, one per
// lane: the tap by a binary search over the wave's per-tap starts, the row as the
// r-th member of the tap's lane set; consecutive lanes then write consecutive
// places of one tap's list, and only real pairs read the neighbour table.
__global__ __launch_bounds__(kCThreads) void k_compact5(
    const uint32_t* __restrict__ mask, const int32_t* __restrict__ nbr, int64_t n, int64_t cap,
    int tile_m, MapState* st, int32_t* __restrict__ pair_in, int32_t* __restrict__ pair_out,
    int32_t* __restrict__ pair_slot, int32_t* __restrict__ rowbase, uint64_t* __restrict__ look,
    uint32_t* ticket, bool by_index, uint32_t epoch, uint32_t* status) {
    __shared__ uint32_t s_bid;
    __shared__ uint32_t s_wc[kCWaves][kK5Cols];   // per-wave counts, then offsets in the chunk
    __shared__ uint32_t s_pre[kK5Cols], s_tot[kK5Cols], s_done[kK5Cols];
    __shared__ uint4 s_m[kCWaves][64];            // the wave's masks
    __shared__ uint64_t s_set[kCWaves][128];      // per tap: the wave's rows with it (bit = lane)
    __shared__ uint32_t s_beg[kCWaves][128];      // per tap: its first pair in the wave's order
    __shared__ uint32_t s_rb[kCWaves][64];        // first slab row of each of the wave's rows
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const uint32_t bid = chunk_of_block(by_index, ticket, &s_bid);
    const int64_t row = (int64_t)bid * kCChunk + tid;
    const bool valid = row < n;
    uint4 mv = make_uint4(0u, 0u, 0u, 0u);
    if (valid) mv = reinterpret_cast<const uint4*>(mask)[row];
    const uint32_t pop = (uint32_t)(__popc(mv.x) + __popc(mv.y) + __popc(mv.z) + __popc(mv.w));
    const uint32_t deg = pop ? pop - 1u : 0u;     // off-centre pairs of the row
    s_m[w][lane] = mv;
    __builtin_amdgcn_wave_barrier();
    // lane j: bit j % 32 of words j / 32 (tap j) and 2 + j / 32 (tap 64 + j) of each row
    uint64_t set_lo = 0, set_hi = 0;
    {
        const int sh = lane & 31;
        const bool upper = lane >= 32;
#pragma unroll 16
        for (int r = 0; r < 64; ++r) {
            const uint4 v = s_m[w][r];
            set_lo |= (uint64_t)(((upper ? v.y : v.x) >> sh) & 1u) << r;
            set_hi |= (uint64_t)(((upper ? v.w : v.z) >> sh) & 1u) << r;
        }
    }
    if (lane >= kK5Taps - 64) set_hi = 0;
    const uint32_t cnt_lo = (uint32_t)__popcll(set_lo), cnt_hi = (uint32_t)__popcll(set_hi);
    uint32_t tot_lo, tot_hi;
    const uint32_t beg_lo = wave_excl_scan<7>(cnt_lo, &tot_lo);
    const uint32_t beg_hi = tot_lo + wave_excl_scan<7>(cnt_hi, &tot_hi);
    const uint32_t n_pairs = tot_lo + tot_hi;     // the wave's pairs, centre ones included
    s_set[w][lane] = set_lo;
    s_set[w][64 + lane] = set_hi;
    s_beg[w][lane] = beg_lo;
    s_beg[w][64 + lane] = lane < kK5Taps - 64 ? beg_hi : n_pairs;
    s_wc[w][lane] = cnt_lo;
    if (lane < kK5Taps - 64) s_wc[w][64 + lane] = cnt_hi;
    uint32_t wave_slab;
    const uint32_t excl = wave_excl_scan<7>(deg, &wave_slab);     // deg < 125
    if (lane == 0) s_wc[w][kK5Taps] = wave_slab;
    __syncthreads();
    if (tid < kK5Cols) {
        uint32_t run = 0;
#pragma unroll
        for (int v = 0; v < kCWaves; ++v) {
            const uint32_t c = s_wc[v][tid];
            s_wc[v][tid] = run;
            run += c;
        }
        s_tot[tid] = run;
        __hip_atomic_store(&look[(int64_t)bid * kK5Cols + tid],
                           lb_pack(epoch, bid == 0 ? kIncl : kAgg, run), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    }
    block_lookback<kK5Cols, 16, 2>(look, (int64_t)bid - 1, epoch, status, s_pre, s_done);
    if (tid < kK5Cols) {
        const uint32_t run = s_tot[tid], prefix = s_pre[tid];
        if (bid > 0)
            __hip_atomic_store(&look[(int64_t)bid * kK5Cols + tid],
                               lb_pack(epoch, kIncl, prefix + run), __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
        if (bid == gridDim.x - 1) {
            const uint32_t tot = prefix + run;
            if (tid < kK5Taps) {
                st->tap_count[tid] = (int32_t)tot;
                st->tap_off[tid] = (int32_t)(tid * cap);
            } else {
                st->totals[3] = (int32_t)tot;
                st->tap_off[kK5Taps] = (int32_t)(kK5Taps * cap);
                rowbase[n] = (int32_t)tot;
            }
        }
    }
    __syncthreads();
    if (bid == gridDim.x - 1) {                   // the last chunk: pairs and padded tiles
        __shared__ int32_t s_red[2][2];
        if (tid < 128) {                          // waves 0 and 1 cover the 125 taps
            int32_t c = tid < kK5Taps ? (int32_t)(s_pre[tid] + s_tot[tid]) : 0;
            int32_t padded = (c + tile_m - 1) / tile_m * tile_m;
#pragma unroll
            for (int o = 32; o > 0; o >>= 1) {
                c += __shfl_xor(c, o, 64);
                padded += __shfl_xor(padded, o, 64);
            }
            if (lane == 0) {
                s_red[w][0] = c;
                s_red[w][1] = padded;
            }
        }
        __syncthreads();
        if (tid == 0) {
            const int32_t padded = s_red[0][1] + s_red[1][1];
            st->totals[0] = s_red[0][0] + s_red[1][0];
            st->totals[1] = padded;
            st->totals[2] = padded / tile_m;
        }
    }
    const uint32_t rb = s_pre[kK5Taps] + s_wc[w][kK5Taps] + excl;
    if (valid) rowbase[row] = (int32_t)rb;
    s_rb[w][lane] = rb;
    __builtin_amdgcn_wave_barrier();
    const uint32_t cap32 = cap < (int64_t)UINT32_MAX ? (uint32_t)cap : UINT32_MAX;
    const int64_t wave_row0 = (int64_t)bid * kCChunk + 64 * w;
    for (uint32_t e0 = 0; e0 < n_pairs; e0 += 64) {
        const uint32_t e = e0 + (uint32_t)lane;
        if (e >= n_pairs) break;
        int k = 0;                                // the last tap whose pairs start at or before e
#pragma unroll
        for (int step = 64; step > 0; step >>= 1)
            if (s_beg[w][k + step] <= e) k += step;
        const uint32_t r = e - s_beg[w][k];       // e is the tap's r-th pair of the wave
        const int rl = select_bit(s_set[w][k], r);
        const uint32_t p = s_pre[k] + s_wc[w][k] + r;
        const int64_t rg = wave_row0 + rl;
        const uint4 m = s_m[w][rl];
        // off-centre taps of the row below k
        const uint32_t lowk = k & 31, q = (uint32_t)k >> 5;
        const uint32_t part = (q == 0 ? m.x : q == 1 ? m.y : q == 2 ? m.z : m.w) & ((1u << lowk) - 1u);
        const uint32_t below = (uint32_t)__popc(part) + (q > 0 ? (uint32_t)__popc(m.x) : 0u) +
                               (q > 1 ? (uint32_t)__popc(m.y) : 0u) +
                               (q > 2 ? (uint32_t)__popc(m.z) : 0u) -
                               (k > kK5Centre ? (m.y >> (kK5Centre - 32)) & 1u : 0u);
        const bool centre = k == kK5Centre;
        if (p < cap32 && rg < n) {                // (only false after a stalled wait)
            const int32_t src = centre ? (int32_t)rg : nbr[rg * kK5Taps + k];
            const int64_t pos = (int64_t)k * cap + p;
            pair_in[pos] = src;
            pair_out[pos] = (int32_t)rg;
            pair_slot[pos] = centre ? -1 : (int32_t)(s_rb[w][rl] + below);
        }
    }
    if (!by_index && bid == gridDim.x - 1 && tid == 0) atomicExch(ticket, 0u);
}

}  // namespace

int mask_sort_bits(const MaskOrder& ord) {
    if (ord.plain) return kMaskBits;
    if (ord.n_groups == 1) return ord.group_bits;
    int gb = 0;
    while ((1 << gb) < ord.n_groups) ++gb;
    return ord.group_bits + 1 + gb;
}

hipError_t launch_mask_hist(const uint32_t* mask, int64_t n, const SortPlan& plan,
                            const MaskOrder& ord, uint32_t* keys, uint32_t* hist, int32_t* tap_tot,
                            int32_t* group_rows, hipStream_t s) {
    if (!ord.plain && !keys) return hipErrorInvalidValue;
    unsigned blocks = (unsigned)((n + kHTile - 1) / kHTile);
    size_t lds = ((size_t)plan.passes * (1u << plan.bits) + kTaps + kMaxGroups) * 4;
    launch(k_mask_hist, blocks, kHThreads, lds, s, mask, n, plan.bits, plan.passes, ord, keys, hist,
           tap_tot, group_rows);
    return hipGetLastError();
}

int64_t compact_chunks(int64_t n) { return (n + kCChunk - 1) / kCChunk; }

size_t compact_look_bytes(int64_t n) { return (size_t)compact_chunks(n) * (kTaps + 1) * 8; }

size_t compact_look_bytes_k(int64_t n, int ksize) {
    return (size_t)compact_chunks(n) * (ksize == 5 ? kK5Cols : kTaps + 1) * 8;
}

// Blocks of 256 threads of `kern` resident at once on the current device
// (occupancy per CU times CUs, queried once per kernel and device; 0 if the
// query failed).
static int64_t resident_blocks(const void* kern, int slot) {
    constexpr int kDevs = 64;
    static std::atomic<int64_t> cache[kDevs][6];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kDevs) return 0;
    int64_t cap = cache[dev][slot].load(std::memory_order_relaxed);
    if (cap == 0) {
        int per_cu = 0, n_cu = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, kCThreads, 0) != hipSuccess ||
            hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
            return 0;
        cap = (int64_t)per_cu * n_cu;
        cache[dev][slot].store(cap > 0 ? cap : -1, std::memory_order_relaxed);
    }
    return cap > 0 ? cap : 0;
}

// Whether `blocks` blocks of `kern` fit on the current device at once.
static bool fits_at_once(const void* kern, int slot, unsigned blocks) {
    const int64_t cap = resident_blocks(kern, slot);
    return cap > 0 && (int64_t)blocks <= cap;
}

static uint32_t next_epoch(SortWork& ws) {
    uint32_t epoch = ++ws.epoch & 0x3FFFFFFFu;
    if (epoch == 0) epoch = ++ws.epoch & 0x3FFFFFFFu;
    return epoch;
}

uint32_t take_epoch(SortWork& ws) { return next_epoch(ws); }

hipError_t launch_compact(const uint32_t* mask, const int32_t* nbr, int64_t n, int ksize,
                          int64_t cap, int tile_m, MapState* st, int32_t* pair_in,
                          int32_t* pair_out, int32_t* pair_slot, int32_t* rowbase,
                          int32_t* chunk_pre, SortWork& ws, uint32_t* status, hipStream_t s,
                          bool dense_centre, const int32_t* n_dev) {
    const uint32_t epoch = next_epoch(ws);
    const unsigned blocks = (unsigned)compact_chunks(n);
    if (ksize == 5) {
        if (n_dev) return hipErrorInvalidValue;   // (a device count comes with 3 x 3 x 3 maps only)
        const bool by_index = fits_at_once((const void*)k_compact5, 0, blocks);
        launch(k_compact5, blocks, kCThreads, 0, s, mask, nbr, n, cap, tile_m, st, pair_in,
               pair_out, pair_slot, rowbase, ws.look, ws.ticket, by_index, epoch, status);
    } else if (n_dev) {
        // chunks up to the device count, strided over at most the resident blocks
        const int64_t res = resident_blocks((const void*)k_compact, 1);
        const unsigned grid = res > 0 && res < (int64_t)blocks ? (unsigned)res : blocks;
        launch(k_compact, grid, kCThreads, 0, s, mask, nbr, n, cap, tile_m, st, pair_in,
               pair_out, pair_slot, rowbase, chunk_pre, ws.look, ws.ticket, false, epoch, status,
               dense_centre, n_dev);
    } else {
        const bool by_index = fits_at_once((const void*)k_compact, 1, blocks);
        launch(k_compact, blocks, kCThreads, 0, s, mask, nbr, n, cap, tile_m, st, pair_in,
               pair_out, pair_slot, rowbase, chunk_pre, ws.look, ws.ticket, by_index, epoch, status,
               dense_centre, n_dev);
    }
    return hipGetLastError();
}

// One launch of k_lookup_compact with lookup lk: by block index when every
// block fits at once (else by ticket), or under a device row count over at most
// the resident blocks.
template <class LOOKUP>
static hipError_t launch_lookup_compact_t(const LOOKUP& lk, int slot, int64_t n, int32_t* nbr,
                                          uint32_t* mask, int64_t cap, int tile_m, MapState* st,
                                          int32_t* pair_in, int32_t* pair_out, int32_t* pair_slot,
                                          int32_t* rowbase, int32_t* chunk_pre, SortWork& ws,
                                          uint32_t* status, hipStream_t s, const int32_t* n_dev) {
    const uint32_t epoch = next_epoch(ws);
    const unsigned blocks = (unsigned)compact_chunks(n);
    const uint32_t spin = ws.force_timeout ? 64u : kSpinLimit;
    const uint32_t wx = ws.force_timeout ? 0x15555555u : 0u;
    const void* kern = (const void*)k_lookup_compact<LOOKUP>;
    unsigned grid_x = blocks;
    bool by_index = false;
    if (n_dev) {
        const int64_t res = resident_blocks(kern, slot);
        if (res > 0 && res < (int64_t)blocks) grid_x = (unsigned)res;
    } else {
        by_index = fits_at_once(kern, slot, blocks);
    }
    launch(k_lookup_compact<LOOKUP>, grid_x, kCThreads, 0, s, lk, n, nbr, mask, cap, tile_m, st,
           pair_in, pair_out, pair_slot, rowbase, chunk_pre, ws.look, ws.ticket, by_index, epoch,
           status, spin, wx, n_dev);
    return hipGetLastError();
}

hipError_t launch_lookup_compact(const int32_t* coords, int64_t n, const Geom& g,
                                 const int32_t* grid, const uint32_t* bits, int32_t* nbr,
                                 uint32_t* mask, int64_t cap,
                                 int tile_m, MapState* st, int32_t* pair_in, int32_t* pair_out,
                                 int32_t* pair_slot, int32_t* rowbase, int32_t* chunk_pre,
                                 SortWork& ws, uint32_t* status, hipStream_t s, bool sparse_centre,
                                 const int32_t* n_dev) {
    // (resident-block cache slots 2 .. 5, one per instance)
    if (sparse_centre && g.brick)
        return launch_lookup_compact_t(DenseLookup<true, true>{coords, g, grid, bits}, 5, n, nbr,
                                       mask, cap, tile_m, st, pair_in, pair_out, pair_slot, rowbase,
                                       chunk_pre, ws, status, s, n_dev);
    if (sparse_centre)
        return launch_lookup_compact_t(DenseLookup<true, false>{coords, g, grid, bits}, 3, n, nbr,
                                       mask, cap, tile_m, st, pair_in, pair_out, pair_slot, rowbase,
                                       chunk_pre, ws, status, s, n_dev);
    if (g.brick)
        return launch_lookup_compact_t(DenseLookup<false, true>{coords, g, grid, bits}, 4, n, nbr,
                                       mask, cap, tile_m, st, pair_in, pair_out, pair_slot, rowbase,
                                       chunk_pre, ws, status, s, n_dev);
    return launch_lookup_compact_t(DenseLookup<false, false>{coords, g, grid, bits}, 2, n, nbr, mask,
                                   cap, tile_m, st, pair_in, pair_out, pair_slot, rowbase, chunk_pre,
                                   ws, status, s, n_dev);
}

}  // namespace smc
