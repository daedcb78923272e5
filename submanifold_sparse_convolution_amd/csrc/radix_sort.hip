// Stable LSD radix sort of (key, value) pairs, 8 bits per pass.
//
// Used twice in the map build: on packed voxel keys in the sorted route
// (the sort the Z-Delta mapper needs; "[Kernel] Add submanifold sparse 3D
// convolution (bf16 implicit GEMM, gfx950)", Design) and on neighbour masks
// to group rows with equal masks ("Sparse convolution in FP32", "Neighbour
// masks and sorted rows": a GPU radix sort orders the rows by mask).
//
// Each pass is reduce-then-scan with no global atomics (the pull request's
// Open questions record an atomic-counter compaction that serialised):
//   count   per tile of 4096 keys, a 256-bin histogram, stored digit-major
//   scan    one block turns the digit-major table into exclusive offsets
//   scatter per tile, a stable rank inside the tile from wave ballots, then
//           offset + rank
#include "smc_internal.h"

namespace smc {
namespace {

constexpr int kRadixBits = 8;
constexpr int kBins = 1 << kRadixBits;
constexpr int kSortBlock = 256;
constexpr int kItems = 16;
constexpr int kTile = kSortBlock * kItems;
constexpr int kScanBlock = 1024;

template <typename K>
__global__ __launch_bounds__(kSortBlock) void k_radix_count(const K* __restrict__ keys, int64_t n,
                                                            int shift, int n_tiles,
                                                            uint32_t* __restrict__ counts) {
    __shared__ uint32_t hist[kBins];
    hist[threadIdx.x] = 0;
    __syncthreads();
    int64_t base = (int64_t)blockIdx.x * kTile;
#pragma unroll 4
    for (int i = 0; i < kItems; ++i) {
        int64_t idx = base + i * kSortBlock + threadIdx.x;
        if (idx < n) atomicAdd(&hist[(uint32_t)(keys[idx] >> shift) & (kBins - 1)], 1u);
    }
    __syncthreads();
    counts[(int64_t)threadIdx.x * n_tiles + blockIdx.x] = hist[threadIdx.x];
}

// Exclusive scan in place over m entries, one block.
__global__ __launch_bounds__(kScanBlock) void k_exclusive_scan(uint32_t* __restrict__ v,
                                                               int64_t m) {
    __shared__ uint32_t wave_tot[kScanBlock / 64];
    __shared__ uint32_t carry_s;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    if (tid == 0) carry_s = 0;
    __syncthreads();
    for (int64_t seg = 0; seg < m; seg += (int64_t)kScanBlock * 4) {
        uint32_t x[4];
        uint32_t sum = 0;
        int64_t i0 = seg + (int64_t)tid * 4;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            x[j] = (i0 + j < m) ? v[i0 + j] : 0u;
            sum += x[j];
        }
        // inclusive wave scan of the per-thread sums
        uint32_t inc = sum;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            uint32_t y = __shfl_up(inc, o);
            if (lane >= o) inc += y;
        }
        if (lane == 63) wave_tot[w] = inc;
        __syncthreads();
        uint32_t before = carry_s;
        for (int j = 0; j < w; ++j) before += wave_tot[j];
        uint32_t run = before + inc - sum;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if (i0 + j < m) v[i0 + j] = run;
            run += x[j];
        }
        __syncthreads();
        if (tid == kScanBlock - 1) carry_s = run;
        __syncthreads();
    }
}

template <typename K>
__global__ __launch_bounds__(kSortBlock) void k_radix_scatter(
    const K* __restrict__ kin, const uint32_t* __restrict__ vin, K* __restrict__ kout,
    uint32_t* __restrict__ vout, int64_t n, int shift, int n_tiles,
    const uint32_t* __restrict__ offsets) {
    __shared__ uint32_t next[kBins];                     // next free slot per digit
    __shared__ uint32_t wave_cnt[kSortBlock / 64][kBins];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    next[tid] = offsets[(int64_t)tid * n_tiles + blockIdx.x];
#pragma unroll
    for (int j = 0; j < kSortBlock / 64; ++j) wave_cnt[j][tid] = 0;
    __syncthreads();
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    int64_t base = (int64_t)blockIdx.x * kTile;
    for (int i = 0; i < kItems; ++i) {
        // processing order (i, wave, lane) is the input order: keeps the sort stable
        int64_t idx = base + i * kSortBlock + tid;
        bool valid = idx < n;
        K key = valid ? kin[idx] : (K)0;
        uint32_t val = valid ? (vin ? vin[idx] : (uint32_t)idx) : 0u;
        uint32_t d = (uint32_t)(key >> shift) & (kBins - 1);
        uint64_t peers = __ballot(valid);
#pragma unroll
        for (int b = 0; b < kRadixBits; ++b) {
            uint64_t bb = __ballot((d >> b) & 1u);
            peers &= ((d >> b) & 1u) ? bb : ~bb;
        }
        uint32_t rank = (uint32_t)__popcll(peers & below);
        if (valid && rank == 0) wave_cnt[w][d] = (uint32_t)__popcll(peers);
        __syncthreads();
        if (valid) {
            uint32_t pos = next[d] + rank;
            for (int j = 0; j < w; ++j) pos += wave_cnt[j][d];
            kout[pos] = key;
            vout[pos] = val;
        }
        __syncthreads();
        uint32_t add = 0;
#pragma unroll
        for (int j = 0; j < kSortBlock / 64; ++j) {
            add += wave_cnt[j][tid];
            wave_cnt[j][tid] = 0;
        }
        next[tid] += add;
        __syncthreads();
    }
}

template <typename K>
hipError_t radix_sort_impl(const K* keys_in, const uint32_t* vals_in, int64_t n, int key_bits,
                           K* kbuf0, K* kbuf1, uint32_t* vbuf0, uint32_t* vbuf1, uint32_t* counts,
                           const K** keys_out, const uint32_t** vals_out, hipStream_t s) {
    const int n_tiles = (int)((n + kTile - 1) / kTile);
    const K* kcur = keys_in;
    const uint32_t* vcur = vals_in;
    K* kdst[2] = {kbuf0, kbuf1};
    uint32_t* vdst[2] = {vbuf0, vbuf1};
    int passes = (key_bits + kRadixBits - 1) / kRadixBits;
    if (passes < 1) passes = 1;   // still produce the value permutation
    for (int p = 0; p < passes; ++p) {
        int shift = p * kRadixBits;
        k_radix_count<K><<<n_tiles, kSortBlock, 0, s>>>(kcur, n, shift, n_tiles, counts);
        k_exclusive_scan<<<1, kScanBlock, 0, s>>>(counts, (int64_t)kBins * n_tiles);
        k_radix_scatter<K><<<n_tiles, kSortBlock, 0, s>>>(kcur, vcur, kdst[p & 1], vdst[p & 1], n,
                                                          shift, n_tiles, counts);
        kcur = kdst[p & 1];
        vcur = vdst[p & 1];
    }
    *keys_out = kcur;
    *vals_out = vcur;
    return hipGetLastError();
}

}  // namespace

size_t radix_counts_elems(int64_t n) {
    int64_t tiles = (n + kTile - 1) / kTile;
    if (tiles < 1) tiles = 1;
    return (size_t)tiles * kBins;
}

hipError_t radix_sort_u32(const uint32_t* keys_in, const uint32_t* vals_in, int64_t n, int key_bits,
                          uint32_t* kbuf0, uint32_t* kbuf1, uint32_t* vbuf0, uint32_t* vbuf1,
                          uint32_t* counts, const uint32_t** keys_out, const uint32_t** vals_out,
                          hipStream_t s) {
    return radix_sort_impl<uint32_t>(keys_in, vals_in, n, key_bits, kbuf0, kbuf1, vbuf0, vbuf1,
                                     counts, keys_out, vals_out, s);
}

hipError_t radix_sort_u64(const uint64_t* keys_in, const uint32_t* vals_in, int64_t n, int key_bits,
                          uint64_t* kbuf0, uint64_t* kbuf1, uint32_t* vbuf0, uint32_t* vbuf1,
                          uint32_t* counts, const uint64_t** keys_out, const uint32_t** vals_out,
                          hipStream_t s) {
    return radix_sort_impl<uint64_t>(keys_in, vals_in, n, key_bits, kbuf0, kbuf1, vbuf0, vbuf1,
                                     counts, keys_out, vals_out, s);
}

}  // namespace smc
