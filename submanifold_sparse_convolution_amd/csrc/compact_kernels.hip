// Compaction of the neighbour table into per-tap pair lists.
//
// Only existing (input, output) pairs are listed, grouped by tap so that a
// GEMM tile shares one weight slab, and each tap's run is padded to a
// multiple of the tile height ("[Kernel] Add submanifold sparse 3D
// convolution (bf16 implicit GEMM, gfx950)", Design "Compaction"). The
// count / scan / write split, with the scan run over the small table of
// per-(tap, chunk) counts rather than over every slot, and the totals kept
// on the device, follows that pull request's commits "move pair compaction
// from torch onto three fx kernels" and "scan the pair counts on the
// device". Rows are visited in mask-sorted order, so within a tap the pairs
// follow that order ("Sparse convolution in FP32", "Neighbour masks and
// sorted rows").
#include "smc_internal.h"

namespace smc {
namespace {

constexpr int kWaves = kChunk / 64;
constexpr int kScanThreads = 1024;

// counts layout: [27][n_chunks], tap-major
__global__ __launch_bounds__(kChunk) void k_pair_count(const uint32_t* __restrict__ perm,
                                                       const uint32_t* __restrict__ mask,
                                                       int64_t n, int n_chunks,
                                                       int32_t* __restrict__ counts) {
    __shared__ int32_t wc[kWaves][kTaps];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    int64_t s = (int64_t)blockIdx.x * kChunk + tid;
    uint32_t m = s < n ? mask[perm[s]] : 0u;
#pragma unroll
    for (int k = 0; k < kTaps; ++k) {
        uint64_t b = __ballot((m >> k) & 1u);
        if (lane == 0) wc[w][k] = __popcll(b);
    }
    __syncthreads();
    if (tid < kTaps) {
        int32_t c = 0;
#pragma unroll
        for (int j = 0; j < kWaves; ++j) c += wc[j][tid];
        counts[(int64_t)tid * n_chunks + blockIdx.x] = c;
    }
}

// One block. Per tap: exclusive scan over the chunks, tap total, padded tap
// offsets; then the chunk offsets become absolute, pad slots get -1 and each
// tile gets its tap.
__global__ __launch_bounds__(kScanThreads) void k_pair_scan(int32_t* __restrict__ counts,
                                                            int n_chunks, int tile_m,
                                                            MapState* st,
                                                            int32_t* __restrict__ pair_in,
                                                            int32_t* __restrict__ pair_out,
                                                            int32_t* __restrict__ tile_tap) {
    __shared__ int32_t wave_tot[kScanThreads / 64];
    __shared__ int32_t tap_tot[kTaps];
    __shared__ int32_t tap_off[kTaps + 1];
    __shared__ int32_t carry_s;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    for (int k = 0; k < kTaps; ++k) {
        int32_t* row = counts + (int64_t)k * n_chunks;
        if (tid == 0) carry_s = 0;
        __syncthreads();
        for (int seg = 0; seg < n_chunks; seg += kScanThreads) {
            int i = seg + tid;
            int32_t x = i < n_chunks ? row[i] : 0;
            int32_t inc = x;
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                int32_t y = __shfl_up(inc, o);
                if (lane >= o) inc += y;
            }
            if (lane == 63) wave_tot[w] = inc;
            __syncthreads();
            int32_t before = carry_s;
            for (int j = 0; j < w; ++j) before += wave_tot[j];
            if (i < n_chunks) row[i] = before + inc - x;
            __syncthreads();
            if (tid == kScanThreads - 1) carry_s = before + inc;
            __syncthreads();
        }
        if (tid == 0) tap_tot[k] = carry_s;
        __syncthreads();
    }
    if (tid == 0) {
        int32_t off = 0;
        for (int k = 0; k < kTaps; ++k) {
            tap_off[k] = off;
            st->tap_off[k] = off;
            st->tap_count[k] = tap_tot[k];
            off += (tap_tot[k] + tile_m - 1) / tile_m * tile_m;
        }
        tap_off[kTaps] = off;
        st->tap_off[kTaps] = off;
        int32_t p = 0;
        for (int k = 0; k < kTaps; ++k) p += tap_tot[k];
        st->totals[0] = p;
        st->totals[1] = off;
        st->totals[2] = off / tile_m;
    }
    __syncthreads();
    for (int k = 0; k < kTaps; ++k) {
        int32_t* row = counts + (int64_t)k * n_chunks;
        for (int i = tid; i < n_chunks; i += kScanThreads) row[i] += tap_off[k];
        for (int p = tap_off[k] + tap_tot[k] + tid; p < tap_off[k + 1]; p += kScanThreads) {
            pair_in[p] = -1;
            pair_out[p] = -1;
        }
        for (int t = tap_off[k] / tile_m + tid; t < tap_off[k + 1] / tile_m; t += kScanThreads)
            tile_tap[t] = k;
    }
}

__global__ __launch_bounds__(kChunk) void k_pair_write(const uint32_t* __restrict__ perm,
                                                       const uint32_t* __restrict__ mask,
                                                       const int32_t* __restrict__ nbr, int64_t n,
                                                       int n_chunks,
                                                       const int32_t* __restrict__ chunk_off,
                                                       int32_t* __restrict__ pair_in,
                                                       int32_t* __restrict__ pair_out) {
    __shared__ int32_t wc[kWaves][kTaps];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    int64_t s = (int64_t)blockIdx.x * kChunk + tid;
    uint32_t r = s < n ? perm[s] : 0u;
    uint32_t m = s < n ? mask[r] : 0u;
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
#pragma unroll
    for (int k = 0; k < kTaps; ++k) {
        uint64_t b = __ballot((m >> k) & 1u);
        if (lane == 0) wc[w][k] = __popcll(b);
    }
    __syncthreads();
    for (int k = 0; k < kTaps; ++k) {
        uint64_t b = __ballot((m >> k) & 1u);
        if ((m >> k) & 1u) {
            int32_t pos = chunk_off[(int64_t)k * n_chunks + blockIdx.x] + __popcll(b & below);
            for (int j = 0; j < w; ++j) pos += wc[j][k];
            pair_in[pos] = nbr[(int64_t)r * kTaps + k];
            pair_out[pos] = (int32_t)r;
        }
    }
}

}  // namespace

hipError_t launch_pair_count(const uint32_t* perm, const uint32_t* mask, int64_t n,
                             int32_t* counts, hipStream_t s) {
    int n_chunks = (int)((n + kChunk - 1) / kChunk);
    k_pair_count<<<n_chunks, kChunk, 0, s>>>(perm, mask, n, n_chunks, counts);
    return hipGetLastError();
}

hipError_t launch_pair_scan(int32_t* counts, int64_t n, int tile_m, MapState* st,
                            int32_t* pair_in, int32_t* pair_out, int32_t* tile_tap,
                            hipStream_t s) {
    int n_chunks = (int)((n + kChunk - 1) / kChunk);
    k_pair_scan<<<1, kScanThreads, 0, s>>>(counts, n_chunks, tile_m, st, pair_in, pair_out,
                                           tile_tap);
    return hipGetLastError();
}

hipError_t launch_pair_write(const uint32_t* perm, const uint32_t* mask, const int32_t* nbr,
                             int64_t n, const int32_t* chunk_off, int32_t* pair_in,
                             int32_t* pair_out, hipStream_t s) {
    int n_chunks = (int)((n + kChunk - 1) / kChunk);
    k_pair_write<<<n_chunks, kChunk, 0, s>>>(perm, mask, nbr, n, n_chunks, chunk_off, pair_in,
                                             pair_out);
    return hipGetLastError();
}

}  // namespace smc
