// Decoupled look-back over per-block counts (the compaction, the strided
// output bitmap). Internal to the library.
//
// A block publishes each count as an entry (epoch << 34) | (state << 32) |
// count, state kAgg (its own count) or kIncl (its count plus every earlier
// block's); entries of other launches carry other epochs, so the table needs
// no clearing between launches. Block indices come from a ticket taken in
// launch order (or are the block index when the grid fits the device at once),
// so a block only waits for blocks that are running. Every wait is bounded:
// one that runs out flags the status word and the block goes on with an
// in-bounds (wrong) prefix.
#pragma once

#include "smc_internal.h"

namespace smc {
namespace {

constexpr uint32_t kSpinLimit = 1u << 22;
constexpr uint64_t kAgg = 1, kIncl = 2;

__device__ inline uint64_t lb_pack(uint32_t epoch, uint64_t state, uint32_t count) {
    return ((uint64_t)epoch << 34) | (state << 32) | count;
}

// Prefix of column k (k < NC) over blocks pb, pb-1, ..., read by the whole
// block: thread t < kLanes NC covers column t % NC and every kLanes-th
// predecessor starting at pb - t / NC, W of them per round trip (kLanes W
// predecessors per column per round). A round finds, per column, the nearest
// entry that holds an inclusive prefix (LDS minimum of the distance), and
// sums the entries up to and including it; columns without one go on to the
// next round. Two barriers per round: the distance minima and the "some
// column still open" flag alternate between two LDS slots by round parity,
// so a slot is reset only after every thread has read it. Every thread of the
// block must call this. The result is in s_sum[k] on return.
// spin_limit bounds the waits of each thread; wait_xor (0 in every build but
// the forced-timeout test, see smc_test_force_lookback_timeout) makes the
// block wait for an epoch no block publishes, so that every wait runs out.
template <int NC, int W, int kLanes>
__device__ void block_lookback(uint64_t* look, int64_t pb, uint32_t epoch, uint32_t* status,
                               uint32_t* s_sum, uint32_t* s_done, uint32_t spin_limit = kSpinLimit,
                               uint32_t wait_xor = 0u) {
    static_assert(kLanes * NC <= 256, "one thread per (column, lane)");
    __shared__ uint32_t s_near[2][NC];
    __shared__ uint32_t s_open[2];
    const int tid = threadIdx.x;
    const int k = tid % NC, j0 = tid / NC;
    const bool active = tid < kLanes * NC;
    const uint32_t ep = (epoch ^ wait_xor) & 0x3FFFFFFFu;
    if (tid < NC) {
        s_sum[tid] = 0;
        s_done[tid] = pb < 0 ? 1u : 0u;
        s_near[0][tid] = 0xFFFFFFFFu;
    }
    __syncthreads();
    uint32_t spins = 0;
    int r = 0;
    for (int64_t top = pb; top >= 0; top -= kLanes * W, r ^= 1) {
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
                if (++spins > spin_limit) {
                    atomicOr(status, kStSortStall);
                    e[j] = 0;
                    break;
                }
                __builtin_amdgcn_s_sleep(1);
                e[j] = __hip_atomic_load(&look[idx * NC + k], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
            if (((e[j] >> 32) & 3u) == kIncl) near = min(near, (uint32_t)(top - idx));
        }
        if (go && near != 0xFFFFFFFFu) atomicMin(&s_near[r][k], near);
        if (tid == 0) s_open[r] = 0u;
        __syncthreads();
        const uint32_t lim = go ? s_near[r][k] : 0u;
        uint32_t part = 0;
#pragma unroll
        for (int j = 0; j < W; ++j) {
            const int64_t idx = top - j0 - (int64_t)j * kLanes;
            if (go && idx >= 0 && (uint32_t)(top - idx) <= lim) part += (uint32_t)e[j];
        }
        if (part) atomicAdd(&s_sum[k], part);
        if (tid < NC) {
            if (!s_done[tid]) {
                if (s_near[r][tid] != 0xFFFFFFFFu || top - kLanes * W < 0)
                    s_done[tid] = 1u;
                else
                    s_open[r] = 1u;
            }
            s_near[r ^ 1][tid] = 0xFFFFFFFFu;     // the next round's slot
        }
        __syncthreads();
        if (!s_open[r]) break;
    }
}

}  // namespace
}  // namespace smc
