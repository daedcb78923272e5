// Row-range implicit GEMM: the whole pair-list layer of a 3 x 3 x 3 map in one
// kernel, for c_in, c_out <= 64.
//
// "[Kernel] Add submanifold sparse 3D convolution (bf16 implicit GEMM, gfx950)",
// section "Design, and the measurements behind it": rows gathered through the
// pair lists times packed weights on mfma_f32_16x16x32_bf16, float32
// accumulation. The two-kernel pair path stores each off-centre pair's product
// row in a device-memory slab (one row per pair, a row's pairs consecutive) and
// adds a row's slab rows in the centre-tap GEMM's epilogue. Here the slab rows
// of one 256-row chunk live in LDS only:
//  * block (x, q) owns column tile q (16 NB2 output columns) and a contiguous
//    range of the compaction's 256-row chunks;
//  * the 16 waves of a block share the 26 off-centre taps, two slots each,
//    assigned by the map's tap counts (largest first, dealt in snake order
//    over the waves); a wave keeps its taps' weights for the column tile in
//    registers for the whole launch, the centre tap's weights sit in LDS;
//  * per chunk, wave w multiplies the chunk's 16 rows 16 w .. 16 w + 15 by the
//    centre weights into registers and, for each of its taps, the chunk's
//    pairs of that tap (one contiguous run of the tap's pair list, from the
//    compaction's per-chunk starts) 16 at a time, writing each pair's product
//    row to LDS at its slab row (relative to the chunk's first). After a
//    barrier each wave adds its rows' slab runs in slab order, rounds, applies
//    the ReLU and stores the rows.
// The sums are formed in the same order as in the two-kernel path (the centre
// product first, then the row's slab rows in order) from the same products, so
// both paths give the same bits, and no atomics are used. A chunk whose slab
// rows exceed the LDS window runs in several passes, each keeping the pairs
// whose slab rows fall in that pass's window.
//
// Loads are issued a chunk ahead: while chunk c is multiplied, the pair
// indices of chunk c + 1's first fragments and the per-chunk starts of chunk
// c + 2 are already in flight, so a chunk waits for one round trip (its
// gathered rows) instead of three.
#include "gemm_common.h"

#include <algorithm>

namespace smc {
namespace {

constexpr int kRowsWaves = 16;
constexpr int kRowsThreads = kRowsWaves * 64;
constexpr int kRowsChunk = 256;                                  // the compaction's chunk
constexpr int kRowsCols = kTaps + 1;                             // per-chunk table columns
constexpr int kRowsSlots = (kTaps - 1 + kRowsWaves - 1) / kRowsWaves;   // off-centre taps per wave
constexpr int kRowsSlabBytes = 128 * 1024;                       // LDS slab window
static_assert(kRowsChunk == 16 * kRowsWaves, "one centre fragment per wave and chunk");

template <int NB2>
constexpr int rows_window() { return kRowsSlabBytes / (16 * NB2 * 4); }

// Per-chunk quantities of one wave, loaded ahead of use.
struct RowsAhead {
    int32_t pa[kRowsSlots], pb[kRowsSlots];     // the chunk's run of each slot's tap list
    int32_t sb0, sb1;                           // the chunk's slab rows [sb0, sb1)
};

__device__ __forceinline__ void rows_ranges(const int32_t* __restrict__ chunk_pre, int64_t c,
                                            const int (&tap)[kRowsSlots], int64_t cap,
                                            RowsAhead& ra) {
    const int32_t* p0 = chunk_pre + c * kRowsCols;
    const int32_t* p1 = p0 + kRowsCols;
    ra.sb0 = p0[kTaps];
    ra.sb1 = p1[kTaps];
#pragma unroll
    for (int j = 0; j < kRowsSlots; ++j) {
        const int t = tap[j] < 0 ? 0 : tap[j];
        ra.pa[j] = p0[t];
        ra.pb[j] = p1[t];
    }
}

// Clamp a loaded chunk's ranges to what a valid map allows (a tap has at most
// one pair per row of the chunk; a chunk at most 26 slab rows per row), so a
// corrupt table cannot send a load out of bounds or a pass loop far.
__device__ __forceinline__ void rows_clamp(RowsAhead& ra, const int (&tap)[kRowsSlots], int64_t cap) {
#pragma unroll
    for (int j = 0; j < kRowsSlots; ++j) {
        int32_t a = ra.pa[j], b = ra.pb[j];
        a = a < 0 ? 0 : (a > cap ? (int32_t)cap : a);
        b = b < a ? a : b;
        b = b > a + kRowsChunk ? a + kRowsChunk : b;
        b = b > cap ? (int32_t)cap : b;
        if (tap[j] < 0) a = b = 0;
        ra.pa[j] = a;
        ra.pb[j] = b;
    }
    const int32_t bound = ra.sb0 + (kTaps - 1) * kRowsChunk;
    ra.sb1 = ra.sb1 < ra.sb0 ? ra.sb0 : (ra.sb1 > bound ? bound : ra.sb1);
}

// NB2 output values of one row at columns col0 .. (bf16 rounded to nearest,
// ties to even, or float), with the optional ReLU.
template <int NB2, bool OUT_F32>
__device__ __forceinline__ void rows_store(void* __restrict__ yv, int64_t row, int c_out, int col0,
                                           const float (&v)[NB2], int relu) {
    if (OUT_F32) {
        float* y = static_cast<float*>(yv) + row * c_out + col0;
        float o[NB2];
#pragma unroll
        for (int nb = 0; nb < NB2; ++nb) o[nb] = (relu && v[nb] < 0.f) ? 0.f : v[nb];
        if (NB2 == 2 && col0 + 2 <= c_out && (c_out & 1) == 0) {
            *reinterpret_cast<float2*>(y) = make_float2(o[0], o[NB2 - 1]);
        } else {
#pragma unroll
            for (int nb = 0; nb < NB2; ++nb)
                if (col0 + nb < c_out) y[nb] = o[nb];
        }
        return;
    }
    uint16_t* y = static_cast<uint16_t*>(yv) + row * c_out + col0;
    uint32_t bb[NB2];
#pragma unroll
    for (int nb = 0; nb < NB2; ++nb) {
        bb[nb] = bf16_rne_bits(v[nb]);
        if (relu && (bb[nb] & 0x8000u)) bb[nb] = 0;
    }
    if (NB2 == 2 && col0 + 2 <= c_out && (c_out & 1) == 0) {
        *reinterpret_cast<uint32_t*>(y) = bb[0] | (bb[NB2 - 1] << 16);
    } else {
#pragma unroll
        for (int nb = 0; nb < NB2; ++nb)
            if (col0 + nb < c_out) y[nb] = (uint16_t)bb[nb];
    }
}

template <int NB2, int STEPS, bool OUT_F32>
__global__ __launch_bounds__(kRowsThreads, 1) void k_gemm_rows(
    const uint16_t* __restrict__ x, int c_in, const u32x4* __restrict__ wp, int n_q, int c_out,
    const int32_t* __restrict__ pair_in, const int32_t* __restrict__ pair_slot,
    const int32_t* __restrict__ chunk_pre, const int32_t* __restrict__ rowbase,
    const MapState* __restrict__ st, int64_t cap, int64_t n, void* __restrict__ yv, int relu) {
    constexpr int kW = 16 * NB2;                  // columns of a tile
    constexpr int kWin = rows_window<NB2>();      // slab rows per pass
    constexpr int kB = STEPS * NB2 * 64;          // 16-byte words of one tap's tile weights
    extern __shared__ float s_slab[];             // [kWin][kW]
    __shared__ u32x4 s_bc[kB];                    // centre weights of the tile
    __shared__ int32_t s_tap[kRowsWaves * kRowsSlots];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int r = lane & 15, g = lane >> 4;
    const int q = blockIdx.y;
    const int64_t n_chunks = (n + kRowsChunk - 1) / kRowsChunk;
    const int64_t c_lo = (int64_t)blockIdx.x * n_chunks / gridDim.x;
    const int64_t c_hi = (int64_t)(blockIdx.x + 1) * n_chunks / gridDim.x;
    if (c_lo >= c_hi) return;                     // the whole block, before any barrier

    // packed weights: [tap][tile][k-step][nb][lane] words; this tile's start
    const u32x4* wq = wp + (int64_t)q * kB;
    for (int i = tid; i < kRowsWaves * kRowsSlots; i += kRowsThreads) s_tap[i] = -1;
    for (int i = tid; i < kB; i += kRowsThreads) s_bc[i] = wq[(int64_t)kCentre * n_q * kB + i];
    __syncthreads();
    if (w == 0) {                                 // slots: lane k ranks off-centre tap k
        const bool off = lane < kTaps && lane != kCentre;
        const int32_t cnt = off ? st->tap_count[lane] : -1;
        int rank = 0;
        for (int j = 0; j < kTaps; ++j) {
            const int32_t cj = __shfl(cnt, j, 64);
            if (j != kCentre && (cj > cnt || (cj == cnt && j < lane))) ++rank;
        }
        if (off) {
            const int slot = rank / kRowsWaves, pos = rank % kRowsWaves;
            s_tap[((slot & 1) ? kRowsWaves - 1 - pos : pos) * kRowsSlots + slot] = lane;
        }
    }
    __syncthreads();
    int tap[kRowsSlots];                          // wave-uniform
    u32x4 bw[kRowsSlots][STEPS][NB2];
#pragma unroll
    for (int j = 0; j < kRowsSlots; ++j) {
        tap[j] = __builtin_amdgcn_readfirstlane(s_tap[w * kRowsSlots + j]);
        const u32x4* src = wq + (int64_t)(tap[j] < 0 ? 0 : tap[j]) * n_q * kB + lane;
#pragma unroll
        for (int s = 0; s < STEPS; ++s)
#pragma unroll
            for (int nb = 0; nb < NB2; ++nb) bw[j][s][nb] = src[(s * NB2 + nb) * 64];
    }
    const int col0 = q * kW + r * NB2;            // this lane's first output column

    // chunk c's ranges (ra) and chunk c + 1's (rn, loaded one chunk ahead), and
    // the pair indices of each slot's first fragment of chunk c (pin0 / psl0)
    RowsAhead ra, rn;
    rows_ranges(chunk_pre, c_lo, tap, cap, ra);
    rows_clamp(ra, tap, cap);
    rows_ranges(chunk_pre, c_lo + 1 < c_hi ? c_lo + 1 : c_lo, tap, cap, rn);
    int32_t pin0[kRowsSlots], psl0[kRowsSlots];
#pragma unroll
    for (int j = 0; j < kRowsSlots; ++j) {
        const int64_t lb = (int64_t)(tap[j] < 0 ? 0 : tap[j]) * cap;
        const int32_t pr = min(ra.pa[j] + r, ra.pb[j] - 1);
        pin0[j] = pair_in[lb + (pr < 0 ? 0 : pr)];
        psl0[j] = pair_slot[lb + (pr < 0 ? 0 : pr)];
    }

    for (int64_t c = c_lo; c < c_hi; ++c) {
        const int64_t t0 = c * kRowsChunk;
        const int64_t fr0 = t0 + 16 * w;          // this wave's centre fragment
        // the centre fragment's rows and its rows' slab runs first
        u32x4 a[STEPS];
        {
            const int64_t ar = fr0 + r;
            const uint16_t* xr = x + (ar < n ? ar : n - 1) * c_in;
#pragma unroll
            for (int s = 0; s < STEPS; ++s) a[s] = load_a4<true>(xr, s * 32 + 8 * g, c_in);
        }
        int32_t rb[5];
#pragma unroll
        for (int j = 0; j < 5; ++j) {
            const int64_t row = fr0 + 4 * g + j;
            rb[j] = rowbase[row < n ? row : n];
        }
        // then slot 0's gathered rows
        int32_t pin[kRowsSlots], psl[kRowsSlots];
#pragma unroll
        for (int j = 0; j < kRowsSlots; ++j) {
            const bool live = ra.pa[j] + r < ra.pb[j];
            pin[j] = live && pin0[j] >= 0 && pin0[j] < n ? pin0[j] : 0;
            psl[j] = live ? psl0[j] : -1;
        }
        u32x4 ag[STEPS];
        {
            const uint16_t* xg = x + (int64_t)pin[0] * c_in;
#pragma unroll
            for (int s = 0; s < STEPS; ++s) ag[s] = load_a4<true>(xg, s * 32 + 8 * g, c_in);
        }
        // ahead: chunk c + 1's first pair indices, chunk c + 2's ranges
        RowsAhead rn2;
        {
            rows_clamp(rn, tap, cap);
            const int64_t c2 = c + 2 < c_hi ? c + 2 : c;
            rows_ranges(chunk_pre, c2, tap, cap, rn2);
#pragma unroll
            for (int j = 0; j < kRowsSlots; ++j) {
                const int64_t lb = (int64_t)(tap[j] < 0 ? 0 : tap[j]) * cap;
                const int32_t pr = min(rn.pa[j] + r, rn.pb[j] - 1);
                pin0[j] = pair_in[lb + (pr < 0 ? 0 : pr)];
                psl0[j] = pair_slot[lb + (pr < 0 ? 0 : pr)];
            }
        }
        float v[4][NB2];
        {
            f32x4 cc[NB2];
#pragma unroll
            for (int nb = 0; nb < NB2; ++nb) cc[nb] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < STEPS; ++s)
#pragma unroll
                for (int nb = 0; nb < NB2; ++nb)
                    cc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        as_bf16x8(a[s]), as_bf16x8(s_bc[(s * NB2 + nb) * 64 + lane]), cc[nb], 0, 0, 0);
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int nb = 0; nb < NB2; ++nb) v[j][nb] = cc[nb][j];
        }
        for (int32_t w0 = ra.sb0;; w0 += kWin) {
#pragma unroll
            for (int j = 0; j < kRowsSlots; ++j) {
                if (tap[j] < 0) continue;
                const int64_t lb = (int64_t)tap[j] * cap;
                for (int32_t p = ra.pa[j]; p < ra.pb[j]; p += 16) {
                    // slot 0's first fragment of the first pass was loaded above
                    if (j != 0 || p != ra.pa[j] || w0 != ra.sb0) {
                        const bool first = p == ra.pa[j] && w0 == ra.sb0;
                        if (!first) {
                            const bool live = p + r < ra.pb[j];
                            const int32_t pr = min(p + r, ra.pb[j] - 1);
                            const int32_t pi = pair_in[lb + pr];
                            psl[j] = live ? pair_slot[lb + pr] : -1;
                            pin[j] = live && pi >= 0 && pi < n ? pi : 0;
                        }
                        const uint16_t* xg = x + (int64_t)pin[j] * c_in;
#pragma unroll
                        for (int s = 0; s < STEPS; ++s) ag[s] = load_a4<true>(xg, s * 32 + 8 * g, c_in);
                    }
                    f32x4 co[NB2];
#pragma unroll
                    for (int nb = 0; nb < NB2; ++nb) co[nb] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int s = 0; s < STEPS; ++s)
#pragma unroll
                        for (int nb = 0; nb < NB2; ++nb)
                            co[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                                as_bf16x8(ag[s]), as_bf16x8(bw[j][s][nb]), co[nb], 0, 0, 0);
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) {
                        const int32_t sl = __shfl(psl[j], 4 * g + jj, 64);
                        const int32_t loc = sl - w0;
                        if (sl < 0 || loc < 0 || loc >= kWin) continue;
                        float* d = s_slab + loc * kW + r * NB2;
                        if (NB2 == 2) {
                            *reinterpret_cast<float2*>(d) = make_float2(co[0][jj], co[NB2 - 1][jj]);
                        } else {
                            d[0] = co[0][jj];
                        }
                    }
                }
            }
            __syncthreads();
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int32_t e0 = rb[j] > w0 ? rb[j] : w0;
                const int32_t e1 = rb[j + 1] < w0 + kWin ? rb[j + 1] : w0 + kWin;
                for (int32_t e = e0; e < e1; ++e) {
                    const float* sp = s_slab + (e - w0) * kW + r * NB2;
#pragma unroll
                    for (int nb = 0; nb < NB2; ++nb) v[j][nb] += sp[nb];
                }
            }
            __syncthreads();
            if (w0 + kWin >= ra.sb1) break;
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int64_t row = fr0 + 4 * g + j;
            if (row < n && col0 < c_out) rows_store<NB2, OUT_F32>(yv, row, c_out, col0, v[j], relu);
        }
            ra = rn;
        rows_clamp(ra, tap, cap);
        rn = rn2;
    }
}

template <typename K>
bool rows_lds_ok(K kernel, size_t bytes) {
    return hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes) == hipSuccess;
}

template <int NB2, int STEPS, bool OUT_F32>
hipError_t rows_launch(dim3 grid, hipStream_t s, const uint16_t* x, int c_in, const u32x4* wp,
                       int n_q, int c_out, const int32_t* pair_in, const int32_t* pair_slot,
                       const int32_t* chunk_pre, const int32_t* rowbase, const MapState* st,
                       int64_t cap, int64_t n, void* y, int relu) {
    constexpr size_t lds = (size_t)kRowsSlabBytes;
    static const bool ok = rows_lds_ok(k_gemm_rows<NB2, STEPS, OUT_F32>, lds);
    if (!ok) return hipErrorInvalidValue;
    launch(k_gemm_rows<NB2, STEPS, OUT_F32>, grid, kRowsThreads, lds, s, x, c_in, wp, n_q,
           c_out, pair_in, pair_slot, chunk_pre, rowbase, st, cap, n, y, relu);
    return hipGetLastError();
}

template <int NB2, int STEPS>
hipError_t rows_launch_s(dim3 grid, hipStream_t s, bool out_f32, const uint16_t* x, int c_in,
                         const u32x4* wp, int n_q, int c_out, const int32_t* pi,
                         const int32_t* ps, const int32_t* cp, const int32_t* rb,
                         const MapState* st, int64_t cap, int64_t n, void* y, int relu) {
    return out_f32 ? rows_launch<NB2, STEPS, true>(grid, s, x, c_in, wp, n_q, c_out, pi, ps, cp, rb, st, cap, n, y, relu)
                   : rows_launch<NB2, STEPS, false>(grid, s, x, c_in, wp, n_q, c_out, pi, ps, cp, rb, st, cap, n, y, relu);
}

template <int NB2>
hipError_t rows_launch_n(dim3 grid, hipStream_t s, int steps, bool out_f32, const uint16_t* x,
                         int c_in, const u32x4* wp, int n_q, int c_out, const int32_t* pi,
                         const int32_t* ps, const int32_t* cp, const int32_t* rb,
                         const MapState* st, int64_t cap, int64_t n, void* y, int relu) {
    static_assert(kRowsMaxC <= 64, "k-steps of 32 channels: 1 or 2");
    if (steps == 1)
        return rows_launch_s<NB2, 1>(grid, s, out_f32, x, c_in, wp, n_q, c_out, pi, ps, cp, rb, st, cap, n, y, relu);
    return rows_launch_s<NB2, 2>(grid, s, out_f32, x, c_in, wp, n_q, c_out, pi, ps, cp, rb, st, cap, n, y, relu);
}

}  // namespace

// Column blocks per tile of the row-range GEMM's packing, and its tiles.
static int rows_nb2(int c_out) { return c_out > 16 ? 2 : 1; }
static int rows_tiles(int c_out) { return (c_out + 16 * rows_nb2(c_out) - 1) / (16 * rows_nb2(c_out)); }

size_t rows_weight_offset(int taps, int c_in, int c_out) {
    if (!rows_eligible(taps, c_in, c_out)) return 0;
    const int steps = (c_in + 31) / 32;
    const int nbw = nbw_for(c_out);
    const int64_t n_wt = (c_out + 16 * nbw - 1) / (16 * nbw);
    // the first packing is already this one when its column blocks per wave tile agree
    if (nbw == rows_nb2(c_out)) return 0;
    return (size_t)taps * n_wt * steps * nbw * 64 * 16;
}

size_t rows_weight_bytes(int taps, int c_in, int c_out) {
    if (!rows_eligible(taps, c_in, c_out) || rows_weight_offset(taps, c_in, c_out) == 0) return 0;
    const int steps = (c_in + 31) / 32;
    return (size_t)taps * rows_tiles(c_out) * steps * rows_nb2(c_out) * 64 * 16;
}

int rows_pack_nbw(int c_out) { return rows_nb2(c_out); }

hipError_t launch_gemm_rows(const uint16_t* x, int c_in, const void* wpacked, int c_out,
                            const int32_t* pair_in, const int32_t* pair_slot,
                            const int32_t* chunk_pre, const int32_t* rowbase, const MapState* st,
                            int64_t cap, int64_t n, void* y, bool out_f32, bool relu, int n_cu,
                            hipStream_t s) {
    if (n <= 0) return hipSuccess;
    const int steps = (c_in + 31) / 32;
    const int nb2 = rows_nb2(c_out);
    const int n_q = rows_tiles(c_out);
    // one block of 16 waves per CU, all blocks resident at once; the column
    // tiles of one chunk range share a die (grid x a multiple of 8: blocks go
    // to the dies round robin by linear index, so block (x, q) is on die x mod
    // 8 for every q). Rounding x down keeps x n_q <= n_cu (rounding up put 264
    // blocks on 256 CUs at three tiles, and the last 8 ran a second round).
    int64_t gx = std::max<int64_t>(1, n_cu / n_q);
    gx = gx >= 8 ? gx / 8 * 8 : gx;
    const dim3 grid((unsigned)gx, (unsigned)n_q);
    const u32x4* wp = reinterpret_cast<const u32x4*>(static_cast<const char*>(wpacked) +
                                                     rows_weight_offset(kTaps, c_in, c_out));
    const int rl = relu ? 1 : 0;
    if (nb2 == 2)
        return rows_launch_n<2>(grid, s, steps, out_f32, x, c_in, wp, n_q, c_out, pair_in,
                                pair_slot, chunk_pre, rowbase, st, cap, n, y, rl);
    return rows_launch_n<1>(grid, s, steps, out_f32, x, c_in, wp, n_q, c_out, pair_in, pair_slot,
                            chunk_pre, rowbase, st, cap, n, y, rl);
}

}  // namespace smc
