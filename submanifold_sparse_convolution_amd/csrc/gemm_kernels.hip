// Implicit GEMM over per-tap pair lists: gather -> MFMA -> scatter.
//
// "[Kernel] Add submanifold sparse 3D convolution (bf16 implicit GEMM, gfx950)", section
// "Design, and the measurements behind it", and commit d4161ef: mfma_f32_16x16x32_bf16 with
// float32 accumulation; A is read through the pair list's input rows, the result goes to the
// output rows through the pair list; weights are packed so a wave reads whole cache lines; the
// loads of a k-step are issued ahead of its MFMAs.
//
// Two kernels per layer, split by tap:
//  * k_gemm_nc: every tap but the centre, tile by tile over the pair lists.
//    Each pair's product row is stored (float32, plain stores) into its own
//    row of a partial-product slab, numbered by the compaction so that the
//    rows of one output row are consecutive;
//  * k_gemm_centre: the centre tap pairs every row with itself, so it is a
//    dense, output-stationary GEMM over consecutive rows. Its epilogue adds
//    the row's slab rows, applies the optional ReLU, rounds to bf16 (to
//    nearest, ties to even) and stores the output.
// No atomics: the pull request scatters with float32 atomic adds, which on
// this GPU (device-scope atomics resolved past the per-die L2s) cost far
// more than the slab's extra write and read.
//
// MFMA operand layout on gfx950 for v_mfma_f32_16x16x32_bf16 (lane l of the
// 64-lane wave): A holds row (l % 16), k = 8 (l / 16) .. +7; B holds column
// (l % 16), the same k; the 16x16 float result holds column (l % 16), rows
// 4 (l / 16) .. +3.
//
// Free orderings used: (1) the input channels: lane group g = l / 16 is
// given a contiguous quarter of the padded input channels, channel
// g Kp/4 + 8 s .. +7 at k-step s, so a lane walks one contiguous stretch of
// its gathered row; (2) the output columns: a wave covers WT = 16 NBW
// columns with NBW MFMA column blocks, and block nb, lane column c stands
// for output column c NBW + nb, so each lane ends up holding NBW
// consecutive output columns of its rows (one vector store per row). The
// packed weights follow both orderings.
#include "gemm_common.h"

namespace smc {
namespace {

// Packed weights: [tap][wave tile][k-step][nb][lane][8] bf16; one MFMA's B
// fragment is 1 KiB contiguous and a k-step's NBW fragments are adjacent.
__global__ __launch_bounds__(kBlock) void k_weight_pack(const uint16_t* __restrict__ w, int c_in,
                                                        int c_out, int nbw, int n_wt, int steps,
                                                        uint4* __restrict__ out) {
    int64_t t = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
    int64_t total = (int64_t)kTaps * n_wt * steps * nbw * 64;
    if (t >= total) return;
    int lane = (int)(t & 63);
    int64_t r = t >> 6;
    int nb = (int)(r % nbw);
    r /= nbw;
    int s = (int)(r % steps);
    r /= steps;
    int wt = (int)(r % n_wt);
    int tap = (int)(r / n_wt);
    int col = wt * 16 * nbw + (lane & 15) * nbw + nb;
    int k0 = (lane >> 4) * (steps * 8) + s * 8;
    uint16_t v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        int k = k0 + j;
        v[j] = (k < c_in && col < c_out) ? w[((int64_t)tap * c_in + k) * c_out + col] : (uint16_t)0;
    }
    uint4 o;
    o.x = v[0] | ((uint32_t)v[1] << 16);
    o.y = v[2] | ((uint32_t)v[3] << 16);
    o.z = v[4] | ((uint32_t)v[5] << 16);
    o.w = v[6] | ((uint32_t)v[7] << 16);
    out[t] = o;
}

// Copy n16 16-byte words of packed weights into LDS with 8 loads in flight
// per thread: whole rounds of 8 x 256 words without conditions, then the rest.
__device__ inline void stage_b(uint4* __restrict__ dst, const uint4* __restrict__ src, int n16) {
    const int full = n16 / (8 * kGemmThreads) * (8 * kGemmThreads);
    for (int i0 = threadIdx.x; i0 < full; i0 += 8 * kGemmThreads) {
        uint4 v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = src[i0 + j * kGemmThreads];
#pragma unroll
        for (int j = 0; j < 8; ++j) dst[i0 + j * kGemmThreads] = v[j];
    }
    for (int i = full + threadIdx.x; i < n16; i += kGemmThreads) dst[i] = src[i];
}

// A fragments of k-steps s0 .. s0+3 for MW gathered rows (steps past the
// last re-read the last one: valid addresses, results unused).
template <int MW, bool VEC>
__device__ __forceinline__ void load_group(const uint16_t* const (&xrow)[MW], int c_in, int steps,
                                           int s0, int g, u32x4 (&a)[4][MW]) {
    const int kq = steps * 8;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int st = min(s0 + i, steps - 1);
#pragma unroll
        for (int m = 0; m < MW; ++m) a[i][m] = load_a4<VEC>(xrow[m], g * kq + st * 8, c_in);
    }
}

// c += A (k-steps s0 .. s0+3, those below steps) x B; b points at this lane's
// word of the (tap, wave tile) fragments, in LDS or in global memory.
template <int NBW, int MW>
__device__ __forceinline__ void mma_group(const u32x4 (&a)[4][MW], const uint4* __restrict__ b,
                                          int s0, int steps, f32x4 (&c)[MW][NBW]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        if (s0 + i >= steps) break;
#pragma unroll
        for (int nb = 0; nb < NBW; ++nb) {
            const uint4 bv = b[((s0 + i) * NBW + nb) * 64];
#pragma unroll
            for (int m = 0; m < MW; ++m)
                c[m][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a[i][m]), as_bf16x8(bv),
                                                                   c[m][nb], 0, 0, 0);
        }
    }
}

// One wave: MW fragments of 16 rows times 16 NBW columns, one tap's weights.
// a holds the first group of k-steps (loaded by the caller, ahead of
// whatever it had to wait for); each later group is loaded while the
// previous one is multiplied.
template <int NBW, int MW, bool VEC>
__device__ __forceinline__ void wave_mma(const uint16_t* const (&xrow)[MW], int c_in, int steps,
                                         const uint4* __restrict__ b, int g, u32x4 (&a)[4][MW],
                                         f32x4 (&c)[MW][NBW]) {
#pragma unroll
    for (int m = 0; m < MW; ++m)
#pragma unroll
        for (int nb = 0; nb < NBW; ++nb) c[m][nb] = (f32x4){0.f, 0.f, 0.f, 0.f};
    u32x4 an[4][MW];
    for (int s0 = 0;; s0 += 8) {
        if (s0 + 4 < steps) load_group<MW, VEC>(xrow, c_in, steps, s0 + 4, g, an);
        mma_group<NBW, MW>(a, b, s0, steps, c);
        if (s0 + 4 >= steps) break;
        if (s0 + 8 < steps) load_group<MW, VEC>(xrow, c_in, steps, s0 + 8, g, a);
        mma_group<NBW, MW>(an, b, s0 + 4, steps, c);
        if (s0 + 8 >= steps) break;
    }
}

// Store NBW float values of one slab or output row (columns col0 ..).
template <int NBW>
__device__ __forceinline__ void store_f32(float* __restrict__ dst, int col0, int c_out,
                                          const float (&v)[NBW]) {
    if (NBW >= 4 && col0 + NBW <= c_out && (c_out & 3) == 0) {
#pragma unroll
        for (int q = 0; q < NBW; q += 4)
            *reinterpret_cast<float4*>(dst + q) = make_float4(v[q], v[q + 1], v[q + 2], v[q + 3]);
    } else {
#pragma unroll
        for (int nb = 0; nb < NBW; ++nb)
            if (col0 + nb < c_out) dst[nb] = v[nb];
    }
}

// Non-centre taps: blocks stride over the tiles of the 26 pair lists (tap k
// holds tap_count[k] pairs from k * cap on; the counts are read on the
// device). With LDS, the tile's weight slab is staged once for the block's
// 4 waves.
template <int NBW, bool LDS, bool VEC>
__global__ __launch_bounds__(kGemmThreads) void k_gemm_nc(
    const uint16_t* __restrict__ x, int c_in, int steps, const uint4* __restrict__ wp, int n_wt,
    int c_out, const int32_t* __restrict__ pair_in, const int32_t* __restrict__ pair_slot,
    const MapState* __restrict__ st, int64_t cap, int64_t n, float* __restrict__ part) {
    extern __shared__ uint4 s_b[];
    __shared__ int32_t s_first[kTaps + 1];      // first tile of each tap (centre: none)
    __shared__ int32_t s_cnt[kTaps];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int r = lane & 15, g = lane >> 4;
    if (threadIdx.x == 0) {
        int32_t t = 0;
        for (int k = 0; k < kTaps; ++k) {
            const int32_t c = k == kCentre ? 0 : st->tap_count[k];
            s_cnt[k] = c;
            s_first[k] = t;
            t += (c + kTileM - 1) / kTileM;
        }
        s_first[kTaps] = t;
    }
    __syncthreads();
    const int n_nc = s_first[kTaps];
    const int wt_i = blockIdx.y;
    const int col0 = wt_i * 16 * NBW + r * NBW;
    const int n16 = steps * NBW * 64;
    for (int u = blockIdx.x; u < n_nc; u += gridDim.x) {
        int tap = 0;
        while (tap + 1 < kTaps && s_first[tap + 1] <= u) ++tap;
        const int j0 = (u - s_first[tap]) * kTileM + w * 16;   // this wave's first pair in the tap
        const int cnt = s_cnt[tap];
        const int64_t base = (int64_t)tap * cap + j0;
        const int pi = pair_in[base + r];
        const int4 ps = *reinterpret_cast<const int4*>(pair_slot + base + 4 * g);
        const bool a_ok = j0 + r < cnt && pi >= 0 && pi < n;
        const uint16_t* xrow[1] = {x + (int64_t)(a_ok ? pi : 0) * c_in};
        u32x4 a[4][1];
        load_group<1, VEC>(xrow, c_in, steps, 0, g, a);   // in flight while weights are staged
        const uint4* src = wp + ((int64_t)tap * n_wt + wt_i) * n16;
        const uint4* b = src + lane;
        if (LDS) {
            __syncthreads();                    // the previous tile's reads of s_b are done
            stage_b(s_b, src, n16);
            __syncthreads();
            b = s_b + lane;
        }
        f32x4 c[1][NBW];
        wave_mma<NBW, 1, VEC>(xrow, c_in, steps, b, g, a, c);
        if (col0 >= c_out) continue;
        const int slots[4] = {ps.x, ps.y, ps.z, ps.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if (j0 + 4 * g + j >= cnt || slots[j] < 0) continue;
            float v[NBW];
#pragma unroll
            for (int nb = 0; nb < NBW; ++nb) v[nb] = c[0][nb][j];
            store_f32<NBW>(part + (int64_t)slots[j] * c_out + col0, col0, c_out, v);
        }
    }
}

// Centre tap + output. Blocks stride over tiles of 64 MW consecutive rows;
// wave w takes rows +16 MW w .. +16 MW w + 16 MW - 1. With LDS the centre
// weight slab is staged once per block. A lane's 4 output rows of a
// fragment are consecutive, so their slab rows form one consecutive run
// [rowbase[first], rowbase[last] + deg(last)). Every load that does not
// depend on another is issued first (gathered rows, run bounds, weights);
// the first kSlabBatch slab rows of the lane's runs are in flight while the
// MFMAs run, and longer runs take further batches afterwards.
constexpr int kSlabBatch = 4;

// Slab row of flat index t over a lane's MW runs [rb[m][0], rb[m][0] + len[m])
// (past the end: row 0, read but unused).
template <int MW>
__device__ __forceinline__ int32_t slab_row(const int32_t (&rb)[MW][4], const int32_t (&len)[MW],
                                            int tot, int t) {
    int32_t sr = 0;
    int before = 0;
#pragma unroll
    for (int m = 0; m < MW; ++m) {
        if (t >= before && t < before + len[m]) sr = rb[m][0] + t - before;
        before += len[m];
    }
    return t < tot ? sr : 0;
}

// kSlabBatch slab rows from flat index t0 on, NBW columns from col.
template <int NBW, int MW>
__device__ __forceinline__ void load_slab(const float* __restrict__ part, int c_out, int col,
                                          bool vec, const int32_t (&rb)[MW][4],
                                          const int32_t (&len)[MW], int tot, int t0,
                                          float (&pv)[kSlabBatch][NBW]) {
#pragma unroll
    for (int u = 0; u < kSlabBatch; ++u) {
        const float* prow = part + (int64_t)slab_row<MW>(rb, len, tot, t0 + u) * c_out + col;
        if (vec) {
#pragma unroll
            for (int q = 0; q < NBW; q += 4) {
                const float4 p4 = *reinterpret_cast<const float4*>(prow + q);
                pv[u][q] = p4.x;
                pv[u][q + 1] = p4.y;
                pv[u][q + 2] = p4.z;
                pv[u][q + 3] = p4.w;
            }
        } else {
#pragma unroll
            for (int nb = 0; nb < NBW; ++nb) pv[u][nb] = prow[col + nb < c_out ? nb : 0];
        }
    }
}

// Add slab rows t0 .. t0 + kSlabBatch - 1 (those below tot) to the output rows
// they belong to.
template <int NBW, int MW>
__device__ __forceinline__ void add_slab(const int32_t (&rb)[MW][4], const int32_t (&re)[MW],
                                         const int32_t (&len)[MW], int tot, int t0,
                                         const float (&pv)[kSlabBatch][NBW],
                                         float (&v)[MW][4][NBW]) {
#pragma unroll
    for (int u = 0; u < kSlabBatch; ++u) {
        const int t = t0 + u;
        if (t >= tot) break;
        const int32_t sl = slab_row<MW>(rb, len, tot, t);
        // every element is written (a select, not a branch): a conditional update of
        // v[m][jr] would become a dynamically indexed array in scratch memory
#pragma unroll
        for (int m = 0; m < MW; ++m) {
            const bool in_m = sl >= rb[m][0] && sl < re[m];
            const int jr = (sl >= rb[m][1]) + (sl >= rb[m][2]) + (sl >= rb[m][3]);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const bool hit = in_m && j == jr;
#pragma unroll
                for (int nb = 0; nb < NBW; ++nb) v[m][j][nb] = hit ? v[m][j][nb] + pv[u][nb] : v[m][j][nb];
            }
        }
    }
}

// Loads of one 64 MW-row tile: gathered rows (first k-group), raw run bounds
// (rowbase and mask of this lane's output rows).
template <int MW, bool VEC>
__device__ __forceinline__ void centre_tile_loads(const uint16_t* __restrict__ x, int c_in, int steps,
                                                  const uint32_t* __restrict__ mask,
                                                  const int32_t* __restrict__ rowbase, int64_t n,
                                                  int64_t row0, int r, int g,
                                                  const uint16_t* (&xrow)[MW], u32x4 (&a)[4][MW],
                                                  int32_t (&rb)[MW][4], uint32_t (&mk)[MW][4]) {
#pragma unroll
    for (int m = 0; m < MW; ++m) {
        const int64_t ir = row0 + m * 16 + r;
        xrow[m] = x + (ir < n ? ir : 0) * c_in;
    }
    load_group<MW, VEC>(xrow, c_in, steps, 0, g, a);
#pragma unroll
    for (int m = 0; m < MW; ++m)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int64_t row = row0 + m * 16 + 4 * g + j;
            const int64_t rc = row < n ? row : n - 1;
            rb[m][j] = rowbase[rc];
            mk[m][j] = mask[rc];
        }
}

// Slab runs from the raw bounds: rows past n get empty runs at the end of the
// last real row's run. Returns the lane's total slab rows.
template <int MW>
__device__ __forceinline__ int centre_runs(int64_t row0, int g, int64_t n, int32_t (&rb)[MW][4],
                                           const uint32_t (&mk)[MW][4], int32_t (&re)[MW],
                                           int32_t (&len)[MW]) {
    int tot = 0;
#pragma unroll
    for (int m = 0; m < MW; ++m) {
        int32_t e = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int64_t row = row0 + m * 16 + 4 * g + j;
            if (row < n) e = rb[m][j] + __popc(mk[m][j] & ~(1u << kCentre));
        }
#pragma unroll
        for (int j = 0; j < 4; ++j)
            if (row0 + m * 16 + 4 * g + j >= n) rb[m][j] = e;
        re[m] = e;
        len[m] = e - rb[m][0];
        tot += len[m];
    }
    return tot;
}

template <int NBW, int MW, bool OUT_F32, bool LDS, bool VEC>
__global__ __launch_bounds__(kGemmThreads) void k_gemm_centre(
    const uint16_t* __restrict__ x, int c_in, int steps, const uint4* __restrict__ wp, int n_wt,
    int c_out, const uint32_t* __restrict__ mask, const int32_t* __restrict__ rowbase, int64_t n,
    const float* __restrict__ part, void* __restrict__ yv, int relu) {
    extern __shared__ uint4 s_b[];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int r = lane & 15, g = lane >> 4;
    const int wt_i = blockIdx.y;
    const int col0 = wt_i * 16 * NBW + r * NBW;
    const int colc = col0 < c_out ? col0 : 0;     // slab column read by lanes past c_out
    const int n16 = steps * NBW * 64;
    const bool vec_part = col0 + NBW <= c_out && (c_out & 3) == 0 && NBW >= 4;
    const int64_t rows_per_tile = 64 * MW;
    const int64_t n_rt = (n + rows_per_tile - 1) / rows_per_tile;
    int64_t rt = blockIdx.x;
    if (rt >= n_rt) return;
    const uint4* src = wp + ((int64_t)kCentre * n_wt + wt_i) * n16;
    // the MFMAs read B from LDS (LDS) or from global memory: fixed at compile time
    const uint4* bmma = LDS ? static_cast<const uint4*>(s_b) + lane : src + lane;

    // first tile: every independent load is issued before any wait
    const uint16_t* xrow[MW];
    u32x4 a[4][MW];
    int32_t rb[MW][4];
    uint32_t mk[MW][4];
    int64_t row0 = rt * rows_per_tile + w * 16 * MW;
    centre_tile_loads<MW, VEC>(x, c_in, steps, mask, rowbase, n, row0, r, g, xrow, a, rb, mk);
    u32x4 bw[8];
    if (LDS) {                                    // first round of the weight slab
        const u32x4* src4 = reinterpret_cast<const u32x4*>(src);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int i = threadIdx.x + j * kGemmThreads;
            bw[j] = src4[i < n16 ? i : n16 - 1];
        }
    }
    int32_t re[MW], len[MW];
    int tot = centre_runs<MW>(row0, g, n, rb, mk, re, len);
    float pv[kSlabBatch][NBW];
    load_slab<NBW, MW>(part, c_out, colc, vec_part, rb, len, tot, 0, pv);
    if (LDS) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int i = threadIdx.x + j * kGemmThreads;
            if (i < n16) reinterpret_cast<u32x4*>(s_b)[i] = bw[j];
        }
        if (n16 > 8 * kGemmThreads)               // wide inputs: the remaining rounds
            for (int i = 8 * kGemmThreads + threadIdx.x; i < n16; i += kGemmThreads) s_b[i] = src[i];
        __syncthreads();
    }

    for (;;) {
        f32x4 c[MW][NBW];
        wave_mma<NBW, MW, VEC>(xrow, c_in, steps, bmma, g, a, c);
        float v[MW][4][NBW];
#pragma unroll
        for (int m = 0; m < MW; ++m)
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int nb = 0; nb < NBW; ++nb) v[m][j][nb] = c[m][nb][j];
        add_slab<NBW, MW>(rb, re, len, tot, 0, pv, v);
        for (int t0 = kSlabBatch; t0 < tot; t0 += kSlabBatch) {
            load_slab<NBW, MW>(part, c_out, colc, vec_part, rb, len, tot, t0, pv);
            add_slab<NBW, MW>(rb, re, len, tot, t0, pv, v);
        }
#pragma unroll
        for (int m = 0; m < MW; ++m)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int64_t row = row0 + m * 16 + 4 * g + j;
                if (row >= n || col0 >= c_out) continue;
                store_row<NBW, OUT_F32>(yv, row, c_out, col0, v[m][j], relu);
            }
        rt += gridDim.x;
        if (rt >= n_rt) break;
        row0 = rt * rows_per_tile + w * 16 * MW;
        centre_tile_loads<MW, VEC>(x, c_in, steps, mask, rowbase, n, row0, r, g, xrow, a, rb, mk);
        tot = centre_runs<MW>(row0, g, n, rb, mk, re, len);
        load_slab<NBW, MW>(part, c_out, colc, vec_part, rb, len, tot, 0, pv);
    }
}

// Largest dynamic LDS a block of these kernels may ask for.
constexpr size_t kLdsCap = 160 * 1024;

template <typename F>
bool allow_lds(F* fn, size_t bytes) {
    if (bytes <= 64 * 1024) return true;
    if (bytes > kLdsCap) return false;
    if (hipFuncSetAttribute(reinterpret_cast<const void*>(fn),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes) != hipSuccess) {
        (void)hipGetLastError();
        return false;
    }
    return true;
}

template <int NBW, bool VEC>
void launch_nc_t(dim3 grid, hipStream_t s, const uint16_t* x, int c_in, int steps,
                 const uint4* wp, int n_wt, int c_out, const int32_t* pi, const int32_t* ps,
                 const MapState* st, int64_t cap, int64_t n, float* part) {
    const size_t lds = (size_t)steps * NBW * 1024;
    if (allow_lds(k_gemm_nc<NBW, true, VEC>, lds))
        launch(k_gemm_nc<NBW, true, VEC>, grid, kGemmThreads, lds, s, x, c_in, steps, wp, n_wt, c_out,
                                                                  pi, ps, st, cap, n, part);
    else
        launch(k_gemm_nc<NBW, false, VEC>, grid, kGemmThreads, 0, s, x, c_in, steps, wp, n_wt, c_out,
                                                                 pi, ps, st, cap, n, part);
}

template <int NBW>
void launch_nc(dim3 grid, hipStream_t s, const uint16_t* x, int c_in, int steps, const uint4* wp,
               int n_wt, int c_out, const int32_t* pi, const int32_t* ps, const MapState* st,
               int64_t cap, int64_t n, float* part) {
    if ((c_in & 7) == 0)
        launch_nc_t<NBW, true>(grid, s, x, c_in, steps, wp, n_wt, c_out, pi, ps, st, cap, n, part);
    else
        launch_nc_t<NBW, false>(grid, s, x, c_in, steps, wp, n_wt, c_out, pi, ps, st, cap, n, part);
}

template <int NBW, int MW, bool OUT_F32, bool VEC>
void launch_centre_t(dim3 grid, hipStream_t s, const uint16_t* x, int c_in, int steps,
                     const uint4* wp, int n_wt, int c_out, const uint32_t* mask,
                     const int32_t* rowbase, int64_t n, const float* part, void* y, int relu) {
    const size_t lds = (size_t)steps * NBW * 1024;
    if (allow_lds(k_gemm_centre<NBW, MW, OUT_F32, true, VEC>, lds))
        launch(k_gemm_centre<NBW, MW, OUT_F32, true, VEC>, grid, kGemmThreads, lds, s, 
            x, c_in, steps, wp, n_wt, c_out, mask, rowbase, n, part, y, relu);
    else
        launch(k_gemm_centre<NBW, MW, OUT_F32, false, VEC>, grid, kGemmThreads, 0, s, 
            x, c_in, steps, wp, n_wt, c_out, mask, rowbase, n, part, y, relu);
}

template <int NBW>
void launch_centre(dim3 grid, hipStream_t s, bool out_f32, const uint16_t* x, int c_in, int steps,
                   const uint4* wp, int n_wt, int c_out, const uint32_t* mask,
                   const int32_t* rowbase, int64_t n, const float* part, void* y, int relu) {
    const bool vec = (c_in & 7) == 0;
    if (out_f32) {
        if (vec) launch_centre_t<NBW, 2, true, true>(grid, s, x, c_in, steps, wp, n_wt, c_out, mask, rowbase, n, part, y, relu);
        else launch_centre_t<NBW, 2, true, false>(grid, s, x, c_in, steps, wp, n_wt, c_out, mask, rowbase, n, part, y, relu);
    } else {
        if (vec) launch_centre_t<NBW, 2, false, true>(grid, s, x, c_in, steps, wp, n_wt, c_out, mask, rowbase, n, part, y, relu);
        else launch_centre_t<NBW, 2, false, false>(grid, s, x, c_in, steps, wp, n_wt, c_out, mask, rowbase, n, part, y, relu);
    }
}

}  // namespace

size_t packed_weight_bytes(int c_in, int c_out) {
    int64_t steps = (c_in + 31) / 32;
    int nbw = nbw_for(c_out);
    int64_t n_wt = (c_out + 16 * nbw - 1) / (16 * nbw);
    return (size_t)(kTaps * n_wt * steps * nbw * 64 * 16);
}

hipError_t launch_weight_pack(const uint16_t* w, int c_in, int c_out, void* out, hipStream_t s) {
    int steps = (c_in + 31) / 32;
    int nbw = nbw_for(c_out);
    int n_wt = (c_out + 16 * nbw - 1) / (16 * nbw);
    int64_t total = (int64_t)kTaps * n_wt * steps * nbw * 64;
    unsigned blocks = (unsigned)((total + kBlock - 1) / kBlock);
    launch(k_weight_pack, blocks, kBlock, 0, s, w, c_in, c_out, nbw, n_wt, steps, (uint4*)out);
    return hipGetLastError();
}

hipError_t launch_gemm_nc(const uint16_t* x, int c_in, const void* wpacked, int c_out,
                          const int32_t* pair_in, const int32_t* pair_slot, const MapState* st,
                          int64_t cap, int64_t n, int n_cu, float* part, hipStream_t s) {
    const int steps = (c_in + 31) / 32;
    const int nbw = nbw_for(c_out);
    const int n_wt = (c_out + 16 * nbw - 1) / (16 * nbw);
    int64_t gx = (kTaps - 1) * (cap / kTileM);     // tiles if every tap were full
    if (gx > (int64_t)n_cu * 2) gx = (int64_t)n_cu * 2;
    if (gx < 1) gx = 1;
    dim3 grid((unsigned)gx, (unsigned)n_wt);
    const uint4* wp = (const uint4*)wpacked;
    switch (nbw) {
        case 1: launch_nc<1>(grid, s, x, c_in, steps, wp, n_wt, c_out, pair_in, pair_slot, st, cap, n, part); break;
        case 2: launch_nc<2>(grid, s, x, c_in, steps, wp, n_wt, c_out, pair_in, pair_slot, st, cap, n, part); break;
        case 4: launch_nc<4>(grid, s, x, c_in, steps, wp, n_wt, c_out, pair_in, pair_slot, st, cap, n, part); break;
        default: launch_nc<8>(grid, s, x, c_in, steps, wp, n_wt, c_out, pair_in, pair_slot, st, cap, n, part); break;
    }
    return hipGetLastError();
}

hipError_t launch_gemm_centre(const uint16_t* x, int c_in, const void* wpacked, int c_out,
                              const uint32_t* mask, const int32_t* rowbase, int64_t n,
                              const float* part, void* y, bool out_f32, bool relu, int n_cu,
                              hipStream_t s) {
    if (n <= 0) return hipSuccess;
    const int steps = (c_in + 31) / 32;
    const int nbw = nbw_for(c_out);
    const int n_wt = (c_out + 16 * nbw - 1) / (16 * nbw);
    int64_t row_tiles = (n + 2 * kTileM - 1) / (2 * kTileM);   // 128-row tiles (MW = 2)
    int64_t gx = row_tiles < (int64_t)n_cu * 2 ? row_tiles : (int64_t)n_cu * 2;
    dim3 grid((unsigned)gx, (unsigned)n_wt);
    const uint4* wp = (const uint4*)wpacked;
    const int rl = relu ? 1 : 0;
    switch (nbw) {
        case 1: launch_centre<1>(grid, s, out_f32, x, c_in, steps, wp, n_wt, c_out, mask, rowbase, n, part, y, rl); break;
        case 2: launch_centre<2>(grid, s, out_f32, x, c_in, steps, wp, n_wt, c_out, mask, rowbase, n, part, y, rl); break;
        case 4: launch_centre<4>(grid, s, out_f32, x, c_in, steps, wp, n_wt, c_out, mask, rowbase, n, part, y, rl); break;
        default: launch_centre<8>(grid, s, out_f32, x, c_in, steps, wp, n_wt, c_out, mask, rowbase, n, part, y, rl); break;
    }
    return hipGetLastError();
}

}  // namespace smc
