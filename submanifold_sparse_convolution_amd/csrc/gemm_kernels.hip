// Implicit GEMM over per-tap pair lists: gather -> MFMA -> scatter.
//
// "[Kernel] Add submanifold sparse 3D convolution (bf16 implicit GEMM,
// gfx950)", Design "GEMM" and commit d4161ef: mfma_f32_16x16x32_bf16 with
// float32 accumulation; A is read through the pair list's input rows, the
// result goes to the output rows through the pair list, nothing per pair is
// materialised; weights are packed so a wave reads whole cache lines; the
// loads of a k-step are issued ahead of its MFMAs.
//
// Two kernels per layer, split by tap:
//  * k_gemm_nc: every tap but the centre, tile by tile over the pair list,
//    float32 atomic adds into a per-map accumulator;
//  * k_gemm_centre: the centre tap pairs every row with itself, so its
//    output rows are distinct and in row order: a dense, output-stationary
//    tile over consecutive rows that also adds the accumulator (only for
//    rows that have a non-centre neighbour, per their mask), applies the
//    optional ReLU, rounds to bf16 (to nearest, ties to even), stores the
//    output and clears the accumulator rows it read.
// The centre tap is the largest tap by far on sparse scans (every row has
// it), so most MACs avoid the atomic read-modify-write, and no separate
// finalize pass or accumulator clear is needed.
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

__global__ __launch_bounds__(kBlock) void k_fill_f32_zero(float* p, int64_t n) {
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x)
        p[i] = 0.0f;
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

// One wave: MW fragments of 16 rows times 16 NBW columns, one tap's weights.
// b points at this lane's word of the (tap, wave tile) fragments, in LDS or
// in global memory. A loads of 4 k-steps are issued before their MFMAs.
template <int NBW, int MW, bool VEC>
__device__ __forceinline__ void wave_mma(const uint16_t* const (&xrow)[MW], int c_in, int steps,
                                         const uint4* __restrict__ b, int lane,
                                         f32x4 (&c)[MW][NBW]) {
    const int g = lane >> 4;
    const int kq = steps * 8;
#pragma unroll
    for (int m = 0; m < MW; ++m)
#pragma unroll
        for (int nb = 0; nb < NBW; ++nb) c[m][nb] = (f32x4){0.f, 0.f, 0.f, 0.f};
    int s0 = 0;
    for (; s0 + 4 <= steps; s0 += 4) {        // groups of 4 k-steps: A loads first
        uint4 a[4][MW];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int m = 0; m < MW; ++m) a[i][m] = load_a<VEC>(xrow[m], g * kq + (s0 + i) * 8, c_in);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int nb = 0; nb < NBW; ++nb) {
                const uint4 bv = b[((s0 + i) * NBW + nb) * 64];
#pragma unroll
                for (int m = 0; m < MW; ++m)
                    c[m][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        as_bf16x8(a[i][m]), as_bf16x8(bv), c[m][nb], 0, 0, 0);
            }
    }
    for (; s0 < steps; ++s0) {                 // remaining k-steps (fewer than 4)
        uint4 a[MW];
#pragma unroll
        for (int m = 0; m < MW; ++m) a[m] = load_a<VEC>(xrow[m], g * kq + s0 * 8, c_in);
#pragma unroll
        for (int nb = 0; nb < NBW; ++nb) {
            const uint4 bv = b[(s0 * NBW + nb) * 64];
#pragma unroll
            for (int m = 0; m < MW; ++m)
                c[m][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a[m]), as_bf16x8(bv),
                                                                   c[m][nb], 0, 0, 0);
        }
    }
}

// Non-centre taps: blocks stride over the pair-list tiles other than the
// centre tap's (tile counts are read on the device). With LDS, the tile's
// weight slab is staged once for the block's 4 waves.
template <int NBW, bool LDS, bool VEC>
__global__ __launch_bounds__(kGemmThreads) void k_gemm_nc(
    const uint16_t* __restrict__ x, int c_in, int steps, const uint4* __restrict__ wp, int n_wt,
    int c_out, const int32_t* __restrict__ pair_in, const int32_t* __restrict__ pair_out,
    const int32_t* __restrict__ tile_tap, const MapState* __restrict__ st, int64_t n,
    float* __restrict__ acc) {
    extern __shared__ uint4 s_b[];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int r = lane & 15, g = lane >> 4;
    const int n_tiles = st->totals[2];
    const int c_lo = st->tap_off[kCentre] / kTileM;
    const int c_n = st->tap_off[kCentre + 1] / kTileM - c_lo;
    const int n_nc = n_tiles - c_n;
    const int wt_i = blockIdx.y;
    const int col0 = wt_i * 16 * NBW + r * NBW;
    const int n16 = steps * NBW * 64;
    const bool full = col0 + NBW <= c_out;
    for (int u = blockIdx.x; u < n_nc; u += gridDim.x) {
        const int t = u < c_lo ? u : u + c_n;
        const int tap = min(max(tile_tap[t], 0), kTaps - 1);
        const int64_t base = (int64_t)t * kTileM + w * 16;
        int in_row = pair_in[base + r];
        const int4 po = *reinterpret_cast<const int4*>(pair_out + base + 4 * g);
        if (in_row >= n) in_row = -1;           // never for a valid map
        const uint16_t* xrow[1] = {x + (int64_t)(in_row < 0 ? 0 : in_row) * c_in};
        const uint4* src = wp + ((int64_t)tap * n_wt + wt_i) * n16;
        const uint4* b = src + lane;
        if (LDS) {
            __syncthreads();                    // the previous tile's reads of s_b are done
            stage_b(s_b, src, n16);
            __syncthreads();
            b = s_b + lane;
        }
        f32x4 c[1][NBW];
        wave_mma<NBW, 1, VEC>(xrow, c_in, steps, b, lane, c);
        const int orows[4] = {po.x, po.y, po.z, po.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int orow = orows[j];
            if (orow < 0 || orow >= n || col0 >= c_out) continue;
            float* yrow = acc + (int64_t)orow * c_out + col0;
            if (full) {
#pragma unroll
                for (int nb = 0; nb < NBW; ++nb) atomicAdd(yrow + nb, c[0][nb][j]);
            } else {
#pragma unroll
                for (int nb = 0; nb < NBW; ++nb)
                    if (col0 + nb < c_out) atomicAdd(yrow + nb, c[0][nb][j]);
            }
        }
    }
}

// Centre tap + output. Blocks stride over tiles of 64 MW consecutive rows;
// wave w takes rows +16 MW w .. +16 MW w + 16 MW - 1. With LDS the centre
// weight slab is staged once per block.
template <int NBW, int MW, bool OUT_F32, bool LDS, bool VEC>
__global__ __launch_bounds__(kGemmThreads) void k_gemm_centre(
    const uint16_t* __restrict__ x, int c_in, int steps, const uint4* __restrict__ wp, int n_wt,
    int c_out, const uint32_t* __restrict__ mask, int64_t n, float* __restrict__ acc,
    void* __restrict__ yv, int relu) {
    extern __shared__ uint4 s_b[];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int r = lane & 15, g = lane >> 4;
    const int wt_i = blockIdx.y;
    const int col0 = wt_i * 16 * NBW + r * NBW;
    const int n16 = steps * NBW * 64;
    const uint4* src = wp + ((int64_t)kCentre * n_wt + wt_i) * n16;
    const uint4* b = src + lane;
    if (LDS) {
        stage_b(s_b, src, n16);
        __syncthreads();
        b = s_b + lane;
    }
    const bool full = col0 + NBW <= c_out;
    const bool vec_acc = full && (c_out & 3) == 0 && NBW >= 4;
    const int64_t rows_per_tile = 64 * MW;
    const int64_t n_rt = (n + rows_per_tile - 1) / rows_per_tile;
    for (int64_t rt = blockIdx.x; rt < n_rt; rt += gridDim.x) {
        const int64_t row0 = rt * rows_per_tile + w * 16 * MW;
        const uint16_t* xrow[MW];
#pragma unroll
        for (int m = 0; m < MW; ++m) {
            const int64_t ir = row0 + m * 16 + r;
            xrow[m] = x + (ir < n ? ir : 0) * c_in;
        }
        // masks of this lane's output rows, loaded before the MFMAs need them
        uint32_t rmask[MW][4];
#pragma unroll
        for (int m = 0; m < MW; ++m)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int64_t row = row0 + m * 16 + 4 * g + j;
                rmask[m][j] = mask[row < n ? row : n - 1];
            }
        f32x4 c[MW][NBW];
        wave_mma<NBW, MW, VEC>(xrow, c_in, steps, b, lane, c);
#pragma unroll
        for (int m = 0; m < MW; ++m) {
            // accumulator rows from the other taps: all loads first, then use
            float av[4][NBW];
            bool has[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int64_t row = row0 + m * 16 + 4 * g + j;
                has[j] = row < n && col0 < c_out && rmask[m][j] != (1u << kCentre);
                const float* arow = acc + (has[j] ? row * c_out + col0 : 0);
                if (vec_acc) {
#pragma unroll
                    for (int q = 0; q < NBW; q += 4) {
                        const float4 a4 = *reinterpret_cast<const float4*>(arow + q);
                        av[j][q] = a4.x;
                        av[j][q + 1] = a4.y;
                        av[j][q + 2] = a4.z;
                        av[j][q + 3] = a4.w;
                    }
                } else {
#pragma unroll
                    for (int nb = 0; nb < NBW; ++nb)
                        av[j][nb] = arow[has[j] && col0 + nb < c_out ? nb : 0];
                }
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int64_t row = row0 + m * 16 + 4 * g + j;
                if (row >= n || col0 >= c_out) continue;
                float v[NBW];
#pragma unroll
                for (int nb = 0; nb < NBW; ++nb) v[nb] = c[m][nb][j] + (has[j] ? av[j][nb] : 0.f);
                if (has[j]) {
                    float* arow = acc + row * c_out + col0;
                    if (vec_acc) {
#pragma unroll
                        for (int q = 0; q < NBW; q += 4)
                            *reinterpret_cast<float4*>(arow + q) = make_float4(0.f, 0.f, 0.f, 0.f);
                    } else {
#pragma unroll
                        for (int nb = 0; nb < NBW; ++nb)
                            if (col0 + nb < c_out) arow[nb] = 0.f;
                    }
                }
                if (OUT_F32) {
                    float* y = static_cast<float*>(yv) + row * c_out + col0;
#pragma unroll
                    for (int nb = 0; nb < NBW; ++nb)
                        if (col0 + nb < c_out) y[nb] = (relu && v[nb] < 0.f) ? 0.f : v[nb];
                } else {
                    uint16_t* y = static_cast<uint16_t*>(yv) + row * c_out + col0;
                    uint32_t bb[8];
#pragma unroll
                    for (int nb = 0; nb < 8; ++nb) {
                        bb[nb] = nb < NBW ? bf16_rne_bits(v[nb < NBW ? nb : 0]) : 0u;
                        if (relu && (bb[nb] & 0x8000u)) bb[nb] = 0;
                    }
                    if (NBW == 8 && full && (c_out & 7) == 0) {
                        uint4 o;
                        o.x = bb[0] | (bb[1] << 16);
                        o.y = bb[2] | (bb[3] << 16);
                        o.z = bb[4] | (bb[5] << 16);
                        o.w = bb[6] | (bb[7] << 16);
                        *reinterpret_cast<uint4*>(y) = o;
                    } else if (NBW == 4 && full && (c_out & 3) == 0) {
                        uint2 o;
                        o.x = bb[0] | (bb[1] << 16);
                        o.y = bb[2] | (bb[3] << 16);
                        *reinterpret_cast<uint2*>(y) = o;
                    } else {
#pragma unroll
                        for (int nb = 0; nb < NBW; ++nb)
                            if (col0 + nb < c_out) y[nb] = (uint16_t)bb[nb];
                    }
                }
            }
        }
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
                 const uint4* wp, int n_wt, int c_out, const int32_t* pi, const int32_t* po,
                 const int32_t* tt, const MapState* st, int64_t n, float* acc) {
    const size_t lds = (size_t)steps * NBW * 1024;
    if (allow_lds(k_gemm_nc<NBW, true, VEC>, lds))
        k_gemm_nc<NBW, true, VEC><<<grid, kGemmThreads, lds, s>>>(x, c_in, steps, wp, n_wt, c_out,
                                                                  pi, po, tt, st, n, acc);
    else
        k_gemm_nc<NBW, false, VEC><<<grid, kGemmThreads, 0, s>>>(x, c_in, steps, wp, n_wt, c_out,
                                                                 pi, po, tt, st, n, acc);
}

template <int NBW>
void launch_nc(dim3 grid, hipStream_t s, const uint16_t* x, int c_in, int steps, const uint4* wp,
               int n_wt, int c_out, const int32_t* pi, const int32_t* po, const int32_t* tt,
               const MapState* st, int64_t n, float* acc) {
    if ((c_in & 7) == 0)
        launch_nc_t<NBW, true>(grid, s, x, c_in, steps, wp, n_wt, c_out, pi, po, tt, st, n, acc);
    else
        launch_nc_t<NBW, false>(grid, s, x, c_in, steps, wp, n_wt, c_out, pi, po, tt, st, n, acc);
}

template <int NBW, int MW, bool OUT_F32, bool VEC>
void launch_centre_t(dim3 grid, hipStream_t s, const uint16_t* x, int c_in, int steps,
                     const uint4* wp, int n_wt, int c_out, const uint32_t* mask, int64_t n,
                     float* acc, void* y, int relu) {
    const size_t lds = (size_t)steps * NBW * 1024;
    if (allow_lds(k_gemm_centre<NBW, MW, OUT_F32, true, VEC>, lds))
        k_gemm_centre<NBW, MW, OUT_F32, true, VEC><<<grid, kGemmThreads, lds, s>>>(
            x, c_in, steps, wp, n_wt, c_out, mask, n, acc, y, relu);
    else
        k_gemm_centre<NBW, MW, OUT_F32, false, VEC><<<grid, kGemmThreads, 0, s>>>(
            x, c_in, steps, wp, n_wt, c_out, mask, n, acc, y, relu);
}

template <int NBW>
void launch_centre(dim3 grid, hipStream_t s, bool out_f32, const uint16_t* x, int c_in, int steps,
                   const uint4* wp, int n_wt, int c_out, const uint32_t* mask, int64_t n,
                   float* acc, void* y, int relu) {
    const bool vec = (c_in & 7) == 0;
    if (out_f32) {
        if (vec) launch_centre_t<NBW, 2, true, true>(grid, s, x, c_in, steps, wp, n_wt, c_out, mask, n, acc, y, relu);
        else launch_centre_t<NBW, 2, true, false>(grid, s, x, c_in, steps, wp, n_wt, c_out, mask, n, acc, y, relu);
    } else {
        if (vec) launch_centre_t<NBW, 2, false, true>(grid, s, x, c_in, steps, wp, n_wt, c_out, mask, n, acc, y, relu);
        else launch_centre_t<NBW, 2, false, false>(grid, s, x, c_in, steps, wp, n_wt, c_out, mask, n, acc, y, relu);
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
    k_weight_pack<<<blocks, kBlock, 0, s>>>(w, c_in, c_out, nbw, n_wt, steps, (uint4*)out);
    return hipGetLastError();
}

hipError_t launch_fill_f32(float* p, int64_t n, hipStream_t s) {
    if (n <= 0) return hipSuccess;
    int64_t b = (n + kBlock - 1) / kBlock;
    unsigned blocks = (unsigned)(b > 65536 ? 65536 : b);
    k_fill_f32_zero<<<blocks, kBlock, 0, s>>>(p, n);
    return hipGetLastError();
}

hipError_t launch_gemm_nc(const uint16_t* x, int c_in, const void* wpacked, int c_out,
                          const int32_t* pair_in, const int32_t* pair_out, const int32_t* tile_tap,
                          const MapState* st, int64_t n, int64_t max_tiles, int n_cu,
                          float* acc, hipStream_t s) {
    const int steps = (c_in + 31) / 32;
    const int nbw = nbw_for(c_out);
    const int n_wt = (c_out + 16 * nbw - 1) / (16 * nbw);
    int64_t gx = max_tiles;
    int64_t cap = (int64_t)n_cu * 2;
    if (gx > cap) gx = cap;
    if (gx < 1) gx = 1;
    dim3 grid((unsigned)gx, (unsigned)n_wt);
    const uint4* wp = (const uint4*)wpacked;
    switch (nbw) {
        case 1: launch_nc<1>(grid, s, x, c_in, steps, wp, n_wt, c_out, pair_in, pair_out, tile_tap, st, n, acc); break;
        case 2: launch_nc<2>(grid, s, x, c_in, steps, wp, n_wt, c_out, pair_in, pair_out, tile_tap, st, n, acc); break;
        case 4: launch_nc<4>(grid, s, x, c_in, steps, wp, n_wt, c_out, pair_in, pair_out, tile_tap, st, n, acc); break;
        default: launch_nc<8>(grid, s, x, c_in, steps, wp, n_wt, c_out, pair_in, pair_out, tile_tap, st, n, acc); break;
    }
    return hipGetLastError();
}

hipError_t launch_gemm_centre(const uint16_t* x, int c_in, const void* wpacked, int c_out,
                              const uint32_t* mask, int64_t n, float* acc, void* y, bool out_f32,
                              bool relu, int n_cu, hipStream_t s) {
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
        case 1: launch_centre<1>(grid, s, out_f32, x, c_in, steps, wp, n_wt, c_out, mask, n, acc, y, rl); break;
        case 2: launch_centre<2>(grid, s, out_f32, x, c_in, steps, wp, n_wt, c_out, mask, n, acc, y, rl); break;
        case 4: launch_centre<4>(grid, s, out_f32, x, c_in, steps, wp, n_wt, c_out, mask, n, acc, y, rl); break;
        default: launch_centre<8>(grid, s, out_f32, x, c_in, steps, wp, n_wt, c_out, mask, n, acc, y, rl); break;
    }
    return hipGetLastError();
}

}  // namespace smc
