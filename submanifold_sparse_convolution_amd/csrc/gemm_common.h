// Device helpers shared by the GEMM kernels (gemm_kernels.hip,
// masktile_kernels.hip). Internal to the library.
//
// MFMA operand layout on gfx950 for v_mfma_f32_16x16x32_bf16 (lane l of the
// 64-lane wave): A holds row (l % 16), k = 8 (l / 16) .. +7; B holds column
// (l % 16), the same k; the 16x16 float result holds column (l % 16), rows
// 4 (l / 16) .. +3.
//
// Packed weights ([tap][wave tile][k-step][nb][lane][8] bf16) assign input
// channels 32 s + 8 g .. +7 to lane group g = l / 16 at k-step s (so a load
// instruction of A reads 64 contiguous bytes per row), and output column
// c NBW + nb (plus the wave tile's base) to column block nb, lane column c
// (each lane ends up holding NBW consecutive output columns).
#pragma once

#include "smc_internal.h"

namespace smc {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));   // native vector: stays in VGPRs

constexpr int kGemmThreads = 256;   // 4 waves, 16 rows each: kTileM = 64 rows per tile

__device__ inline bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }
__device__ inline bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

inline int nbw_for(int c_out) {
    int nb = (c_out + 15) / 16;
    return nb >= 8 ? 8 : nb >= 4 ? (nb == 4 ? 4 : 8) : nb >= 2 ? (nb == 2 ? 2 : 4) : 1;
}

// 8 input channels k0..k0+7 of a gathered row. Reads that fall outside the
// data are redirected, never masked: channels past c_in read the row's own
// first channels (the packed weights are zero there, and those values are
// finite whenever the row's output is), and absent rows (pad pairs, rows past
// n) read row 0 (their output row is discarded). Only the address is
// selected, so a batch of these loads issues back to back.
template <bool VEC>
__device__ __forceinline__ uint4 load_a(const uint16_t* __restrict__ xrow, int k0, int c_in) {
    if (VEC) return *reinterpret_cast<const uint4*>(xrow + (k0 < c_in ? k0 : 0));
    uint32_t h[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) h[j] = xrow[k0 + j < c_in ? k0 + j : 0];
    return make_uint4(h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16),
                      h[6] | (h[7] << 16));
}

// The same read as load_a, as a native vector.
template <bool VEC>
__device__ __forceinline__ u32x4 load_a4(const uint16_t* __restrict__ xrow, int k0, int c_in) {
    if (VEC) return *reinterpret_cast<const u32x4*>(xrow + (k0 < c_in ? k0 : 0));
    const uint4 v = load_a<VEC>(xrow, k0, c_in);
    return (u32x4){v.x, v.y, v.z, v.w};
}

__device__ inline uint32_t bf16_rne_bits(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;   // NaN stays NaN
    u += 0x7fffu + ((u >> 16) & 1u);
    return u >> 16;
}

// Write NBW consecutive output values of one row (columns col0 ..), as bf16
// (rounded to nearest, ties to even) or float, with optional ReLU. Full
// 8-column bf16 rows go out as one 16-byte store, a plain (cached) one: the
// next layer reads the output at once, and the lines kept in the caches make
// that read cheaper (six 91k-row layers on one map: 34.1 -> 32.5 us per layer
// against streaming stores).
template <int NBW, bool OUT_F32>
__device__ __forceinline__ void store_row(void* __restrict__ yv, int64_t row, int c_out, int col0,
                                          const float (&v)[NBW], int relu) {
    const bool full = col0 + NBW <= c_out;
    if (OUT_F32) {
        float* y = static_cast<float*>(yv) + row * c_out + col0;
#pragma unroll
        for (int nb = 0; nb < NBW; ++nb)
            if (col0 + nb < c_out) y[nb] = (relu && v[nb] < 0.f) ? 0.f : v[nb];
        return;
    }
    uint16_t* y = static_cast<uint16_t*>(yv) + row * c_out + col0;
    uint32_t bb[8];
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) {
        bb[nb] = nb < NBW ? bf16_rne_bits(v[nb < NBW ? nb : 0]) : 0u;
        if (relu && (bb[nb] & 0x8000u)) bb[nb] = 0;
    }
    if (NBW == 8 && full && (c_out & 7) == 0) {
        *reinterpret_cast<u32x4*>(y) = (u32x4){bb[0] | (bb[1] << 16), bb[2] | (bb[3] << 16),
                                               bb[4] | (bb[5] << 16), bb[6] | (bb[7] << 16)};
    } else if (NBW == 4 && full && (c_out & 3) == 0) {
        *reinterpret_cast<uint2*>(y) = make_uint2(bb[0] | (bb[1] << 16), bb[2] | (bb[3] << 16));
    } else {
#pragma unroll
        for (int nb = 0; nb < NBW; ++nb)
            if (col0 + nb < c_out) y[nb] = (uint16_t)bb[nb];
    }
}

}  // namespace
}  // namespace smc
