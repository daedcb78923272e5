// Implicit GEMM over per-tap pair lists: gather -> MFMA -> scatter-add.
//
// "[Kernel] Add submanifold sparse 3D convolution (bf16 implicit GEMM,
// gfx950)", Design "GEMM" and commit d4161ef: mfma_f32_16x16x32_bf16 with
// float32 accumulation; A is read through the pair list's input rows, the
// result is atomically added through its output rows, nothing per pair is
// materialised; the centre tap is just another tap of the pair list; loads
// for the k-steps are issued ahead of their MFMAs; weights are packed so a
// wave reads whole cache lines.
//
// MFMA operand layout on gfx950 for v_mfma_f32_16x16x32_bf16 (per lane l of
// the 64-lane wave): A holds row (l % 16), k = 8 (l / 16) .. +7; B holds
// column (l % 16), the same k; the 16x16 float result holds column (l % 16),
// rows 4 (l / 16) .. +3.
//
// The contraction order over input channels is free, so each lane group
// g = l / 16 is given its own contiguous quarter of the (padded) input
// channels: at k-step s it takes channels g Kp/4 + 8 s .. +7. A lane then
// walks one contiguous stretch of its gathered row, and the packed weights
// use the same assignment.
#include "smc_internal.h"

namespace smc {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kGemmThreads = 256;   // 4 waves, 16 pairs each

__device__ inline bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

// Packed weights: [tap][col block of 16][k-step][lane][8] bf16, so the B
// fragment of one MFMA is 1 KiB contiguous (64 lanes x 16 bytes).
__global__ __launch_bounds__(kBlock) void k_weight_pack(const uint16_t* __restrict__ w, int c_in,
                                                        int c_out, int nb_total, int steps,
                                                        uint4* __restrict__ out) {
    int64_t t = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
    int64_t total = (int64_t)kTaps * nb_total * steps * 64;
    if (t >= total) return;
    int lane = (int)(t & 63);
    int64_t r = t >> 6;
    int s = (int)(r % steps);
    r /= steps;
    int nb = (int)(r % nb_total);
    int tap = (int)(r / nb_total);
    int col = nb * 16 + (lane & 15);
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

// 8 input channels k0..k0+7 of a gathered row, zero past c_in or for a pad pair.
__device__ inline uint4 load_a(const uint16_t* __restrict__ xrow, bool valid, int k0, int c_in,
                               bool vec) {
    uint4 z = {0u, 0u, 0u, 0u};
    if (!valid) return z;
    if (vec) {
        if (k0 < c_in) return *reinterpret_cast<const uint4*>(xrow + k0);
        return z;
    }
    uint16_t v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = (k0 + j < c_in) ? xrow[k0 + j] : (uint16_t)0;
    z.x = v[0] | ((uint32_t)v[1] << 16);
    z.y = v[2] | ((uint32_t)v[3] << 16);
    z.z = v[4] | ((uint32_t)v[5] << 16);
    z.w = v[6] | ((uint32_t)v[7] << 16);
    return z;
}

// Each wave: 16 pairs x (16 NBW) output columns. Blocks stride over the
// tiles; the tile count is read on the device, so no host read of the map's
// totals is needed before launch.
template <int NBW>
__global__ __launch_bounds__(kGemmThreads) void k_gemm(
    const uint16_t* __restrict__ x, int c_in, int steps, const uint4* __restrict__ wp, int nb_total,
    int c_out, const int32_t* __restrict__ pair_in, const int32_t* __restrict__ pair_out,
    const int32_t* __restrict__ tile_tap, const MapState* __restrict__ st,
    float* __restrict__ acc) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int r = lane & 15, g = lane >> 4;
    const int n_tiles = st->totals[2];
    const int nb0 = blockIdx.y * NBW;
    const int kq = steps * 8;
    const bool vec = (c_in & 7) == 0;
    for (int t = blockIdx.x; t < n_tiles; t += gridDim.x) {
        const int tap = tile_tap[t];
        const int64_t base = (int64_t)t * kTileM + w * 16;
        const int in_row = pair_in[base + r];
        const uint16_t* xrow = x + (int64_t)(in_row < 0 ? 0 : in_row) * c_in;
        const uint4* wt = wp + ((int64_t)tap * nb_total + nb0) * steps * 64 + lane;
        f32x4 c[NBW];
#pragma unroll
        for (int nb = 0; nb < NBW; ++nb) c[nb] = (f32x4){0.f, 0.f, 0.f, 0.f};
        for (int s = 0; s < steps; ++s) {
            uint4 a = load_a(xrow, in_row >= 0, g * kq + s * 8, c_in, vec);
            uint4 b[NBW];
#pragma unroll
            for (int nb = 0; nb < NBW; ++nb)
                if (nb0 + nb < nb_total) b[nb] = wt[((int64_t)nb * steps + s) * 64];
#pragma unroll
            for (int nb = 0; nb < NBW; ++nb)
                if (nb0 + nb < nb_total)
                    c[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(b[nb]),
                                                                    c[nb], 0, 0, 0);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int orow = pair_out[base + 4 * g + j];
            if (orow < 0) continue;
            float* yrow = acc + (int64_t)orow * c_out;
#pragma unroll
            for (int nb = 0; nb < NBW; ++nb) {
                const int col = (nb0 + nb) * 16 + r;
                if (nb0 + nb < nb_total && col < c_out) atomicAdd(yrow + col, c[nb][j]);
            }
        }
    }
}

__device__ inline uint32_t bf16_rne_bits(float f, bool relu) {
    uint32_t u = __float_as_uint(f);
    uint32_t b;
    if ((u & 0x7fffffffu) > 0x7f800000u) {
        b = 0x7fc0u;                                   // NaN stays NaN
    } else {
        u += 0x7fffu + ((u >> 16) & 1u);
        b = u >> 16;
    }
    if (relu && (b & 0x8000u)) b = 0;
    return b;
}

// y = bf16(acc) (+ReLU), and acc is left zeroed for the next layer.
__global__ __launch_bounds__(kBlock) void k_finalize(float* __restrict__ acc,
                                                     uint16_t* __restrict__ y, int64_t count,
                                                     int relu, int vec) {
    int64_t stride = (int64_t)gridDim.x * blockDim.x;
    int64_t t0 = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
    if (vec) {
        int64_t n4 = count >> 2;
        float4* a4 = reinterpret_cast<float4*>(acc);
        uint2* y4 = reinterpret_cast<uint2*>(y);
        for (int64_t i = t0; i < n4; i += stride) {
            float4 v = a4[i];
            a4[i] = make_float4(0.f, 0.f, 0.f, 0.f);
            uint2 o;
            o.x = bf16_rne_bits(v.x, relu) | (bf16_rne_bits(v.y, relu) << 16);
            o.y = bf16_rne_bits(v.z, relu) | (bf16_rne_bits(v.w, relu) << 16);
            y4[i] = o;
        }
        for (int64_t i = (n4 << 2) + t0; i < count; i += stride) {
            y[i] = (uint16_t)bf16_rne_bits(acc[i], relu);
            acc[i] = 0.f;
        }
    } else {
        for (int64_t i = t0; i < count; i += stride) {
            y[i] = (uint16_t)bf16_rne_bits(acc[i], relu);
            acc[i] = 0.f;
        }
    }
}

template <int NBW>
void gemm_launch(dim3 grid, hipStream_t s, const uint16_t* x, int c_in, int steps, const uint4* wp,
                 int nb_total, int c_out, const int32_t* pair_in, const int32_t* pair_out,
                 const int32_t* tile_tap, const MapState* st, float* acc) {
    k_gemm<NBW><<<grid, kGemmThreads, 0, s>>>(x, c_in, steps, wp, nb_total, c_out, pair_in,
                                              pair_out, tile_tap, st, acc);
}

}  // namespace

size_t packed_weight_bytes(int c_in, int c_out) {
    int64_t steps = (c_in + 31) / 32;
    int64_t nb = (c_out + 15) / 16;
    return (size_t)(kTaps * nb * steps * 64 * 16);
}

hipError_t launch_weight_pack(const uint16_t* w, int c_in, int c_out, void* out, hipStream_t s) {
    int steps = (c_in + 31) / 32;
    int nb = (c_out + 15) / 16;
    int64_t total = (int64_t)kTaps * nb * steps * 64;
    unsigned blocks = (unsigned)((total + kBlock - 1) / kBlock);
    k_weight_pack<<<blocks, kBlock, 0, s>>>(w, c_in, c_out, nb, steps, (uint4*)out);
    return hipGetLastError();
}

hipError_t launch_fill_f32(float* p, int64_t n, hipStream_t s) {
    if (n <= 0) return hipSuccess;
    int64_t b = (n + kBlock - 1) / kBlock;
    unsigned blocks = (unsigned)(b > 65536 ? 65536 : b);
    k_fill_f32_zero<<<blocks, kBlock, 0, s>>>(p, n);
    return hipGetLastError();
}

hipError_t launch_gemm(const uint16_t* x, int c_in, const void* wpacked, int c_out,
                       const int32_t* pair_in, const int32_t* pair_out, const int32_t* tile_tap,
                       const MapState* st, int64_t max_tiles, int n_cu, float* acc,
                       hipStream_t s) {
    const int steps = (c_in + 31) / 32;
    const int nb_total = (c_out + 15) / 16;
    int nbw = nb_total >= 8 ? 8 : nb_total >= 4 ? 4 : nb_total >= 2 ? 2 : 1;
    if (nbw < nb_total && nb_total < 8) nbw *= 2;
    int64_t gx = max_tiles;
    int64_t cap = (int64_t)n_cu * 8;
    if (gx > cap) gx = cap;
    if (gx < 1) gx = 1;
    dim3 grid((unsigned)gx, (unsigned)((nb_total + nbw - 1) / nbw));
    const uint4* wp = (const uint4*)wpacked;
    switch (nbw) {
        case 1: gemm_launch<1>(grid, s, x, c_in, steps, wp, nb_total, c_out, pair_in, pair_out, tile_tap, st, acc); break;
        case 2: gemm_launch<2>(grid, s, x, c_in, steps, wp, nb_total, c_out, pair_in, pair_out, tile_tap, st, acc); break;
        case 4: gemm_launch<4>(grid, s, x, c_in, steps, wp, nb_total, c_out, pair_in, pair_out, tile_tap, st, acc); break;
        default: gemm_launch<8>(grid, s, x, c_in, steps, wp, nb_total, c_out, pair_in, pair_out, tile_tap, st, acc); break;
    }
    return hipGetLastError();
}

// float32 output: y = acc (+ReLU), acc left zeroed.
__global__ __launch_bounds__(kBlock) void k_finalize_f32(float* __restrict__ acc,
                                                         float* __restrict__ y, int64_t count,
                                                         int relu) {
    int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < count; i += stride) {
        float v = acc[i];
        acc[i] = 0.f;
        y[i] = (relu && v < 0.f) ? 0.f : v;
    }
}

hipError_t launch_finalize(float* acc, void* yv, bool out_f32, int64_t count, bool relu,
                           hipStream_t s) {
    if (count <= 0) return hipSuccess;
    if (out_f32) {
        int64_t b = (count + kBlock - 1) / kBlock;
        unsigned blocks = (unsigned)(b > 16384 ? 16384 : b);
        k_finalize_f32<<<blocks, kBlock, 0, s>>>(acc, (float*)yv, count, relu ? 1 : 0);
        return hipGetLastError();
    }
    uint16_t* y = (uint16_t*)yv;
    int vec = (((uintptr_t)y & 7) == 0) ? 1 : 0;
    int64_t b = (count / 4 + kBlock - 1) / kBlock;
    if (b < 1) b = 1;
    unsigned blocks = (unsigned)(b > 16384 ? 16384 : b);
    k_finalize<<<blocks, kBlock, 0, s>>>(acc, y, count, relu ? 1 : 0, vec);
    return hipGetLastError();
}

}  // namespace smc
