// Attainable-peak probes: a bf16 MFMA loop and a plain device copy. They
// compute nothing of the convolution; the benchmark times them on the same GPU to
// put the spec peaks (2.5 PFLOP/s dense bf16, 8 TB/s HBM) next to what this
// part reaches under its power and clock limits.
#include "smconv.h"
#include "smc_internal.h"

namespace smc {
namespace {

typedef __bf16 bf16x8_p __attribute__((ext_vector_type(8)));
typedef float f32x4_p __attribute__((ext_vector_type(4)));

constexpr int kProbeChains = 8;     // independent accumulators per wave: hides the MFMA latency

// Every wave runs iters (rounded up to a multiple of 16) rounds of
// kProbeChains independent 16x16x32 bf16 MFMAs on register operands, then
// writes one float per lane (the sum of its accumulators), so nothing is
// dead code.
__global__ __launch_bounds__(256) void k_probe_mfma(int64_t iters, float* __restrict__ out) {
    const int lane = threadIdx.x & 63;
    const float fa = 1.0f / (float)(lane + 1);
    bf16x8_p a, b;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        a[j] = (__bf16)(fa * (float)(j + 1));
        b[j] = (__bf16)(fa * (float)(8 - j));
    }
    // eight named accumulators: an array of them was register-allocated with
    // overlapping tuples and reshuffled every iteration
    // (distinct starting values, so no two chains are the same computation)
    f32x4_p c0 = {fa, 0.f, 0.f, 0.f}, c1 = c0 + 1.f, c2 = c0 + 2.f, c3 = c0 + 3.f, c4 = c0 + 4.f,
            c5 = c0 + 5.f, c6 = c0 + 6.f, c7 = c0 + 7.f;
    // rounds of 16 unrolled: the loop-carried accumulators are copied between
    // register tuples once per 128 MFMAs instead of once per 8
    for (int64_t i = 0; i < iters; i += 16) {
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            c0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c0, 0, 0, 0);
            c1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c1, 0, 0, 0);
            c2 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c2, 0, 0, 0);
            c3 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c3, 0, 0, 0);
            c4 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c4, 0, 0, 0);
            c5 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c5, 0, 0, 0);
            c6 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c6, 0, 0, 0);
            c7 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c7, 0, 0, 0);
        }
    }
    const f32x4_p t = c0 + c1 + c2 + c3 + c4 + c5 + c6 + c7;
    const float s = t[0] + t[1] + t[2] + t[3];
    out[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// dst[i] = src[i] over n 16-byte words, grid-stride, eight words per thread
// in flight.
typedef uint32_t u32x4_p __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void k_probe_copy(const u32x4_p* __restrict__ src,
                                                    u32x4_p* __restrict__ dst, int64_t n) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    for (; i + 7 * stride < n; i += 8 * stride) {
        u32x4_p v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = __builtin_nontemporal_load(src + i + j * stride);
#pragma unroll
        for (int j = 0; j < 8; ++j) __builtin_nontemporal_store(v[j], dst + i + j * stride);
    }
    for (; i < n; i += stride) dst[i] = src[i];
}

}  // namespace
}  // namespace smc

using namespace smc;

extern "C" {

size_t smc_probe_mfma_out_bytes(int n_cu) { return (size_t)n_cu * 2 * 256 * sizeof(float); }

int smc_probe_mfma_bf16(int64_t iters, float* out, size_t out_bytes, double* flops,
                        void* stream) {
    if (iters < 1 || !out) return SMC_ERR_ARG;
    int dev = 0, n_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return SMC_ERR_HIP;
    if (out_bytes < smc_probe_mfma_out_bytes(n_cu)) return SMC_ERR_ARG;
    const int blocks = n_cu * 2;     // two blocks of 4 waves per CU: two waves per SIMD
    launch(k_probe_mfma, dim3(blocks), dim3(256), 0, (hipStream_t)stream, iters, out);
    if (hipGetLastError() != hipSuccess) return SMC_ERR_HIP;
    const double rounds = (double)((iters + 15) / 16 * 16);
    if (flops) *flops = (double)blocks * 4 * rounds * kProbeChains * 16.0 * 16.0 * 32.0 * 2.0;
    return SMC_OK;
}

int smc_probe_copy(void* dst, const void* src, size_t bytes, void* stream) {
    if (!dst || !src || (bytes & 15) || ((uintptr_t)dst & 15) || ((uintptr_t)src & 15))
        return SMC_ERR_ARG;
    int dev = 0, n_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return SMC_ERR_HIP;
    const int64_t n = (int64_t)(bytes / 16);
    int64_t blocks = (n + 255) / 256;
    if (blocks > (int64_t)n_cu * 8) blocks = (int64_t)n_cu * 8;
    if (blocks < 1) blocks = 1;
    launch(k_probe_copy, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream,
           (const u32x4_p*)src, (u32x4_p*)dst, n);
    return hipGetLastError() == hipSuccess ? SMC_OK : SMC_ERR_HIP;
}

}  // extern "C"
