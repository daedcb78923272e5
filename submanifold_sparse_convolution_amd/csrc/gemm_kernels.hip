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
// Orderings used: (1) the input channels: k-step s covers channels
// 32 s .. 32 s + 31 and lane group g = l / 16 takes 32 s + 8 g .. +7, so one
// load instruction reads 64 contiguous bytes of each of its 16 rows (a
// quarter-per-lane-group order instead spreads an instruction over 64 cache
// lines and, at C = 512, thrashes L1 across k-steps); (2) the output
// columns (a free choice): a wave covers WT = 16 NBW columns with NBW MFMA
// column blocks, and block nb, lane column c stands for output column
// c NBW + nb, so each lane ends up holding NBW consecutive output columns
// of its rows (one vector store per row). The packed weights follow both.
#include "gemm_common.h"

#include <algorithm>

namespace smc {
namespace {

// Packed weights: [tap][wave tile][k-step][nb][lane][8] bf16; one MFMA's B
// fragment is 1 KiB contiguous and a k-step's NBW fragments are adjacent.
__global__ __launch_bounds__(kBlock) void k_weight_pack(const uint16_t* __restrict__ w, int taps,
                                                        int c_in, int c_out, int nbw, int n_wt,
                                                        int steps, uint4* __restrict__ out) {
    int64_t t = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
    int64_t total = (int64_t)taps * n_wt * steps * nbw * 64;
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
    int k0 = s * 32 + (lane >> 4) * 8;
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

// A fragments of k-steps s0 .. s0+3 for MW gathered rows (steps past the
// last re-read the last one: valid addresses, results unused).
template <int MW, bool VEC>
__device__ __forceinline__ void load_group(const uint16_t* const (&xrow)[MW], int c_in, int steps,
                                           int s0, int g, u32x4 (&a)[4][MW]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int st = min(s0 + i, steps - 1);
#pragma unroll
        for (int m = 0; m < MW; ++m) a[i][m] = load_a4<VEC>(xrow[m], st * 32 + g * 8, c_in);
    }
}

constexpr int kChunk = 4;    // k-steps per streamed weight chunk (the A group size too)

// c += A (k-steps s0 .. s0+3, those below steps) x the weight chunk at b
// (this lane's word of the chunk's first fragment, in LDS).
template <int NBW, int MW>
__device__ __forceinline__ void mma_chunk(const u32x4 (&a)[4][MW], const u32x4* b, int s0, int steps,
                                          f32x4 (&c)[MW][NBW]) {
#pragma unroll
    for (int i = 0; i < kChunk; ++i) {
        if (s0 + i >= steps) break;
#pragma unroll
        for (int nb = 0; nb < NBW; ++nb) {
            const u32x4 bv = b[(i * NBW + nb) * 64];
#pragma unroll
            for (int m = 0; m < MW; ++m)
                c[m][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a[i][m]), as_bf16x8(bv),
                                                                   c[m][nb], 0, 0, 0);
        }
    }
}

// Weight words of one streamed chunk per thread.
template <int NBW>
constexpr int bg_per() { return kChunk * NBW * 64 / kGemmThreads; }

// First chunk of a weight slab into registers (issued early, before the
// caller's other waits).
template <int NBW>
__device__ __forceinline__ void bg_fetch0(const u32x4* __restrict__ src, int steps,
                                          u32x4 (&bw)[bg_per<NBW>()]) {
    const int n_words = steps * NBW * 64;
#pragma unroll
    for (int j = 0; j < bg_per<NBW>(); ++j) {
        const int i = threadIdx.x + j * kGemmThreads;
        bw[j] = src[i < n_words ? i : n_words - 1];
    }
}

// One block tile: every wave multiplies its MW row fragments (16 rows each)
// by one (tap, wave tile) weight slab src ([k-step][nb][lane] words). The
// slab streams through two LDS buffers kChunk k-steps at a time: chunk ch+1
// (weights and this wave's gathered rows) is loaded while chunk ch is
// multiplied, one barrier per chunk. The caller has loaded the first A
// group into a and the first weight chunk into bw (bg_fetch0), and must
// have finished every read of s_b from before -- unless resident: a slab of
// one chunk already in buffer 0 from the previous tile, which is reused
// as is. All threads of the block call this. Loads past the last chunk
// re-read it (valid addresses, unused), so the loop has no conditional
// loads.
template <int NBW, int MW, bool VEC, bool STREAM, int BWN>
__device__ __forceinline__ void block_gemm(const uint16_t* const (&xrow)[MW], int c_in, int steps,
                                           const u32x4* __restrict__ src, u32x4* s_b, int lane, int g,
                                           u32x4 (&a)[4][MW], u32x4 (&bw)[BWN],
                                           bool resident, f32x4 (&c)[MW][NBW]) {
    constexpr int kBufW = kChunk * NBW * 64;           // words per LDS buffer
    constexpr int kPer = bg_per<NBW>();                // words per thread per chunk
    const int tid = threadIdx.x;
    const int n_words = steps * NBW * 64;
    const int n_ch = (steps + kChunk - 1) / kChunk;
#pragma unroll
    for (int m = 0; m < MW; ++m)
#pragma unroll
        for (int nb = 0; nb < NBW; ++nb) c[m][nb] = (f32x4){0.f, 0.f, 0.f, 0.f};
    if (STREAM || !resident) {
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            const int i = tid + j * kGemmThreads;
            if (i < n_words) s_b[i] = bw[j];
        }
        __syncthreads();
    }
    if (!STREAM) {                                // one chunk (steps <= kChunk): nothing to stream
        mma_chunk<NBW, MW>(a, s_b + lane, 0, steps, c);
        return;
    }
    u32x4 an[4][MW];
// chunk CH (its weights in buffer CH & 1, rows in ACUR); prefetch chunk CH + 1 into ANEXT
#define SMC_BG_STEP(ACUR, ANEXT)                                                                  \
    {                                                                                             \
        const int nx_ = min(ch + 1, n_ch - 1);                                                    \
        _Pragma("unroll") for (int j = 0; j < kPer; ++j) {                                        \
            const int i_ = nx_ * kBufW + tid + j * kGemmThreads;                                  \
            bw[j] = src[i_ < n_words ? i_ : n_words - 1];                                         \
        }                                                                                         \
        load_group<MW, VEC>(xrow, c_in, steps, nx_ * kChunk, g, ANEXT);                           \
        mma_chunk<NBW, MW>(ACUR, s_b + (ch & 1) * kBufW + lane, ch * kChunk, steps, c);           \
        if (ch + 1 >= n_ch) break;                                                                \
        _Pragma("unroll") for (int j = 0; j < kPer; ++j) {                                        \
            const int i_ = tid + j * kGemmThreads;                                                \
            if ((ch + 1) * kBufW + i_ < n_words) s_b[((ch + 1) & 1) * kBufW + i_] = bw[j];        \
        }                                                                                         \
        __syncthreads();                                                                          \
        ++ch;                                                                                     \
    }
    int ch = 0;
    while (true) {
        SMC_BG_STEP(a, an)
        SMC_BG_STEP(an, a)
    }
#undef SMC_BG_STEP
}

// Store NBW float values of one slab row (columns col0 ..). Plain stores: the
// centre-tap GEMM that follows reads the slab, and lines kept in the caches
// make that read cheaper than the store's extra write-back costs (measured:
// 91k-row set, off-centre + centre 31.9 -> 31.6 us, wide 32.0 -> 29.9 us,
// against streaming stores).
template <int NBW>
__device__ __forceinline__ void store_f32(float* __restrict__ dst, int col0, int c_out,
                                          const float (&v)[NBW]) {
    if (NBW >= 4 && col0 + NBW <= c_out && (c_out & 3) == 0) {
#pragma unroll
        for (int q = 0; q < NBW; q += 4)
            *reinterpret_cast<f32x4*>(dst + q) = (f32x4){v[q], v[q + 1], v[q + 2], v[q + 3]};
    } else {
#pragma unroll
        for (int nb = 0; nb < NBW; ++nb)
            if (col0 + nb < c_out) dst[nb] = v[nb];
    }
}

// One pair's product row: to its slab row (slot >= 0); for the only pair of a
// strided map's output row (slot = -2 - row) straight to that row's output,
// as the sum the slab would have given (0 + product), rounded to bf16 or kept
// in float (ymode bit 0), with the optional ReLU (bit 1); slot -1: none.
template <int NBW>
__device__ __forceinline__ void pair_row_out(float* __restrict__ part, void* __restrict__ yv,
                                             int ymode, int32_t slot, int col0, int c_out,
                                             const float (&v)[NBW]) {
    if (slot >= 0) {
        store_f32<NBW>(part + (int64_t)slot * c_out + col0, col0, c_out, v);
        return;
    }
    if (slot == -1) return;
    const int64_t row = -2 - (int64_t)slot;
    float o[NBW];
#pragma unroll
    for (int nb = 0; nb < NBW; ++nb) o[nb] = 0.f + v[nb];
    if (ymode & 1)
        store_row<NBW, true>(yv, row, c_out, col0, o, ymode >> 1);
    else
        store_row<NBW, false>(yv, row, c_out, col0, o, ymode >> 1);
}

// Tile table of the taps, tiles of kRows pairs: on return s_first[k] is tap
// k's first tile (s_first[taps]: the tile count) and s_cnt[k] its pairs (the
// centre: none when skip_centre, i.e. when the centre is a dense GEMM of its
// own). Per-tap counts are read in parallel (one thread per tap), tiles per
// tap scanned over the first two waves. Every thread of the block calls this.
template <int kRows>
__device__ __forceinline__ void nc_tap_table(int taps, const MapState* __restrict__ st,
                                             int32_t* s_first, int32_t* s_cnt, int32_t* s_wave0,
                                             int skip_centre) {
    static_assert(kMaxTaps <= 128 && kGemmThreads >= 128, "two waves scan the taps");
    const int centre = taps / 2;
    const int lane = threadIdx.x & 63;
    const int k = threadIdx.x;
    int32_t tiles = 0;
    if (k < taps) {
        const int32_t c = skip_centre && k == centre ? 0 : st->tap_count[k];
        s_cnt[k] = c;
        tiles = (c + kRows - 1) / kRows;
    }
    int32_t inc = tiles;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int32_t t = __shfl_up(inc, o, 64);
        if (lane >= o) inc += t;
    }
    if (k == 63) *s_wave0 = inc;
    __syncthreads();
    const int32_t ex = inc - tiles + (k >= 64 ? *s_wave0 : 0);
    if (k < taps) s_first[k] = ex;
    if (k == taps - 1) s_first[taps] = ex + tiles;
    __syncthreads();
}

// Non-centre taps (every tap when skip_centre is 0): blocks stride over tiles
// of 64 MW pairs of one tap (tap k holds tap_count[k] pairs from k * cap on,
// cap a multiple of 256; the counts are read on the device). Each pair's
// product row goes to its slab row. n: the input rows (bounds the gathers).
template <int NBW, int MW, bool VEC, bool STREAM>
__global__ __launch_bounds__(kGemmThreads, 2) void k_gemm_nc(
    const uint16_t* __restrict__ x, int c_in, int steps, const u32x4* __restrict__ wp, int n_wt,
    int c_out, int taps, const int32_t* __restrict__ pair_in,
    const int32_t* __restrict__ pair_slot, const MapState* __restrict__ st, int64_t cap, int64_t n,
    float* __restrict__ part, int skip_centre, void* __restrict__ yv, int ymode) {
    constexpr int kRows = 64 * MW;                 // pairs per tile
    extern __shared__ u32x4 s_b[];
    __shared__ int32_t s_first[kMaxTaps + 1];     // first tile of each tap (centre: none)
    __shared__ int32_t s_cnt[kMaxTaps];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int r = lane & 15, g = lane >> 4;
    __shared__ int32_t s_wave0;
    nc_tap_table<kRows>(taps, st, s_first, s_cnt, &s_wave0, skip_centre);
    const int n_nc = s_first[taps];
    const int wt_i = blockIdx.y;
    const int col0 = wt_i * 16 * NBW + r * NBW;
    const int64_t n16 = (int64_t)steps * NBW * 64;
    int last_tap = -1;                            // tap whose one-chunk slab is in LDS
    int tap = 0;                                  // u only grows: the tap search resumes
    for (int u = blockIdx.x; u < n_nc; u += gridDim.x) {
        while (tap + 1 < taps && s_first[tap + 1] <= u) ++tap;
        const int j0 = (u - s_first[tap]) * kRows + w * 16 * MW;   // this wave's first pair
        const int cnt = s_cnt[tap];
        const int64_t base = (int64_t)tap * cap + j0;
        const uint16_t* xrow[MW];
        int4 ps[MW];
#pragma unroll
        for (int m = 0; m < MW; ++m) {
            const int pi = pair_in[base + m * 16 + r];
            ps[m] = *reinterpret_cast<const int4*>(pair_slot + base + m * 16 + 4 * g);
            const bool ok = j0 + m * 16 + r < cnt && pi >= 0 && pi < n;
            xrow[m] = x + (int64_t)(ok ? pi : 0) * c_in;
        }
        const u32x4* src = wp + ((int64_t)tap * n_wt + wt_i) * n16;
        const bool resident = !STREAM && tap == last_tap;     // a one-chunk slab stays in LDS
        last_tap = tap;
        u32x4 a[4][MW];
        load_group<MW, VEC>(xrow, c_in, steps, 0, g, a);
        u32x4 bw[bg_per<NBW>()];
        bg_fetch0<NBW>(src, steps, bw);
        if (!resident) __syncthreads();            // the previous tile's reads of s_b are done
        f32x4 c[MW][NBW];
        block_gemm<NBW, MW, VEC, STREAM, bg_per<NBW>()>(xrow, c_in, steps, src, s_b, lane, g, a, bw, resident, c);
        if (col0 >= c_out) continue;
#pragma unroll
        for (int m = 0; m < MW; ++m) {
            const int slots[4] = {ps[m].x, ps[m].y, ps[m].z, ps[m].w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                if (j0 + m * 16 + 4 * g + j >= cnt || slots[j] == -1) continue;
                float v[NBW];
#pragma unroll
                for (int nb = 0; nb < NBW; ++nb) v[nb] = c[m][nb][j];
                pair_row_out<NBW>(part, yv, ymode, slots[j], col0, c_out, v);
            }
        }
    }
}

// Centre tap + output. Blocks stride over tiles of 64 MW consecutive rows;
// wave w takes rows +16 MW w .. +16 MW w + 16 MW - 1. A lane's 4 output rows
// of a fragment are consecutive, so their slab rows form one consecutive run
// [rowbase[first], rowbase[last] + deg(last)). The tile's independent loads
// (gathered rows, run bounds) are issued first; the first slab_batch() slab
// rows of the lane's runs are in flight while the weights stream and the
// MFMAs run; longer runs take further batches afterwards. With the weights
// resident (C_in <= 128) they are staged in LDS once, before the tile loop,
// and the batch is 2, which keeps a wave within 128 registers: four waves per
// SIMD (measured on the 91k-row set: 19.6 -> 18.9 us).
template <bool STREAM>
constexpr int slab_batch() { return STREAM ? 4 : 2; }

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

// SB slab rows from flat index t0 on, NBW columns from col. Full 4-column
// groups are read with the non-temporal hint: nothing reads a slab row again,
// and the lines it would keep hold the layer's input and output (91k-row set:
// centre GEMM 16.2 -> 15.7 us).
template <int NBW, int MW, int SB>
__device__ __forceinline__ void load_slab(const float* __restrict__ part, int c_out, int col,
                                          bool vec, const int32_t (&rb)[MW][4],
                                          const int32_t (&len)[MW], int tot, int t0,
                                          float (&pv)[SB][NBW]) {
#pragma unroll
    for (int u = 0; u < SB; ++u) {
        const float* prow = part + (int64_t)slab_row<MW>(rb, len, tot, t0 + u) * c_out + col;
        if (vec) {
#pragma unroll
            for (int q = 0; q < NBW; q += 4) {
                const f32x4 p4 = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(prow + q));
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

// Add slab rows t0 .. t0 + SB - 1 (those below tot) to the output rows they
// belong to.
template <int NBW, int MW, int SB>
__device__ __forceinline__ void add_slab(const int32_t (&rb)[MW][4], const int32_t (&re)[MW],
                                         const int32_t (&len)[MW], int tot, int t0,
                                         const float (&pv)[SB][NBW],
                                         float (&v)[MW][4][NBW]) {
#pragma unroll
    for (int u = 0; u < SB; ++u) {
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
// (rowbase of this lane's 4 output rows, and the end of the last one's run:
// rowbase[row + 1], rowbase[n] being the slab's size).
template <int MW, bool VEC>
__device__ __forceinline__ void centre_tile_loads(const uint16_t* __restrict__ x, int c_in, int steps,
                                                  const int32_t* __restrict__ rowbase, int64_t n,
                                                  int64_t row0, int r, int g,
                                                  const uint16_t* (&xrow)[MW], u32x4 (&a)[4][MW],
                                                  int32_t (&rb)[MW][4], int32_t (&rend)[MW]) {
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
        }
#pragma unroll
    for (int m = 0; m < MW; ++m) {
        const int64_t e = row0 + m * 16 + 4 * g + 4;          // one past the lane's last row
        rend[m] = rowbase[e < n ? e : n];
    }
}

// Slab runs from the raw bounds: rows past n get empty runs at the end of the
// last real row's run. Returns the lane's total slab rows.
template <int MW>
__device__ __forceinline__ int centre_runs(int64_t row0, int g, int64_t n, int32_t (&rb)[MW][4],
                                           const int32_t (&rend)[MW], int32_t (&re)[MW],
                                           int32_t (&len)[MW]) {
    int tot = 0;
#pragma unroll
    for (int m = 0; m < MW; ++m) {
        const int32_t e = rend[m];
#pragma unroll
        for (int j = 0; j < 4; ++j)
            if (row0 + m * 16 + 4 * g + j >= n) rb[m][j] = e;
        re[m] = e;
        len[m] = e - rb[m][0];
        tot += len[m];
    }
    return tot;
}

template <int NBW, int MW, bool OUT_F32, bool VEC, bool STREAM>
__global__ __launch_bounds__(kGemmThreads, (STREAM && MW == 2) ? 1 : (STREAM ? 2 : 4)) void k_gemm_centre(
    const uint16_t* __restrict__ x, int c_in, int steps, const u32x4* __restrict__ wp, int n_wt,
    int c_out, int centre, const int32_t* __restrict__ rowbase, int64_t n,
    const float* __restrict__ part, void* __restrict__ yv, int relu) {
    extern __shared__ u32x4 s_b[];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int r = lane & 15, g = lane >> 4;
    const int wt_i = blockIdx.y;
    const int col0 = wt_i * 16 * NBW + r * NBW;
    const int colc = col0 < c_out ? col0 : 0;     // slab column read by lanes past c_out
    const int64_t n16 = (int64_t)steps * NBW * 64;
    const bool vec_part = col0 + NBW <= c_out && (c_out & 3) == 0 && NBW >= 4;
    const int64_t rows_per_tile = 64 * MW;
    const int64_t n_rt = (n + rows_per_tile - 1) / rows_per_tile;
    const u32x4* src = wp + ((int64_t)centre * n_wt + wt_i) * n16;
    if (!STREAM) {
        constexpr int kPer = bg_per<NBW>();
        u32x4 wv[kPer];
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            const int i = threadIdx.x + j * kGemmThreads;
            wv[j] = src[i < n16 ? i : n16 - 1];
        }
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            const int i = threadIdx.x + j * kGemmThreads;
            if (i < n16) s_b[i] = wv[j];
        }
        __syncthreads();
    }
    for (int64_t rt = blockIdx.x; rt < n_rt; rt += gridDim.x) {
        const int64_t row0 = rt * rows_per_tile + w * 16 * MW;
        const uint16_t* xrow[MW];
        u32x4 a[4][MW];
        int32_t rb[MW][4];
        int32_t rend[MW];
        const bool resident = !STREAM;                        // loaded before the loop
        centre_tile_loads<MW, VEC>(x, c_in, steps, rowbase, n, row0, r, g, xrow, a, rb, rend);
        u32x4 bw[STREAM ? bg_per<NBW>() : 1];
        if constexpr (STREAM) bg_fetch0<NBW>(src, steps, bw);
        int32_t re[MW], len[MW];
        const int tot = centre_runs<MW>(row0, g, n, rb, rend, re, len);
        constexpr int SB = slab_batch<STREAM>();
        float pv[SB][NBW];
        load_slab<NBW, MW, SB>(part, c_out, colc, vec_part, rb, len, tot, 0, pv);
        if (!resident) __syncthreads();            // the previous tile's reads of s_b are done
        f32x4 c[MW][NBW];
        block_gemm<NBW, MW, VEC, STREAM, STREAM ? bg_per<NBW>() : 1>(xrow, c_in, steps, src, s_b, lane, g, a, bw, resident, c);
        float v[MW][4][NBW];
#pragma unroll
        for (int m = 0; m < MW; ++m)
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int nb = 0; nb < NBW; ++nb) v[m][j][nb] = c[m][nb][j];
        add_slab<NBW, MW, SB>(rb, re, len, tot, 0, pv, v);
        for (int t0 = SB; t0 < tot; t0 += SB) {
            load_slab<NBW, MW, SB>(part, c_out, colc, vec_part, rb, len, tot, t0, pv);
            add_slab<NBW, MW, SB>(rb, re, len, tot, t0, pv, v);
        }
#pragma unroll
        for (int m = 0; m < MW; ++m)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int64_t row = row0 + m * 16 + 4 * g + j;
                if (row >= n || col0 >= c_out) continue;
                store_row<NBW, OUT_F32>(yv, row, c_out, col0, v[m][j], relu);
            }
    }
}

// Output rows of a map whose centre tap is a tap like the others (strided
// maps): row i is the sum of its slab rows rowbase[i] .. rowbase[i+1] - 1 in
// order, rounded to bf16 (to nearest, ties to even) or kept in float, with the
// optional ReLU. A row with no slab rows had a single pair, whose product the
// off-centre GEMM already wrote as the row's output. Thread t takes four columns (VEC4, c_out a multiple of 4) or
// one column of one row; a row's threads read each slab row contiguously.
template <bool VEC4, bool OUT_F32>
__global__ __launch_bounds__(kBlock) void k_slab_sum(const float* __restrict__ part,
                                                     const int32_t* __restrict__ rowbase, int64_t m,
                                                     int c_out, void* __restrict__ yv, int relu) {
    const int per = VEC4 ? c_out / 4 : c_out;      // threads per row
    const int64_t total = m * per;
    for (int64_t t = (int64_t)blockIdx.x * kBlock + threadIdx.x; t < total;
         t += (int64_t)gridDim.x * kBlock) {
        const int64_t row = t / per;
        const int col = (int)(t - row * per) * (VEC4 ? 4 : 1);
        const int32_t e0 = rowbase[row], e1 = rowbase[row + 1];
        if (e1 <= e0) continue;                       // one pair: the GEMM wrote the row
        float v[4] = {0.f, 0.f, 0.f, 0.f};
        for (int32_t e = e0; e < e1; ++e) {
            const float* p = part + (int64_t)e * c_out + col;
            if (VEC4) {
                const float4 q = *reinterpret_cast<const float4*>(p);
                v[0] += q.x;
                v[1] += q.y;
                v[2] += q.z;
                v[3] += q.w;
            } else {
                v[0] += p[0];
            }
        }
        if (OUT_F32) {
            float* y = static_cast<float*>(yv) + row * c_out + col;
#pragma unroll
            for (int j = 0; j < (VEC4 ? 4 : 1); ++j) y[j] = (relu && v[j] < 0.f) ? 0.f : v[j];
        } else {
            uint16_t* y = static_cast<uint16_t*>(yv) + row * c_out + col;
            uint32_t b[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                b[j] = bf16_rne_bits(v[j]);
                if (relu && (b[j] & 0x8000u)) b[j] = 0;
            }
            if (VEC4)
                *reinterpret_cast<uint2*>(y) = make_uint2(b[0] | (b[1] << 16), b[2] | (b[3] << 16));
            else
                y[0] = (uint16_t)b[0];
        }
    }
}

// ---------------------------------------------------------------------------
// Wide inputs (C_in above 128, up to kBigMaxSteps k-steps): one (tap, column
// tile) weight slab stays in LDS for the whole launch -- steps x NBW KiB, 128
// KiB at C_in = 512 -- and eight waves stream 16-row fragments through it,
// each fragment's rows loaded four k-steps at a time with the next four in
// flight. No barrier in the loops. The chunked kernels above instead stream
// the slab in 32 KiB chunks through two LDS buffers per 64-row tile, which
// pays one L2 round trip per chunk per tile.
constexpr int kBigThreads = 512;
constexpr int kBigWaves = kBigThreads / 64;
constexpr int kBigMaxSteps = 18;             // LDS: steps x NBW x 1 KiB <= 144 KiB

inline bool big_ok(int steps, int nbw) {
    return steps > kChunk && steps <= kBigMaxSteps && steps * nbw <= kBigMaxSteps * 8;
}

// k-steps s0 .. s0 + 3 of a fragment row (steps past the last re-read it).
template <bool VEC>
__device__ __forceinline__ void load_k4(const uint16_t* __restrict__ xrow, int c_in, int steps, int s0,
                                        int g, u32x4 (&a)[kChunk]) {
#pragma unroll
    for (int i = 0; i < kChunk; ++i) a[i] = load_a4<VEC>(xrow, min(s0 + i, steps - 1) * 32 + g * 8, c_in);
}

template <int NBW>
__device__ __forceinline__ void mma_k4(const u32x4 (&a)[kChunk], const u32x4* sb, int s0, int steps,
                                       f32x4 (&c)[NBW]) {
#pragma unroll
    for (int i = 0; i < kChunk; ++i) {
        if (s0 + i < steps) {
#pragma unroll
            for (int nb = 0; nb < NBW; ++nb)
                c[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    as_bf16x8(a[i]), as_bf16x8(sb[((s0 + i) * NBW + nb) * 64]), c[nb], 0, 0, 0);
        }
    }
}

// The whole k loop of one 16-row fragment, four k-steps of rows at a time with
// the next four in flight; a holds k-steps 0 .. 3 on entry (and is
// overwritten). sb: this lane's word of the slab in LDS. (Loading every k-step
// of the fragment at once, 16 per lane at C_in = 512, was slower: Deep centre
// 22.3 -> 26.1 us, off-centre 25.5 -> 31.2 us.)
template <int NBW, bool VEC>
__device__ __forceinline__ void frag_gemm(const uint16_t* __restrict__ xrow, int c_in, int steps, int g,
                                          const u32x4* sb, u32x4 (&a)[kChunk], f32x4 (&c)[NBW]) {
#pragma unroll
    for (int nb = 0; nb < NBW; ++nb) c[nb] = (f32x4){0.f, 0.f, 0.f, 0.f};
    u32x4 b[kChunk];
    for (int s0 = 0; s0 < steps; s0 += 2 * kChunk) {
        load_k4<VEC>(xrow, c_in, steps, s0 + kChunk, g, b);
        mma_k4<NBW>(a, sb, s0, steps, c);
        if (s0 + kChunk >= steps) break;
        if (s0 + 2 * kChunk < steps) load_k4<VEC>(xrow, c_in, steps, s0 + 2 * kChunk, g, a);
        mma_k4<NBW>(b, sb, s0 + kChunk, steps, c);
    }
}

// The (tap, column tile) slab of n16 words into LDS, 8 loads per thread in
// flight per round.
__device__ __forceinline__ void stage_slab(const u32x4* __restrict__ src, int n16, u32x4* s_b) {
    for (int base = 0; base < n16; base += 8 * kBigThreads) {
        u32x4 v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int i = base + (int)threadIdx.x + j * kBigThreads;
            v[j] = src[i < n16 ? i : n16 - 1];
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int i = base + (int)threadIdx.x + j * kBigThreads;
            if (i < n16) s_b[i] = v[j];
        }
    }
}

// Off-centre taps, wide inputs: work items of kBigWaves x 16 pairs of one tap
// (tap k's items from s_first[k]); block x takes the consecutive items
// [x per, (x + 1) per), per = ceil(items / gridDim.x), so it reloads the slab
// only when the tap changes. Each pair's product row goes to its slab row.
template <int NBW>
__global__ __launch_bounds__(kBigThreads, 2) void k_gemm_nc_big(
    const uint16_t* __restrict__ x, int c_in, int steps, const u32x4* __restrict__ wp, int n_wt,
    int c_out, int taps, const int32_t* __restrict__ pair_in,
    const int32_t* __restrict__ pair_slot, const MapState* __restrict__ st, int64_t cap, int64_t n,
    float* __restrict__ part, int skip_centre, void* __restrict__ yv, int ymode) {
    constexpr int kRows = kBigWaves * 16;          // pairs per item
    extern __shared__ u32x4 s_b[];
    __shared__ int32_t s_first[kMaxTaps + 1];
    __shared__ int32_t s_cnt[kMaxTaps];
    __shared__ int32_t s_wave0;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int r = lane & 15, g = lane >> 4;
    nc_tap_table<kRows>(taps, st, s_first, s_cnt, &s_wave0, skip_centre);
    const int n_items = s_first[taps];
    const int per = (n_items + (int)gridDim.x - 1) / (int)gridDim.x;
    const int u0 = (int)blockIdx.x * per;
    const int u1 = min(u0 + per, n_items);
    const int wt_i = blockIdx.y;
    const int col0 = wt_i * 16 * NBW + r * NBW;
    const int n16 = steps * NBW * 64;
    int tap = 0, slab_tap = -1;
    for (int u = u0; u < u1; ++u) {
        while (tap + 1 < taps && s_first[tap + 1] <= u) ++tap;
        const int j0 = (u - s_first[tap]) * kRows + w * 16;     // this wave's first pair
        const int cnt = s_cnt[tap];
        const int64_t base = (int64_t)tap * cap + j0;
        // the fragment's loads go out before any slab staging
        const int pi = pair_in[base + r];
        const int4 ps = *reinterpret_cast<const int4*>(pair_slot + base + 4 * g);
        const bool ok = j0 + r < cnt && pi >= 0 && pi < n;
        const uint16_t* xrow = x + (int64_t)(ok ? pi : 0) * c_in;
        u32x4 a[kChunk];
        load_k4<true>(xrow, c_in, steps, 0, g, a);
        if (tap != slab_tap) {
            __syncthreads();                       // earlier items' reads of s_b are done
            stage_slab(wp + ((int64_t)tap * n_wt + wt_i) * n16, n16, s_b);
            __syncthreads();
            slab_tap = tap;
        }
        if (j0 >= cnt) continue;                   // a wave past the tap's pairs
        f32x4 c[NBW];
        frag_gemm<NBW, true>(xrow, c_in, steps, g, s_b + lane, a, c);
        if (col0 >= c_out) continue;
        const int slots[4] = {ps.x, ps.y, ps.z, ps.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if (j0 + 4 * g + j >= cnt || slots[j] == -1) continue;
            float v[NBW];
#pragma unroll
            for (int nb = 0; nb < NBW; ++nb) v[nb] = c[nb][j];
            pair_row_out<NBW>(part, yv, ymode, slots[j], col0, c_out, v);
        }
    }
}

// Centre tap + output, wide inputs: the centre slab stays in LDS; wave
// fragments of 16 consecutive rows (fragment = global wave index, stride =
// all waves), the slab-run epilogue of the chunked kernel.
template <int NBW, bool OUT_F32>
__global__ __launch_bounds__(kBigThreads, 2) void k_gemm_centre_big(
    const uint16_t* __restrict__ x, int c_in, int steps, const u32x4* __restrict__ wp, int n_wt,
    int c_out, int centre, const int32_t* __restrict__ rowbase, int64_t n,
    const float* __restrict__ part, void* __restrict__ yv, int relu) {
    extern __shared__ u32x4 s_b[];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int r = lane & 15, g = lane >> 4;
    const int wt_i = blockIdx.y;
    const int col0 = wt_i * 16 * NBW + r * NBW;
    const int colc = col0 < c_out ? col0 : 0;
    const bool vec_part = col0 + NBW <= c_out && (c_out & 3) == 0 && NBW >= 4;
    const int n16 = steps * NBW * 64;
    const int64_t n_t = (n + 15) / 16;
    const int64_t stride = (int64_t)gridDim.x * kBigWaves;
    int64_t t = (int64_t)blockIdx.x * kBigWaves + w;
    const bool live = t < n_t;
    // a fragment's loads: its rows (k-steps 0 .. 3) and the run bounds of this lane's 4 rows
    u32x4 a[kChunk];
    const uint16_t* xr = x;
    int32_t rb[1][4], rend[1];
    auto frag_loads = [&](int64_t tt) {
        const int64_t row0 = tt * 16;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int64_t row = row0 + 4 * g + j;
            rb[0][j] = rowbase[row < n ? row : n - 1];
        }
        const int64_t e = row0 + 4 * g + 4;
        rend[0] = rowbase[e < n ? e : n];
        const int64_t ir = row0 + r;
        xr = x + (ir < n ? ir : 0) * c_in;
        load_k4<true>(xr, c_in, steps, 0, g, a);
    };
    frag_loads(live ? t : 0);
    stage_slab(wp + ((int64_t)centre * n_wt + wt_i) * n16, n16, s_b);
    __syncthreads();
    if (!live) return;
    while (true) {
        const int64_t row0 = t * 16;
        int32_t re[1], len[1];
        const int tot = centre_runs<1>(row0, g, n, rb, rend, re, len);
        constexpr int SB = 4;
        float pv[SB][NBW];
        load_slab<NBW, 1, SB>(part, c_out, colc, vec_part, rb, len, tot, 0, pv);
        f32x4 c[NBW];
        frag_gemm<NBW, true>(xr, c_in, steps, g, s_b + lane, a, c);
        const int64_t tn = t + stride;
        int32_t rbc[1][4];
#pragma unroll
        for (int j = 0; j < 4; ++j) rbc[0][j] = rb[0][j];
        if (tn < n_t) frag_loads(tn);                  // next fragment's loads before the epilogue
        float v[1][4][NBW];
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int nb = 0; nb < NBW; ++nb) v[0][j][nb] = c[nb][j];
        add_slab<NBW, 1, SB>(rbc, re, len, tot, 0, pv, v);
        for (int t0 = SB; t0 < tot; t0 += SB) {
            load_slab<NBW, 1, SB>(part, c_out, colc, vec_part, rbc, len, tot, t0, pv);
            add_slab<NBW, 1, SB>(rbc, re, len, tot, t0, pv, v);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int64_t row = row0 + 4 * g + j;
            if (row >= n || col0 >= c_out) continue;
            store_row<NBW, OUT_F32>(yv, row, c_out, col0, v[0][j], relu);
        }
        if (tn >= n_t) break;
        t = tn;
    }
}

// LDS of both kernels: two weight chunks when streaming, else one.
template <int NBW, bool STREAM>
constexpr size_t gemm_lds_bytes() { return (STREAM ? 2 : 1) * (size_t)kChunk * NBW * 64 * 16; }

// Row fragments per wave. The centre GEMM with 16-byte row loads uses 1:
// twice the blocks of 2, and registers for two blocks per CU, so the
// serial chain of a tile (row and weight loads, the slab epilogue) overlaps
// another block's (centre at C = 128: LiDAR 11.0 -> 9.4 us, the 91k-row set
// 22.5 -> 17.6 us; streamed at C = 512: forward 62.5 -> 49.7 us). Measured
// on the C = 512 set, the streamed off-centre GEMM is best at 2 (4 left too
// few blocks: 31 -> 24 us with 2); at C <= 128 it uses 1 (the pair lists of
// a sparse scan are short). A tile's loads are latency-bound at one block
// per CU: with 128 KiB of weights in LDS and every load issued at once, one
// block per CU took longer (Deep forward 62 -> 73 us) than two streaming.
inline int mw_for(int c_in) { return (c_in & 7) == 0 || (c_in + 31) / 32 <= kChunk ? 1 : 2; }
inline int mw_nc_for(int c_in) { return (c_in + 31) / 32 > kChunk && (c_in & 7) == 0 ? 2 : 1; }

// Grid x rounded up to a multiple of 8: block (x, y) is then on die x mod 8
// for every y (blocks go to the 8 dies round robin by linear index), so the
// wave tiles of one row tile share that die's L2 for the rows they gather.
inline int64_t xcd_round(int64_t gx) { return (gx + 7) / 8 * 8; }

// Lets a kernel take `bytes` of dynamic LDS (once per kernel; the default cap
// is 64 KiB including the kernel's static LDS).
template <typename K>
bool lds_ok(K kernel, size_t bytes) {
    if (bytes + 1024 <= 64 * 1024) return true;
    return hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes) == hipSuccess;
}

template <int NBW, int MW, bool VEC, bool STREAM>
void launch_nc_t(dim3 grid, hipStream_t s, const uint16_t* x, int c_in, int steps, const u32x4* wp,
                 int n_wt, int c_out, int taps, const int32_t* pi, const int32_t* ps,
                 const MapState* st, int64_t cap, int64_t n, float* part, int sc, void* y,
                 int ym) {
    constexpr size_t lds = gemm_lds_bytes<NBW, STREAM>();
    static const bool ok = lds_ok(k_gemm_nc<NBW, MW, VEC, STREAM>, lds);
    (void)ok;
    launch(k_gemm_nc<NBW, MW, VEC, STREAM>, grid, kGemmThreads, lds, s, x, c_in, steps, wp, n_wt,
           c_out, taps, pi, ps, st, cap, n, part, sc, y, ym);
}

template <int NBW>
void launch_nc(dim3 grid, hipStream_t s, int mw, const uint16_t* x, int c_in, int steps,
               const u32x4* wp, int n_wt, int c_out, int taps, const int32_t* pi,
               const int32_t* ps, const MapState* st, int64_t cap, int64_t n, float* part, int sc,
               void* y, int ym) {
    const bool vec = (c_in & 7) == 0;
    if (mw == 2)                                   // mw_nc_for: streamed, 16-byte row loads
        launch_nc_t<NBW, 2, true, true>(grid, s, x, c_in, steps, wp, n_wt, c_out, taps, pi, ps, st, cap, n, part, sc, y, ym);
    else if (steps > kChunk)
        launch_nc_t<NBW, 1, false, true>(grid, s, x, c_in, steps, wp, n_wt, c_out, taps, pi, ps, st, cap, n, part, sc, y, ym);
    else if (vec)
        launch_nc_t<NBW, 1, true, false>(grid, s, x, c_in, steps, wp, n_wt, c_out, taps, pi, ps, st, cap, n, part, sc, y, ym);
    else
        launch_nc_t<NBW, 1, false, false>(grid, s, x, c_in, steps, wp, n_wt, c_out, taps, pi, ps, st, cap, n, part, sc, y, ym);
}

template <int NBW, int MW, bool OUT_F32, bool VEC, bool STREAM>
void launch_centre_t(dim3 grid, hipStream_t s, const uint16_t* x, int c_in, int steps,
                     const u32x4* wp, int n_wt, int c_out, int centre,
                     const int32_t* rowbase, int64_t n, const float* part, void* y, int relu) {
    constexpr size_t lds = gemm_lds_bytes<NBW, STREAM>();
    static const bool ok = lds_ok(k_gemm_centre<NBW, MW, OUT_F32, VEC, STREAM>, lds);
    (void)ok;
    launch(k_gemm_centre<NBW, MW, OUT_F32, VEC, STREAM>, grid, kGemmThreads, lds, s, x, c_in,
           steps, wp, n_wt, c_out, centre, rowbase, n, part, y, relu);
}

template <int NBW, int MW, bool VEC, bool STREAM>
void launch_centre_mw(dim3 grid, hipStream_t s, bool out_f32, const uint16_t* x, int c_in,
                      int steps, const u32x4* wp, int n_wt, int c_out, int centre,
                      const int32_t* rowbase, int64_t n, const float* part, void* y, int relu) {
    if (out_f32)
        launch_centre_t<NBW, MW, true, VEC, STREAM>(grid, s, x, c_in, steps, wp, n_wt, c_out, centre, rowbase, n, part, y, relu);
    else
        launch_centre_t<NBW, MW, false, VEC, STREAM>(grid, s, x, c_in, steps, wp, n_wt, c_out, centre, rowbase, n, part, y, relu);
}

template <int NBW>
void launch_centre(dim3 grid, hipStream_t s, int mw, bool out_f32, const uint16_t* x, int c_in,
                   int steps, const u32x4* wp, int n_wt, int c_out, int centre,
                   const int32_t* rowbase, int64_t n, const float* part, void* y, int relu) {
    const bool vec = (c_in & 7) == 0;
    (void)mw;
    if (steps > kChunk && vec)                     // streamed, 16-byte row loads
        launch_centre_mw<NBW, 1, true, true>(grid, s, out_f32, x, c_in, steps, wp, n_wt, c_out, centre, rowbase, n, part, y, relu);
    else if (steps > kChunk)
        launch_centre_mw<NBW, 2, false, true>(grid, s, out_f32, x, c_in, steps, wp, n_wt, c_out, centre, rowbase, n, part, y, relu);
    else if (vec)
        launch_centre_mw<NBW, 1, true, false>(grid, s, out_f32, x, c_in, steps, wp, n_wt, c_out, centre, rowbase, n, part, y, relu);
    else
        launch_centre_mw<NBW, 1, false, false>(grid, s, out_f32, x, c_in, steps, wp, n_wt, c_out, centre, rowbase, n, part, y, relu);
}

template <int NBW>
void launch_nc_big(dim3 grid, size_t lds, hipStream_t s, const uint16_t* x, int c_in, int steps,
                   const u32x4* wp, int n_wt, int c_out, int taps, const int32_t* pi,
                   const int32_t* ps, const MapState* st, int64_t cap, int64_t n, float* part,
                   int sc, void* y, int ym) {
    static const bool ok = lds_ok(k_gemm_nc_big<NBW>, (size_t)kBigMaxSteps * 8 * 1024);
    (void)ok;
    launch(k_gemm_nc_big<NBW>, grid, kBigThreads, lds, s, x, c_in, steps, wp, n_wt, c_out, taps,
           pi, ps, st, cap, n, part, sc, y, ym);
}

template <int NBW>
void launch_centre_big(dim3 grid, size_t lds, hipStream_t s, bool out_f32, const uint16_t* x,
                       int c_in, int steps, const u32x4* wp, int n_wt, int c_out, int centre,
                       const int32_t* rowbase, int64_t n, const float* part, void* y, int relu) {
    if (out_f32) {
        static const bool ok = lds_ok(k_gemm_centre_big<NBW, true>, (size_t)kBigMaxSteps * 8 * 1024);
        (void)ok;
        launch(k_gemm_centre_big<NBW, true>, grid, kBigThreads, lds, s, x, c_in, steps, wp, n_wt,
               c_out, centre, rowbase, n, part, y, relu);
    } else {
        static const bool ok = lds_ok(k_gemm_centre_big<NBW, false>, (size_t)kBigMaxSteps * 8 * 1024);
        (void)ok;
        launch(k_gemm_centre_big<NBW, false>, grid, kBigThreads, lds, s, x, c_in, steps, wp, n_wt,
               c_out, centre, rowbase, n, part, y, relu);
    }
}

// Column blocks per wave tile of the off-centre GEMM's own packing, or 0 when it
// reads the first packing. Where one chunk of weights is resident (C_in <= 128)
// and the first packing has 8 blocks (128 columns), the off-centre kernel takes
// tiles of 64 columns: twice the blocks, each staging half the weights, and its
// gathered rows read once more from L2 (measured on the 91k-row set: 13.1 ->
// 11.8 us; the centre GEMM stays at 128 columns: 64 made it slower, 17.7 ->
// 18.1 us there and 15.8 -> 18.8 us on the 95k-row set).
int nc_pack_nbw(int c_in, int c_out) {
    return (c_in + 31) / 32 <= kChunk && nbw_for(c_out) == 8 ? 4 : 0;
}

size_t first_pack_bytes(int taps, int c_in, int c_out) {
    const int64_t steps = (c_in + 31) / 32;
    const int nbw = nbw_for(c_out);
    const int64_t n_wt = (c_out + 16 * nbw - 1) / (16 * nbw);
    return (size_t)(taps * n_wt * steps * nbw * 64 * 16);
}

size_t nc_pack_bytes(int taps, int c_in, int c_out) {
    const int nb = nc_pack_nbw(c_in, c_out);
    if (nb == 0) return 0;
    const int64_t steps = (c_in + 31) / 32;
    const int64_t n_wt = (c_out + 16 * nb - 1) / (16 * nb);
    return (size_t)(taps * n_wt * steps * nb * 64 * 16);
}

}  // namespace

// The first packing, then (where the row-range GEMM runs and needs other
// column tiles) that kernel's packing, or (nc_pack_nbw) the off-centre
// kernel's; the two never occur together (C_out <= 64 against > 64).
size_t packed_weight_bytes(int taps, int c_in, int c_out) {
    return first_pack_bytes(taps, c_in, c_out) + rows_weight_bytes(taps, c_in, c_out) +
           nc_pack_bytes(taps, c_in, c_out);
}

// The packings above, each with its own tile width.
hipError_t launch_weight_pack(const uint16_t* w, int taps, int c_in, int c_out, void* out,
                              hipStream_t s) {
    int steps = (c_in + 31) / 32;
    int nbw = nbw_for(c_out);
    int n_wt = (c_out + 16 * nbw - 1) / (16 * nbw);
    int64_t total = (int64_t)taps * n_wt * steps * nbw * 64;
    unsigned blocks = (unsigned)((total + kBlock - 1) / kBlock);
    launch(k_weight_pack, blocks, kBlock, 0, s, w, taps, c_in, c_out, nbw, n_wt, steps,
           (uint4*)out);
    if (rows_weight_bytes(taps, c_in, c_out) > 0) {
        const int nb2 = rows_pack_nbw(c_out);
        const int n_q = (c_out + 16 * nb2 - 1) / (16 * nb2);
        const int64_t total2 = (int64_t)taps * n_q * steps * nb2 * 64;
        launch(k_weight_pack, (unsigned)((total2 + kBlock - 1) / kBlock), kBlock, 0, s, w, taps,
               c_in, c_out, nb2, n_q, steps,
               (uint4*)((char*)out + rows_weight_offset(taps, c_in, c_out)));
    }
    if (nc_pack_bytes(taps, c_in, c_out) > 0) {
        const int nb3 = nc_pack_nbw(c_in, c_out);
        const int n_q = (c_out + 16 * nb3 - 1) / (16 * nb3);
        const int64_t total3 = (int64_t)taps * n_q * steps * nb3 * 64;
        launch(k_weight_pack, (unsigned)((total3 + kBlock - 1) / kBlock), kBlock, 0, s, w, taps,
               c_in, c_out, nb3, n_q, steps,
               (uint4*)((char*)out + first_pack_bytes(taps, c_in, c_out)));
    }
    return hipGetLastError();
}

hipError_t launch_gemm_nc(const uint16_t* x, int c_in, const void* wpacked, int c_out, int taps,
                          const int32_t* pair_in, const int32_t* pair_slot, const MapState* st,
                          int64_t cap, int64_t n, int n_cu, float* part, hipStream_t s,
                          bool skip_centre, void* y, bool out_f32, bool relu) {
    const int sc = skip_centre ? 1 : 0;
    const int ym = (out_f32 ? 1 : 0) | (relu ? 2 : 0);
    const int steps = (c_in + 31) / 32;
    const int nbw = nbw_for(c_out);
    const int n_wt = (c_out + 16 * nbw - 1) / (16 * nbw);
    if (big_ok(steps, nbw) && (c_in & 7) == 0) {
        // one block per CU in all, column tiles of one item range on one die
        const int64_t gx = xcd_round(std::max<int64_t>(1, n_cu / n_wt));
        const dim3 grid((unsigned)gx, (unsigned)n_wt);
        const size_t lds = (size_t)steps * nbw * 64 * 16;
        const u32x4* wp = (const u32x4*)wpacked;
        switch (nbw) {
            case 1: launch_nc_big<1>(grid, lds, s, x, c_in, steps, wp, n_wt, c_out, taps, pair_in, pair_slot, st, cap, n, part, sc, y, ym); break;
            case 2: launch_nc_big<2>(grid, lds, s, x, c_in, steps, wp, n_wt, c_out, taps, pair_in, pair_slot, st, cap, n, part, sc, y, ym); break;
            case 4: launch_nc_big<4>(grid, lds, s, x, c_in, steps, wp, n_wt, c_out, taps, pair_in, pair_slot, st, cap, n, part, sc, y, ym); break;
            default: launch_nc_big<8>(grid, lds, s, x, c_in, steps, wp, n_wt, c_out, taps, pair_in, pair_slot, st, cap, n, part, sc, y, ym); break;
        }
        return hipGetLastError();
    }
    const int mw = mw_nc_for(c_in);
    // tiles if every tap were full, at most four blocks per CU: a launch holds
    // every tile of the sets here at once (measured against two per CU: 91k-row
    // off-centre GEMM 14.1 -> 13.1 us, its strided layer's 48.5 -> 39.1 us)
    int64_t gx = (taps - 1) * (cap / (64 * mw));
    if (gx > (int64_t)n_cu * 4) gx = (int64_t)n_cu * 4;
    if (gx < 1) gx = 1;
    gx = xcd_round(gx);
    // its own packing where it has one (nc_pack_nbw), on submanifold maps: a
    // strided map's 27 taps of pair lists were slower in 64-column tiles
    // (91k-input layer 39.4 -> 51.9 us, 32k-input 20.3 -> 24.7 us)
    const int nb_own = skip_centre ? nc_pack_nbw(c_in, c_out) : 0;
    const int nbw_nc = nb_own ? nb_own : nbw;
    const int n_wt_nc = nb_own ? (c_out + 16 * nb_own - 1) / (16 * nb_own) : n_wt;
    const u32x4* wp = (const u32x4*)((const char*)wpacked +
                                     (nb_own ? first_pack_bytes(taps, c_in, c_out) : 0));
    dim3 grid((unsigned)gx, (unsigned)n_wt_nc);
    switch (nbw_nc) {
        case 1: launch_nc<1>(grid, s, mw, x, c_in, steps, wp, n_wt_nc, c_out, taps, pair_in, pair_slot, st, cap, n, part, sc, y, ym); break;
        case 2: launch_nc<2>(grid, s, mw, x, c_in, steps, wp, n_wt_nc, c_out, taps, pair_in, pair_slot, st, cap, n, part, sc, y, ym); break;
        case 4: launch_nc<4>(grid, s, mw, x, c_in, steps, wp, n_wt_nc, c_out, taps, pair_in, pair_slot, st, cap, n, part, sc, y, ym); break;
        default: launch_nc<8>(grid, s, mw, x, c_in, steps, wp, n_wt_nc, c_out, taps, pair_in, pair_slot, st, cap, n, part, sc, y, ym); break;
    }
    return hipGetLastError();
}

hipError_t launch_slab_sum(const float* part, const int32_t* rowbase, int64_t m, int c_out,
                           void* y, bool out_f32, bool relu, int n_cu, hipStream_t s) {
    if (m <= 0) return hipSuccess;
    const bool vec4 = (c_out & 3) == 0;
    const int64_t total = m * (vec4 ? c_out / 4 : c_out);
    int64_t blocks = (total + kBlock - 1) / kBlock;
    if (blocks > (int64_t)n_cu * 16) blocks = (int64_t)n_cu * 16;
    const dim3 grid((unsigned)blocks);
    const int rl = relu ? 1 : 0;
    if (vec4) {
        if (out_f32) launch(k_slab_sum<true, true>, grid, kBlock, 0, s, part, rowbase, m, c_out, y, rl);
        else launch(k_slab_sum<true, false>, grid, kBlock, 0, s, part, rowbase, m, c_out, y, rl);
    } else {
        if (out_f32) launch(k_slab_sum<false, true>, grid, kBlock, 0, s, part, rowbase, m, c_out, y, rl);
        else launch(k_slab_sum<false, false>, grid, kBlock, 0, s, part, rowbase, m, c_out, y, rl);
    }
    return hipGetLastError();
}

hipError_t launch_gemm_centre(const uint16_t* x, int c_in, const void* wpacked, int c_out,
                              int taps, const int32_t* rowbase, int64_t n, const float* part,
                              void* y, bool out_f32, bool relu, int n_cu, hipStream_t s) {
    const int centre = taps / 2;
    if (n <= 0) return hipSuccess;
    const int steps = (c_in + 31) / 32;
    const int nbw = nbw_for(c_out);
    const int n_wt = (c_out + 16 * nbw - 1) / (16 * nbw);
    if (big_ok(steps, nbw) && (c_in & 7) == 0) {
        const int64_t frags = (n + 15) / 16;
        const int64_t need = (frags + kBigWaves - 1) / kBigWaves;
        const int64_t gx = xcd_round(std::min<int64_t>(need, std::max<int64_t>(1, n_cu / n_wt)));
        const dim3 grid((unsigned)gx, (unsigned)n_wt);
        const size_t lds = (size_t)steps * nbw * 64 * 16;
        const u32x4* wp = (const u32x4*)wpacked;
        const int rl = relu ? 1 : 0;
        switch (nbw) {
            case 1: launch_centre_big<1>(grid, lds, s, out_f32, x, c_in, steps, wp, n_wt, c_out, centre, rowbase, n, part, y, rl); break;
            case 2: launch_centre_big<2>(grid, lds, s, out_f32, x, c_in, steps, wp, n_wt, c_out, centre, rowbase, n, part, y, rl); break;
            case 4: launch_centre_big<4>(grid, lds, s, out_f32, x, c_in, steps, wp, n_wt, c_out, centre, rowbase, n, part, y, rl); break;
            default: launch_centre_big<8>(grid, lds, s, out_f32, x, c_in, steps, wp, n_wt, c_out, centre, rowbase, n, part, y, rl); break;
        }
        return hipGetLastError();
    }
    const int mw = mw_for(c_in);
    const int64_t row_tiles = (n + 64 * mw - 1) / (64 * mw);
    const int64_t cap_b = (int64_t)n_cu * (steps <= kChunk ? 4 : 2);
    const int64_t gx = xcd_round(row_tiles < cap_b ? row_tiles : cap_b);
    dim3 grid((unsigned)gx, (unsigned)n_wt);
    const u32x4* wp = (const u32x4*)wpacked;
    const int rl = relu ? 1 : 0;
    switch (nbw) {
        case 1: launch_centre<1>(grid, s, mw, out_f32, x, c_in, steps, wp, n_wt, c_out, centre, rowbase, n, part, y, rl); break;
        case 2: launch_centre<2>(grid, s, mw, out_f32, x, c_in, steps, wp, n_wt, c_out, centre, rowbase, n, part, y, rl); break;
        case 4: launch_centre<4>(grid, s, mw, out_f32, x, c_in, steps, wp, n_wt, c_out, centre, rowbase, n, part, y, rl); break;
        default: launch_centre<8>(grid, s, mw, out_f32, x, c_in, steps, wp, n_wt, c_out, centre, rowbase, n, part, y, rl); break;
    }
    return hipGetLastError();
}

}  // namespace smc
