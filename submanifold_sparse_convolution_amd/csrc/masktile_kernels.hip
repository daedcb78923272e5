// Output-stationary mask-tile GEMM: one kernel per layer, no atomics.
//
// "Sparse convolution in FP32" (DriveRT), "Neighbour masks and sorted rows":
// rows sorted by their 27-bit neighbour mask are processed a tile at a time,
// and a tile only loads the offsets present in the union of its rows' masks;
// the outputs go back to the rows' original positions. Here a block takes 64
// consecutive mask-sorted rows (4 waves x 16 rows) and one wave tile of
// output columns, walks the taps of the union (the centre tap first: every
// row has it), gathers each wave's 16 input rows through the neighbour table
// (an absent neighbour reads a zero row), and accumulates every tap in
// registers with v_mfma_f32_16x16x32_bf16. Each output row is written once,
// as bf16 with the optional ReLU: no float32 accumulator in memory and no
// read-modify-write, which on this GPU's multi-die L2 is the cost that
// dominates a scatter-add GEMM.
//
// Offset groups ("Sparse convolution in FP32", "Offset-group partitioning"):
// the taps may be split into groups, each with its own row order. A launch
// then covers one group: the rows that have a tap of it, tiles taking the
// union of their masks restricted to the group. Earlier groups leave float32
// partial sums of their rows in a buffer; a row that has one adds it in the
// epilogue. The last group holds the centre tap, so its pass reaches every
// row and is the one that writes the output (and applies the ReLU).
//
// Work items are (tap, chunk of 4 k-steps = 128 input channels). A chunk of
// the tap's packed weights is staged in LDS (two buffers). The gathered rows
// come from scattered rows of the feature matrix, so each costs a full
// memory round trip: they are fetched three items ahead (neighbour ids of
// the whole tile are read into LDS once), the weights two items ahead.
#include "gemm_common.h"

namespace smc {
namespace {

constexpr int kMtRows = 64;          // mask-sorted rows per block
constexpr int kChunkSteps = 4;       // k-steps (of 32 channels) per staged weight chunk
constexpr int kMaxLightItems = 4;    // heavier tiles take the k-split path (heavy_tile)

// acc += a (the wave's 16 gathered rows, k-steps first .. first+3) x the
// staged weight chunk (this lane's words in LDS at bl).
template <int NBW>
__device__ __forceinline__ void mma_chunk(const u32x4* bl, const u32x4 (&a)[kChunkSteps], int first,
                                          int steps, f32x4 (&acc)[NBW]) {
#pragma unroll
    for (int i = 0; i < kChunkSteps; ++i) {
        if (first + i >= steps) break;
#pragma unroll
        for (int nb = 0; nb < NBW; ++nb) {
            const u32x4 b = bl[(i * NBW + nb) * 64];
            acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a[i]), as_bf16x8(b), acc[nb],
                                                              0, 0, 0);
        }
    }
}

// Tap of item i: items run (centre, chunks 0..) when the pass has the centre
// tap (CF), then each tap of `rest` (the union without the centre) in
// ascending order.
template <bool CF>
__device__ __forceinline__ int item_tap(int i, int n_chunks, uint32_t rest) {
    int idx = i / n_chunks;
    if (CF) {
        if (idx == 0) return kCentre;
        --idx;
    }
    for (int j = 0; j < idx; ++j) rest &= rest - 1;
    return __builtin_ctz(rest);
}

// Where one pass reads its rows and leaves its sums.
struct PassArgs {
    const uint32_t* perm;      // item indices; row = entry - goff
    int64_t goff;
    int64_t cnt;               // listed rows of the pass
    uint32_t gm, prev;         // taps of the pass, taps of the earlier passes
    int last;                  // writes the output (else the float32 partial sums)
    float* partial;            // [n, c_out] float32 partial sums
};

// Row at position sp of the pass's order (sp clamped to the listed rows, the
// row to the table).
__device__ __forceinline__ uint32_t pass_row(const PassArgs& pa, int64_t sp, int64_t n) {
    const uint32_t e = pa.perm[sp < pa.cnt ? sp : pa.cnt - 1];
    return min((uint32_t)(e - (uint32_t)pa.goff), (uint32_t)(n - 1));
}

// v += the partial sums of row `row`, columns col0 .. col0 + NB - 1 (< c_out).
template <int NB>
__device__ __forceinline__ void add_partial(const float* __restrict__ part, int64_t row, int c_out,
                                            int col0, float (&v)[NB]) {
    const float* src = part + row * c_out + col0;
    if (NB >= 4 && col0 + NB <= c_out && (c_out & 3) == 0) {
#pragma unroll
        for (int q = 0; q < NB / 4; ++q) {
            const float4 f = *reinterpret_cast<const float4*>(src + 4 * q);
            v[4 * q] += f.x;
            v[4 * q + 1] += f.y;
            v[4 * q + 2] += f.z;
            v[4 * q + 3] += f.w;
        }
    } else {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
            if (col0 + nb < c_out) v[nb] += src[nb];
    }
}

// Epilogue of one output row: earlier groups' partial sums, then the output
// or this pass's partial sums.
template <int NB, bool OUT_F32>
__device__ __forceinline__ void finish_row(const PassArgs& pa, void* __restrict__ yv, int64_t row,
                                           uint32_t row_mask, int c_out, int col0, float (&v)[NB],
                                           int relu) {
    if (row_mask & pa.prev) add_partial<NB>(pa.partial, row, c_out, col0, v);
    if (pa.last)
        store_row<NB, OUT_F32>(yv, row, c_out, col0, v, relu);
    else
        store_row<NB, true>(pa.partial, row, c_out, col0, v, 0);
}

// Column blocks of a heavy tile per block: NBW of them are split over
// blockIdx.z in slices of kNbh(NBW).
constexpr int nbh_for(int nbw) { return nbw > 4 ? 4 : nbw; }

// LDS bytes ahead of the neighbour-id table: the light path's two weight
// buffers, or the heavy path's per-wave partial sums, whichever is larger.
constexpr size_t mt_region_bytes(int nbw) {
    return 2 * (size_t)kChunkSteps * nbw * 64 * 16 > 4 * (size_t)kMtRows * 16 * nbh_for(nbw) * 4
               ? 2 * (size_t)kChunkSteps * nbw * 64 * 16
               : 4 * (size_t)kMtRows * 16 * nbh_for(nbw) * 4;
}
constexpr size_t mt_lds_bytes(int nbw) {
    return mt_region_bytes(nbw) + (size_t)kMtRows * kTaps * 4 + 64;
}

// A heavy tile (more work items than kMaxLightItems): the 4 waves split the
// k-steps instead of the rows. Wave w takes k-steps w, w + 4, ... of every
// tap of the union, for all 64 rows of the tile (4 row fragments) and column
// blocks z*NBH .. z*NBH + NBH-1 of the wave tile, so a wave's serial chain is
// a quarter as long and each step needs few registers: the gathered rows (4
// fragments x 16 bytes per lane) and the weights (NBH fragments x 16 bytes,
// straight from L2, where every block of the layer finds them). Steps are
// fetched two ahead with no block barrier in the loop. The four partial
// sums meet in LDS (region s_part) at the end.
template <int NBW, int NBH, bool OUT_F32, bool VEC, bool CF>
__device__ __forceinline__ void heavy_tile(
    const uint16_t* __restrict__ x, int c_in, int steps, const u32x4* __restrict__ wp, int n_wt,
    int c_out, const int32_t* __restrict__ nbr, const uint32_t* __restrict__ mask,
    const PassArgs& pa, int64_t n, int64_t n_in, const uint16_t* __restrict__ zrow,
    void* __restrict__ yv, int relu, uint32_t rest, int z, float* s_part, int32_t* s_nb) {
    constexpr int kWh = 16 * NBH;                     // columns of the slice
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int r = lane & 15, g = lane >> 4;
    const int wt = blockIdx.y;
    const int64_t t0 = (int64_t)blockIdx.x * kMtRows;
    const int64_t n16 = (int64_t)steps * NBW * 64;
    const int n_taps = (CF ? 1 : 0) + __builtin_popcount(rest);

    // neighbour ids of the 64 rows (thread t: row t / 4, 7 taps); rows of the 4 fragments
    {
        const int rr = tid >> 2, k0 = (tid & 3) * 7;
        const int32_t* src = nbr + (int64_t)pass_row(pa, t0 + rr, n) * kTaps;
        int32_t v[7];
#pragma unroll
        for (int q = 0; q < 7; ++q) v[q] = src[min(k0 + q, kTaps - 1)];
#pragma unroll
        for (int q = 0; q < 7; ++q)
            if (k0 + q < kTaps) s_nb[rr * kTaps + k0 + q] = v[q];
    }
    uint32_t rowf[4];
#pragma unroll
    for (int f = 0; f < 4; ++f) rowf[f] = pass_row(pa, t0 + f * 16 + r, n);
    __syncthreads();

    const int per_tap = steps > w ? (steps - w + 3) / 4 : 0;
    const int n_steps = n_taps * per_tap;
    f32x4 acc[4][NBH];
#pragma unroll
    for (int f = 0; f < 4; ++f)
#pragma unroll
        for (int nb = 0; nb < NBH; ++nb) acc[f][nb] = (f32x4){0.f, 0.f, 0.f, 0.f};
    const u32x4* wbase = wp + (int64_t)wt * n16 + (int64_t)z * NBH * 64 + lane;

// data of step P (clamped to the last step: valid addresses, results unused)
#define SMC_HV_FETCH(A, B, P)                                                                     \
    {                                                                                             \
        const int p_ = min((P), n_steps - 1);                                                     \
        const int tap_ = item_tap<CF>(p_ / per_tap, 1, rest);                                     \
        const int st_ = w + 4 * (p_ % per_tap);                                                   \
        const u32x4* bsrc_ = wbase + (int64_t)tap_ * n_wt * n16 + (int64_t)st_ * NBW * 64;        \
        _Pragma("unroll") for (int nb_ = 0; nb_ < NBH; ++nb_) B[nb_] = bsrc_[nb_ * 64];         \
        _Pragma("unroll") for (int f_ = 0; f_ < 4; ++f_) {                                        \
            const int id_ = CF && tap_ == kCentre ? (int)rowf[f_] : s_nb[(f_ * 16 + r) * kTaps + tap_]; \
            const uint16_t* xr_ = id_ >= 0 && id_ < n_in ? x + (int64_t)id_ * c_in : zrow;       \
            A[f_] = load_a4<VEC>(xr_, st_ * 32 + g * 8, c_in);                                    \
        }                                                                                         \
    }
#define SMC_HV_MMA(A, B)                                                                          \
    _Pragma("unroll") for (int nb_ = 0; nb_ < NBH; ++nb_)                                         \
    _Pragma("unroll") for (int f_ = 0; f_ < 4; ++f_)                                              \
        acc[f_][nb_] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(A[f_]), as_bf16x8(B[nb_]), \
                                                               acc[f_][nb_], 0, 0, 0);
    if (n_steps > 0) {
        u32x4 a0[4], a1[4], a2[4], b0[NBH], b1[NBH], b2[NBH];
        SMC_HV_FETCH(a0, b0, 0)
        SMC_HV_FETCH(a1, b1, 1)
        int p = 0;
        while (true) {
            SMC_HV_FETCH(a2, b2, p + 2)
            SMC_HV_MMA(a0, b0)
            if (++p >= n_steps) break;
            SMC_HV_FETCH(a0, b0, p + 2)
            SMC_HV_MMA(a1, b1)
            if (++p >= n_steps) break;
            SMC_HV_FETCH(a1, b1, p + 2)
            SMC_HV_MMA(a2, b2)
            if (++p >= n_steps) break;
        }
    }
#undef SMC_HV_FETCH
#undef SMC_HV_MMA

    // partial sums: fragment f, block nb, lane (r, g), element j is tile row f*16 + 4g + j,
    // slice column r*NBH + nb
    float* mine = s_part + (size_t)w * kMtRows * kWh;
#pragma unroll
    for (int f = 0; f < 4; ++f)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int nb = 0; nb < NBH; ++nb)
                mine[(f * 16 + 4 * g + j) * kWh + r * NBH + nb] = acc[f][nb][j];
    __syncthreads();
    // wave w finishes tile rows w*16 + 4g + j; columns r*NBW + z*NBH .. of the wave tile
    const int col0 = wt * 16 * NBW + r * NBW + z * NBH;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int tr = w * 16 + 4 * g + j;
        const int64_t so = t0 + tr;
        if (so >= pa.cnt || col0 >= c_out) continue;
        float v[NBH];
#pragma unroll
        for (int nb = 0; nb < NBH; ++nb) {
            float sum = 0.f;
#pragma unroll
            for (int q = 0; q < 4; ++q) sum += s_part[((size_t)q * kMtRows + tr) * kWh + r * NBH + nb];
            v[nb] = sum;
        }
        const uint32_t row = pass_row(pa, so, n);
        finish_row<NBH, OUT_F32>(pa, yv, row, pa.prev ? mask[row] : 0u, c_out, col0, v, relu);
    }
}

template <int NBW, bool OUT_F32, bool VEC, bool CF>
__global__ __launch_bounds__(kGemmThreads) void k_conv_masktile(
    const uint16_t* __restrict__ x, int c_in, int steps, const u32x4* __restrict__ wp, int n_wt,
    int c_out, const int32_t* __restrict__ nbr, const uint32_t* __restrict__ mask,
    const uint32_t* __restrict__ perm, int64_t goff, const int32_t* __restrict__ rows,
    uint32_t gm, uint32_t prev, int last, float* __restrict__ partial, int64_t n, int64_t n_in,
    const uint16_t* __restrict__ zrow, void* __restrict__ yv, int relu, int max_items) {
    constexpr int kBuf = kChunkSteps * NBW * 64;    // 16-byte words per staged chunk
    constexpr int kPer = kChunkSteps * NBW / 4;     // words per thread
    constexpr int NBH = nbh_for(NBW);
    // LDS: 2 weight buffers (or the heavy path's partial sums), the tile's neighbour ids
    // [64][kTaps], the wave unions
    extern __shared__ u32x4 s_b[];
    int32_t* s_nb = reinterpret_cast<int32_t*>(reinterpret_cast<char*>(s_b) + mt_region_bytes(NBW));
    uint32_t* s_u = reinterpret_cast<uint32_t*>(s_nb + kMtRows * kTaps);
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int r = lane & 15, g = lane >> 4;
    const int wt = blockIdx.y;
    const int col0 = wt * 16 * NBW + r * NBW;
    const int n_chunks = (steps + kChunkSteps - 1) / kChunkSteps;
    const int64_t t0 = (int64_t)blockIdx.x * kMtRows;     // first position of the tile
    const int64_t s0 = t0 + w * 16;
    const int64_t n16 = (int64_t)steps * NBW * 64;        // words of one (tap, wave tile) slab
    PassArgs pa;
    pa.perm = perm;
    pa.goff = goff;
    pa.cnt = rows ? (int64_t)*rows : n;
    pa.gm = gm;
    pa.prev = prev;
    pa.last = last;
    pa.partial = partial;
    if (t0 >= pa.cnt) return;                              // the whole tile is past the pass's rows

// weights of item (tap K, chunk C) -> register set B (thread t: words t, t + 256, ...)
#define SMC_FETCH_B(B, K, C)                                                                      \
    {                                                                                             \
        const int first_ = (C) * kChunkSteps;                                                     \
        const int cnt_ = min(kChunkSteps, steps - first_) * NBW * 64;                             \
        const u32x4* src_ = wp + ((int64_t)(K) * n_wt + wt) * n16 + (int64_t)first_ * NBW * 64;   \
        _Pragma("unroll") for (int j_ = 0; j_ < kPer; ++j_) {                                     \
            const int i_ = tid + j_ * kGemmThreads;                                               \
            B[j_] = src_[i_ < cnt_ ? i_ : cnt_ - 1];                                              \
        }                                                                                         \
    }
#define SMC_PUT_B(DST, B)                                                                         \
    _Pragma("unroll") for (int j_ = 0; j_ < kPer; ++j_) (DST)[tid + j_ * kGemmThreads] = B[j_];
// gathered rows of chunk C from row pointer XR -> register set A
#define SMC_FETCH_A(A, XR, C)                                                                     \
    {                                                                                             \
        const uint16_t* xr_ = (XR);                                                               \
        _Pragma("unroll") for (int q_ = 0; q_ < kChunkSteps; ++q_) {                              \
            const int st_ = (C) * kChunkSteps + q_;                                               \
            A[q_] = load_a4<VEC>(xr_, st_ < steps ? st_ * 32 + g * 8 : c_in, c_in);               \
        }                                                                                         \
    }
// neighbour ids of the tile's 64 rows, all at once (thread t: row t / 4, 7 taps)
#define SMC_FILL_NB()                                                                             \
    {                                                                                             \
        const int rr_ = tid >> 2, k0_ = (tid & 3) * 7;                                            \
        const int32_t* src_ = nbr + (int64_t)pass_row(pa, t0 + rr_, n) * kTaps;                   \
        int32_t v_[7];                                                                            \
        _Pragma("unroll") for (int q_ = 0; q_ < 7; ++q_) v_[q_] = src_[min(k0_ + q_, kTaps - 1)]; \
        _Pragma("unroll") for (int q_ = 0; q_ < 7; ++q_)                                          \
            if (k0_ + q_ < kTaps) s_nb[rr_ * kTaps + k0_ + q_] = v_[q_];                          \
    }

    if (blockIdx.z > 0) {
        // a further column slice: only heavy tiles have one
        uint32_t m = 0;
#pragma unroll
        for (int f = 0; f < 4; ++f) {
            const int64_t sp = t0 + f * 16 + r;
            const uint32_t mv = mask[pass_row(pa, sp, n)];
            m |= sp < pa.cnt ? mv & gm : 0u;
        }
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) m |= __shfl_xor(m, o, 16);
        const uint32_t rest = CF ? m & ~(1u << kCentre) : m;
        if (((CF ? 1 : 0) + __builtin_popcount(rest)) * n_chunks <= max_items) return;
        heavy_tile<NBW, NBH, OUT_F32, VEC, CF>(x, c_in, steps, wp, n_wt, c_out, nbr, mask, pa, n,
                                               n_in, zrow, yv, relu, rest, blockIdx.z,
                                               reinterpret_cast<float*>(s_b), s_nb);
        return;
    }

    // With the centre tap, item 0 = (centre, chunk 0) needs nothing from the map:
    // its weights and rows (each lane's own row) are fetched before the union is known.
    u32x4 bA[kPer], bB[kPer];
    if (CF) SMC_FETCH_B(bA, kCentre, 0)
    // this lane's A row (tile row r), the 4 output rows it writes, and its mask
    const int64_t sa = s0 + r;
    const uint32_t row_a = pass_row(pa, sa, n);
    uint32_t orow[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) orow[j] = pass_row(pa, s0 + 4 * g + j, n);
    const uint32_t m_raw = mask[row_a];
    const uint16_t* xself = x + (int64_t)row_a * c_in;
    u32x4 a0[kChunkSteps], a1[kChunkSteps], a2[kChunkSteps], a3[kChunkSteps];
    if (CF) {
        SMC_FETCH_A(a0, xself, 0)
        SMC_PUT_B(s_b, bA)
    }
    uint32_t m = sa < pa.cnt ? m_raw & gm : 0u;
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) m |= __shfl_xor(m, o, 16);
    if (lane == 0) s_u[w] = m;
    if (!CF) SMC_FILL_NB()                            // every row of the pass has a tap of it
    __syncthreads();                                  // wave unions (and buffer 0 / ids) in LDS
    uint32_t u = 0;
#pragma unroll
    for (int v = 0; v < kGemmThreads / 64; ++v) u |= s_u[v];
    // without CF (a group without the centre, or a strided map whose centre tap
    // is an ordinary gathered input) every tap of the union is read through s_nb
    const uint32_t rest = CF ? u & ~(1u << kCentre) : u;
    const int n_items = ((CF ? 1 : 0) + __builtin_popcount(rest)) * n_chunks;
    const int last_item = n_items - 1;
    if (n_items > max_items) {                        // heavy tile: column slice 0
        heavy_tile<NBW, NBH, OUT_F32, VEC, CF>(x, c_in, steps, wp, n_wt, c_out, nbr, mask, pa, n,
                                               n_in, zrow, yv, relu, rest, 0,
                                               reinterpret_cast<float*>(s_b), s_nb);
        return;
    }
    const int my_nb = w * 16 + r;                     // this lane's row in s_nb
    // this lane's input row for item j (centre: itself)
#define SMC_XROW(J)                                                                               \
    ({                                                                                            \
        const int kk_ = item_tap<CF>(J, n_chunks, rest);                                          \
        const int nb_ = CF && kk_ == kCentre ? (int)row_a : s_nb[my_nb * kTaps + kk_];            \
        nb_ >= 0 && nb_ < n_in ? x + (int64_t)nb_ * c_in : zrow;                                  \
    })
    if (!CF) {                                        // item 0 now that the union is known
        SMC_FETCH_B(bA, item_tap<CF>(0, n_chunks, rest), 0)
        SMC_FETCH_A(a0, SMC_XROW(0), 0)
        SMC_PUT_B(s_b, bA)
        __syncthreads();
    }
    f32x4 acc[NBW];
#pragma unroll
    for (int nb = 0; nb < NBW; ++nb) acc[nb] = (f32x4){0.f, 0.f, 0.f, 0.f};
    if (n_items == 1) {                               // one item: nothing to prefetch
        mma_chunk<NBW>(s_b + lane, a0, 0, steps, acc);
    } else {
    if (CF && rest) {
        SMC_FILL_NB()
        __syncthreads();
    }

    // Pipeline: gathered rows 3 items ahead (4 register sets), weights 2 items ahead
    // (2 register sets + 2 LDS buffers). At the top of iteration i: weights of item i in
    // LDS buffer (i & 1), rows of items i..i+2 in A sets i%4..(i+2)%4, weights of item i+1
    // in B set (i+1)%2. Fetches past the last item re-read the last item (valid
    // addresses, results unused), so every register set is always written.
    {
        const int j1 = min(1, last_item), j2 = min(2, last_item);
        SMC_FETCH_A(a1, SMC_XROW(j1), j1 % n_chunks)
        SMC_FETCH_A(a2, SMC_XROW(j2), j2 % n_chunks)
        SMC_FETCH_B(bB, item_tap<CF>(j1, n_chunks, rest), j1 % n_chunks)
    }

#define SMC_MT_STEP(ACUR, ANEW, BFREE, BNEXT)                                                     \
    {                                                                                             \
        const int i2 = min(i + 2, last_item), i3 = min(i + 3, last_item);                         \
        SMC_FETCH_B(BFREE, item_tap<CF>(i2, n_chunks, rest), i2 % n_chunks)                       \
        SMC_FETCH_A(ANEW, SMC_XROW(i3), i3 % n_chunks)                                            \
        mma_chunk<NBW>(s_b + (i & 1) * kBuf + lane, ACUR, (i % n_chunks) * kChunkSteps, steps,   \
                       acc);                                                                      \
        if (i + 1 >= n_items) break;                                                              \
        SMC_PUT_B(s_b + ((i + 1) & 1) * kBuf, BNEXT)                                              \
        __syncthreads();                                                                          \
        ++i;                                                                                      \
    }

    int i = 0;
    while (true) {
        SMC_MT_STEP(a0, a3, bA, bB)
        SMC_MT_STEP(a1, a0, bB, bA)
        SMC_MT_STEP(a2, a1, bA, bB)
        SMC_MT_STEP(a3, a2, bB, bA)
    }
    }                                                 // n_items > 1
#undef SMC_MT_STEP
#undef SMC_XROW
#undef SMC_FETCH_B
#undef SMC_PUT_B
#undef SMC_FETCH_A
#undef SMC_FILL_NB

    // write the 4 output rows this lane holds (row 4g + j of the wave: lane 4g + j has its mask)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int64_t so = s0 + 4 * g + j;
        const uint32_t mj = __shfl(m_raw, 4 * g + j);
        if (so >= pa.cnt || col0 >= c_out) continue;
        float v[NBW];
#pragma unroll
        for (int nb = 0; nb < NBW; ++nb) v[nb] = acc[nb][j];
        finish_row<NBW, OUT_F32>(pa, yv, (int64_t)orow[j], mj, c_out, col0, v, relu);
    }
}

template <int NBW, bool OUT_F32, bool VEC, bool CF>
hipError_t launch_mt(dim3 grid, hipStream_t s, const uint16_t* x, int c_in, int steps,
                     const u32x4* wp, int n_wt, int c_out, const int32_t* nbr, const uint32_t* mask,
                     const GroupPass& gp, int64_t n, const uint16_t* zrow, void* y, int relu) {
    static bool attr_ok = false;                      // one attribute call per instantiation
    constexpr size_t lds = mt_lds_bytes(NBW);
    if (!attr_ok && lds > 64 * 1024) {
        if (hipFuncSetAttribute(reinterpret_cast<const void*>(k_conv_masktile<NBW, OUT_F32, VEC, CF>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess) {
            (void)hipGetLastError();
            return hipErrorInvalidValue;
        }
    }
    attr_ok = true;
    grid.z = NBW / nbh_for(NBW);
    launch(k_conv_masktile<NBW, OUT_F32, VEC, CF>, grid, kGemmThreads, lds, s, x, c_in, steps, wp,
           n_wt, c_out, nbr, mask, gp.perm, gp.goff, gp.rows, gp.gm, gp.prev, gp.last ? 1 : 0,
           gp.partial, n, gp.n_in > 0 ? gp.n_in : n, zrow, y, relu, kMaxLightItems);
    return hipGetLastError();
}

template <int NBW, bool OUT_F32>
hipError_t launch_mt_v(dim3 grid, hipStream_t s, const uint16_t* x, int c_in, int steps,
                       const u32x4* wp, int n_wt, int c_out, const int32_t* nbr,
                       const uint32_t* mask, const GroupPass& gp, int64_t n, const uint16_t* zrow,
                       void* y, int relu) {
    const bool vec = (c_in & 7) == 0;
    const bool cf = ((gp.gm >> kCentre) & 1u) && gp.centre_self;
    if (vec) {
        if (cf) return launch_mt<NBW, OUT_F32, true, true>(grid, s, x, c_in, steps, wp, n_wt, c_out, nbr, mask, gp, n, zrow, y, relu);
        return launch_mt<NBW, OUT_F32, true, false>(grid, s, x, c_in, steps, wp, n_wt, c_out, nbr, mask, gp, n, zrow, y, relu);
    }
    if (cf) return launch_mt<NBW, OUT_F32, false, true>(grid, s, x, c_in, steps, wp, n_wt, c_out, nbr, mask, gp, n, zrow, y, relu);
    return launch_mt<NBW, OUT_F32, false, false>(grid, s, x, c_in, steps, wp, n_wt, c_out, nbr, mask, gp, n, zrow, y, relu);
}

template <int NBW>
hipError_t launch_mt_nbw(dim3 grid, hipStream_t s, bool out_f32, const uint16_t* x, int c_in,
                         int steps, const u32x4* wp, int n_wt, int c_out, const int32_t* nbr,
                         const uint32_t* mask, const GroupPass& gp, int64_t n,
                         const uint16_t* zrow, void* y, int relu) {
    if (out_f32) return launch_mt_v<NBW, true>(grid, s, x, c_in, steps, wp, n_wt, c_out, nbr, mask, gp, n, zrow, y, relu);
    return launch_mt_v<NBW, false>(grid, s, x, c_in, steps, wp, n_wt, c_out, nbr, mask, gp, n, zrow, y, relu);
}

}  // namespace

hipError_t launch_conv_masktile(const uint16_t* x, int c_in, const void* wpacked, int c_out,
                                const int32_t* nbr, const uint32_t* mask, const GroupPass& gp,
                                int64_t n, const uint16_t* zrow, void* y, bool out_f32, bool relu,
                                hipStream_t s) {
    if (n <= 0) return hipSuccess;
    if (!gp.perm || (!gp.last && !gp.partial) || (gp.prev && !gp.partial) || !gp.gm)
        return hipErrorInvalidValue;
    if (!gp.last && ((gp.gm >> kCentre) & 1u) && gp.centre_self)
        return hipErrorInvalidValue;                                           // centre is last
    const int steps = (c_in + 31) / 32;
    const int nbw = nbw_for(c_out);
    const int n_wt = (c_out + 16 * nbw - 1) / (16 * nbw);
    dim3 grid((unsigned)((n + kMtRows - 1) / kMtRows), (unsigned)n_wt);
    const u32x4* wp = (const u32x4*)wpacked;
    const int rl = relu ? 1 : 0;
    switch (nbw) {
        case 1: return launch_mt_nbw<1>(grid, s, out_f32, x, c_in, steps, wp, n_wt, c_out, nbr, mask, gp, n, zrow, y, rl);
        case 2: return launch_mt_nbw<2>(grid, s, out_f32, x, c_in, steps, wp, n_wt, c_out, nbr, mask, gp, n, zrow, y, rl);
        case 4: return launch_mt_nbw<4>(grid, s, out_f32, x, c_in, steps, wp, n_wt, c_out, nbr, mask, gp, n, zrow, y, rl);
        default: return launch_mt_nbw<8>(grid, s, out_f32, x, c_in, steps, wp, n_wt, c_out, nbr, mask, gp, n, zrow, y, rl);
    }
}

}  // namespace smc
