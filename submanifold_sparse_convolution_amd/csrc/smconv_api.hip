// C ABI: map handles, the map build pipeline, weight packing and the
// forward layer. See include/smconv.h for the contract of each call.
#include "smconv.h"
#include "smc_internal.h"

#include <mutex>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

using namespace smc;

namespace smc {
thread_local KernelTimer g_ktimer;
}

// One copy per GPU, held until the process ends; calls on one GPU share it.
static __device__ __align__(256) unsigned char scratch[(size_t)32 << 20];

namespace {

thread_local std::string g_last_error;

int fail(int status, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int status, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return status;
}

#define SMC_HIP(call)                                                                          \
    do {                                                                                       \
        hipError_t e_ = (call);                                                                \
        if (e_ != hipSuccess)                                                                  \
            return fail(SMC_ERR_HIP, "%s failed: %s (%s:%d)", #call, hipGetErrorString(e_),    \
                        __FILE__, __LINE__);                                                   \
    } while (0)

// Device allocator of the process (smc_set_allocator); both null: hipMalloc
// and hipFree.
struct Allocator {
    smc_alloc_fn alloc = nullptr;
    smc_free_fn free = nullptr;
    void* ctx = nullptr;
};
std::mutex g_alloc_mu;
Allocator g_alloc;

Allocator current_allocator() {
    std::lock_guard<std::mutex> lock(g_alloc_mu);
    return g_alloc;
}

// Grow-only device buffer. It keeps the allocator that made it and frees
// with that one, whatever the process allocator is by then; s is the stream
// the buffer is about to be used on (handed to a caller's allocator).
struct DevBuf {
    void* p = nullptr;
    size_t bytes = 0;
    Allocator by;
    int ensure(size_t want, hipStream_t s = nullptr) {
        if (want <= bytes) return SMC_OK;
        release(s);
        const size_t alloc = want < 256 ? 256 : want;
        const Allocator a = current_allocator();
        if (a.alloc) {
            p = a.alloc(a.ctx, alloc, (void*)s);
            if (!p) return fail(SMC_ERR_ALLOC, "the caller's allocator returned NULL for %zu bytes", alloc);
            if (((uintptr_t)p & 255) != 0) {     // the kernels read rows in 16-byte words
                a.free(a.ctx, p, (void*)s);
                p = nullptr;
                return fail(SMC_ERR_ALLOC, "the caller's allocator returned a pointer not aligned to 256 bytes");
            }
        } else if (hipMalloc(&p, alloc) != hipSuccess) {
            (void)hipGetLastError();
            p = nullptr;
            return fail(SMC_ERR_ALLOC, "hipMalloc(%zu) failed", alloc);
        }
        by = a;
        bytes = alloc;
        return SMC_OK;
    }
    void release(hipStream_t s = nullptr) {
        if (p) {
            if (by.free)
                by.free(by.ctx, p, (void*)s);
            else
                (void)hipFree(p);
        }
        p = nullptr;
        bytes = 0;
        by = Allocator();
    }
    template <typename T> T* as() const { return static_cast<T*>(p); }
};

// Scratch of the no-allocation forward (smc_conv_forward_noalloc): the
// pair-list slab or the grouped mask tiles' float32 partial sums. The array is
// a host-side stand-in in host code; kernels get its device address, looked
// up once per device (scratch_ptr).
constexpr size_t kScratchBytes = (size_t)32 << 20;
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

constexpr int64_t kMaxRows = (int64_t)1 << 26;
constexpr int64_t kMaxStridedRows = (int64_t)1 << 24;            // 8 candidates per input
constexpr int kMaxChannels = 4096;
constexpr int kZeroRowBytes = kMaxChannels * 2;                 // keeps 27 n + pads < 2^31
// auto route: the dense grid (4 bytes a cell, two bitmaps of 1 bit) takes at most
// 1/16 of the device's memory and at most 16 GiB
constexpr int64_t kDenseBudgetMaxBytes = (int64_t)16 << 30;
constexpr double kDenseMaxCells = 68719476736.0;                 // 2^36: bitmap words fit int32
constexpr int64_t kSlabBoundBytes = (int64_t)4 << 30;          // unread counts: bound the slab

int bit_len(int64_t v) {   // bits needed to hold 0..v
    int b = 0;
    while (v > 0) {
        ++b;
        v >>= 1;
    }
    return b;
}

}  // namespace

struct smc_map {
    int device = -1;
    int n_cu = 0;
    int64_t dense_budget = 0;         // bytes the auto route may spend on a dense grid
    hipEvent_t done = nullptr;        // end of a synchronous build (system-scope fence)
    hipEvent_t done_nf = nullptr;     // end of an asynchronous build (no fence, see build_map)
    hipEvent_t done_last = nullptr;   // the one the last build recorded
    hipEvent_t rows_ev = nullptr;     // a strided build's output count copied to the host
    bool rows_pending = false;        // n is that build's bound until rows_ev is read
    MapState* host_state = nullptr;   // pinned
    bool built = false;
    bool pending = false;             // a build whose device checks are not read yet
    int build_status = SMC_OK;
    int64_t n = 0;
    int route = 0;
    int key_bits = 0;
    bool wide = false;
    Geom geom{};
    int64_t grid_cells = 0;
    // device buffers
    DevBuf state;                     // two MapState records: builds alternate between them
    int slot = 1;                     // record of the last build
    bool slot_clean[2] = {true, true};  // record in its starting state
    // Dense route: one int32 id grid and two occupancy bitmaps, used by alternate
    // dense builds and kept all zero between them. A build writes the ids of its
    // own cells only and reads ids only under its own bits, so the id grid is
    // never cleared. cells[i] records the bitmap word of every row of the last
    // build on bitmap i; the next dense build (on the other bitmap) or, before a
    // sorted build, a small kernel clears those words.
    DevBuf grid;                             // int32 row ids (read only where a bit is set)
    DevBuf bits[2];                          // one occupancy bit per cell (+2 words)
    int64_t bits_clean_words[2] = {0, 0};    // prefix of each bitmap known to be zero
    DevBuf cells[2];
    int next_grid = 0;                       // bitmap of the next dense build
    PrevCells stale;                         // cells not yet put back (stale.n = 0: none)
    DevBuf keys0, keys1, keys2;       // packed keys (u32 or u64)
    DevBuf vals0, vals1;              // u32
    DevBuf hist;                      // per record: digit histograms, mask sort then key sort
    DevBuf look, ticket;              // look-back table and block ticket (zeroed when allocated)
    DevBuf sticky;                    // status bits of recycled records not read yet (one word)
    SortWork ws;
    bool state_copied = false;        // host_state already holds the last build's record
    DevBuf nbr, mask, mkey0, mkey1, mval0, mval1;
    const uint32_t* perm = nullptr;   // points into mval0 or mval1: [groups][n] item indices
    MaskOrder order;                  // bit order and offset groups of the next builds' mask sort
    MaskOrder sorted_order;           // the order the last build's mask sort used
    DevBuf okeys;                     // per-group sort keys ([groups][n])
    DevBuf pair_in, pair_out, pair_slot, rowbase;
    DevBuf chunk_pre;                 // per 256-row chunk: pairs of each tap and slab rows before it
    int64_t cap = 0;                  // pairs per tap the pair arrays hold (n rounded up to a tile)
    DevBuf part;                      // float32 partial-product slab of the pair-list forward
    DevBuf split;                     // splitter table of the sorted route's key sort
    DevBuf zrow;                      // zero row read for absent neighbours (mask-tile GEMM)
    bool has_pairs = false;
    bool has_sort = false;
    bool has_table = false;           // nbr holds the last build's neighbour table
    int ksize = 3;                    // kernel size of the last build (taps = ksize^3)
    // strided builds: outputs differ from inputs (n = output rows, n_in = input rows)
    bool strided = false;
    int64_t n_in = 0;
    StrideGeom sgeom{};
    DevBuf ck0, ck1, ck2, cv0, cv1, chist, ucounts, ocoords, qcoords;
    DevBuf obits;                 // output-grid bitmap of strided builds (kept zero between builds)
    DevBuf scan;                      // count table of many-tile sorts
    // stage timers
    bool timing = false;
    std::vector<hipEvent_t> ev_pool;
    struct TimedKernel {
        hipEvent_t start;             // set on the first kernel of a sequence
        hipEvent_t stop;
        int stage;
        bool in_build;
    };
    std::vector<TimedKernel> seq;     // timed kernels in launch order, not yet read
    bool seq_open = false;            // the last timed kernel's stop starts the next interval
    bool in_build = false;            // inside a timed build
    double stage_ms[SMC_STAGE_COUNT] = {};
    int64_t stage_calls[SMC_STAGE_COUNT] = {};
    int64_t stage_exec[SMC_STAGE_COUNT] = {};   // timed executions not yet read
};

namespace {

// Device address of this GPU's copy of `scratch`, looked up once per device
// with that device current (the library's first map use on it). A failed
// lookup leaves it null: only the no-allocation forward needs it, and it
// reports the failure.
void lookup_scratch(int dev) {
    static_assert(sizeof(scratch) == kScratchBytes, "scratch size");
    if (dev < 0 || dev >= kMaxDevices) return;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev]) return;
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) {
        (void)hipGetLastError();
        return;
    }
    g_scratch_ptr[dev] = p;
}

void* scratch_ptr(int dev) {
    if (dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    return g_scratch_ptr[dev];
}

// First use of a handle: its device, event, pinned record and small buffers.
// Every step can be repeated, and the handle counts as initialised (device
// set) only once all of them succeeded, so a handle whose first build failed
// to allocate is initialised again by its next build, never used half-made.
int ensure_device(smc_map* m) {
    int dev = 0;
    SMC_HIP(hipGetDevice(&dev));
    if (m->device < 0) {
        lookup_scratch(dev);
        SMC_HIP(hipDeviceGetAttribute(&m->n_cu, hipDeviceAttributeMultiprocessorCount, dev));
        size_t total = 0;
        SMC_HIP(hipDeviceTotalMem(&total, dev));
        m->dense_budget = std::min<int64_t>(kDenseBudgetMaxBytes, (int64_t)(total / 16));
        if (!m->done) SMC_HIP(hipEventCreateWithFlags(&m->done, hipEventDisableTiming));
        if (!m->done_nf)
            SMC_HIP(hipEventCreateWithFlags(&m->done_nf,
                                            hipEventDisableTiming | hipEventDisableSystemFence));
        if (!m->rows_ev) SMC_HIP(hipEventCreateWithFlags(&m->rows_ev, hipEventDisableTiming));
        if (!m->host_state &&
            hipHostMalloc((void**)&m->host_state, sizeof(MapState), hipHostMallocDefault) !=
                hipSuccess) {
            (void)hipGetLastError();
            m->host_state = nullptr;
            return fail(SMC_ERR_ALLOC, "hipHostMalloc of the readback record failed");
        }
        int rc = m->state.ensure(2 * sizeof(MapState));
        if (rc) return rc;
        if ((rc = m->ticket.ensure(256)) || (rc = m->hist.ensure((size_t)2 * kHistInts * 4)) ||
            (rc = m->zrow.ensure(kZeroRowBytes)) || (rc = m->sticky.ensure(256)))
            return rc;
        SMC_HIP(launch_fill_i32(m->ticket.as<int32_t>(), 64, 0, nullptr));
        SMC_HIP(launch_fill_i32(m->sticky.as<int32_t>(), 64, 0, nullptr));
        for (int k = 0; k < 2; ++k)
            SMC_HIP(launch_state_init(m->state.as<MapState>() + k, m->hist.as<uint32_t>() + k * kHistInts,
                                      kHistInts, nullptr, nullptr));
        SMC_HIP(launch_fill_i32(m->zrow.as<int32_t>(), kZeroRowBytes / 4, 0, nullptr));
        SMC_HIP(hipDeviceSynchronize());
        m->ws.ticket = m->ticket.as<uint32_t>();
        m->device = dev;
    } else if (dev != m->device) {
        return fail(SMC_ERR_STATE, "map was created on device %d, current device is %d",
                    m->device, dev);
    }
    return SMC_OK;
}

// A strided pair-list build sizes its lookup and compaction by a bound (8
// candidates per input) and leaves its output count on the device; the count
// reaches the host with an event of its own, read here on first use.
int resolve_rows(smc_map* m) {
    if (!m->rows_pending) return SMC_OK;
    SMC_HIP(hipEventSynchronize(m->rows_ev));
    m->rows_pending = false;
    const int64_t c = m->host_state->n_out;
    if (c < 0 || c > m->n) {
        m->n = 0;
        m->build_status = SMC_ERR_STATE;
        return fail(SMC_ERR_STATE, "output count %lld", (long long)c);
    }
    m->n = c;
    return SMC_OK;
}

// Waits for the handle's last build and reads its record. Asynchronous builds
// do not wait for each other: a build recycles the record of the build before
// it, carrying that record's status bits into the sticky word first, so the
// checks of every build since the last wait are reported here.
int wait_build(smc_map* m) {
    if (int rc = resolve_rows(m)) return rc;
    if (!m->pending) return SMC_OK;
    SMC_HIP(hipEventSynchronize(m->done_last));
    if (!m->state_copied) {
        SMC_HIP(hipMemcpy(m->host_state, m->state.as<MapState>() + m->slot, sizeof(MapState),
                          hipMemcpyDeviceToHost));
        m->state_copied = true;
    }
    m->pending = false;
    uint32_t sticky = 0;
    SMC_HIP(hipMemcpy(&sticky, m->sticky.p, sizeof(sticky), hipMemcpyDeviceToHost));
    if (sticky) {                                 // every build is done: nothing else writes it
        const uint32_t zero = 0;
        SMC_HIP(hipMemcpy(m->sticky.p, &zero, sizeof(zero), hipMemcpyHostToDevice));
    }
    uint32_t st = m->host_state->status | sticky;
    if (st & kStSortStall) {
        m->build_status = SMC_ERR_HIP;
        return fail(SMC_ERR_HIP, "a look-back wait of the map build ran out (results invalid)");
    }
    if (st & kStDuplicate) {
        m->build_status = SMC_ERR_DUPLICATE;
        return fail(SMC_ERR_DUPLICATE, "two rows share the same (b, x, y, z)");
    }
    if (st & kStRange) {
        m->build_status = SMC_ERR_RANGE;
        return fail(SMC_ERR_RANGE, "a coordinate lies outside the spatial shape or batch range");
    }
    m->build_status = SMC_OK;
    return SMC_OK;
}

int ensure_grid(smc_map* m, int gi, int64_t cells, hipStream_t s) {
    const int64_t words = cells / 32 + 2;
    DevBuf& grid = m->grid;
    DevBuf& bits = m->bits[gi];
    int rc = grid.ensure((size_t)cells * 4, s);       // never filled: read only under a set bit
    if (rc) return rc;
    if ((size_t)words * 4 > bits.bytes) {
        if (m->stale.n > 0 && m->stale.bits == bits.as<uint32_t>()) m->stale = PrevCells();
        if ((rc = bits.ensure((size_t)words * 4, s))) return rc;
        m->bits_clean_words[gi] = 0;
    }
    if (m->bits_clean_words[gi] < words) {
        // zero the whole allocation once; later builds only clear the words they used
        const int64_t all = (int64_t)(bits.bytes / 4);
        SMC_HIP(launch_fill_i32(bits.as<int32_t>(), all, 0, s));
        m->bits_clean_words[gi] = all;
    }
    return SMC_OK;
}

hipEvent_t take_event(smc_map* m) {
    if (!m->ev_pool.empty()) {
        hipEvent_t e = m->ev_pool.back();
        m->ev_pool.pop_back();
        return e;
    }
    // timing only: no system-scope fence (cache write-back and invalidate) at
    // the event, which would lengthen the kernel it is bound to
    hipEvent_t e = nullptr;
    if (hipEventCreateWithFlags(&e, hipEventDisableSystemFence) != hipSuccess) {
        (void)hipGetLastError();
        return nullptr;
    }
    return e;
}

// Stage timer (only while timing is on). Every kernel launched while a timer
// is active carries one stop event, stamped by its own dispatch
// (hipExtLaunchKernel), and a kernel's time is the interval from the stop of
// the kernel before it in the handle's timed sequence (or from a start marker
// recorded before the sequence's first kernel) to its own stop. On a stream
// the GPU runs back to back, that is the kernel's duration plus the dispatch
// gap before it, and the times of a sequence add up to its elapsed time. A
// start event beside each kernel instead adds its own marker's latency to
// every kernel (about 2 us each on MI355X). Kernel mode: the kernels count
// for the timer's stage (and for SMC_STAGE_MAP inside a build). Bracket mode
// (the whole build): kernels not inside a nested stage count for the build
// only.
struct StageTimer {
    smc_map* m;
    int stage;
    hipStream_t s;
    bool bracket;
    bool active = false;
    KernelTimer saved;
    static bool take_stop(void* ctx, hipEvent_t* stop) {
        StageTimer* t = static_cast<StageTimer*>(ctx);
        smc_map* mm = t->m;
        hipEvent_t start = nullptr;
        if (!mm->seq_open) {
            start = take_event(mm);
            if (!start) return false;
            if (hipEventRecord(start, t->s) != hipSuccess) {
                (void)hipGetLastError();
                mm->ev_pool.push_back(start);
                return false;
            }
            mm->seq_open = true;
        }
        hipEvent_t e = take_event(mm);
        if (!e) {
            if (start) mm->ev_pool.push_back(start);
            mm->seq_open = false;
            return false;
        }
        mm->seq.push_back({start, e, t->stage, mm->in_build});
        *stop = e;
        return true;
    }
    StageTimer(smc_map* m_, int stage_, hipStream_t s_, bool bracket_ = false, bool enable = true)
        : m(m_), stage(stage_), s(s_), bracket(bracket_) {
        if (!m->timing || !enable) return;
        active = true;
        saved = g_ktimer;
        g_ktimer.ctx = this;
        g_ktimer.take = &take_stop;
        if (bracket) m->in_build = true;
    }
    ~StageTimer() { finish(); }
    void finish() {
        if (!active) return;
        active = false;
        g_ktimer = saved;
        if (bracket) m->in_build = false;
        m->stage_exec[stage] += 1;
    }
};

}  // namespace

extern "C" {

int smc_version(void) { return 100; }

int smc_set_allocator(smc_alloc_fn alloc, smc_free_fn free_fn, void* ctx) {
    if ((alloc == nullptr) != (free_fn == nullptr))
        return fail(SMC_ERR_ARG, "alloc and free must both be set or both be NULL");
    std::lock_guard<std::mutex> lock(g_alloc_mu);
    g_alloc.alloc = alloc;
    g_alloc.free = free_fn;
    g_alloc.ctx = alloc ? ctx : nullptr;
    return SMC_OK;
}

const char* smc_status_string(int status) {
    switch (status) {
        case SMC_OK: return "ok";
        case SMC_ERR_ARG: return "invalid argument";
        case SMC_ERR_DUPLICATE: return "duplicate coordinates";
        case SMC_ERR_RANGE: return "coordinate out of range";
        case SMC_ERR_KEY_OVERFLOW: return "packed key needs more than 64 bits";
        case SMC_ERR_ALLOC: return "allocation failed";
        case SMC_ERR_HIP: return "HIP runtime error";
        case SMC_ERR_STATE: return "map not built or built with an error";
        case SMC_ERR_UNSUPPORTED: return "unsupported";
        case SMC_ERR_GRID: return "dense grid too large";
        default: return "unknown status";
    }
}

const char* smc_last_error(void) { return g_last_error.c_str(); }

int smc_map_create(smc_map** out) {
    if (!out) return fail(SMC_ERR_ARG, "out is NULL");
    smc_map* m = new (std::nothrow) smc_map();
    if (!m) return fail(SMC_ERR_ALLOC, "out of host memory");
    *out = m;
    return SMC_OK;
}

int smc_map_destroy(smc_map* m) {
    if (!m) return SMC_OK;
    // (a handle whose first build failed part-way holds some buffers with no device set)
    const bool touched =
        m->device >= 0 || m->done || m->done_nf || m->rows_ev || m->host_state || m->state.p;
    if (touched) {
        int cur = 0;
        (void)hipGetDevice(&cur);
        if (m->device >= 0) (void)hipSetDevice(m->device);
        (void)hipDeviceSynchronize();
        DevBuf* bufs[] = {&m->state, &m->grid, &m->bits[0], &m->bits[1],
                          &m->cells[0], &m->cells[1], &m->keys0, &m->keys1, &m->keys2,
                          &m->vals0, &m->vals1, &m->hist, &m->look, &m->ticket, &m->nbr,
                          &m->mask, &m->mkey0, &m->mkey1, &m->mval0, &m->mval1, &m->okeys,
                          &m->pair_in, &m->pair_out, &m->pair_slot, &m->rowbase,
                          &m->chunk_pre, &m->part,
                          &m->zrow, &m->ck0, &m->ck1, &m->ck2, &m->cv0, &m->cv1, &m->chist,
                          &m->ucounts, &m->ocoords, &m->qcoords, &m->scan, &m->split,
                          &m->obits, &m->sticky};
        for (DevBuf* b : bufs) b->release();
        for (auto& tk : m->seq) {
            if (tk.start) m->ev_pool.push_back(tk.start);
            m->ev_pool.push_back(tk.stop);
        }
        for (hipEvent_t e : m->ev_pool) (void)hipEventDestroy(e);
        if (m->host_state) (void)hipHostFree(m->host_state);
        if (m->done) (void)hipEventDestroy(m->done);
        if (m->done_nf) (void)hipEventDestroy(m->done_nf);
        if (m->rows_ev) (void)hipEventDestroy(m->rows_ev);
        (void)hipSetDevice(cur);
    }
    delete m;
    return SMC_OK;
}

// Strided map, output side: the output cells (a bitmap of the output grid, or
// for a larger grid candidate output keys of every input, one radix sort and
// unique), as output coords + query points. *rows: the output count, read
// back at once, or with defer the bound 8 n (the count stays on the device in
// st->n_out for the kernels after, and reaches the host through rows_ev). The
// input-side structure (grid or sorted keys) is built by the caller.
// The output-grid bitmap (zero when allocated and between builds) and the
// per-block counts of its bitmap route.
static int prepare_obits(smc_map* m, int64_t words, hipStream_t s) {
    const size_t want = (size_t)words * 4 + 4;
    int rc;
    if (want > m->obits.bytes) {
        if ((rc = m->obits.ensure(want, s))) return rc;
        SMC_HIP(launch_fill_i32(m->obits.as<int32_t>(), (int64_t)(m->obits.bytes / 4), 0, s));
    }
    const int64_t nb = out_bitmap_blocks(words);
    if ((size_t)nb * 4 > m->ucounts.bytes && (rc = m->ucounts.ensure((size_t)nb * 4, s))) return rc;
    return SMC_OK;
}

// marked: the dense scatter has set the output bits already (bitmap route).
static int strided_outputs(smc_map* m, const int32_t* coords, int64_t n, const Geom& g,
                           const StrideGeom& sg, MapState* st, uint32_t* status, hipStream_t s,
                           int64_t* rows, bool defer, bool marked) {
    const int64_t n_cand = 8 * n;
    // a small output grid: its cells through a bitmap, no candidate sort
    const int64_t words = out_bitmap_words(sg, g.batch);
    if (words <= kOutBitmapWords) {
        int rc;
        if ((rc = prepare_obits(m, words, s))) return rc;
        SMC_HIP(launch_stride_bitmap(coords, n, g, sg, m->obits.as<uint32_t>(), words,
                                     m->ucounts.as<uint32_t>(), m->ocoords.as<int32_t>(),
                                     m->qcoords.as<int32_t>(), st, m->ws, m->n_cu, s, marked));
    } else {
        SMC_HIP(launch_stride_candidates(coords, n, g, sg, m->ck0.as<uint64_t>(), st, s));
        int bits = 1;
        while (((uint64_t)1 << bits) <= sg.sentinel) ++bits;   // key bits including the sentinel's
        const SortPlan plan = sort_plan(bits);
        if (plan.passes * (1 << plan.bits) > kHistKeyInts)
            return fail(SMC_ERR_UNSUPPORTED, "output key sort needs %d bins", plan.passes * (1 << plan.bits));
        // (a many-tile sort counts per tile itself: no global histogram needed)
        if (sort_scan_ints(n_cand) == 0 || !m->ws.cnt) {
            SMC_HIP(launch_fill_i32(m->chist.as<int32_t>(), kHistKeyInts, 0, s));
            SMC_HIP(launch_key_hist(m->ck0.p, true, n_cand, plan, m->chist.as<uint32_t>(), s));
        }
        const uint64_t* sorted = nullptr;
        const uint32_t* sv = nullptr;
        SMC_HIP(radix_sort_u64(m->ck0.as<uint64_t>(), nullptr, n_cand, plan, m->chist.as<uint32_t>(),
                               m->ck1.as<uint64_t>(), m->ck2.as<uint64_t>(), m->cv0.as<uint32_t>(),
                               m->cv1.as<uint32_t>(), m->ws, status, &sorted, &sv, s));
        SMC_HIP(launch_unique(sorted, n_cand, sg, m->ucounts.as<uint32_t>(), m->ocoords.as<int32_t>(),
                              m->qcoords.as<int32_t>(), st, s));
    }
    int32_t count = 0;
    SMC_HIP(hipMemcpyAsync(&m->host_state->n_out, &st->n_out, sizeof(int32_t),
                           hipMemcpyDeviceToHost, s));
    if (defer) {                                  // the count is read on first use
        SMC_HIP(hipEventRecord(m->rows_ev, s));
        *rows = n_cand;
        return SMC_OK;
    }
    SMC_HIP(hipStreamSynchronize(s));
    count = m->host_state->n_out;
    if (count < 0 || count > n_cand) return fail(SMC_ERR_STATE, "output count %d", count);
    *rows = count;
    return SMC_OK;
}

static int build_map(smc_map* m, const int32_t* coords, int64_t n, int ncols,
                     const int32_t* spatial_shape, int batch_size, int kernel_size, int route,
                     unsigned flags, void* stream, bool strided) {
    if (!m) return fail(SMC_ERR_ARG, "map is NULL");
    if (kernel_size != 3 && kernel_size != 5)
        return fail(SMC_ERR_UNSUPPORTED, "kernel_size %d (3 or 5)", kernel_size);
    if (kernel_size == 5 && (flags & SMC_BUILD_NO_PAIRS))
        return fail(SMC_ERR_UNSUPPORTED, "kernel_size 5 maps always carry pair lists");
    if (ncols != 3 && ncols != 4) return fail(SMC_ERR_ARG, "ncols must be 3 or 4, got %d", ncols);
    if (n < 0 || n > kMaxRows) return fail(SMC_ERR_ARG, "n = %lld out of [0, 2^26]", (long long)n);
    if (n > 0 && !coords) return fail(SMC_ERR_ARG, "coords is NULL");
    if (route < SMC_ROUTE_AUTO || route > SMC_ROUTE_SORTED)
        return fail(SMC_ERR_ARG, "bad route %d", route);
    if (spatial_shape)
        for (int d = 0; d < 3; ++d)
            if (spatial_shape[d] < 1)
                return fail(SMC_ERR_ARG, "spatial_shape[%d] = %d", d, spatial_shape[d]);
    int rc = ensure_device(m);
    if (rc) return rc;
    hipStream_t s = (hipStream_t)stream;
    // an earlier build not waited for yet: its checks reach the sticky word when
    // this build's first kernel recycles its record (stream order), and the next
    // wait reports them (a build that fails before any kernel, or an empty one,
    // drops them with the earlier map). A record already read is recycled
    // without carrying anything.
    const bool carry = m->pending;
    m->pending = false;
    m->built = false;
    m->rows_pending = false;                      // (a failed build leaves no count to read)
    m->perm = nullptr;
    // this build's record and histograms; the other slot is cleared by its first kernel
    const int slot = m->slot ^ 1;
    m->slot = slot;
    MapState* st = m->state.as<MapState>() + slot;
    uint32_t* hist_mask = m->hist.as<uint32_t>() + slot * kHistInts;
    uint32_t* hist_key = hist_mask + kHistMaskInts;
    NextRecord next;
    next.st = m->state.as<MapState>() + (slot ^ 1);
    next.hist = m->hist.as<uint32_t>() + (slot ^ 1) * kHistInts;
    next.hist_ints = kHistInts;
    next.sticky = carry ? m->sticky.as<uint32_t>() : nullptr;
    StageTimer t_map(m, SMC_STAGE_MAP, s, /*bracket=*/true);
    if (!m->slot_clean[slot]) SMC_HIP(launch_state_init(st, hist_mask, kHistInts, nullptr, s));
    if (n > 0) m->slot_clean[slot] = false;

    // ---- geometry: explicit shape, or the bounding box (one read) ----
    Geom g{};
    g.ncols = ncols;
    g.ksize = kernel_size;
    g.pad = (kernel_size - 1) / 2;
    const int taps = kernel_size * kernel_size * kernel_size;
    const int mwords = kernel_size == 3 ? 1 : kMaxMaskWords;
    const bool need_bbox = n > 0 && (!spatial_shape || (ncols == 4 && batch_size <= 0));
    int32_t bbox[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    if (need_bbox) {
        SMC_HIP(launch_bbox(coords, n, ncols, st, s));
        SMC_HIP(hipMemcpyAsync(m->host_state, st, sizeof(MapState), hipMemcpyDeviceToHost, s));
        SMC_HIP(hipStreamSynchronize(s));
        memcpy(bbox, m->host_state->bbox, sizeof(bbox));
    }
    if (spatial_shape) {
        for (int d = 0; d < 3; ++d) {
            g.origin[d] = 0;
            g.ext[d] = spatial_shape[d];
        }
    } else if (n > 0 && strided) {
        // output cells are counted from coordinate 0: the grid is [0, max + 1)
        for (int d = 0; d < 3; ++d) {
            if (bbox[d] < 0) return fail(SMC_ERR_RANGE, "negative coordinate %d", bbox[d]);
            int64_t e = (int64_t)bbox[3 + d] + 1;
            if (e > ((int64_t)1 << 30)) return fail(SMC_ERR_RANGE, "extent %lld too large", (long long)e);
            g.origin[d] = 0;
            g.ext[d] = (int32_t)e;
        }
    } else if (n > 0) {
        for (int d = 0; d < 3; ++d) {
            g.origin[d] = bbox[d];
            int64_t e = (int64_t)bbox[3 + d] - bbox[d] + 1;
            if (e > ((int64_t)1 << 30)) return fail(SMC_ERR_RANGE, "extent %lld too large", (long long)e);
            g.ext[d] = (int32_t)e;
        }
    } else {
        for (int d = 0; d < 3; ++d) g.ext[d] = 1;
    }
    if (ncols == 3) {
        g.batch = 1;
    } else if (batch_size > 0) {
        g.batch = batch_size;
    } else if (n > 0) {
        if (bbox[6] < 0) return fail(SMC_ERR_RANGE, "negative batch index %d", bbox[6]);
        g.batch = bbox[7] + 1;
    } else {
        g.batch = 1;
    }

    // ---- route by grid volume ----
    const double pad2 = 2.0 * g.pad;
    const double cells_d =
        (double)g.batch * (g.ext[0] + pad2) * (g.ext[1] + pad2) * (g.ext[2] + pad2);
    // the dense route's cells: tall grids in whole bricks of 8 x 8 x 16 (brick_cell)
    const bool brick = g.ext[2] + 2 * g.pad >= kBrickMinZ;
    const double grid_cells_d = brick ? (double)g.batch * std::ceil((g.ext[0] + pad2) / 8.0) *
                                            std::ceil((g.ext[1] + pad2) / 8.0) *
                                            std::ceil((g.ext[2] + pad2) / 16.0) * 1024.0
                                      : cells_d;
    const bool dense_addressable = grid_cells_d < kDenseMaxCells;
    int chosen;
    if (route == SMC_ROUTE_DENSE) {
        if (!dense_addressable)
            return fail(SMC_ERR_GRID, "dense grid of %.3g cells exceeds 2^36", grid_cells_d);
        chosen = SMC_ROUTE_DENSE;
    } else if (route == SMC_ROUTE_SORTED) {
        chosen = SMC_ROUTE_SORTED;
    } else {
        // ids (4 bytes a cell) and the two bitmaps; a grid this handle has not
        // allocated yet must also fit half the device memory free now
        const double need = grid_cells_d * 4.25;
        bool fits = dense_addressable && need <= (double)m->dense_budget;
        if (fits && (double)m->grid.bytes < grid_cells_d * 4.0) {
            size_t free_b = 0, total_b = 0;
            if (hipMemGetInfo(&free_b, &total_b) != hipSuccess) {
                (void)hipGetLastError();
                fits = false;
            } else if (need > (double)free_b / 2) {
                fits = false;
            }
        }
        chosen = fits ? SMC_ROUTE_DENSE : SMC_ROUTE_SORTED;
    }
    g.sz_y = g.ext[2] + 2 * g.pad;
    g.sz_x = (int64_t)(g.ext[1] + 2 * g.pad) * g.sz_y;
    g.sz_b = (int64_t)(g.ext[0] + 2 * g.pad) * g.sz_x;
    g.bs_y = (g.ext[2] + 2 * g.pad + 15) / 16;
    g.bs_x = (int64_t)((g.ext[1] + 2 * g.pad + 7) / 8) * g.bs_y;
    g.bs_b = (int64_t)((g.ext[0] + 2 * g.pad + 7) / 8) * g.bs_x;
    g.brick = chosen == SMC_ROUTE_DENSE && brick ? 1 : 0;
    int key_bits = 0;
    if (chosen == SMC_ROUTE_SORTED) {
        // keys are cells of the padded grid: 0 .. cells - 1
        if (cells_d >= 9.0e18)
            return fail(SMC_ERR_KEY_OVERFLOW, "packed key of %.3g cells exceeds 63 bits", cells_d);
        key_bits = bit_len((int64_t)g.batch * g.sz_b - 1);
    }
    StrideGeom sg{};
    if (strided) {
        sg.stride = 2;
        sg.pad = 1;
        sg.ksize = 3;
        for (int d = 0; d < 3; ++d) {
            sg.oext[d] = (g.ext[d] + 2 * sg.pad - sg.ksize) / sg.stride + 1;
            sg.origin[d] = 0;
        }
        sg.wb = bit_len((int64_t)g.batch - 1);
        sg.wx = bit_len((int64_t)sg.oext[0] - 1);
        sg.wy = bit_len((int64_t)sg.oext[1] - 1);
        sg.wz = bit_len((int64_t)sg.oext[2] - 1);
        const int ob = sg.wb + sg.wx + sg.wy + sg.wz;
        if (ob > 62) return fail(SMC_ERR_KEY_OVERFLOW, "output key needs %d bits", ob);
        sg.sentinel = (uint64_t)1 << ob;
    }
    m->geom = g;
    m->route = chosen;
    m->key_bits = key_bits;
    m->wide = key_bits > 32;
    m->grid_cells = chosen != SMC_ROUTE_DENSE ? 0
                    : g.brick ? (int64_t)g.batch * g.bs_b * 1024 : (int64_t)g.batch * g.sz_b;
    m->n = n;

    // ---- buffers ----
    // a strided map: pair lists over its output rows (sized once the output
    // count is known), the plain mask order
    const bool want_pairs = !(flags & SMC_BUILD_NO_PAIRS);
    const bool want_sort = !(flags & SMC_BUILD_NO_SORT) && kernel_size == 3;
    const int64_t nn = n > 0 ? n : 1;
    const int64_t n_cand = strided ? 8 * nn : 0;      // candidate output cells (8 per input)
    const int64_t rows_cap = strided ? n_cand : nn;   // rows of the map's tables
    const int64_t cap = (nn + kCapAlign - 1) / kCapAlign * kCapAlign;
    const MaskOrder ord = want_sort && !strided ? m->order : MaskOrder();
    const int64_t items = rows_cap * ord.n_groups;    // mask-sort items: one per (group, row)
    size_t look_bytes = sort_look_bytes(items > nn ? items : nn);
    const size_t look_c = compact_look_bytes_k(rows_cap, kernel_size);
    if (look_c > look_bytes) look_bytes = look_c;
    if (strided && out_bitmap_words(sg, g.batch) <= kOutBitmapWords) {   // the bitmap's chunks
        const size_t look_o = (size_t)out_bitmap_blocks(out_bitmap_words(sg, g.batch)) * 8;
        if (look_o > look_bytes) look_bytes = look_o;
    }
    const size_t look_before = m->look.bytes;
    // (the neighbour table is read in whole 16-byte words: keep the last one readable)
    if ((rc = m->nbr.ensure((size_t)rows_cap * taps * 4 + 16, s)) ||
        (rc = m->mask.ensure((size_t)rows_cap * mwords * 4, s)) ||
        (rc = m->mkey0.ensure((size_t)items * 4, s)) || (rc = m->mkey1.ensure((size_t)items * 4, s)) ||
        (rc = m->mval0.ensure((size_t)items * 4, s)) || (rc = m->mval1.ensure((size_t)items * 4, s)) ||
        (rc = m->look.ensure(look_bytes, s)))
        return rc;
    if (!ord.plain && (rc = m->okeys.ensure((size_t)items * 4, s))) return rc;
    // strided outputs: a small output grid goes through a bitmap (no candidate
    // buffers); a larger one sorts 8 candidate keys per input
    const bool cand_sort = strided && out_bitmap_words(sg, g.batch) > kOutBitmapWords;
    if (strided &&
        ((rc = m->ocoords.ensure((size_t)n_cand * 16, s)) ||
         (rc = m->qcoords.ensure((size_t)n_cand * 16, s))))
        return rc;
    if (cand_sort &&
        ((rc = m->ck0.ensure((size_t)n_cand * 8, s)) || (rc = m->ck1.ensure((size_t)n_cand * 8, s)) ||
         (rc = m->ck2.ensure((size_t)n_cand * 8, s)) || (rc = m->cv0.ensure((size_t)n_cand * 4, s)) ||
         (rc = m->cv1.ensure((size_t)n_cand * 4, s)) ||
         (rc = m->chist.ensure((size_t)kHistKeyInts * 4, s)) ||
         (rc = m->ucounts.ensure((size_t)unique_blocks(n_cand) * 4, s))))
        return rc;
    if (want_pairs && !strided &&
        ((rc = m->pair_in.ensure((size_t)taps * cap * 4, s)) ||
         (rc = m->pair_out.ensure((size_t)taps * cap * 4, s)) ||
         (rc = m->pair_slot.ensure((size_t)taps * cap * 4, s)) ||
         (rc = m->rowbase.ensure((size_t)(nn + 1) * 4, s)) ||
         (rc = m->chunk_pre.ensure((size_t)(compact_chunks(nn) + 1) * (kTaps + 1) * 4, s))))
        return rc;
    {
        // the largest sort of the build: input keys, strided candidates or mask-sort items
        int64_t big = nn;
        if (cand_sort && n_cand > big) big = n_cand;
        if (items > big) big = items;
        const int64_t scan_ints = sort_scan_ints(big);
        if (scan_ints > 0 && (rc = m->scan.ensure((size_t)scan_ints * 4, s))) return rc;
        m->ws.cnt = scan_ints > 0 ? m->scan.as<uint32_t>() : nullptr;
        m->ws.cnt_ints = scan_ints > 0 ? (int64_t)(m->scan.bytes / 4) : 0;
    }
    if (m->look.bytes != look_before || look_before == 0)   // new table: epoch 0 everywhere
        SMC_HIP(launch_fill_i32(m->look.as<int32_t>(), (int64_t)(m->look.bytes / 4), 0, s));
    m->ws.look = m->look.as<uint64_t>();
    m->cap = cap;
    uint32_t* status = &st->status;

    int64_t rows = strided ? 0 : n;                  // rows of the map (strided: output cells)
    // strided pair-list builds size everything after the output cells by the
    // bound 8 n and read the count on the device: no wait inside the build (up
    // to a bound of 2^23 rows, whose pair lists take 2.7 GB; larger builds read
    // the count back and size by it)
    constexpr int64_t kDeferMaxRows = (int64_t)1 << 23;
    const bool defer_rows = strided && want_pairs && !want_sort && n > 0 && 8 * n <= kDeferMaxRows;
    const int32_t* n_out_dev = defer_rows ? &st->n_out : nullptr;
    // a strided map's pair lists over its (bound of) rows: every tap sparse
    auto strided_pair_bufs = [&](int64_t rr) -> int {
        const int64_t cap_s = (rr + kCapAlign - 1) / kCapAlign * kCapAlign;
        int rc2;
        if ((rc2 = m->pair_in.ensure((size_t)taps * cap_s * 4, s)) ||
            (rc2 = m->pair_out.ensure((size_t)taps * cap_s * 4, s)) ||
            (rc2 = m->pair_slot.ensure((size_t)taps * cap_s * 4, s)) ||
            (rc2 = m->rowbase.ensure((size_t)(rr + 1) * 4, s)) ||
            (rc2 = m->chunk_pre.ensure((size_t)(compact_chunks(rr) + 1) * (kTaps + 1) * 4, s)))
            return rc2;
        m->cap = cap_s;
        return SMC_OK;
    };
    bool compacted = false;                          // the pair lists came with the lookup
    if (n > 0) {
        int32_t* nbr = m->nbr.as<int32_t>();
        uint32_t* mask = m->mask.as<uint32_t>();
        const bool fused = chosen == SMC_ROUTE_DENSE && want_pairs && kernel_size == 3 && !strided;
        // the fused kernel writes the table only when asked to or when the mask-tile
        // path (which gathers through it) may run on this map
        int32_t* nbr_out = fused && !want_sort && !(flags & SMC_BUILD_TABLE) ? nullptr : nbr;
        StageTimer t_nb(m, SMC_STAGE_NEIGHBOURS, s);
        if (chosen == SMC_ROUTE_DENSE) {
            const int gi = m->next_grid;
            if ((rc = ensure_grid(m, gi, m->grid_cells, s)) ||
                (rc = m->cells[gi].ensure((size_t)nn * 4, s)))
                return rc;
            int32_t* grid = m->grid.as<int32_t>();
            uint32_t* bits = m->bits[gi].as<uint32_t>();
            // a strided build on the output bitmap's route marks its output cells
            // in the same pass
            const bool mark = strided && out_bitmap_words(sg, g.batch) <= kOutBitmapWords;
            if (mark && (rc = prepare_obits(m, out_bitmap_words(sg, g.batch), s))) return rc;
            SMC_HIP(launch_dense_scatter(coords, n, g, grid, bits, m->cells[gi].as<int32_t>(), st,
                                         next, m->stale, s, mark ? m->obits.as<uint32_t>() : nullptr,
                                         &sg));
            m->slot_clean[slot ^ 1] = true;
            m->stale.cells = m->cells[gi].as<int32_t>();
            m->stale.n = n;
            m->stale.bits = bits;
            m->next_grid = gi ^ 1;
            if (fused) {
                t_nb.finish();
                StageTimer t_cp(m, SMC_STAGE_COMPACT, s);
                SMC_HIP(launch_lookup_compact(coords, n, g, grid, bits, nbr_out, mask, cap, kTileM, st,
                                              m->pair_in.as<int32_t>(), m->pair_out.as<int32_t>(),
                                              m->pair_slot.as<int32_t>(),
                                              m->rowbase.as<int32_t>(),
                                              m->chunk_pre.as<int32_t>(), m->ws, status, s));
                t_cp.finish();
            } else if (strided) {
                if ((rc = strided_outputs(m, coords, n, g, sg, st, status, s, &rows, defer_rows,
                                          mark)))
                    return rc;
                Geom gq = g;                          // query points: [M, 4] in input coordinates
                gq.ncols = 4;
                if (want_pairs && !want_sort && kernel_size == 3 && rows > 0) {
                    // lookup and compaction in one kernel (the centre a sparse tap); the
                    // table only when asked for: nothing after the pair lists reads it
                    if ((rc = strided_pair_bufs(rows))) return rc;
                    t_nb.finish();
                    StageTimer t_cp(m, SMC_STAGE_COMPACT, s);
                    SMC_HIP(launch_lookup_compact(m->qcoords.as<int32_t>(), rows, gq, grid, bits,
                                                  (flags & SMC_BUILD_TABLE) ? nbr : nullptr,
                                                  mask, m->cap, kTileM, st,
                                                  m->pair_in.as<int32_t>(),
                                                  m->pair_out.as<int32_t>(),
                                                  m->pair_slot.as<int32_t>(),
                                                  m->rowbase.as<int32_t>(),
                                                  m->chunk_pre.as<int32_t>(), m->ws, status, s,
                                                  true, n_out_dev));
                    t_cp.finish();
                    compacted = true;
                } else {                              // (rows exact: no device count)
                    SMC_HIP(launch_dense_lookup(m->qcoords.as<int32_t>(), rows, gq, grid, bits,
                                                nbr, mask, s));
                }
            } else {
                SMC_HIP(launch_dense_lookup(coords, n, g, grid, bits, nbr, mask, s));
            }
        } else {
            if (m->stale.n > 0) {             // the last dense build's cells
                SMC_HIP(launch_clear_cells(m->stale, s));
                m->stale = PrevCells();
            }
            const size_t kb = (size_t)nn * (m->wide ? 8 : 4);
            if ((rc = m->keys0.ensure(kb, s)) || (rc = m->keys1.ensure(kb, s)) ||
                (rc = m->keys2.ensure(kb, s)) || (rc = m->vals0.ensure((size_t)nn * 4, s)) ||
                (rc = m->vals1.ensure((size_t)nn * 4, s)))
                return rc;
            const SortPlan kp = key_sort_plan(key_bits, n);
            SMC_HIP(launch_make_keys(coords, n, g, m->wide, m->keys0.p, st, next, kp, hist_key, s));
            m->slot_clean[slot ^ 1] = true;
            const void* skeys;
            const uint32_t* svals;
            // the key sort's last pass also lists splitters for the lookup's searches
            const int sh = split_shift_for(n);
            void* split = nullptr;
            if (!strided) {
                if ((rc = m->split.ensure((size_t)kMaxSplit * 8, s))) return rc;
                split = m->split.p;
            }
            if (m->wide) {
                SMC_HIP(radix_sort_u64(m->keys0.as<uint64_t>(), nullptr, n, kp, hist_key,
                                       m->keys1.as<uint64_t>(), m->keys2.as<uint64_t>(),
                                       m->vals0.as<uint32_t>(), m->vals1.as<uint32_t>(), m->ws,
                                       status, (const uint64_t**)&skeys, &svals, s, split, sh));
            } else {
                SMC_HIP(radix_sort_u32(m->keys0.as<uint32_t>(), nullptr, n, kp, hist_key,
                                       m->keys1.as<uint32_t>(), m->keys2.as<uint32_t>(),
                                       m->vals0.as<uint32_t>(), m->vals1.as<uint32_t>(), m->ws,
                                       status, (const uint32_t**)&skeys, &svals, s, split, sh));
            }
            if (strided) {
                SMC_HIP(launch_key_dups(skeys, m->wide, n, st, s));
                if ((rc = strided_outputs(m, coords, n, g, sg, st, status, s, &rows, defer_rows,
                                          false)))
                    return rc;
                SMC_HIP(launch_query_lookup(skeys, svals, n, g, m->wide, m->qcoords.as<int32_t>(),
                                            rows, nbr, mask, s, n_out_dev));
            } else {
                SMC_HIP(launch_sorted_lookup(skeys, svals, n, g, m->wide, split, sh, nbr, mask, st,
                                             s));
            }
        }
        t_nb.finish();
        // the mask histogram also gives the per-tap counts of a map without pair lists
        if (want_sort || !want_pairs) {
            // rows ordered by (mask, row): histograms (+ per-tap totals), then passes
            StageTimer t_ms(m, SMC_STAGE_MASK_SORT, s);
            // (with a calibrated order or offset groups: per-group keys, one sort of them all)
            SortPlan mp = sort_plan(mask_sort_bits(ord));
            if (!want_sort) mp.passes = 0;
            if (mp.passes * (1 << mp.bits) > kHistMaskInts)
                return fail(SMC_ERR_UNSUPPORTED, "mask sort needs %d histogram bins",
                            mp.passes * (1 << mp.bits));
            uint32_t* okeys = ord.plain ? nullptr : m->okeys.as<uint32_t>();
            if (rows > 0)
                SMC_HIP(launch_mask_hist(mask, rows, mp, ord, okeys, hist_mask, st->tap_tot,
                                         st->group_rows, s));
            if (want_sort && rows > 0) {
                const uint32_t* sorted_keys;
                SMC_HIP(radix_sort_u32(ord.plain ? mask : okeys, nullptr, rows * ord.n_groups, mp,
                                       hist_mask, m->mkey0.as<uint32_t>(),
                                       m->mkey1.as<uint32_t>(), m->mval0.as<uint32_t>(),
                                       m->mval1.as<uint32_t>(), m->ws, status, &sorted_keys,
                                       &m->perm, s));
            }
            t_ms.finish();
        }
        if (want_pairs && !fused && strided && !compacted) {
            // the output rows' pair lists: every tap sparse, the centre too
            if ((rc = strided_pair_bufs(rows > 0 ? rows : 1))) return rc;
            const int64_t cap_s = m->cap;
            if (rows > 0) {
                StageTimer t_cp(m, SMC_STAGE_COMPACT, s);
                SMC_HIP(launch_compact(mask, nbr, rows, kernel_size, cap_s, kTileM, st,
                                       m->pair_in.as<int32_t>(), m->pair_out.as<int32_t>(),
                                       m->pair_slot.as<int32_t>(), m->rowbase.as<int32_t>(),
                                       m->chunk_pre.as<int32_t>(), m->ws, status, s, false,
                                       n_out_dev));
                t_cp.finish();
            }
        } else if (want_pairs && !fused && !strided) {
            StageTimer t_cp(m, SMC_STAGE_COMPACT, s);
            SMC_HIP(launch_compact(mask, nbr, n, kernel_size, cap, kTileM, st,
                                   m->pair_in.as<int32_t>(),
                                   m->pair_out.as<int32_t>(), m->pair_slot.as<int32_t>(),
                                   m->rowbase.as<int32_t>(), m->chunk_pre.as<int32_t>(), m->ws,
                                   status, s));
            t_cp.finish();
        }
    }
    m->has_pairs = want_pairs;
    m->has_sort = want_sort;
    m->has_table = !(chosen == SMC_ROUTE_DENSE && want_pairs && kernel_size == 3 && !want_sort &&
                     !(flags & SMC_BUILD_TABLE)) || n == 0;
    m->sorted_order = ord;
    m->ksize = kernel_size;
    m->strided = strided;
    m->n_in = n;
    m->n = rows;
    m->rows_pending = n_out_dev != nullptr;
    m->sgeom = sg;
    t_map.finish();
    const bool async = (flags & SMC_BUILD_ASYNC) != 0;
    if (!async)
        SMC_HIP(hipMemcpyAsync(m->host_state, st, sizeof(MapState), hipMemcpyDeviceToHost, s));
    m->state_copied = !async;
    // A synchronous build has copied its record into pinned host memory before
    // this event, so the event's system-scope fence makes that copy visible. An
    // asynchronous build's record is read later by hipMemcpy, after the event:
    // its fence (a write-back of the caches, about 4 us on MI355X between the
    // build and the first GEMM) buys nothing there, and the event goes without.
    m->done_last = async ? m->done_nf : m->done;
    SMC_HIP(hipEventRecord(m->done_last, s));
    m->pending = true;
    m->built = true;
    m->build_status = SMC_OK;
    if (async) return SMC_OK;
    return wait_build(m);
}

int smc_map_build(smc_map* m, const int32_t* coords, int64_t n, int ncols,
                  const int32_t* spatial_shape, int batch_size, int kernel_size, int route,
                  unsigned flags, void* stream) {
    return build_map(m, coords, n, ncols, spatial_shape, batch_size, kernel_size, route, flags,
                     stream, false);
}

int smc_map_build_strided(smc_map* m, const int32_t* coords, int64_t n, int ncols,
                          const int32_t* spatial_shape, int batch_size, int kernel_size,
                          int stride, int route, unsigned flags, void* stream) {
    if (!m) return fail(SMC_ERR_ARG, "map is NULL");
    if (kernel_size != 3 || stride != 2)
        return fail(SMC_ERR_UNSUPPORTED, "strided maps: kernel 3, stride 2 (got %d, %d)",
                    kernel_size, stride);
    if (n > kMaxStridedRows)
        return fail(SMC_ERR_ARG, "n = %lld above 2^24 for a strided map", (long long)n);
    return build_map(m, coords, n, ncols, spatial_shape, batch_size, kernel_size, route, flags,
                     stream, true);
}

int smc_map_export_out_coords(smc_map* m, int32_t* out_coords) {
    if (!m) return fail(SMC_ERR_ARG, "map is NULL");
    if (!m->built) return fail(SMC_ERR_STATE, "map was never built");
    if (!m->strided) return fail(SMC_ERR_STATE, "not a strided map (outputs are the inputs)");
    SMC_HIP(hipSetDevice(m->device));
    (void)wait_build(m);
    SMC_HIP(hipDeviceSynchronize());
    if (m->n > 0 && out_coords)
        SMC_HIP(hipMemcpy(out_coords, m->ocoords.p, (size_t)m->n * 16, hipMemcpyDeviceToHost));
    return SMC_OK;
}

int smc_map_sync(smc_map* m) {
    if (!m) return fail(SMC_ERR_ARG, "map is NULL");
    if (!m->built) return fail(SMC_ERR_STATE, "map was never built");
    int rc = wait_build(m);
    if (rc) return rc;
    return m->build_status;
}

int smc_map_rows(smc_map* m, int64_t* n, int64_t* n_in) {
    if (!m) return fail(SMC_ERR_ARG, "map is NULL");
    if (!m->built) return fail(SMC_ERR_STATE, "map was never built");
    if (int rc = resolve_rows(m)) return rc;
    if (n) *n = m->n;
    if (n_in) *n_in = m->n_in;
    return SMC_OK;
}

int smc_map_info(smc_map* m, smc_map_info_t* info) {
    if (!m || !info) return fail(SMC_ERR_ARG, "NULL argument");
    if (!m->built) return fail(SMC_ERR_STATE, "map was never built");
    int rc = wait_build(m);
    memset(info, 0, sizeof(*info));
    info->n = m->n;
    info->route = m->route;
    info->key_bits = m->key_bits;
    for (int d = 0; d < 3; ++d) {
        info->origin[d] = m->geom.origin[d];
        info->extent[d] = m->geom.ext[d];
    }
    info->batch = m->geom.batch;
    info->tile_m = kTileM;
    info->grid_cells = m->grid_cells;
    info->kernel_size = m->ksize;
    info->n_in = m->n_in;
    info->strided = m->strided ? 1 : 0;
    for (int d = 0; d < 3; ++d) info->out_extent[d] = m->strided ? m->sgeom.oext[d] : m->geom.ext[d];
    const int taps = m->ksize * m->ksize * m->ksize;
    info->taps = taps;
    const MapState& hs = *m->host_state;
    if (m->n == 0) {
        // nothing was counted
    } else if (m->has_pairs) {
        info->pairs = hs.totals[0];
        info->pairs_padded = hs.totals[1];
        info->n_tiles = hs.totals[2];
        for (int k = 0; k < taps; ++k) info->tap_count[k] = hs.tap_count[k];
    } else {                           // counts from the mask histogram; no lists were written
        for (int k = 0; k < kTaps; ++k) {
            info->tap_count[k] = hs.tap_tot[k];
            info->pairs += hs.tap_tot[k];
        }
    }
    info->status = rc ? rc : m->build_status;
    info->n_groups = m->has_sort ? m->sorted_order.n_groups : 0;
    if (m->has_sort) {
        for (int g = 0; g < info->n_groups; ++g)
            info->group_rows[g] = m->sorted_order.plain || g == info->n_groups - 1 ? m->n
                                                                                   : hs.group_rows[g];
    }
    return SMC_OK;
}

int smc_map_export(smc_map* m, int32_t* nbr, uint32_t* mask, int32_t* perm, int32_t* pair_in,
                   int32_t* pair_out, int64_t* tap_off) {
    if (!m) return fail(SMC_ERR_ARG, "map is NULL");
    if (!m->built) return fail(SMC_ERR_STATE, "map was never built");
    if ((pair_in || pair_out) && !m->has_pairs)
        return fail(SMC_ERR_STATE, "map was built without pair lists (SMC_BUILD_NO_PAIRS)");
    if (perm && !m->has_sort)
        return fail(SMC_ERR_STATE, "map was built without the mask order (SMC_BUILD_NO_SORT)");
    SMC_HIP(hipSetDevice(m->device));
    (void)wait_build(m);
    SMC_HIP(hipDeviceSynchronize());
    const int64_t n = m->n;
    const MapState& hs = *m->host_state;
    const int taps = m->ksize * m->ksize * m->ksize;
    const int mwords = m->ksize == 3 ? 1 : kMaxMaskWords;
    if (n > 0) {
        if (nbr && m->has_table)
            SMC_HIP(hipMemcpy(nbr, m->nbr.p, (size_t)n * taps * 4, hipMemcpyDeviceToHost));
        if (nbr && !m->has_table) {
            // the table was not kept: every entry is a pair of the lists
            std::vector<int32_t> pin, pout;
            for (int64_t i = 0; i < n * taps; ++i) nbr[i] = -1;
            for (int k = 0; k < taps; ++k) {
                const int64_t c = hs.tap_count[k];
                if (c > m->cap) return fail(SMC_ERR_STATE, "tap %d holds %lld pairs", k, (long long)c);
                if (c == 0) continue;
                pin.resize((size_t)c);
                pout.resize((size_t)c);
                SMC_HIP(hipMemcpy(pin.data(), m->pair_in.as<int32_t>() + (int64_t)k * m->cap,
                                  (size_t)c * 4, hipMemcpyDeviceToHost));
                SMC_HIP(hipMemcpy(pout.data(), m->pair_out.as<int32_t>() + (int64_t)k * m->cap,
                                  (size_t)c * 4, hipMemcpyDeviceToHost));
                for (int64_t j = 0; j < c; ++j) {
                    if (pout[j] < 0 || pout[j] >= n)
                        return fail(SMC_ERR_STATE, "pair output row %d out of range", pout[j]);
                    nbr[(int64_t)pout[j] * taps + k] = pin[j];
                }
            }
        }
        if (mask)
            SMC_HIP(hipMemcpy(mask, m->mask.p, (size_t)n * mwords * 4, hipMemcpyDeviceToHost));
        if (perm) {
            // item indices g n + row -> rows, group by group
            const int G = m->sorted_order.n_groups;
            SMC_HIP(hipMemcpy(perm, m->perm, (size_t)G * n * 4, hipMemcpyDeviceToHost));
            for (int g = 1; g < G; ++g)
                for (int64_t i = 0; i < n; ++i) perm[g * n + i] -= (int32_t)(g * n);
        }
    }
    if (tap_off) {
        tap_off[0] = 0;
        for (int k = 0; k < taps; ++k)
            tap_off[k + 1] = tap_off[k] + (n == 0 ? 0 : m->has_pairs ? hs.tap_count[k] : hs.tap_tot[k]);
    }
    if ((pair_in || pair_out) && n > 0) {
        // tap k's run starts at k * cap on the device
        for (int which = 0; which < 2; ++which) {
            int32_t* dst = which == 0 ? pair_in : pair_out;
            if (!dst) continue;
            const int32_t* src = (which == 0 ? m->pair_in : m->pair_out).as<int32_t>();
            int64_t o = 0;
            for (int k = 0; k < taps; ++k) {
                const int64_t c = hs.tap_count[k];
                if (c > m->cap) return fail(SMC_ERR_STATE, "tap %d holds %lld pairs", k, (long long)c);
                if (c > 0)
                    SMC_HIP(hipMemcpy(dst + o, src + (int64_t)k * m->cap, (size_t)c * 4,
                                      hipMemcpyDeviceToHost));
                o += c;
            }
        }
    }
    return SMC_OK;
}

size_t smc_weight_packed_bytes(int kernel_size, int c_in, int c_out) {
    if (c_in < 1 || c_out < 1 || (kernel_size != 3 && kernel_size != 5)) return 0;
    return packed_weight_bytes(kernel_size * kernel_size * kernel_size, c_in, c_out);
}

int smc_weight_pack(const uint16_t* w, int kernel_size, int c_in, int c_out, void* out,
                    void* stream) {
    if (!w || !out) return fail(SMC_ERR_ARG, "NULL pointer");
    if (kernel_size != 3 && kernel_size != 5)
        return fail(SMC_ERR_UNSUPPORTED, "kernel_size %d (3 or 5)", kernel_size);
    if (c_in < 1 || c_out < 1) return fail(SMC_ERR_ARG, "c_in = %d, c_out = %d", c_in, c_out);
    if (((uintptr_t)out & 15) != 0) return fail(SMC_ERR_ARG, "packed buffer not 16-byte aligned");
    SMC_HIP(launch_weight_pack(w, kernel_size * kernel_size * kernel_size, c_in, c_out, out,
                               (hipStream_t)stream));
    return SMC_OK;
}

}  // extern "C"

// The forward of both entry points. fixed == nullptr: the handle's slab
// (grow-only, allocated here when short). Otherwise fixed (fixed_bytes long)
// holds the slab or partial sums, nothing is allocated and no stage timer
// runs (an event pool may grow).
static int conv_forward(smc_map* m, const uint16_t* x, int c_in, const void* wpacked, int c_out,
                        void* y, unsigned flags, void* stream, float* fixed, size_t fixed_bytes) {
    if (!m) return fail(SMC_ERR_ARG, "map is NULL");
    if (!m->built) return fail(SMC_ERR_STATE, "map was never built");
    if (int rc = resolve_rows(m)) return rc;
    if (!m->pending && m->build_status != SMC_OK)
        return fail(SMC_ERR_STATE, "map build failed: %s", smc_status_string(m->build_status));
    if (c_in < 1 || c_out < 1) return fail(SMC_ERR_ARG, "c_in = %d, c_out = %d", c_in, c_out);
    if (c_in > kMaxChannels || c_out > kMaxChannels)
        return fail(SMC_ERR_UNSUPPORTED, "channels above 4096");
    // a strided map without pair lists has mask tiles only
    const bool mask_tiles = (flags & SMC_FWD_MASK_TILES) != 0 || (m->strided && !m->has_pairs);
    if (!mask_tiles && !m->has_pairs)
        return fail(SMC_ERR_STATE, "map was built without pair lists (SMC_BUILD_NO_PAIRS)");
    if (mask_tiles && m->ksize != 3)
        return fail(SMC_ERR_UNSUPPORTED, "mask tiles need a 3x3x3 map (this one is %d^3)",
                    m->ksize);
    if (mask_tiles && !m->has_sort)
        return fail(SMC_ERR_STATE, "map was built without the mask order (SMC_BUILD_NO_SORT)");
    if (m->n == 0) return SMC_OK;
    if (!x || !wpacked || !y) return fail(SMC_ERR_ARG, "NULL pointer");
    if (((uintptr_t)wpacked & 15) != 0) return fail(SMC_ERR_ARG, "packed weights not 16-byte aligned");
    if ((c_in & 7) == 0 && ((uintptr_t)x & 15) != 0)
        return fail(SMC_ERR_ARG, "x must be 16-byte aligned when c_in is a multiple of 8");
    if (((uintptr_t)y & 15) != 0) return fail(SMC_ERR_ARG, "y must be 16-byte aligned");
    int dev = 0;
    SMC_HIP(hipGetDevice(&dev));
    if (dev != m->device) return fail(SMC_ERR_STATE, "map lives on device %d", m->device);
    hipStream_t s = (hipStream_t)stream;
    if (mask_tiles) {
        // one pass per offset group; the earlier ones leave float32 partial sums
        const MaskOrder& o = m->sorted_order;
        float* partial = nullptr;
        if (o.n_groups > 1) {
            const size_t need = (size_t)m->n * c_out * 4;
            if (fixed) {
                if (need > fixed_bytes)
                    return fail(SMC_ERR_UNSUPPORTED,
                                "partial sums of %zu bytes exceed the fixed scratch of %zu bytes",
                                need, fixed_bytes);
                partial = fixed;
            } else {
                int rc = m->part.ensure(need, s);
                if (rc) return rc;
                partial = m->part.as<float>();
            }
        }
        const MapState* dst = m->state.as<MapState>() + m->slot;
        StageTimer t_mt(m, SMC_STAGE_GEMM, s, false, fixed == nullptr);
        uint32_t prev = 0;
        for (int g = 0; g < o.n_groups; ++g) {
            GroupPass gp;
            gp.gm = 0;
            for (int t = 0; t < kTaps; ++t)
                if (o.grp[t] == g || o.plain) gp.gm |= 1u << t;
            gp.prev = prev;
            gp.last = g == o.n_groups - 1;
            gp.perm = m->perm + (int64_t)g * m->n;
            gp.goff = (int64_t)g * m->n;
            gp.rows = gp.last ? nullptr : dst->group_rows + g;
            gp.partial = partial;
            gp.centre_self = !m->strided;
            gp.n_in = m->n_in;
            SMC_HIP(launch_conv_masktile(x, c_in, wpacked, c_out, m->nbr.as<int32_t>(),
                                         m->mask.as<uint32_t>(), gp, m->n,
                                         m->zrow.as<uint16_t>(), y, (flags & SMC_FWD_OUT_F32) != 0,
                                         (flags & SMC_FWD_RELU) != 0, s));
            prev |= gp.gm;
        }
        t_mt.finish();
        return SMC_OK;
    }
    const int taps = m->ksize * m->ksize * m->ksize;
    if (rows_eligible(taps, c_in, c_out) && !m->strided && !(flags & SMC_FWD_SLAB_IN_MEMORY)) {
        // one kernel, the slab in LDS: nothing to allocate, no count to read
        StageTimer t_r(m, SMC_STAGE_GEMM, s, false, fixed == nullptr);
        SMC_HIP(launch_gemm_rows(x, c_in, wpacked, c_out, m->pair_in.as<int32_t>(),
                                 m->pair_slot.as<int32_t>(), m->chunk_pre.as<int32_t>(),
                                 m->rowbase.as<int32_t>(), m->state.as<MapState>() + m->slot,
                                 m->cap, m->n, y, (flags & SMC_FWD_OUT_F32) != 0,
                                 (flags & SMC_FWD_RELU) != 0, m->n_cu, s));
        t_r.finish();
        return SMC_OK;
    }
    // slab: 4 c_out bytes per off-centre pair (a strided map: per pair); without
    // the build's counts, taps - 1 (taps) a row
    double slab = (double)(m->strided ? taps : taps - 1) * m->n * c_out * 4.0;
    if (m->pending && slab > (double)kSlabBoundBytes) {
        int rc = wait_build(m);
        if (rc) return rc;
    }
    if (fixed && m->pending && slab > (double)fixed_bytes) {
        int rc = wait_build(m);                  // the exact count decides
        if (rc) return rc;
    }
    if (!m->pending) slab = (double)m->host_state->totals[3] * c_out * 4.0;
    if (slab > (double)((size_t)1 << 46)) return fail(SMC_ERR_ALLOC, "slab of %.3g bytes", slab);
    // at least one row: lanes with nothing to add read row 0
    if (slab < (double)c_out * 4.0) slab = (double)c_out * 4.0;
    float* part = fixed;
    if (fixed) {
        if (slab > (double)fixed_bytes)
            return fail(SMC_ERR_UNSUPPORTED, "slab of %.0f bytes exceeds the fixed scratch of %zu bytes",
                        slab, fixed_bytes);
    } else {
        int rc = m->part.ensure((size_t)slab, s);
        if (rc) return rc;
        part = m->part.as<float>();
    }
    StageTimer t_g(m, SMC_STAGE_GEMM, s, false, fixed == nullptr);
    SMC_HIP(launch_gemm_nc(x, c_in, wpacked, c_out, taps, m->pair_in.as<int32_t>(),
                           m->pair_slot.as<int32_t>(), m->state.as<MapState>() + m->slot, m->cap,
                           m->n_in, m->n_cu, part, s, !m->strided, y,
                           (flags & SMC_FWD_OUT_F32) != 0, (flags & SMC_FWD_RELU) != 0));
    t_g.finish();
    StageTimer t_f(m, SMC_STAGE_CENTRE, s, false, fixed == nullptr);
    if (m->strided) {
        // every tap went to the slab: each output row is its slab run's sum
        SMC_HIP(launch_slab_sum(part, m->rowbase.as<int32_t>(), m->n, c_out, y,
                                (flags & SMC_FWD_OUT_F32) != 0, (flags & SMC_FWD_RELU) != 0,
                                m->n_cu, s));
    } else {
        SMC_HIP(launch_gemm_centre(x, c_in, wpacked, c_out, taps,
                                   m->rowbase.as<int32_t>(), m->n, part, y,
                                   (flags & SMC_FWD_OUT_F32) != 0, (flags & SMC_FWD_RELU) != 0,
                                   m->n_cu, s));
    }
    t_f.finish();
    return SMC_OK;
}

extern "C" {

int smc_conv_forward(smc_map* m, const uint16_t* x, int c_in, const void* wpacked, int c_out,
                     void* y, unsigned flags, void* stream) {
    return conv_forward(m, x, c_in, wpacked, c_out, y, flags, stream, nullptr, 0);
}

int smc_conv_forward_noalloc(smc_map* m, const uint16_t* x, int c_in, const void* wpacked,
                             int c_out, void* y, unsigned flags, void* stream) {
    if (!m) return fail(SMC_ERR_ARG, "map is NULL");
    if (!m->built) return fail(SMC_ERR_STATE, "map was never built");
    void* p = scratch_ptr(m->device);
    if (!p) return fail(SMC_ERR_HIP, "device address of the fixed scratch unavailable on device %d",
                        m->device);
    return conv_forward(m, x, c_in, wpacked, c_out, y, flags, stream, static_cast<float*>(p),
                        kScratchBytes);
}

int smc_map_set_order(smc_map* m, const int32_t* bit_order, const int32_t* group_of) {
    if (!m) return fail(SMC_ERR_ARG, "map is NULL");
    int order[kTaps], grp[kTaps];
    for (int j = 0; j < kTaps; ++j) order[j] = bit_order ? bit_order[j] : kTaps - 1 - j;
    for (int t = 0; t < kTaps; ++t) grp[t] = group_of ? group_of[t] : 0;
    bool seen[kTaps] = {};
    for (int j = 0; j < kTaps; ++j) {
        if (order[j] < 0 || order[j] >= kTaps || seen[order[j]])
            return fail(SMC_ERR_ARG, "bit_order must list each of the 27 taps once");
        seen[order[j]] = true;
    }
    int n_groups = 0;
    for (int t = 0; t < kTaps; ++t) {
        if (grp[t] < 0 || grp[t] >= kMaxGroups)
            return fail(SMC_ERR_ARG, "group_of[%d] = %d outside [0, %d)", t, grp[t], kMaxGroups);
        if (grp[t] + 1 > n_groups) n_groups = grp[t] + 1;
    }
    int size[kMaxGroups] = {};
    for (int t = 0; t < kTaps; ++t) ++size[grp[t]];
    for (int g = 0; g < n_groups; ++g)
        if (size[g] == 0) return fail(SMC_ERR_ARG, "group %d has no tap", g);
    if (grp[kCentre] != n_groups - 1)
        return fail(SMC_ERR_ARG, "the centre tap (13) must be in the last group");
    MaskOrder o;
    o.n_groups = n_groups;
    o.group_bits = 0;
    int left[kMaxGroups];
    for (int g = 0; g < n_groups; ++g) {
        left[g] = size[g];
        if (size[g] > o.group_bits) o.group_bits = size[g];
    }
    // the first tap of a group in bit order takes its group key's highest bit
    for (int j = 0; j < kTaps; ++j) {
        const int t = order[j];
        o.grp[t] = (uint8_t)grp[t];
        o.pos[t] = (uint8_t)(--left[grp[t]]);
    }
    bool identity = n_groups == 1;
    for (int t = 0; t < kTaps; ++t) identity = identity && o.pos[t] == t;
    o.plain = identity ? 1 : 0;
    if (o.plain) o.group_bits = kMaskBits;
    m->order = o;
    return SMC_OK;
}

namespace {

// Executed tap-rows of the mask tiles when the rows are sorted by the key
// that the bit order `order` gives (one group, kMtRows rows per tile): a
// stable LSD radix sort of the keys, then per tile its rows times the
// popcount of the OR of their masks.
int64_t calib_work(const std::vector<uint32_t>& mask, const int* order, std::vector<uint32_t>& key,
                   std::vector<uint32_t>& idx, std::vector<uint32_t>& tmp) {
    const int64_t n = (int64_t)mask.size();
    uint32_t tab[4][256];
    for (int b = 0; b < 4; ++b)
        for (int v = 0; v < 256; ++v) {
            uint32_t k = 0;
            for (int j = 0; j < kTaps; ++j) {
                const int t = order[j];
                if (t / 8 == b && ((v >> (t % 8)) & 1)) k |= 1u << (kTaps - 1 - j);
            }
            tab[b][v] = k;
        }
    for (int64_t i = 0; i < n; ++i) {
        const uint32_t m = mask[i];
        key[i] = tab[0][m & 255] | tab[1][(m >> 8) & 255] | tab[2][(m >> 16) & 255] |
                 tab[3][(m >> 24) & 255];
        idx[i] = (uint32_t)i;
    }
    for (int pass = 0; pass < 3; ++pass) {
        const int sh = 9 * pass;
        int64_t cnt[513] = {};
        for (int64_t i = 0; i < n; ++i) ++cnt[((key[idx[i]] >> sh) & 511) + 1];
        for (int d = 0; d < 512; ++d) cnt[d + 1] += cnt[d];
        for (int64_t i = 0; i < n; ++i) tmp[cnt[(key[idx[i]] >> sh) & 511]++] = idx[i];
        idx.swap(tmp);
    }
    int64_t work = 0;
    for (int64_t s0 = 0; s0 < n; s0 += kTileM) {
        const int64_t e = s0 + kTileM < n ? s0 + kTileM : n;
        uint32_t u = 0;
        for (int64_t i = s0; i < e; ++i) u |= mask[idx[i]];
        work += (e - s0) * __builtin_popcount(u);
    }
    return work;
}

}  // namespace

int smc_map_calibrate(smc_map* m, int n_groups, int32_t* bit_order, int32_t* group_of) {
    if (!m || !bit_order || !group_of) return fail(SMC_ERR_ARG, "NULL argument");
    if (!m->built) return fail(SMC_ERR_STATE, "map was never built");
    if (m->ksize != 3) return fail(SMC_ERR_UNSUPPORTED, "row orders are for 3x3x3 maps");
    if (n_groups < 1 || n_groups > kMaxGroups)
        return fail(SMC_ERR_ARG, "n_groups = %d outside [1, %d]", n_groups, kMaxGroups);
    SMC_HIP(hipSetDevice(m->device));
    int rc = wait_build(m);
    if (rc) return rc;
    if (m->build_status != SMC_OK) return fail(SMC_ERR_STATE, "map build failed");
    const int64_t n = m->n;
    std::vector<uint32_t> mask((size_t)n), key((size_t)n), idx((size_t)n), tmp((size_t)n);
    if (n > 0) SMC_HIP(hipMemcpy(mask.data(), m->mask.p, (size_t)n * 4, hipMemcpyDeviceToHost));
    int64_t cnt[kTaps] = {};
    for (int64_t i = 0; i < n; ++i)
        for (int t = 0; t < kTaps; ++t) cnt[t] += (mask[i] >> t) & 1u;
    // start: off-centre taps by ascending count (ties: lower tap); centre always last
    std::vector<int> rem;
    for (int t = 0; t < kTaps; ++t)
        if (t != kCentre) rem.push_back(t);
    std::stable_sort(rem.begin(), rem.end(), [&](int a, int b) { return cnt[a] < cnt[b]; });
    std::vector<int> chosen;
    int cand[kTaps];
    while (!rem.empty()) {
        int best = -1;
        int64_t best_w = 0;
        for (size_t c = 0; c < rem.size(); ++c) {
            int q = 0;
            for (int t : chosen) cand[q++] = t;
            cand[q++] = rem[c];
            for (size_t r = 0; r < rem.size(); ++r)
                if (r != c) cand[q++] = rem[r];
            cand[q++] = kCentre;
            const int64_t w = n > 0 ? calib_work(mask, cand, key, idx, tmp) : 0;
            if (best < 0 || w < best_w) {
                best = (int)c;
                best_w = w;
            }
        }
        chosen.push_back(rem[best]);
        rem.erase(rem.begin() + best);
    }
    for (int j = 0; j < kTaps - 1; ++j) bit_order[j] = chosen[j];
    bit_order[kTaps - 1] = kCentre;
    for (int g = 0; g < n_groups; ++g)
        for (int p = (26 * g) / n_groups; p < (26 * (g + 1)) / n_groups; ++p)
            group_of[chosen[p]] = g;
    group_of[kCentre] = n_groups - 1;
    return SMC_OK;
}

int smc_test_force_lookback_timeout(smc_map* m, int on) {
    if (!m) return fail(SMC_ERR_ARG, "map is NULL");
    m->ws.force_timeout = on != 0;
    return SMC_OK;
}

int smc_timing_enable(smc_map* m, int on) {
    if (!m) return fail(SMC_ERR_ARG, "map is NULL");
    m->timing = on != 0;
    m->seq_open = false;              // untimed work may follow: the next kernel starts anew
    return SMC_OK;
}

int smc_timing_read(smc_map* m, double* ms, int64_t* calls, int reset) {
    if (!m) return fail(SMC_ERR_ARG, "map is NULL");
    hipEvent_t prev = nullptr;
    for (const auto& tk : m->seq) {
        if (tk.start) prev = tk.start;
        SMC_HIP(hipEventSynchronize(tk.stop));
        float e = 0.f;
        if (prev) SMC_HIP(hipEventElapsedTime(&e, prev, tk.stop));
        m->stage_ms[tk.stage] += e;
        if (tk.in_build && tk.stage != SMC_STAGE_MAP) m->stage_ms[SMC_STAGE_MAP] += e;
        prev = tk.stop;
    }
    for (const auto& tk : m->seq) {
        if (tk.start) m->ev_pool.push_back(tk.start);
        m->ev_pool.push_back(tk.stop);
    }
    m->seq.clear();
    m->seq_open = false;
    for (int st = 0; st < SMC_STAGE_COUNT; ++st) {
        m->stage_calls[st] += m->stage_exec[st];
        m->stage_exec[st] = 0;
        if (ms) ms[st] = m->stage_ms[st];
        if (calls) calls[st] = m->stage_calls[st];
        if (reset) {
            m->stage_ms[st] = 0;
            m->stage_calls[st] = 0;
        }
    }
    return SMC_OK;
}

}  // extern "C"
