// Host runtime of libag: symmetric heap, argument validation, launch
// planning and the C ABI declared in include/ag.h.
//
// The heap follows the symmetric-heap model of iris (ROCm/iris #626,
// "Summary"; ROCm/iris #591, "Hoist the peer heap bases"): every rank owns
// a heap, tensors sit at the same offset in every heap, and kernels find a
// peer's copy through a device array heap_bases.  Here the rank heaps are
// regions of one device allocation (ROCm/iris #594, "Local validation":
// logical ranks as separate memory on one GPU).

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <memory>
#include <mutex>
#include <string>
#include <vector>

#include "ag.h"
#include "ag_internal.h"

static_assert(AG_NOALLOC_MAX_RANKS == ag::kNoAllocMaxRanks, "one limit for the allocation-free entry point");

namespace {

thread_local std::string g_last_error;

ag_status_t ok()
{
    g_last_error.clear();
    return AG_OK;
}

ag_status_t fail(ag_status_t s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
ag_status_t fail(ag_status_t s, const char* fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    std::vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return s;
}

ag_status_t fail_hip(hipError_t e, const char* what)
{
    const ag_status_t s = (e == hipErrorOutOfMemory) ? AG_ERR_OUT_OF_MEMORY : AG_ERR_HIP;
    return fail(s, "%s failed: %s (%d)", what, hipGetErrorString(e), static_cast<int>(e));
}

bool is_pow2(uint64_t v) { return v != 0 && (v & (v - 1)) == 0; }
int log2_exact(uint64_t v)
{
    int l = 0;
    while ((uint64_t{1} << l) < v) ++l;
    return l;
}
uint64_t ceil_div(uint64_t a, uint64_t b) { return (a + b - 1) / b; }

int elem_bytes(ag_dtype_t d)
{
    switch (d) {
    case AG_F16: return 2;
    case AG_BF16: return 2;
    case AG_F32: return 4;
    default: return 0;
    }
}

// Half-open byte ranges [a0, a0+an) and [b0, b0+bn) intersect.
bool overlaps(uint64_t a0, uint64_t an, uint64_t b0, uint64_t bn)
{
    return an != 0 && bn != 0 && a0 < b0 + bn && b0 < a0 + an;
}

// Bytes of device memory per rank for its tile counter (ticket order): two uint32 words used, one
// 64-byte block per rank so that no two ranks' counters share a line.
constexpr uint64_t kTicketBytes = 64;

struct HeapCore {
    void* slab = nullptr;
    uint64_t* table = nullptr;  // device uint64_t[n_ranks], followed (256-byte aligned) by the tile counters
    uint32_t* tickets = nullptr;  // device, kTicketBytes per rank; zero between calls
    int n_ranks = 0;
    uint64_t bytes_per_rank = 0;
    bool owns_slab = false;
    int device = 0;
    int num_cus = 0;
    std::mutex mu;
    uint64_t bump = 0;

    ~HeapCore()
    {
        if (table) (void)hipFree(table);
        if (owns_slab && slab) (void)hipFree(slab);
    }
};

}  // namespace

struct ag_heap {
    std::shared_ptr<HeapCore> core;
    int rank = -1;
};

namespace {

// Common part of create and wrap: record the device, build and upload the table.
ag_status_t finish_heap(std::shared_ptr<HeapCore> core, ag_heap_t** out)
{
    hipError_t e = hipGetDevice(&core->device);
    if (e != hipSuccess) return fail_hip(e, "hipGetDevice");
    e = hipDeviceGetAttribute(&core->num_cus, hipDeviceAttributeMultiprocessorCount, core->device);
    if (e != hipSuccess) return fail_hip(e, "hipDeviceGetAttribute(multiProcessorCount)");
    // one device allocation: the base table, then (256-byte aligned) one zeroed tile counter per rank
    const uint64_t table_bytes = ceil_div(sizeof(uint64_t) * core->n_ranks, 256) * 256;
    const uint64_t total = table_bytes + kTicketBytes * core->n_ranks;
    std::vector<uint64_t> host(total / sizeof(uint64_t), 0);
    for (int r = 0; r < core->n_ranks; ++r)
        host[r] = reinterpret_cast<uint64_t>(core->slab) + static_cast<uint64_t>(r) * core->bytes_per_rank;
    e = hipMalloc(reinterpret_cast<void**>(&core->table), total);
    if (e != hipSuccess) {
        core->table = nullptr;
        return fail_hip(e, "hipMalloc(heap_bases)");
    }
    e = hipMemcpy(core->table, host.data(), total, hipMemcpyHostToDevice);
    if (e != hipSuccess) return fail_hip(e, "hipMemcpy(heap_bases)");
    core->tickets = reinterpret_cast<uint32_t*>(reinterpret_cast<uint8_t*>(core->table) + table_bytes);
    auto* h = new (std::nothrow) ag_heap;
    if (!h) return fail(AG_ERR_OUT_OF_MEMORY, "host allocation of the heap handle failed");
    h->core = std::move(core);
    h->rank = -1;
    *out = h;
    return ok();
}

// Launches run on the current HIP device; the heap's slab and base table
// live on the device that was current when it was created or wrapped.
ag_status_t check_device(const ag_heap_t* heap)
{
    int dev = -1;
    const hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail_hip(e, "hipGetDevice");
    if (dev != heap->core->device)
        return fail(AG_ERR_INVALID_ARG, "the heap lives on device %d but device %d is current", heap->core->device, dev);
    return AG_OK;
}

ag_status_t check_geometry(const ag_heap_geometry_t* g)
{
    if (!g) return fail(AG_ERR_INVALID_ARG, "geometry is NULL");
    if (g->n_ranks < 1) return fail(AG_ERR_INVALID_ARG, "n_ranks %d < 1", g->n_ranks);
    if (g->bytes_per_rank == 0 || g->bytes_per_rank % 256 != 0)
        return fail(AG_ERR_INVALID_ARG, "bytes_per_rank %llu is not a positive multiple of 256",
                    static_cast<unsigned long long>(g->bytes_per_rank));
    if (g->slab_addr == 0 || g->slab_addr % 256 != 0)
        return fail(AG_ERR_INVALID_ARG, "slab address is null or not 256-byte aligned");
    if (g->num_cus < 1) return fail(AG_ERR_INVALID_ARG, "num_cus %d < 1", g->num_cus);
    if (g->rank < 0 || g->rank >= g->n_ranks)
        return fail(AG_ERR_INVALID_ARG, "the heap handle is not a view of a rank (rank %d, n_ranks %d); use ag_heap_view",
                    g->rank, g->n_ranks);
    return AG_OK;
}

// Group checks shared by both operations; sets *g_out to the group rank.
ag_status_t check_group(const ag_heap_geometry_t* geom, int W, int rank_start, int rank_stride, int* g_out)
{
    if (W < 1) return fail(AG_ERR_INVALID_ARG, "W %d < 1", W);
    if (W > AG_MAX_WORLD) return fail(AG_ERR_UNSUPPORTED, "W %d > %d", W, AG_MAX_WORLD);
    if (rank_start < 0) return fail(AG_ERR_INVALID_ARG, "rank_start %d < 0", rank_start);
    if (rank_stride < 1) return fail(AG_ERR_INVALID_ARG, "rank_stride %d < 1", rank_stride);
    const int64_t last = static_cast<int64_t>(rank_start) + static_cast<int64_t>(W - 1) * rank_stride;
    if (last >= geom->n_ranks)
        return fail(AG_ERR_INVALID_ARG, "group member %lld is past the last region (n_ranks %d)",
                    static_cast<long long>(last), geom->n_ranks);
    const int d = geom->rank - rank_start;
    if (d < 0 || d % rank_stride != 0 || d / rank_stride >= W)
        return fail(AG_ERR_INVALID_ARG, "rank %d is not a member of the group (start %d, stride %d, W %d)",
                    geom->rank, rank_start, rank_stride, W);
    *g_out = d / rank_stride;
    return AG_OK;
}

// Tuning constants of the copy kernel: concurrent 256-thread tile slices per
// workgroup.  One measured best at 128 and 256 programs; launches on fewer
// than half the CUs take up to four (at 64 programs: 5.26 against 4.91 TB/s
// at W=8, 1024x4096 fp16, 2.55 against 2.47-2.50 at 16384x8192; two slices
// were 3% slower on the larger shape).
#ifndef AG_COPY_MAX_SLICES
#define AG_COPY_MAX_SLICES 1
#endif
#ifndef AG_COPY_NARROW_SLICES
#define AG_COPY_NARROW_SLICES 4
#endif
// Ticket order, tiles per ticket G.  Each ticket is one increment of the calling rank's counter, and
// increments of one address retire about one per 12 ns: at W=2 and W=4, 16384x8192 fp16, 256 programs,
// the call took the ticket count times that (W=2: 263 / 204 / 125 us per call with 3 / 4 / 8 tiles per
// ticket; W=4: 266 / 207 / 203).  So a ticket must move at least AG_TICKETS_MIN_BYTES of HBM traffic (its
// tiles read once and written W times).  Above that floor fewer tiles per ticket keep the tiles in flight
// in a narrower window: a launch on fewer programs than CUs takes the largest of 16, 8 and 4 whose
// tickets over all programs cover at most AG_TICKETS_WINDOW_TILES tiles, a launch with a program per CU
// the smallest G the floor allows.  Measured at W=8, 16384x8192, 8x256 tiles, us per call with
// 4 / 8 / 16 tiles per ticket: 192 programs fp16 356 / 360 / -, fp32 700 / 728 / -; 128 programs fp16
// 380 / 377 / 391, fp32 750 / 733 / -; 96 programs fp16 - / 399 / 406; 64 programs fp16 - / 542 / 502;
// 256 programs fp16 with 2 / 3 / 4: 390 / 357 / 362.  AG_TICKETS_MIN_TILES_PER_PROGRAM is the tiles per
// program from which AG_ORDER_AUTO chooses tickets over the grid stride.
#ifndef AG_TICKETS_WINDOW_TILES
#define AG_TICKETS_WINDOW_TILES 1024
#endif
#ifndef AG_TICKETS_MIN_BYTES
#define AG_TICKETS_MIN_BYTES (96u << 10)
#endif
#ifndef AG_TICKETS_MIN_TILES_PER_PROGRAM
#define AG_TICKETS_MIN_TILES_PER_PROGRAM 64
#endif
constexpr int kCopyMaxVpt = 8;
constexpr int kCopyMaxSlices = AG_COPY_MAX_SLICES;
constexpr uint64_t kCopyNarrowSlices = AG_COPY_NARROW_SLICES;   // launches on fewer than half the CUs

}  // namespace

extern "C" {

const char* ag_status_string(ag_status_t s)
{
    switch (s) {
    case AG_OK: return "AG_OK";
    case AG_ERR_INVALID_ARG: return "AG_ERR_INVALID_ARG";
    case AG_ERR_UNSUPPORTED: return "AG_ERR_UNSUPPORTED";
    case AG_ERR_OUT_OF_MEMORY: return "AG_ERR_OUT_OF_MEMORY";
    case AG_ERR_HIP: return "AG_ERR_HIP";
    default: return "AG_ERR_UNKNOWN";
    }
}

const char* ag_last_error_message(void) { return g_last_error.c_str(); }

const char* ag_version(void) { return "libag 0.1 (gfx950)"; }

// Region stride for bytes_per_rank: whole 2 MiB units, and one unit more when that is a power of two of
// 512 MiB or more.  The W copies of a tile are stored at the same offset of W regions at once; with a
// large power-of-two stride those addresses alias in the HBM channel interleave.  Measured at W=8, N=8192
// fp16, 256 programs, us per call with the stride at the size / plus 2 MiB: 16384 rows (2 GiB) 354.2-359.5
// / 348.8-353.8 over five runs, 4096 rows (0.5 GiB) 97.5-98.1 / 96.1-96.6, 8192 rows (1 GiB) 182.4-182.8 /
// 182.1 (adding 4 MiB instead was 2-8% slower at every size).
ag_status_t ag_heap_region_bytes(size_t bytes_per_rank, size_t* region_bytes)
{
    if (!region_bytes) return fail(AG_ERR_INVALID_ARG, "region_bytes is NULL");
    if (bytes_per_rank == 0) return fail(AG_ERR_INVALID_ARG, "bytes_per_rank is 0");
    if (bytes_per_rank > (size_t{1} << 40)) return fail(AG_ERR_INVALID_ARG, "bytes_per_rank above 1 TiB");
    uint64_t S = ceil_div(bytes_per_rank, AG_REGION_ALIGN) * AG_REGION_ALIGN;
    if (S >= (uint64_t{512} << 20) && (S & (S - 1)) == 0) S += AG_REGION_ALIGN;
    *region_bytes = S;
    return ok();
}

ag_status_t ag_heap_create(int n_ranks, size_t bytes_per_rank, ag_heap_t** out)
{
    if (!out) return fail(AG_ERR_INVALID_ARG, "out is NULL");
    if (n_ranks < 1 || n_ranks > 1024) return fail(AG_ERR_INVALID_ARG, "n_ranks %d not in [1, 1024]", n_ranks);
    if (bytes_per_rank == 0) return fail(AG_ERR_INVALID_ARG, "bytes_per_rank is 0");
    size_t region = 0;
    const ag_status_t rs = ag_heap_region_bytes(bytes_per_rank, &region);
    if (rs != AG_OK) return rs;
    const uint64_t S = region;
    if (S / AG_REGION_ALIGN > (uint64_t{1} << 40) / static_cast<uint64_t>(n_ranks))
        return fail(AG_ERR_INVALID_ARG, "heap size overflows");
    auto core = std::make_shared<HeapCore>();
    core->n_ranks = n_ranks;
    core->bytes_per_rank = S;
    core->owns_slab = true;
    const hipError_t e = hipMalloc(&core->slab, S * static_cast<uint64_t>(n_ranks));
    if (e != hipSuccess) {
        core->slab = nullptr;
        return fail_hip(e, "hipMalloc(slab)");
    }
    return finish_heap(std::move(core), out);
}

ag_status_t ag_heap_wrap(void* dev_slab, int n_ranks, size_t bytes_per_rank, ag_heap_t** out)
{
    if (!out) return fail(AG_ERR_INVALID_ARG, "out is NULL");
    if (!dev_slab || reinterpret_cast<uint64_t>(dev_slab) % 256 != 0)
        return fail(AG_ERR_INVALID_ARG, "dev_slab is NULL or not 256-byte aligned");
    if (n_ranks < 1 || n_ranks > 1024) return fail(AG_ERR_INVALID_ARG, "n_ranks %d not in [1, 1024]", n_ranks);
    if (bytes_per_rank == 0 || bytes_per_rank % 256 != 0)
        return fail(AG_ERR_INVALID_ARG, "bytes_per_rank %zu is not a positive multiple of 256", bytes_per_rank);
    if (bytes_per_rank > (uint64_t{1} << 50) / static_cast<uint64_t>(n_ranks))
        return fail(AG_ERR_INVALID_ARG, "heap size overflows");
    // The slab must be device memory of the current device, and the n_ranks regions must lie inside
    // its allocation: a kernel would otherwise fault on the first launch.
    {
        hipPointerAttribute_t attr{};
        hipError_t e = hipPointerGetAttributes(&attr, dev_slab);
        if (e != hipSuccess) {
            (void)hipGetLastError();   // a failed query must not surface as a later launch error
            return fail(AG_ERR_INVALID_ARG, "dev_slab is not device memory known to HIP (%s)", hipGetErrorString(e));
        }
        int dev = -1;
        e = hipGetDevice(&dev);
        if (e != hipSuccess) return fail_hip(e, "hipGetDevice");
        if ((attr.type != hipMemoryTypeDevice && !attr.isManaged) || attr.device != dev)
            return fail(AG_ERR_INVALID_ARG, "dev_slab is not device memory of the current device %d", dev);
        // the allocation's extent, where the runtime knows it (memory mapped through the virtual
        // memory API may not report one: then only the checks above apply)
        void* base = nullptr;
        size_t size = 0;
        e = hipMemGetAddressRange(reinterpret_cast<hipDeviceptr_t*>(&base), &size, dev_slab);
        if (e != hipSuccess || base == nullptr || size == 0) {
            (void)hipGetLastError();
        } else {
            const uint64_t need = static_cast<uint64_t>(n_ranks) * bytes_per_rank;
            const uint64_t avail = reinterpret_cast<uint64_t>(base) + size - reinterpret_cast<uint64_t>(dev_slab);
            if (need > avail)
                return fail(AG_ERR_INVALID_ARG,
                            "%d regions of %zu bytes need %llu bytes, the allocation holds %llu from dev_slab", n_ranks,
                            bytes_per_rank, static_cast<unsigned long long>(need),
                            static_cast<unsigned long long>(avail));
        }
    }
    auto core = std::make_shared<HeapCore>();
    core->slab = dev_slab;
    core->n_ranks = n_ranks;
    core->bytes_per_rank = bytes_per_rank;
    core->owns_slab = false;
    return finish_heap(std::move(core), out);
}

ag_status_t ag_heap_view(const ag_heap_t* heap, int rank, ag_heap_t** view)
{
    if (!heap || !view) return fail(AG_ERR_INVALID_ARG, "heap or view is NULL");
    if (rank < 0 || rank >= heap->core->n_ranks)
        return fail(AG_ERR_INVALID_ARG, "rank %d not in [0, %d)", rank, heap->core->n_ranks);
    auto* v = new (std::nothrow) ag_heap;
    if (!v) return fail(AG_ERR_OUT_OF_MEMORY, "host allocation of the view failed");
    v->core = heap->core;
    v->rank = rank;
    *view = v;
    return ok();
}

ag_status_t ag_heap_destroy(ag_heap_t* heap)
{
    delete heap;   // the shared state goes with its last handle
    return ok();
}

ag_status_t ag_heap_alloc(ag_heap_t* heap, size_t bytes, size_t align, size_t* offset)
{
    if (!heap || !offset) return fail(AG_ERR_INVALID_ARG, "heap or offset is NULL");
    if (align == 0) align = 256;
    if (!is_pow2(align) || align < 256) return fail(AG_ERR_INVALID_ARG, "align %zu is not a power of two >= 256", align);
    HeapCore& c = *heap->core;
    std::lock_guard<std::mutex> lock(c.mu);
    const uint64_t off = ceil_div(c.bump, align) * align;
    if (off > c.bytes_per_rank || bytes > c.bytes_per_rank - off)
        return fail(AG_ERR_OUT_OF_MEMORY, "symmetric heap exhausted: %zu bytes at offset %llu, region %llu bytes",
                    bytes, static_cast<unsigned long long>(off), static_cast<unsigned long long>(c.bytes_per_rank));
    c.bump = off + bytes;
    *offset = off;
    return ok();
}

ag_status_t ag_heap_reset(ag_heap_t* heap)
{
    if (!heap) return fail(AG_ERR_INVALID_ARG, "heap is NULL");
    std::lock_guard<std::mutex> lock(heap->core->mu);
    heap->core->bump = 0;
    return ok();
}

ag_status_t ag_heap_rank_ptr(const ag_heap_t* heap, int rank, size_t offset, void** dev_ptr)
{
    if (!heap || !dev_ptr) return fail(AG_ERR_INVALID_ARG, "heap or dev_ptr is NULL");
    const HeapCore& c = *heap->core;
    if (rank < 0 || rank >= c.n_ranks) return fail(AG_ERR_INVALID_ARG, "rank %d not in [0, %d)", rank, c.n_ranks);
    if (offset > c.bytes_per_rank) return fail(AG_ERR_INVALID_ARG, "offset %zu past the region", offset);
    *dev_ptr = static_cast<char*>(c.slab) + static_cast<uint64_t>(rank) * c.bytes_per_rank + offset;
    return ok();
}

ag_status_t ag_heap_base_table(const ag_heap_t* heap, const uint64_t** dev_table)
{
    if (!heap || !dev_table) return fail(AG_ERR_INVALID_ARG, "heap or dev_table is NULL");
    *dev_table = heap->core->table;
    return ok();
}

ag_status_t ag_heap_geometry(const ag_heap_t* heap, ag_heap_geometry_t* geom)
{
    if (!heap || !geom) return fail(AG_ERR_INVALID_ARG, "heap or geom is NULL");
    const HeapCore& c = *heap->core;
    geom->slab_addr = reinterpret_cast<uint64_t>(c.slab);
    geom->bytes_per_rank = c.bytes_per_rank;
    geom->n_ranks = c.n_ranks;
    geom->rank = heap->rank;
    geom->num_cus = c.num_cus;
    geom->reserved = 0;
    return ok();
}

ag_status_t ag_heap_info(const ag_heap_t* heap, int* n_ranks, int* rank, size_t* bytes_per_rank,
                         const uint64_t** dev_base_table)
{
    if (!heap) return fail(AG_ERR_INVALID_ARG, "heap is NULL");
    const HeapCore& c = *heap->core;
    if (n_ranks) *n_ranks = c.n_ranks;
    if (rank) *rank = heap->rank;
    if (bytes_per_rank) *bytes_per_rank = static_cast<size_t>(c.bytes_per_rank);
    if (dev_base_table) *dev_base_table = c.table;
    return ok();
}

ag_status_t ag_heap_clear_tickets(const ag_heap_t* heap, void* stream)
{
    if (!heap) return fail(AG_ERR_INVALID_ARG, "heap is NULL");
    ag_status_t s = check_device(heap);
    if (s != AG_OK) return s;
    const HeapCore& c = *heap->core;
    const hipError_t e = ag::clear_counters(c.tickets, static_cast<uint32_t>(c.n_ranks) * (kTicketBytes / sizeof(uint32_t)),
                                            static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail_hip(e, "clear_counters");
    return ok();
}

// ---------------------------------------------------------------------------
// all-gather (default, grouped, partitioned) and all-to-all: one planner
// ---------------------------------------------------------------------------

}  // extern "C"

namespace {

// The rows the copy kernels walk.  A block (this rank's input, or one all-to-
// all chunk, and its place in every output block) is M rows of N elements
// with ld = N, so its M*N*e bytes are contiguous and any rows x cols = M x N
// addresses the same bytes in the same order.  When N*e is not a multiple of
// 16 bytes but the block's size, the input and the output block are, the
// kernels walk rows of cols elements instead, cols*e a multiple of 16 (the
// divisor of the block's 16-byte vector count nearest N*e/16, searched within
// 4096 vectors of it), so that they move 16-byte vectors.  Every destination
// receives the same bytes; only the grouping of bytes into tiles differs.
void copy_rows(uint64_t M, uint64_t N, int e, uint64_t input_addr, uint64_t out_addr, uint64_t* rows, uint64_t* cols)
{
    *rows = M;
    *cols = N;
    const uint64_t row_bytes = N * static_cast<uint64_t>(e);
    const uint64_t bytes = M * row_bytes;
    if (M < 2 || row_bytes % 16 == 0 || bytes % 16 != 0 || input_addr % 16 != 0 || out_addr % 16 != 0) return;
    const uint64_t q = bytes / 16;                                  // 16-byte vectors in the block
    const uint64_t t = std::max<uint64_t>(1, row_bytes / 16);
    for (uint64_t dist = 0; dist <= 4096; ++dist) {
        for (int below = 0; below < 2; ++below) {
            if (below && (dist == 0 || dist >= t)) continue;
            const uint64_t d = below ? t - dist : t + dist;         // vectors per row
            if (d > q || q % d != 0 || q / d >= (uint64_t{1} << 31) || d * 16 / e >= (uint64_t{1} << 31)) continue;
            *cols = d * 16 / static_cast<uint64_t>(e);
            *rows = q / d;
            return;
        }
    }
}

// Validation and launch decisions shared by every copy entry point.  kind:
// ag::kCopyAllGather (M = M_local rows per rank) or ag::kCopyAllToAll (M =
// M_chunk rows per chunk, W chunks in the input).
ag_status_t plan_copy(const ag_heap_geometry_t* geom, int kind, int W, int rank_start, int rank_stride,
                      uint64_t input_addr, size_t out_offset, int64_t M, int64_t N, ag_dtype_t dtype, int tile_m,
                      int tile_n, int n_programs, const ag_copy_options_t* options, ag_plan_t* plan)
{
    ag_status_t s = check_geometry(geom);
    if (s != AG_OK) return s;
    if (!plan) return fail(AG_ERR_INVALID_ARG, "plan is NULL");
    const bool a2a = kind == ag::kCopyAllToAll;
    const char* mname = a2a ? "M_chunk" : "M_local";
    ag_copy_options_t opt{};
    if (options) opt = *options;
    for (int i = 0; i < 5; ++i)
        if (opt.reserved[i] != 0) return fail(AG_ERR_INVALID_ARG, "options->reserved[%d] is not 0", i);
    if (opt.schedule != AG_SCHEDULE_TILES && opt.schedule != AG_SCHEDULE_PARTITIONED)
        return fail(AG_ERR_INVALID_ARG, "unknown schedule %d", opt.schedule);
    if (opt.tile_order != AG_ORDER_AUTO && opt.tile_order != AG_ORDER_STRIDE && opt.tile_order != AG_ORDER_TICKETS)
        return fail(AG_ERR_INVALID_ARG, "unknown tile_order %d", opt.tile_order);
    if (opt.tile_order != AG_ORDER_AUTO && opt.schedule != AG_SCHEDULE_TILES)
        return fail(AG_ERR_INVALID_ARG, "tile_order applies to the tile schedule only");
    if (opt.dest_group < 0) return fail(AG_ERR_INVALID_ARG, "dest_group %d < 0", opt.dest_group);
    if (opt.dest_group != 0 && opt.dest_group != 1 && opt.dest_group != 2 && opt.dest_group != 4)
        return fail(AG_ERR_UNSUPPORTED, "dest_group %d: 0, 1, 2 or 4 are supported", opt.dest_group);
    if (opt.schedule == AG_SCHEDULE_PARTITIONED && opt.dest_group != 0)
        return fail(AG_ERR_INVALID_ARG, "a partitioned program has one destination: dest_group must be 0");
    int g = 0;
    s = check_group(geom, W, rank_start, rank_stride, &g);
    if (s != AG_OK) return s;
    const int e = elem_bytes(dtype);
    if (e == 0) return fail(AG_ERR_INVALID_ARG, "unknown dtype %d", static_cast<int>(dtype));
    if (M < 0) return fail(AG_ERR_INVALID_ARG, "%s %lld < 0", mname, static_cast<long long>(M));
    if (N < 1) return fail(AG_ERR_INVALID_ARG, "N %lld < 1", static_cast<long long>(N));
    if (M > (int64_t{1} << 31) - 1 || N > (int64_t{1} << 31) - 1)
        return fail(AG_ERR_UNSUPPORTED, "%s or N >= 2^31", mname);
    if (n_programs < 0) return fail(AG_ERR_INVALID_ARG, "n_programs %d < 0", n_programs);
    if (tile_m == 0 && tile_n == 0) {
        tile_m = 8;
        tile_n = 256;
    } else if (tile_m <= 0 || tile_n <= 0) {
        return fail(AG_ERR_INVALID_ARG, "tile %dx%d: give both sides, or 0,0 for the 8x256 default", tile_m, tile_n);
    }
    if (!is_pow2(tile_m) || !is_pow2(tile_n) || tile_m > 256 || tile_n < 8 || tile_n > 4096)
        return fail(AG_ERR_UNSUPPORTED, "tile %dx%d: tile_m must be a power of two <= 256 and tile_n a power of two in [8, 4096]",
                    tile_m, tile_n);
    const uint64_t row_bytes = static_cast<uint64_t>(N) * e;
    const uint64_t blk = static_cast<uint64_t>(M) * row_bytes;   // this rank's rows in every output block
    if (out_offset % e != 0)
        return fail(AG_ERR_INVALID_ARG, "out_offset %zu is not a multiple of the element size %d", out_offset, e);
    if (blk > geom->bytes_per_rank / W || out_offset > geom->bytes_per_rank - W * blk)
        return fail(AG_ERR_INVALID_ARG, "output block (%d x %llu bytes at offset %zu) exceeds the region (%llu bytes)",
                    W, static_cast<unsigned long long>(blk), out_offset,
                    static_cast<unsigned long long>(geom->bytes_per_rank));

    const bool part = opt.schedule == AG_SCHEDULE_PARTITIONED;
    const uint64_t in_bytes = a2a ? W * blk : blk;
    ag_plan_t p{};
    p.group_rank = g;
    p.tile_m = tile_m;
    p.tile_n = tile_n;
    p.threads = 256;
    p.rank_block_offset = out_offset + static_cast<uint64_t>(g) * blk;
    p.bytes_read = part ? W * blk : in_bytes;
    p.bytes_written = W * blk;
    p.schedule = part ? AG_SCHEDULE_PARTITIONED : AG_SCHEDULE_TILES;
    p.dest_group = (!a2a && opt.dest_group < W) ? opt.dest_group : 0;
    if (a2a && opt.dest_group != 0) return fail(AG_ERR_INVALID_ARG, "the all-to-all takes no destination groups");
    if (M == 0) {   // nothing to move: valid no-op
        *plan = p;
        return ok();
    }
    if (input_addr == 0) return fail(AG_ERR_INVALID_ARG, "input is NULL");
    if (input_addr % e != 0) return fail(AG_ERR_INVALID_ARG, "input is not aligned to the element size");

    // The input must not overlap any member's output block; the all-gather
    // input may be exactly this rank's own rows in its own region (in place).
    const uint64_t own = geom->slab_addr + static_cast<uint64_t>(geom->rank) * geom->bytes_per_rank + p.rank_block_offset;
    if (a2a || input_addr != own) {
        for (int j = 0; j < W; ++j) {
            const uint64_t region = geom->slab_addr +
                static_cast<uint64_t>(rank_start + j * rank_stride) * geom->bytes_per_rank;
            if (overlaps(input_addr, in_bytes, region + out_offset, W * blk))
                return fail(AG_ERR_INVALID_ARG, "input overlaps the output block of region %d", rank_start + j * rank_stride);
        }
    }

    // widest vector that every row start, the input and every output block allow
    const uint64_t out_addr = geom->slab_addr + p.rank_block_offset;   // same alignment in every region
    auto widest = [&](uint64_t rb) {
        int v = 16;
        while (v > e && ((rb % v) != 0 || (input_addr % v) != 0 || (out_addr % v) != 0)) v /= 2;
        return v;
    };
    const uint64_t tile_row_bytes = static_cast<uint64_t>(tile_n) * e;
    auto tile_fits = [&](int v) {
        const uint64_t tv = static_cast<uint64_t>(tile_m) * tile_row_bytes / v;
        return tv % 256 == 0 && tv / 256 <= static_cast<uint64_t>(kCopyMaxVpt);
    };
    int vec = widest(row_bytes);
    uint64_t rows = static_cast<uint64_t>(M), cols = static_cast<uint64_t>(N);
    if (vec < 16) {   // the kernels' view of the block as rows of a multiple of 16 bytes, if the tile fits it
        uint64_t r2 = 0, c2 = 0;
        copy_rows(rows, cols, e, input_addr, out_addr, &r2, &c2);
        if (c2 != cols && widest(c2 * e) == 16 && tile_fits(16)) {
            rows = r2;
            cols = c2;
            vec = 16;
        }
    }
    const uint64_t view_row_bytes = cols * static_cast<uint64_t>(e);
    const uint64_t tile_vecs = static_cast<uint64_t>(tile_m) * tile_row_bytes / vec;
    if (tile_vecs % 256 != 0 || tile_vecs / 256 > static_cast<uint64_t>(kCopyMaxVpt))
        return fail(AG_ERR_UNSUPPORTED, "tile %dx%d holds %llu %d-byte vectors; 256 to %d are supported",
                    tile_m, tile_n, static_cast<unsigned long long>(tile_vecs), vec, 256 * kCopyMaxVpt);
    if (static_cast<uint64_t>(tile_m) * view_row_bytes >= (uint64_t{1} << 31))
        return fail(AG_ERR_UNSUPPORTED, "a tile spans 2 GiB or more of the input");
    if (p.dest_group > 0 && vec < 8)
        return fail(AG_ERR_UNSUPPORTED, "destination groups need 16- or 8-byte vectors (this call gets %d)", vec);

    const uint64_t tiles_m = ceil_div(rows, tile_m);
    const uint64_t tiles_n = ceil_div(cols, tile_n);
    const uint64_t total = tiles_m * tiles_n;
    if (total >= (uint64_t{1} << 31)) return fail(AG_ERR_UNSUPPORTED, "more than 2^31 tiles");
    // the all-to-all kernel walks the W chunks' tiles as one sequence
    if (a2a && total * static_cast<uint64_t>(W) >= (uint64_t{1} << 31))
        return fail(AG_ERR_UNSUPPORTED, "more than 2^31 tiles over the W chunks");

    const uint64_t programs = n_programs == 0 ? geom->num_cus : n_programs;
    // Tile order of the tile schedule.  Tickets (consecutive tiles handed out in increasing order
    // from the rank's counter) keep the tiles in flight in one compact window; they pay a counter
    // round trip per ticket, which long calls hide and short ones do not (at 1024x4096 fp16, W=8,
    // 16 tiles per program: 15.9 against 11.8 us per call).
    int ticket = 0;
    const int tvpt = static_cast<int>(tile_vecs / 256);   // 16-byte vectors per thread and tile (tickets)
    // the tiles the programs share out: the all-to-all's W chunk copies are one sequence of W x total
    const uint64_t seq_tiles = a2a ? total * static_cast<uint64_t>(W) : total;
    {
        // tiles per ticket: the ticket kernels exist for 3, 4, 8 and 16 tiles with one vector per
        // thread and 2, 4 and 8 with two
        static constexpr int kSizesVpt1[] = {3, 4, 8, 16};
        static constexpr int kSizesVpt2[] = {2, 4, 8};
        const int* sizes = tvpt == 2 ? kSizesVpt2 : kSizesVpt1;
        const int n_sizes = tvpt == 2 ? 3 : 4;
        // HBM bytes a tile moves: read once, then written W times (the all-to-all: once)
        const uint64_t hbm_bytes_per_tile = tile_vecs * vec * (a2a ? 2 : 1 + static_cast<uint64_t>(W));
        int g_floor = sizes[n_sizes - 1];
        for (int i = 0; i < n_sizes; ++i) {
            if (sizes[i] * hbm_bytes_per_tile >= AG_TICKETS_MIN_BYTES) {
                g_floor = sizes[i];
                break;
            }
        }
        int g = sizes[0];
        if (programs < static_cast<uint64_t>(geom->num_cus)) {
            g = 16;
            while (g > 4 && static_cast<uint64_t>(g) * programs > AG_TICKETS_WINDOW_TILES) g /= 2;
            g = std::min(g, sizes[n_sizes - 1]);
        }
        g = std::max(g, g_floor);
        // the ticket kernel's tile offsets are 32-bit: every tile row of the block must lie below 2 GiB
        const bool small = tiles_m * tile_m * view_row_bytes < (uint64_t{1} << 31);
        const bool fits = !part && p.dest_group == 0 && small && ag::copy_ticket_supported(kind, vec, W, tvpt, g);
        if (opt.tile_order == AG_ORDER_TICKETS) {
            if (!fits)
                return fail(AG_ERR_UNSUPPORTED, "no ticket-order kernel for this call (%d-byte vectors, %d per thread, "
                            "destination group %d, %s 2 GiB of tile rows)", vec, tvpt, p.dest_group,
                            small ? "under" : "not under");
            ticket = g;
        } else if (opt.tile_order == AG_ORDER_AUTO && fits) {
            // The all-gather takes tickets from 64 tiles per program.  The all-to-all's grid stride already
            // keeps only two or four streams open (one chunk at a time), so tickets pay off only where few
            // vectors are in flight per CU and the call is long: programs x vectors per thread below twice
            // the CU count, and 64 tiles per program per vector.  Measured at W=8, fp16, us per call, grid
            // stride / tickets: 8 chunks of 2048x8192 with 8x512 tiles 85.1 / 87.4 at 256 programs, 105.7 /
            // 98.3 at 128, 186.9 / 146.9 at 64; with 8x256 tiles 104.5 / 89.1 at 256; 8 chunks of 1024x4096
            // with 8x512 tiles 22.9 / 27.1 at 256, 28.1 / 30.3 at 128, 48.8 / 42.2 at 64.
            const uint64_t per_vec = a2a ? static_cast<uint64_t>(tvpt) : 1;
            const bool few_in_flight = !a2a || programs * per_vec < 2 * static_cast<uint64_t>(geom->num_cus);
            if (few_in_flight && seq_tiles >= AG_TICKETS_MIN_TILES_PER_PROGRAM * per_vec * programs) ticket = g;
        }
    }
    uint64_t slices = 1, grid = 0;
    if (ticket) {
        grid = std::min<uint64_t>(programs, ceil_div(seq_tiles, static_cast<uint64_t>(ticket)));
    } else if (part) {
        // W equal sets of programs, one per destination, each walking all tiles
        const uint64_t per_dest = std::min<uint64_t>(std::max<uint64_t>(programs / W, 1), total);
        grid = per_dest * W;
    } else {
        // concurrent tiles per program: up to kCopyMaxSlices while every slice still gets a tile
        const uint64_t max_slices = 2 * programs < static_cast<uint64_t>(geom->num_cus) ? kCopyNarrowSlices
                                                                                     : static_cast<uint64_t>(kCopyMaxSlices);
        while (!a2a && slices < max_slices && programs * slices * 2 <= total) slices *= 2;
        grid = std::min<uint64_t>(programs, ceil_div(seq_tiles, slices));
    }
    if (grid >= (uint64_t{1} << 31)) return fail(AG_ERR_UNSUPPORTED, "n_programs too large");
    const int vpt = static_cast<int>(tile_vecs / 256);
    if (!ag::copy_supported(kind, vec, part ? 1 : W, p.dest_group, vpt, part))
        return fail(AG_ERR_UNSUPPORTED, "no kernel for %d-byte vectors, %d destinations, group %d, %d vectors per thread",
                    vec, part ? 1 : W, p.dest_group, vpt);

    p.vec_bytes = vec;
    p.vectors_per_thread = vpt;
    p.tiles_m = static_cast<int64_t>(tiles_m);
    p.tiles_n = static_cast<int64_t>(tiles_n);
    p.total_tiles = static_cast<int64_t>(total);
    p.n_programs = static_cast<int32_t>(grid);
    p.threads = static_cast<int32_t>(256 * slices);
    p.variant = kind;
    p.tile_order = ticket ? AG_ORDER_TICKETS : AG_ORDER_STRIDE;
    p.tiles_per_ticket = ticket;
    // Wide launches take each ticket after the stores of the batch before it (the program's first wave
    // waits for them, the others at the barrier that hands the ticket out).  Measured at W=8,
    // 16384x8192 on 256 CUs, it pays from 192 programs with one 16-byte vector per thread and tile
    // (360 against 383 us per call at 192 programs, 361 against 389 at 256; 391 against 377 at 128)
    // and from 96 with two (fp32: 731 against 776 us at 128 programs, 771 against 780 at 96; 1058
    // against 1007 at 64): from three quarters of the CUs' worth of vectors in flight.
    p.ticket_wait = (ticket && grid * static_cast<uint64_t>(tvpt) * 4 >= 3 * static_cast<uint64_t>(geom->num_cus)) ? 1 : 0;
    *plan = p;
    return ok();
}

// noalloc: the ticket order's counter comes from the library's fixed device array (ag_all_gather_noalloc)
ag_status_t launch_copy_call(const ag_heap_t* heap, int kind, int W, int rank_start, int rank_stride,
                             const void* input, size_t out_offset, int64_t M, int64_t N, ag_dtype_t dtype,
                             int tile_m, int tile_n, int n_programs, const ag_copy_options_t* options, void* stream,
                             bool noalloc = false)
{
    if (!heap) return fail(AG_ERR_INVALID_ARG, "heap is NULL");
    if (noalloc && heap->core->n_ranks > AG_NOALLOC_MAX_RANKS)
        return fail(AG_ERR_UNSUPPORTED, "ag_all_gather_noalloc keeps tile counters for heaps of at most %d ranks "
                    "(this heap has %d)", AG_NOALLOC_MAX_RANKS, heap->core->n_ranks);
    ag_heap_geometry_t geom;
    ag_heap_geometry(heap, &geom);
    ag_plan_t p;
    ag_status_t s = plan_copy(&geom, kind, W, rank_start, rank_stride, reinterpret_cast<uint64_t>(input), out_offset,
                              M, N, dtype, tile_m, tile_n, n_programs, options, &p);
    if (s != AG_OK) return s;
    if (p.total_tiles == 0) return ok();
    s = check_device(heap);
    if (s != AG_OK) return s;
    const int e = elem_bytes(dtype);
    const bool part = p.schedule == AG_SCHEDULE_PARTITIONED;
    ag::CopyLaunch l{};
    l.args.heap_bases = heap->core->table;
    l.args.input = static_cast<const uint8_t*>(input);
    l.args.rank_block_offset = p.rank_block_offset;
    // the planner's view of the block: rows of a multiple of 16 bytes when it chose 16-byte vectors
    // for rows that are not
    uint64_t rows = static_cast<uint64_t>(M), cols = static_cast<uint64_t>(N);
    if (p.vec_bytes == 16 && (static_cast<uint64_t>(N) * e) % 16 != 0)
        copy_rows(static_cast<uint64_t>(M), static_cast<uint64_t>(N), e, reinterpret_cast<uint64_t>(input),
                  geom.slab_addr + p.rank_block_offset, &rows, &cols);
    l.args.row_bytes = cols * static_cast<uint64_t>(e);
    l.args.chunk_bytes = kind == ag::kCopyAllToAll ? static_cast<uint64_t>(M) * N * e : 0;
    l.args.rows = static_cast<uint32_t>(rows);
    l.args.tile_m = static_cast<uint32_t>(p.tile_m);
    l.args.tile_row_bytes = static_cast<uint32_t>(p.tile_n) * e;
    l.args.vecs_per_row_log2 = static_cast<uint32_t>(log2_exact(static_cast<uint64_t>(p.tile_n) * e / p.vec_bytes));
    l.args.tiles_n = static_cast<uint32_t>(p.tiles_n);
    l.args.total_tiles = static_cast<uint32_t>(p.total_tiles);
    l.args.rank = geom.rank;
    l.args.rank_start = rank_start;
    l.args.rank_stride = rank_stride;
    l.args.group_rank = p.group_rank;
    l.args.slices = static_cast<uint32_t>(p.threads / 256);
    l.args.world = static_cast<uint32_t>(W);
    l.args.partitioned = part ? 1u : 0u;
    l.kind = kind;
    l.vec_bytes = p.vec_bytes;
    l.dests = part ? 1 : W;
    l.group = p.dest_group;
    l.vpt = p.vectors_per_thread;
    l.grid = p.n_programs;
    // streaming stores with system scope on wide launches whose stores are never waited for
    l.wide = (p.dest_group == 0 && 2 * static_cast<int64_t>(p.n_programs) >= geom.num_cus) ? 1 : 0;
    // ticket order: the calling rank's counter (zero between calls; calls of one rank never overlap)
    l.ticket = p.tiles_per_ticket;
    l.drain = p.ticket_wait;
    l.args.tickets = p.tiles_per_ticket
                         ? heap->core->tickets + (kTicketBytes / sizeof(uint32_t)) * static_cast<uint64_t>(geom.rank)
                         : nullptr;
    if (noalloc && p.tiles_per_ticket) {
        const hipError_t e1 = ag::noalloc_tickets(geom.rank, static_cast<hipStream_t>(stream), &l.args.tickets);
        if (e1 != hipSuccess) return fail_hip(e1, "tile counter of the allocation-free entry point");
    }
    const hipError_t e2 = ag::launch_copy(l, static_cast<hipStream_t>(stream));
    if (e2 != hipSuccess) return fail_hip(e2, kind == ag::kCopyAllToAll ? "all-to-all kernel launch" : "all-gather kernel launch");
    return ok();
}

}  // namespace

extern "C" {

ag_status_t ag_plan_all_gather(const ag_heap_geometry_t* geom, int W, int rank_start, int rank_stride,
                               uint64_t input_addr, size_t out_offset, int64_t M_local, int64_t N,
                               ag_dtype_t dtype, int tile_m, int tile_n, int n_programs, ag_plan_t* plan)
{
    return plan_copy(geom, ag::kCopyAllGather, W, rank_start, rank_stride, input_addr, out_offset, M_local, N, dtype,
                     tile_m, tile_n, n_programs, nullptr, plan);
}

ag_status_t ag_plan_all_gather_ex(const ag_heap_geometry_t* geom, int W, int rank_start, int rank_stride,
                                  uint64_t input_addr, size_t out_offset, int64_t M_local, int64_t N,
                                  ag_dtype_t dtype, int tile_m, int tile_n, int n_programs,
                                  const ag_copy_options_t* options, ag_plan_t* plan)
{
    return plan_copy(geom, ag::kCopyAllGather, W, rank_start, rank_stride, input_addr, out_offset, M_local, N, dtype,
                     tile_m, tile_n, n_programs, options, plan);
}

ag_status_t ag_plan_all_to_all(const ag_heap_geometry_t* geom, int W, int rank_start, int rank_stride,
                               uint64_t input_addr, size_t out_offset, int64_t M_chunk, int64_t N,
                               ag_dtype_t dtype, int tile_m, int tile_n, int n_programs, ag_plan_t* plan)
{
    return plan_copy(geom, ag::kCopyAllToAll, W, rank_start, rank_stride, input_addr, out_offset, M_chunk, N, dtype,
                     tile_m, tile_n, n_programs, nullptr, plan);
}

ag_status_t ag_plan_all_to_all_ex(const ag_heap_geometry_t* geom, int W, int rank_start, int rank_stride,
                                  uint64_t input_addr, size_t out_offset, int64_t M_chunk, int64_t N,
                                  ag_dtype_t dtype, int tile_m, int tile_n, int n_programs,
                                  const ag_copy_options_t* options, ag_plan_t* plan)
{
    return plan_copy(geom, ag::kCopyAllToAll, W, rank_start, rank_stride, input_addr, out_offset, M_chunk, N, dtype,
                     tile_m, tile_n, n_programs, options, plan);
}

ag_status_t ag_all_gather(const ag_heap_t* heap, int W, int rank_start, int rank_stride,
                          const void* input, size_t out_offset, int64_t M_local, int64_t N,
                          ag_dtype_t dtype, int tile_m, int tile_n, int n_programs, void* stream)
{
    return launch_copy_call(heap, ag::kCopyAllGather, W, rank_start, rank_stride, input, out_offset, M_local, N,
                            dtype, tile_m, tile_n, n_programs, nullptr, stream);
}

ag_status_t ag_all_gather_ex(const ag_heap_t* heap, int W, int rank_start, int rank_stride,
                             const void* input, size_t out_offset, int64_t M_local, int64_t N,
                             ag_dtype_t dtype, int tile_m, int tile_n, int n_programs,
                             const ag_copy_options_t* options, void* stream)
{
    return launch_copy_call(heap, ag::kCopyAllGather, W, rank_start, rank_stride, input, out_offset, M_local, N,
                            dtype, tile_m, tile_n, n_programs, options, stream);
}

ag_status_t ag_all_gather_noalloc(const ag_heap_t* heap, int W, int rank_start, int rank_stride,
                                  const void* input, size_t out_offset, int64_t M_local, int64_t N,
                                  ag_dtype_t dtype, int tile_m, int tile_n, int n_programs,
                                  const ag_copy_options_t* options, void* stream)
{
    return launch_copy_call(heap, ag::kCopyAllGather, W, rank_start, rank_stride, input, out_offset, M_local, N,
                            dtype, tile_m, tile_n, n_programs, options, stream, true);
}

ag_status_t ag_all_to_all(const ag_heap_t* heap, int W, int rank_start, int rank_stride,
                          const void* input, size_t out_offset, int64_t M_chunk, int64_t N,
                          ag_dtype_t dtype, int tile_m, int tile_n, int n_programs, void* stream)
{
    return launch_copy_call(heap, ag::kCopyAllToAll, W, rank_start, rank_stride, input, out_offset, M_chunk, N,
                            dtype, tile_m, tile_n, n_programs, nullptr, stream);
}

ag_status_t ag_all_to_all_ex(const ag_heap_t* heap, int W, int rank_start, int rank_stride,
                             const void* input, size_t out_offset, int64_t M_chunk, int64_t N,
                             ag_dtype_t dtype, int tile_m, int tile_n, int n_programs,
                             const ag_copy_options_t* options, void* stream)
{
    return launch_copy_call(heap, ag::kCopyAllToAll, W, rank_start, rank_stride, input, out_offset, M_chunk, N,
                            dtype, tile_m, tile_n, n_programs, options, stream);
}

// ---------------------------------------------------------------------------
// fused GEMM + all-gather
// ---------------------------------------------------------------------------

}  // extern "C"

namespace {

// bt: B stored N-contiguous (element (k,n) at B[k*ldb + n]); otherwise K-contiguous.
ag_status_t plan_gemm(const ag_heap_geometry_t* geom, int W, int rank_start, int rank_stride, uint64_t a_addr,
                      int64_t lda, uint64_t b_addr, int64_t ldb, size_t out_offset, int64_t M_local, int64_t N,
                      int64_t K, ag_dtype_t dtype, int tile_m, int tile_n, int tile_k, int n_programs, bool bt,
                      ag_plan_t* plan)
{
    ag_status_t s = check_geometry(geom);
    if (s != AG_OK) return s;
    if (!plan) return fail(AG_ERR_INVALID_ARG, "plan is NULL");
    int g = 0;
    s = check_group(geom, W, rank_start, rank_stride, &g);
    if (s != AG_OK) return s;
    if (dtype == AG_F32) return fail(AG_ERR_UNSUPPORTED, "the fused GEMM takes fp16 or bf16 operands");
    if (dtype != AG_F16 && dtype != AG_BF16) return fail(AG_ERR_INVALID_ARG, "unknown dtype %d", static_cast<int>(dtype));
    if (M_local < 0) return fail(AG_ERR_INVALID_ARG, "M_local %lld < 0", static_cast<long long>(M_local));
    if (N < 1) return fail(AG_ERR_INVALID_ARG, "N %lld < 1", static_cast<long long>(N));
    if (K < 1) return fail(AG_ERR_INVALID_ARG, "K %lld < 1", static_cast<long long>(K));
    if (n_programs < 0) return fail(AG_ERR_INVALID_ARG, "n_programs %d < 0", n_programs);
    if (M_local > (int64_t{1} << 30) || N > (int64_t{1} << 30) || K > (int64_t{1} << 30))
        return fail(AG_ERR_UNSUPPORTED, "M_local, N or K > 2^30");
    if (K % 64 != 0) return fail(AG_ERR_UNSUPPORTED, "K %lld is not a multiple of 64", static_cast<long long>(K));
    if (N % 8 != 0) return fail(AG_ERR_UNSUPPORTED, "N %lld is not a multiple of 8", static_cast<long long>(N));
    if (lda < K) return fail(AG_ERR_INVALID_ARG, "lda %lld < K %lld", static_cast<long long>(lda),
                             static_cast<long long>(K));
    if (!bt && ldb < K) return fail(AG_ERR_INVALID_ARG, "ldb %lld < K %lld (B K-contiguous)",
                                    static_cast<long long>(ldb), static_cast<long long>(K));
    if (bt && ldb < N) return fail(AG_ERR_INVALID_ARG, "ldb %lld < N %lld (B N-contiguous)",
                                   static_cast<long long>(ldb), static_cast<long long>(N));
    if (lda % 8 != 0 || ldb % 8 != 0) return fail(AG_ERR_UNSUPPORTED, "lda and ldb must be multiples of 8");
    if (out_offset % 16 != 0) return fail(AG_ERR_UNSUPPORTED, "out_offset %zu is not a multiple of 16", out_offset);
    const uint64_t row_bytes = static_cast<uint64_t>(N) * 2;
    const uint64_t blk = static_cast<uint64_t>(M_local) * row_bytes;
    if (blk > geom->bytes_per_rank / W || out_offset > geom->bytes_per_rank - W * blk)
        return fail(AG_ERR_INVALID_ARG, "output block (%d x %llu bytes at offset %zu) exceeds the region (%llu bytes)",
                    W, static_cast<unsigned long long>(blk), out_offset,
                    static_cast<unsigned long long>(geom->bytes_per_rank));
    // tile configurations the kernel is instantiated for: {TM, TN}, K step 64
    struct TileCfg { int tm, tn, id; };
    static const TileCfg kTiles[] = {{256, 256, ag::kGemmTile256x256}, {256, 224, ag::kGemmTile256x224},
                                     {128, 128, ag::kGemmTile128x128}};
    // an N-contiguous B reads two LDS fragments per 16 columns: no 256x256 kernel for it
    auto available = [&](const TileCfg& t) { return !(bt && t.id == ag::kGemmTile256x256); };
    const uint64_t programs_req = n_programs == 0 ? geom->num_cus : n_programs;
    const TileCfg* cfg = nullptr;
    if (tile_m == 0 && tile_n == 0 && tile_k == 0) {
        // fewest MFMA-cycles on the busiest program: rounds of tiles x tile area;
        // ties go to the larger tile (less operand traffic per flop)
        uint64_t best = ~uint64_t{0};
        for (const TileCfg& t : kTiles) {
            if (!available(t)) continue;
            const uint64_t tiles = ceil_div(M_local > 0 ? M_local : 1, t.tm) * ceil_div(N, t.tn);
            const uint64_t cost = ceil_div(tiles, programs_req) * static_cast<uint64_t>(t.tm) * t.tn;
            if (cost < best) {
                best = cost;
                cfg = &t;
            }
        }
    } else {
        for (const TileCfg& t : kTiles)
            if (tile_m == t.tm && tile_n == t.tn && tile_k == 64) cfg = &t;
        if (!cfg)
            return fail(AG_ERR_UNSUPPORTED,
                        "tile %dx%dx%d: supported are 256x256x64, 256x224x64 and 128x128x64 (0,0,0 = choose)",
                        tile_m, tile_n, tile_k);
        if (!available(*cfg))
            return fail(AG_ERR_UNSUPPORTED, "tile 256x256x64 takes B K-contiguous only; use 256x224x64 or 128x128x64");
    }
    ag_plan_t p{};
    p.group_rank = g;
    p.tile_m = cfg->tm;
    p.tile_n = cfg->tn;
    p.tile_k = 64;
    p.vec_bytes = 16;
    p.rank_block_offset = out_offset + static_cast<uint64_t>(g) * blk;
    p.bytes_read = (static_cast<uint64_t>(M_local) + static_cast<uint64_t>(N)) * static_cast<uint64_t>(K) * 2;
    p.bytes_written = blk * W;
    p.flops = 2.0 * static_cast<double>(M_local) * static_cast<double>(N) * static_cast<double>(K);
    if (M_local == 0) {
        p.bytes_read = 0;
        *plan = p;
        return ok();
    }
    if (a_addr == 0 || b_addr == 0) return fail(AG_ERR_INVALID_ARG, "A or B is NULL");
    if (a_addr % 16 != 0 || b_addr % 16 != 0) return fail(AG_ERR_UNSUPPORTED, "A and B must be 16-byte aligned");
    const uint64_t a_bytes = (static_cast<uint64_t>(M_local - 1) * lda + K) * 2;
    const uint64_t b_bytes = bt ? (static_cast<uint64_t>(K - 1) * ldb + N) * 2 : (static_cast<uint64_t>(N - 1) * ldb + K) * 2;
    for (int j = 0; j < W; ++j) {
        const uint64_t region = geom->slab_addr + static_cast<uint64_t>(rank_start + j * rank_stride) * geom->bytes_per_rank;
        if (overlaps(a_addr, a_bytes, region + out_offset, W * blk) ||
            overlaps(b_addr, b_bytes, region + out_offset, W * blk))
            return fail(AG_ERR_INVALID_ARG, "A or B overlaps the output block of region %d", rank_start + j * rank_stride);
    }
    // per-tile buffer descriptors address at most one tile of rows with 32-bit offsets (an N-contiguous B:
    // one K stage of 64 rows, plus the tile's columns)
    if (static_cast<uint64_t>(cfg->tm) * lda * 2 >= (uint64_t{1} << 31) ||
        (!bt && static_cast<uint64_t>(cfg->tn) * ldb * 2 >= (uint64_t{1} << 31)) ||
        (bt && (uint64_t{64} * ldb + cfg->tn) * 2 >= (uint64_t{1} << 31)) ||
        static_cast<uint64_t>(cfg->tm) * row_bytes >= (uint64_t{1} << 31))
        return fail(AG_ERR_UNSUPPORTED, "a tile of rows (or a K stage of an N-contiguous B) spans 2 GiB or more");
    const uint64_t tiles_m = ceil_div(M_local, cfg->tm);
    const uint64_t tiles_n = ceil_div(N, cfg->tn);
    const uint64_t total = tiles_m * tiles_n;
    if (total >= (uint64_t{1} << 31)) return fail(AG_ERR_UNSUPPORTED, "more than 2^31 tiles");
    p.tiles_m = static_cast<int64_t>(tiles_m);
    p.tiles_n = static_cast<int64_t>(tiles_n);
    p.total_tiles = static_cast<int64_t>(total);
    p.n_programs = static_cast<int32_t>(std::min<uint64_t>(programs_req, total));
    ag::gemm_resources(cfg->id, &p.threads, &p.lds_bytes);
    p.variant = cfg->id;
    *plan = p;
    return ok();
}

ag_status_t gemm_options(const ag_gemm_options_t* options, bool* bt)
{
    ag_gemm_options_t opt{};
    if (options) opt = *options;
    for (int i = 0; i < 7; ++i)
        if (opt.reserved[i] != 0) return fail(AG_ERR_INVALID_ARG, "options->reserved[%d] is not 0", i);
    if (opt.b_layout != AG_B_K_CONTIGUOUS && opt.b_layout != AG_B_N_CONTIGUOUS)
        return fail(AG_ERR_INVALID_ARG, "unknown b_layout %d", opt.b_layout);
    *bt = opt.b_layout == AG_B_N_CONTIGUOUS;
    return AG_OK;
}

ag_status_t launch_gemm_call(const ag_heap_t* heap, int W, int rank_start, int rank_stride, const void* A,
                             int64_t lda, const void* B, int64_t ldb, size_t out_offset, int64_t M_local, int64_t N,
                             int64_t K, ag_dtype_t dtype, int tile_m, int tile_n, int tile_k, int n_programs,
                             const ag_gemm_options_t* options, void* stream)
{
    if (!heap) return fail(AG_ERR_INVALID_ARG, "heap is NULL");
    bool bt = false;
    ag_status_t s = gemm_options(options, &bt);
    if (s != AG_OK) return s;
    ag_heap_geometry_t geom;
    ag_heap_geometry(heap, &geom);
    ag_plan_t p;
    s = plan_gemm(&geom, W, rank_start, rank_stride, reinterpret_cast<uint64_t>(A), lda,
                  reinterpret_cast<uint64_t>(B), ldb, out_offset, M_local, N, K, dtype, tile_m, tile_n, tile_k,
                  n_programs, bt, &p);
    if (s != AG_OK) return s;
    if (p.total_tiles == 0) return ok();
    s = check_device(heap);
    if (s != AG_OK) return s;
    ag::GemmLaunch l{};
    l.args.heap_bases = heap->core->table;
    l.args.A = static_cast<const uint16_t*>(A);
    l.args.B = static_cast<const uint16_t*>(B);
    l.args.rank_block_offset = p.rank_block_offset;
    l.args.lda = lda;
    l.args.ldb = ldb;
    l.args.M = static_cast<int32_t>(M_local);
    l.args.N = static_cast<int32_t>(N);
    l.args.K = static_cast<int32_t>(K);
    l.args.tiles_m = static_cast<int32_t>(p.tiles_m);
    l.args.tiles_n = static_cast<int32_t>(p.tiles_n);
    l.args.total_tiles = static_cast<int32_t>(p.total_tiles);
    l.args.rank = geom.rank;
    l.args.rank_start = rank_start;
    l.args.rank_stride = rank_stride;
    l.args.group_rank = p.group_rank;
    l.bf16 = dtype == AG_BF16 ? 1 : 0;
    l.world = W;
    l.cfg = p.variant;
    l.grid = p.n_programs;
    l.b_n_contiguous = bt ? 1 : 0;
    const hipError_t e = ag::launch_gemm(l, static_cast<hipStream_t>(stream));
    if (e == hipErrorNotSupported) return fail(AG_ERR_UNSUPPORTED, "fused GEMM kernel variant not available");
    if (e != hipSuccess) return fail_hip(e, "fused GEMM kernel launch");
    return ok();
}

}  // namespace

extern "C" {

ag_status_t ag_plan_gemm_all_gather(const ag_heap_geometry_t* geom, int W, int rank_start, int rank_stride,
                                    uint64_t a_addr, int64_t lda, uint64_t b_addr, int64_t ldb,
                                    size_t out_offset, int64_t M_local, int64_t N, int64_t K,
                                    ag_dtype_t dtype, int tile_m, int tile_n, int tile_k,
                                    int n_programs, ag_plan_t* plan)
{
    return plan_gemm(geom, W, rank_start, rank_stride, a_addr, lda, b_addr, ldb, out_offset, M_local, N, K, dtype,
                     tile_m, tile_n, tile_k, n_programs, false, plan);
}

ag_status_t ag_plan_gemm_all_gather_ex(const ag_heap_geometry_t* geom, int W, int rank_start, int rank_stride,
                                       uint64_t a_addr, int64_t lda, uint64_t b_addr, int64_t ldb,
                                       size_t out_offset, int64_t M_local, int64_t N, int64_t K,
                                       ag_dtype_t dtype, int tile_m, int tile_n, int tile_k,
                                       int n_programs, const ag_gemm_options_t* options, ag_plan_t* plan)
{
    bool bt = false;
    const ag_status_t s = gemm_options(options, &bt);
    if (s != AG_OK) return s;
    return plan_gemm(geom, W, rank_start, rank_stride, a_addr, lda, b_addr, ldb, out_offset, M_local, N, K, dtype,
                     tile_m, tile_n, tile_k, n_programs, bt, plan);
}

ag_status_t ag_gemm_all_gather(const ag_heap_t* heap, int W, int rank_start, int rank_stride,
                               const void* A, int64_t lda, const void* B, int64_t ldb,
                               size_t out_offset, int64_t M_local, int64_t N, int64_t K,
                               ag_dtype_t dtype, int tile_m, int tile_n, int tile_k,
                               int n_programs, void* stream)
{
    return launch_gemm_call(heap, W, rank_start, rank_stride, A, lda, B, ldb, out_offset, M_local, N, K, dtype,
                            tile_m, tile_n, tile_k, n_programs, nullptr, stream);
}

ag_status_t ag_gemm_all_gather_ex(const ag_heap_t* heap, int W, int rank_start, int rank_stride,
                                  const void* A, int64_t lda, const void* B, int64_t ldb,
                                  size_t out_offset, int64_t M_local, int64_t N, int64_t K,
                                  ag_dtype_t dtype, int tile_m, int tile_n, int tile_k,
                                  int n_programs, const ag_gemm_options_t* options, void* stream)
{
    return launch_gemm_call(heap, W, rank_start, rank_stride, A, lda, B, ldb, out_offset, M_local, N, K, dtype,
                            tile_m, tile_n, tile_k, n_programs, options, stream);
}

}  // extern "C"
