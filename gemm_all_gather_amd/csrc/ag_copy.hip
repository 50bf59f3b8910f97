// Persistent tiled multi-destination all-gather store loop for gfx950.
//
// Method (ROCm/iris #626, "Summary" and "Triton CCL all-gather"; ROCm/iris
// #591, "Hoist the peer heap bases"):
//   * before the tile loop, load the local heap base and every destination's
//     heap base from the device table heap_bases once, and keep each
//     destination as a 64-bit pointer delta (dest_base - local_base) in
//     scalar registers (one vector load of the W entries, issued just ahead
//     of the first two input tiles' loads so the latencies overlap, then
//     readlane);
//   * walk the tiles of the M_local x N input with a grid stride;
//   * load each input tile once and store it to every destination: the
//     local region first, then the peers in rotated group order
//     (g+1, g+2, ... mod W), with a statically unrolled destination loop.
//
// gfx950 specifics:
//   * one 256-thread slice owns one tile at a time; a workgroup has U slices
//     (blockDim.x = 256*U) so a CU keeps U tiles' loads and W*U tiles' stores
//     in flight;
//   * 16-byte vector accesses when N*e, the input and the output block are
//     16-byte aligned (8/4/2 otherwise);
//   * the per-lane byte offsets inside a tile do not depend on the tile, so
//     they are computed once; each tile only rebases buffer descriptors
//     (scalar registers), and every access is a buffer load or store with a
//     32-bit VGPR offset, bounds-checked by the descriptor;
//   * the next tile's loads are issued before the current tile's stores, so
//     waiting for them never waits for the stores (the memory counter is in
//     issue order), and no destination store is preceded by a full drain;
//   * the destination stores stream (non-temporal), with system coherence
//     scope added on launches over at least half the CUs whose stores are
//     never waited for (the WIDE kernels).
//
// Variants (ROCm/iris #594, "Reviewer performance evaluation" and "Compiler
// inspection and grouping"; ROCm/iris #591, "INLINE grouping"; ROCm/iris
// #626, "Triton CCL all-gather" on the partitioned kernel):
//   * destination groups (G > 0): after every G destinations' stores, wait
//     until everything issued before that group has completed, so at most
//     two groups of stores are in flight;
//   * partitioned schedule: program p stores only to destination p % W
//     (rotated order, 0 = local) and walks every (grid/W)-th tile from
//     p / W, reading each input tile once per destination;
//   * all-to-all (ag_a2a_kernel): for each tile, destination i receives
//     the tile of input chunk (g + i) mod W, the chunk meant for it.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "ag_internal.h"

namespace ag {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

// Cache-policy bits of the destination stores.  The W written copies are not
// re-read by these kernels, so they are streamed: non-temporal (nt, bit 1),
// about twice as fast as the default policy (or sc1 alone) on a 75 MB/call
// workload.  Launches on at least half the CUs whose stores are never waited
// for use nt with system coherence scope (sc1, bit 4): 1.5-2% faster again
// (6.54 against 6.43 TB/s at W=8, 1024x4096 fp16, 128 programs; 458 against
// 466-473 us at 16384x8192).  Those stores take longer to retire, so kernels
// that wait on them (destination groups: 3.1 against 5.0 TB/s with groups of
// one) or with few programs (64: 4.4 against 4.9 TB/s) keep nt alone.  nt with
// sc0 equals nt alone.
#ifndef AG_COPY_STORE_AUX
#define AG_COPY_STORE_AUX 2
#endif
#ifndef AG_COPY_STORE_AUX_WIDE
#define AG_COPY_STORE_AUX_WIDE 18
#endif
// Cache-policy bits of the input loads (each input byte is read once):
// default.  Non-temporal loads measured 1.8x slower on the 1024x4096 workload.
#ifndef AG_COPY_LOAD_AUX
#define AG_COPY_LOAD_AUX 0
#endif

// Word 3 of a raw (stride 0) buffer descriptor on gfx9-family parts:
// 32-bit data format, no swizzle, bounds-checked by num_records.
constexpr int kRawBufferWord3 = 0x00020000;
// A lane offset that is always past num_records (<= 0x7fffffff): the access
// is dropped by the hardware (store) or returns zero (load).
constexpr uint32_t kOutOfRange = 0x80000000u;

// s_waitcnt with only the vector-memory counter limited (gfx9 encoding).
template <int N>
__device__ inline void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(uint64_t base, uint32_t num_records)
{
    return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(base), static_cast<short>(0),
                                             static_cast<int>(num_records), kRawBufferWord3);
}

template <int VEC> struct Vec;
template <> struct Vec<16> {
    using T = u32x4;
    static __device__ T load(__amdgpu_buffer_rsrc_t r, uint32_t o) { return __builtin_amdgcn_raw_buffer_load_b128(r, o, 0, AG_COPY_LOAD_AUX); }
    template <int AUX>
    static __device__ void store(T v, __amdgpu_buffer_rsrc_t r, uint32_t o) { __builtin_amdgcn_raw_buffer_store_b128(v, r, o, 0, AUX); }
};
template <> struct Vec<8> {
    using T = u32x2;
    static __device__ T load(__amdgpu_buffer_rsrc_t r, uint32_t o) { return __builtin_amdgcn_raw_buffer_load_b64(r, o, 0, AG_COPY_LOAD_AUX); }
    template <int AUX>
    static __device__ void store(T v, __amdgpu_buffer_rsrc_t r, uint32_t o) { __builtin_amdgcn_raw_buffer_store_b64(v, r, o, 0, AUX); }
};
template <> struct Vec<4> {
    using T = unsigned int;
    static __device__ T load(__amdgpu_buffer_rsrc_t r, uint32_t o) { return __builtin_amdgcn_raw_buffer_load_b32(r, o, 0, AG_COPY_LOAD_AUX); }
    template <int AUX>
    static __device__ void store(T v, __amdgpu_buffer_rsrc_t r, uint32_t o) { __builtin_amdgcn_raw_buffer_store_b32(v, r, o, 0, AUX); }
};
template <> struct Vec<2> {
    using T = unsigned short;
    static __device__ T load(__amdgpu_buffer_rsrc_t r, uint32_t o) { return __builtin_amdgcn_raw_buffer_load_b16(r, o, 0, AG_COPY_LOAD_AUX); }
    template <int AUX>
    static __device__ void store(T v, __amdgpu_buffer_rsrc_t r, uint32_t o) { __builtin_amdgcn_raw_buffer_store_b16(v, r, o, 0, AUX); }
};

struct TileRef {
    uint64_t off;        // byte offset of the tile's first element in the rank's block
    uint32_t records;    // bytes addressable from off (0: no tile, every access dropped)
    bool full;           // every column of the tile lies inside the row
    uint32_t col0;       // byte column of the tile's first element
};

// W destinations per tile; G destinations per wait (0: none).  PART: the
// partitioned schedule (W = 1, the group size is a.world at run time).  A
// partitioned program of the all-to-all (a.chunk_bytes > 0) reads the chunk
// its destination receives: chunk (g + i) mod W for destination i.  WIDE: the
// stores' cache policy for launches on at least half the CUs (never with G).
template <int VEC, int W, int VPT, int G, bool PART, bool WIDE>
__global__ __launch_bounds__(1024) void ag_copy_kernel(CopyKernelArgs a)
{
    constexpr int kAux = WIDE ? AG_COPY_STORE_AUX_WIDE : AG_COPY_STORE_AUX;
    static_assert(!WIDE || G == 0, "waited-for stores keep the plain streaming policy");
    using VT = Vec<VEC>;
    using V = typename VT::T;
    static_assert(G == 0 || G < W, "a group smaller than the destination count");
    static_assert(!PART || (W == 1 && G == 0), "a partitioned program has one destination");

    uint64_t input = reinterpret_cast<uint64_t>(a.input);
    if constexpr (PART) {
        int c = a.group_rank + static_cast<int>(blockIdx.x % a.world);   // < 2 * world
        if (c >= static_cast<int>(a.world)) c -= static_cast<int>(a.world);
        input += static_cast<uint64_t>(c) * a.chunk_bytes;
    }
    const uint64_t block_bytes = static_cast<uint64_t>(a.rows) * a.row_bytes;

    // ---- tile-invariant lane geometry
    const uint32_t lane = threadIdx.x & 255u;
    // a wave never straddles two slices, so the slice index is wave-uniform
    const uint32_t slice = __builtin_amdgcn_readfirstlane(threadIdx.x >> 8);
    const uint32_t vpr_mask = (1u << a.vecs_per_row_log2) - 1u;
    uint32_t lane_off[VPT];   // byte offset of this lane's vector j inside a tile
    uint32_t lane_col[VPT];   // byte column of vector j inside the tile
#pragma unroll
    for (int j = 0; j < VPT; ++j) {
        const uint32_t idx = lane + 256u * j;
        lane_col[j] = (idx & vpr_mask) * VEC;
        lane_off[j] = (idx >> a.vecs_per_row_log2) * static_cast<uint32_t>(a.row_bytes) + lane_col[j];
    }

    // partitioned: the programs of one destination walk the tiles among themselves
    const uint32_t stride = PART ? gridDim.x / a.world : gridDim.x * a.slices;
    uint32_t t = PART ? blockIdx.x / a.world : blockIdx.x * a.slices + slice;
    if (t >= a.total_tiles) return;

    // Tile -> (tm, tn), row-major over tiles.  Rows past M_local fall past the
    // end of the block and are dropped by the descriptor's bounds check;
    // columns past N are redirected out of range explicitly.
    auto origin = [&](uint32_t tile, bool valid) {
        TileRef r;
        const uint32_t tm = tile / a.tiles_n;
        const uint32_t tn = tile - tm * a.tiles_n;
        r.col0 = tn * a.tile_row_bytes;
        r.off = static_cast<uint64_t>(tm) * a.tile_m * a.row_bytes + r.col0;
        const uint64_t left = valid ? block_bytes - r.off : 0;
        r.records = static_cast<uint32_t>(left < 0x7fffffffull ? left : 0x7fffffffull);
        r.full = r.col0 + a.tile_row_bytes <= a.row_bytes;
        return r;
    };
    auto offsets = [&](const TileRef& r, uint32_t (&vo)[VPT]) {
#pragma unroll
        for (int j = 0; j < VPT; ++j)
            vo[j] = (r.full || r.col0 + lane_col[j] < a.row_bytes) ? lane_off[j] : kOutOfRange;
    };
    auto load_tile = [&](const TileRef& r, const uint32_t (&vo)[VPT], V (&v)[VPT]) {
        const __amdgpu_buffer_rsrc_t src = make_rsrc(input + r.off, r.records);
#pragma unroll
        for (int j = 0; j < VPT; ++j) v[j] = VT::load(src, vo[j]);
    };

    // ---- translate every destination once, before the tile loop.
    // Destination i is group member (g + i) mod W (i = 0: the calling rank);
    // a partitioned program owns destination p mod world of that order.  One
    // vector load fetches every table entry (lane i: destination i, lane W:
    // the local base); it is issued ahead of the first two tiles' loads, so
    // the three latencies overlap and waiting for the table never waits for
    // a tile; readlane then moves the entries to scalar registers.
    const int world = PART ? static_cast<int>(a.world) : W;
    const int first = PART ? static_cast<int>(blockIdx.x % a.world) : 0;
    uint64_t table_entry;
    {
        const int l = static_cast<int>(threadIdx.x & 63u);
        int entry = a.rank;
        if (l < W) {
            int gi = a.group_rank + first + l;   // < 2 * world
            if (gi >= world) gi -= world;
            entry = a.rank_start + gi * a.rank_stride;
        }
        table_entry = a.heap_bases[entry];
    }
    __builtin_amdgcn_sched_barrier(0);   // the table load goes out first
    // ---- the first two tiles
    TileRef ta = origin(t, true), tb;
    uint32_t oa[VPT], ob[VPT];
    V va[VPT], vb[VPT];
    offsets(ta, oa);
    load_tile(ta, oa, va);
    uint32_t tn = t + stride;
    bool more = tn < a.total_tiles && tn > t;   // tn > t: no wrap-around
    tb = origin(more ? tn : t, more);
    offsets(tb, ob);
    load_tile(tb, ob, vb);                      // prefetch (dropped when !more)

    uint64_t base[W];
    uint64_t local_base;
    {
        const uint64_t v = table_entry;
        const uint32_t lo = static_cast<uint32_t>(v), hi = static_cast<uint32_t>(v >> 32);
#pragma unroll
        for (int i = 0; i <= W; ++i) {
            const uint64_t b = (static_cast<uint64_t>(static_cast<uint32_t>(__builtin_amdgcn_readlane(hi, i))) << 32) |
                               static_cast<uint32_t>(__builtin_amdgcn_readlane(lo, i));
            if (i < W) base[i] = b;
            else local_base = b;
        }
    }
    const uint64_t out_local = local_base + a.rank_block_offset;
    uint64_t dest[W];   // out_local + (dest_base - local_base): local region first, then rotated peers
#pragma unroll
    for (int i = 0; i < W; ++i) dest[i] = out_local + static_cast<uint64_t>(static_cast<int64_t>(base[i] - local_base));

    auto store_tile = [&](const TileRef& r, const uint32_t (&vo)[VPT], const V (&v)[VPT]) {
#pragma unroll
        for (int i = 0; i < W; ++i) {   // local region first, then the rotated peers
            const __amdgpu_buffer_rsrc_t dst = make_rsrc(dest[i] + r.off, r.records);
#pragma unroll
            for (int j = 0; j < VPT; ++j) VT::template store<kAux>(v[j], dst, vo[j]);
            // end of a destination group: retire everything issued before it
            if (G > 0 && (i + 1) % G == 0 && i + 1 < W) wait_vmcnt<G * VPT>();
        }
    };

    // Two register sets used in turn: the next tile is loaded into one while
    // the other is stored, with no register copy (which would wait on the
    // prefetched loads).  Loads and stores are unconditional buffer accesses;
    // the first step is peeled so that the loop is always entered with the
    // same accesses in flight (one tile load issued before W*VPT stores) and
    // each wait covers only the prefetched loads, never the stores.
    store_tile(ta, oa, va);
    if (!more) return;
    t = tn;
    for (;;) {
        tn = t + stride;
        more = tn < a.total_tiles && tn > t;
        ta = origin(more ? tn : t, more);
        offsets(ta, oa);
        load_tile(ta, oa, va);
        store_tile(tb, ob, vb);
        if (!more) break;
        t = tn;

        tn = t + stride;
        more = tn < a.total_tiles && tn > t;
        tb = origin(more ? tn : t, more);
        offsets(tb, ob);
        load_tile(tb, ob, vb);
        store_tile(ta, oa, va);
        if (!more) break;
        t = tn;
    }
}

// Ticket order.  The same persistent programs and the same per-tile work (each
// tile loaded once, then stored to the local region and the rotated peers),
// but the programs take their tiles from a device counter in increasing
// order, G consecutive tiles per ticket, instead of walking a fixed grid
// stride.  Programs of a grid stride drift apart, so over a long call the
// tiles in flight spread over an ever wider address range of the W+1
// streams; tickets keep them in one compact window, as the hardware
// dispatcher does for a grid of one workgroup per tile, and the HBM streams
// stay dense (W=8, 16384x8192 fp16, 256 programs: 373 against 448 us per call
// in a measured replica).  Each ticket is one relaxed device-scope atomic
// increment by one thread, handed to the workgroup through LDS; the last
// program to finish resets the counter, so it is zero at every launch.  One
// counter serves about one increment per 12 ns, so the planner sizes G for
// at least 96 KiB of HBM traffic per ticket where a kernel that large exists
// (at W=4, 3 tiles of 8x256 fp16 per ticket made the call counter-bound).  Two
// batches of G tiles live in registers: the next one loading while the one in
// hand is stored.
//
// Addressing: a tile is a byte offset into the block, its extent, and the
// columns a lane may touch in it (all uniform); the batch's first tile costs
// one division, the next ones an increment.  Each access rebases a descriptor
// on the tile (the same lane offsets in every tile): measured 5-10% faster
// than one descriptor per stream with the tile in each lane's 32-bit offset.
// Rows past M fall past the tile's extent; columns past N of the last tile
// column get an out-of-range lane offset.
//
// DRAIN false: the next ticket is taken before the stores of the batch in
// hand, so waiting for it never waits for those stores.
// DRAIN true (wide launches: programs x vectors per thread from three
// quarters of the CU count, as the planner decides): the ticket is taken
// after the batch's stores; thread 0 needs its value, so wave 0 waits for
// everything it has issued, and the barrier that hands the ticket out holds
// the other waves until then.  The next batch's loads go out right after, in
// front of the stores of the batch in hand.  With every CU storing, fewer
// stores in flight keep the HBM write streams denser (W=8, 16384x8192 fp16,
// 256 programs: 360 against 387 us per call in a measured replica); with half
// the CUs the wait costs more than it saves.
//
// A2A (the all-to-all in ticket order): the tiles are the W chunk copies as
// one sequence, destination by destination, as in ag_a2a_kernel; each tile
// has one source (chunk (g + i) mod W) and one destination (i) instead of
// one source and W destinations.
template <int VEC, int W, int VPT, int G, bool WIDE, bool DRAIN, bool A2A>
__device__ __forceinline__ void ticket_copy(const CopyKernelArgs& a)
{
    constexpr int kAux = WIDE ? AG_COPY_STORE_AUX_WIDE : AG_COPY_STORE_AUX;
    using VT = Vec<VEC>;
    using V = typename VT::T;
    __shared__ uint32_t s_ticket[2];

    const uint32_t row_bytes = static_cast<uint32_t>(a.row_bytes);
    const uint32_t block_bytes = a.rows * row_bytes;             // < 2^31 (planner); one chunk for A2A
    const uint32_t tile_rows_bytes = a.tile_m * row_bytes;       // bytes from one tile row to the next
    const uint32_t last_col_bytes = row_bytes - (a.tiles_n - 1u) * a.tile_row_bytes;
    const uint64_t input = reinterpret_cast<uint64_t>(a.input);
    uint32_t* const counter = a.tickets;
    const uint32_t per_dest = a.total_tiles;                     // A2A: tiles of one chunk
    const uint32_t total = A2A ? per_dest * static_cast<uint32_t>(W) : per_dest;   // < 2^31 (planner)
    const uint32_t chunk_rows_bytes = (per_dest / a.tiles_n) * tile_rows_bytes;    // A2A: a chunk's tile rows

    const uint32_t lane = threadIdx.x;
    const uint32_t vpr_mask = (1u << a.vecs_per_row_log2) - 1u;
    uint32_t lane_off[VPT], lane_col[VPT];
#pragma unroll
    for (int j = 0; j < VPT; ++j) {
        const uint32_t idx = lane + 256u * j;
        lane_col[j] = (idx & vpr_mask) * VEC;
        lane_off[j] = (idx >> a.vecs_per_row_log2) * row_bytes + lane_col[j];
    }
    // Walk the G tiles first, first+1, ... (row-major over the tile grid; A2A: chunk after chunk), calling
    // f(b, i, off, records, lim) for each: the destination index (A2A; 0 otherwise and past the last
    // tile), its byte offset in the block, the bytes addressable from there (0 past the last tile: every
    // access dropped) and the bytes of its row a lane may touch (the last tile column's width).
    auto for_tiles = [&](uint32_t first, auto&& f) {
        uint32_t i = 0, t = first;
        if constexpr (A2A) {
            i = first / per_dest;
            t = first - i * per_dest;
        }
        uint32_t tm = t / a.tiles_n;
        uint32_t tn = t - tm * a.tiles_n;
        uint32_t row0 = tm * tile_rows_bytes;
#pragma unroll
        for (int b = 0; b < G; ++b) {
            const bool valid = first + static_cast<uint32_t>(b) < total;
            const uint32_t off = valid ? row0 + tn * a.tile_row_bytes : 0u;
            const uint32_t lim = tn + 1u == a.tiles_n ? last_col_bytes : 0xffffffffu;
            f(b, valid ? i : 0u, off, valid ? block_bytes - off : 0u, lim);
            if (++tn == a.tiles_n) {
                tn = 0;
                row0 += tile_rows_bytes;
                if constexpr (A2A) {
                    if (row0 == chunk_rows_bytes) {   // on to the next destination's chunk
                        row0 = 0;
                        ++i;
                    }
                }
            }
        }
    };
    auto lane_offset = [&](int j, uint32_t lim) { return lane_col[j] < lim ? lane_off[j] : kOutOfRange; };
    auto load_batch = [&](uint32_t first, V (&v)[G][VPT]) {
        for_tiles(first, [&](int b, uint32_t i, uint32_t off, uint32_t records, uint32_t lim) {
            uint64_t base = input;
            if constexpr (A2A) {   // chunk (g + i) mod W is meant for destination i
                uint32_t gi = static_cast<uint32_t>(a.group_rank) + i;
                if (gi >= static_cast<uint32_t>(W)) gi -= W;
                base += static_cast<uint64_t>(gi) * block_bytes;
            }
            const __amdgpu_buffer_rsrc_t src = make_rsrc(base + off, records);
#pragma unroll
            for (int j = 0; j < VPT; ++j) v[b][j] = VT::load(src, lane_offset(j, lim));
        });
    };
    // The next ticket: G tiles from the counter, which counts tickets (thread 0; the others get it
    // through LDS).  An increment (atomic inc with no wrap point), not an add: the compiler rewrites a
    // lone add into a wave-wide add whose result it distributes to the lanes at once, which would wait
    // for the atomic right where it is issued.  The ticket number goes through LDS as it comes back
    // (nothing is computed from it in thread 0); the batch's first tile is G times the number.
    auto take = [&]() -> uint32_t {
        return __builtin_amdgcn_atomic_inc32(counter, 0xffffffffu, __ATOMIC_RELAXED, "agent");
    };
    auto post = [&](uint32_t tk, int slot) -> uint32_t {
        if (threadIdx.x == 0) s_ticket[slot] = tk;
        __syncthreads();
        return s_ticket[slot] * static_cast<uint32_t>(G);
    };

    // ---- destinations, once, before the tile loop: one vector load of the table (lane i:
    // destination i = member (g + i) mod W, lane W: the local base), then readlane
    uint64_t table_entry;
    {
        const int l = static_cast<int>(threadIdx.x & 63u);
        int entry = a.rank;
        if (l < W) {
            int gi = a.group_rank + l;
            if (gi >= W) gi -= W;
            entry = a.rank_start + gi * a.rank_stride;
        }
        table_entry = a.heap_bases[entry];
    }
    __builtin_amdgcn_sched_barrier(0);   // the table load goes out first

    uint32_t first = post(threadIdx.x == 0 ? take() : 0u, 0);
    int slot = 1;
    V va[G][VPT], vb[G][VPT];
    uint32_t ta = first, tb = 0;
    if (ta < total) {
        load_batch(ta, va);
        if constexpr (!DRAIN) {
            tb = post(threadIdx.x == 0 ? take() : 0u, slot);
            slot ^= 1;
            load_batch(tb, vb);
        }

        uint64_t dest[A2A ? 1 : W];
        if constexpr (!A2A) {
            const uint32_t lo = static_cast<uint32_t>(table_entry), hi = static_cast<uint32_t>(table_entry >> 32);
            const uint64_t local_base = (static_cast<uint64_t>(static_cast<uint32_t>(__builtin_amdgcn_readlane(hi, W))) << 32) |
                                        static_cast<uint32_t>(__builtin_amdgcn_readlane(lo, W));
            const uint64_t out_local = local_base + a.rank_block_offset;
#pragma unroll
            for (int i = 0; i < W; ++i) {
                const uint64_t b = (static_cast<uint64_t>(static_cast<uint32_t>(__builtin_amdgcn_readlane(hi, i))) << 32) |
                                   static_cast<uint32_t>(__builtin_amdgcn_readlane(lo, i));
                dest[i] = out_local + static_cast<uint64_t>(static_cast<int64_t>(b - local_base));
            }
        }
        // A2A: lane i < W holds this rank's block in destination i's region (its heap base plus the
        // block offset), set once; a tile reads its destination's with readlane
        const uint64_t dest_lane = table_entry + a.rank_block_offset;
        auto store_batch = [&](uint32_t first_tile, const V (&v)[G][VPT]) {
            for_tiles(first_tile, [&](int b, uint32_t di, uint32_t off, uint32_t records, uint32_t lim) {
                if constexpr (A2A) {
                    const int li = static_cast<int>(di);
                    const int lo = static_cast<int>(static_cast<uint32_t>(dest_lane));
                    const int hi = static_cast<int>(static_cast<uint32_t>(dest_lane >> 32));
                    const uint64_t d = (static_cast<uint64_t>(static_cast<uint32_t>(__builtin_amdgcn_readlane(hi, li))) << 32) |
                                       static_cast<uint32_t>(__builtin_amdgcn_readlane(lo, li));
                    const __amdgpu_buffer_rsrc_t dst = make_rsrc(d + off, records);
#pragma unroll
                    for (int j = 0; j < VPT; ++j) VT::template store<kAux>(v[b][j], dst, lane_offset(j, lim));
                } else {
#pragma unroll
                    for (int i = 0; i < W; ++i) {   // local region first, then the rotated peers
                        const __amdgpu_buffer_rsrc_t dst = make_rsrc(dest[i] + off, records);
#pragma unroll
                        for (int j = 0; j < VPT; ++j) VT::template store<kAux>(v[b][j], dst, lane_offset(j, lim));
                    }
                }
            });
        };
        if constexpr (DRAIN) {
            // Invariant: va holds batch ta (ta < total, landed or loading); each ticket is taken after
            // the stores of the batch before it.
            for (;;) {
                tb = post(threadIdx.x == 0 ? take() : 0u, slot);
                slot ^= 1;
                load_batch(tb, vb);
                store_batch(ta, va);
                if (tb >= total) break;
                ta = post(threadIdx.x == 0 ? take() : 0u, slot);
                slot ^= 1;
                load_batch(ta, va);
                store_batch(tb, vb);
                if (ta >= total) break;
            }
        } else {
            // Invariant: va holds batch ta (in hand, ta < total), vb batch tb (loading); tickets rise.
            // The ticket is defined only in thread 0 and used only there: no value is merged in for the
            // other lanes, so nothing overwrites its register while the atomic is in flight and its wait
            // (at the LDS write, after the stores) covers only what was issued before it.
            for (;;) {
                bool more = tb < total;
                uint32_t tk;
                if (more && threadIdx.x == 0) tk = take();   // the batch after tb, before ta's stores
                store_batch(ta, va);
                if (!more) break;
                ta = post(tk, slot);
                slot ^= 1;
                load_batch(ta, va);

                more = ta < total;
                if (more && threadIdx.x == 0) tk = take();
                store_batch(tb, vb);
                if (!more) break;
                tb = post(tk, slot);
                slot ^= 1;
                load_batch(tb, vb);
            }
        }
    }
    // the last program to finish puts the counter back to zero for the next launch
    if (threadIdx.x == 0) {
        const uint32_t done = __hip_atomic_fetch_add(counter + 1, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (done + 1 == gridDim.x) {
            __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(counter + 1, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

template <int VEC, int W, int VPT, int G, bool WIDE, bool DRAIN>
__global__ __launch_bounds__(256) void ag_copy_ticket_kernel(CopyKernelArgs a)
{
    ticket_copy<VEC, W, VPT, G, WIDE, DRAIN, false>(a);
}

// The all-to-all in ticket order (16-byte vectors).
template <int W, int VPT, int G, bool WIDE, bool DRAIN>
__global__ __launch_bounds__(256) void ag_a2a_ticket_kernel(CopyKernelArgs a)
{
    ticket_copy<16, W, VPT, G, WIDE, DRAIN, true>(a);
}

// All-to-all: destination i (group member (g + i) mod W, i = 0 the local
// region) receives input chunk (g + i) mod W at this rank's block.  The W
// chunk copies are walked as one sequence of W x T tiles, destination by
// destination (tile u is tile u mod T of destination u / T: the local region
// first, then the rotated peers), with a grid stride.  At any time the
// programs are on one or two chunks, so two HBM streams are open rather than
// 2W: a tile-by-tile order that loaded the W chunk tiles of one tile index
// and then stored them ran 25.0 us per call at W=8, 8 chunks of 1024x4096
// fp16, where a plain 64 MiB copy takes 19.2.  The destination bases are
// translated once, before the tile loop, one per lane; each tile reads its
// own with readlane.  The next tile is loaded before the current one is
// stored.  WIDE: as for the all-gather kernel.
template <int VEC, int W, int VPT, bool WIDE>
__global__ __launch_bounds__(256) void ag_a2a_kernel(CopyKernelArgs a)
{
    using VT = Vec<VEC>;
    using V = typename VT::T;
    constexpr int kAux = WIDE ? AG_COPY_STORE_AUX_WIDE : AG_COPY_STORE_AUX;

    const uint64_t block_bytes = a.chunk_bytes;
    const uint64_t input = reinterpret_cast<uint64_t>(a.input);
    const uint32_t lane = threadIdx.x;
    const uint32_t vpr_mask = (1u << a.vecs_per_row_log2) - 1u;
    uint32_t lane_off[VPT], lane_col[VPT];
#pragma unroll
    for (int j = 0; j < VPT; ++j) {
        const uint32_t idx = lane + 256u * j;
        lane_col[j] = (idx & vpr_mask) * VEC;
        lane_off[j] = (idx >> a.vecs_per_row_log2) * static_cast<uint32_t>(a.row_bytes) + lane_col[j];
    }
    const uint32_t per_dest = a.total_tiles;                        // tiles of one chunk
    const uint32_t total = per_dest * static_cast<uint32_t>(W);     // < 2^31 (planner)
    const uint32_t stride = gridDim.x;
    uint32_t u = blockIdx.x;
    if (u >= total) return;

    // destination bases, once: one vector load of the table (lane i < W: the
    // heap base of member (g + i) mod W), issued ahead of the first two tiles'
    // loads
    uint64_t table_entry;
    {
        const int l = static_cast<int>(threadIdx.x & 63u);
        int entry = a.rank;
        if (l < W) {
            int gi = a.group_rank + l;
            if (gi >= W) gi -= W;
            entry = a.rank_start + gi * a.rank_stride;
        }
        table_entry = a.heap_bases[entry];
    }
    __builtin_amdgcn_sched_barrier(0);   // the table load goes out first

    struct Tile {
        TileRef r;
        uint32_t i;   // destination index (uniform)
    };
    auto origin = [&](uint32_t tile, bool valid) {
        Tile x;
        x.i = tile / per_dest;
        const uint32_t t = tile - x.i * per_dest;
        const uint32_t tm = t / a.tiles_n;
        const uint32_t tn = t - tm * a.tiles_n;
        x.r.col0 = tn * a.tile_row_bytes;
        x.r.off = static_cast<uint64_t>(tm) * a.tile_m * a.row_bytes + x.r.col0;
        const uint64_t left = valid ? block_bytes - x.r.off : 0;
        x.r.records = static_cast<uint32_t>(left < 0x7fffffffull ? left : 0x7fffffffull);
        x.r.full = x.r.col0 + a.tile_row_bytes <= a.row_bytes;
        return x;
    };
    auto offsets = [&](const TileRef& r, uint32_t (&vo)[VPT]) {
#pragma unroll
        for (int j = 0; j < VPT; ++j)
            vo[j] = (r.full || r.col0 + lane_col[j] < a.row_bytes) ? lane_off[j] : kOutOfRange;
    };
    auto load_tile = [&](const Tile& x, const uint32_t (&vo)[VPT], V (&v)[VPT]) {
        uint32_t gi = static_cast<uint32_t>(a.group_rank) + x.i;    // input chunk meant for destination i
        if (gi >= static_cast<uint32_t>(W)) gi -= W;
        const __amdgpu_buffer_rsrc_t s = make_rsrc(input + static_cast<uint64_t>(gi) * block_bytes + x.r.off,
                                                   x.r.records);
#pragma unroll
        for (int j = 0; j < VPT; ++j) v[j] = VT::load(s, vo[j]);
    };

    // same two-register-set pipeline as the all-gather loop
    Tile ta = origin(u, true), tb;
    uint32_t oa[VPT], ob[VPT];
    V va[VPT], vb[VPT];
    offsets(ta.r, oa);
    load_tile(ta, oa, va);
    uint32_t un = u + stride;
    bool more = un < total && un > u;
    tb = origin(more ? un : u, more);
    offsets(tb.r, ob);
    load_tile(tb, ob, vb);

    // lane i < W: this rank's block in the region of destination i, once.  (The local block's address
    // translated by destination i's base minus the local base is that base plus the block offset.)
    const uint64_t dest_lane = table_entry + a.rank_block_offset;
    const uint32_t dest_lo = static_cast<uint32_t>(dest_lane), dest_hi = static_cast<uint32_t>(dest_lane >> 32);
    auto store_tile = [&](const Tile& x, const uint32_t (&vo)[VPT], const V (&v)[VPT]) {
        const int i = __builtin_amdgcn_readfirstlane(static_cast<int>(x.i));
        const uint64_t d = (static_cast<uint64_t>(static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(dest_hi), i))) << 32) |
                           static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(dest_lo), i));
        const __amdgpu_buffer_rsrc_t dst = make_rsrc(d + x.r.off, x.r.records);
#pragma unroll
        for (int j = 0; j < VPT; ++j) VT::template store<kAux>(v[j], dst, vo[j]);
    };
    store_tile(ta, oa, va);
    if (!more) return;
    u = un;
    for (;;) {
        un = u + stride;
        more = un < total && un > u;
        ta = origin(more ? un : u, more);
        offsets(ta.r, oa);
        load_tile(ta, oa, va);
        store_tile(tb, ob, vb);
        if (!more) break;
        u = un;

        un = u + stride;
        more = un < total && un > u;
        tb = origin(more ? un : u, more);
        offsets(tb.r, ob);
        load_tile(tb, ob, vb);
        store_tile(ta, oa, va);
        if (!more) break;
        u = un;
    }
}

using CopyFn = void (*)(CopyKernelArgs);

// ---- all-gather instantiations: VEC x W x VPT, destination groups G for
// 16- and 8-byte vectors (G < W)
// (the partitioned schedule: W = 1, G = 0, PART)
template <int VEC, int W, int VPT>
CopyFn pick_group(int g, bool part, bool wide)
{
    if (part) {
        if constexpr (W == 1)
            if (g == 0) return wide ? ag_copy_kernel<VEC, 1, VPT, 0, true, true> : ag_copy_kernel<VEC, 1, VPT, 0, true, false>;
        return nullptr;
    }
    if (g == 0) return wide ? ag_copy_kernel<VEC, W, VPT, 0, false, true> : ag_copy_kernel<VEC, W, VPT, 0, false, false>;
    if constexpr (VEC >= 8) {
        if constexpr (W > 1) if (g == 1) return ag_copy_kernel<VEC, W, VPT, 1, false, false>;
        if constexpr (W > 2) if (g == 2) return ag_copy_kernel<VEC, W, VPT, 2, false, false>;
        if constexpr (W > 4) if (g == 4) return ag_copy_kernel<VEC, W, VPT, 4, false, false>;
    }
    return nullptr;
}

template <int VEC, int W>
CopyFn pick_vpt(int vpt, int g, bool part, bool wide)
{
    switch (vpt) {
    case 1: return pick_group<VEC, W, 1>(g, part, wide);
    case 2: return pick_group<VEC, W, 2>(g, part, wide);
    case 4: return pick_group<VEC, W, 4>(g, part, wide);
    case 8: return pick_group<VEC, W, 8>(g, part, wide);
    default: return nullptr;
    }
}

template <int VEC>
CopyFn pick_world(int w, int vpt, int g, bool part, bool wide)
{
    switch (w) {
    case 1: return pick_vpt<VEC, 1>(vpt, g, part, wide);
    case 2: return pick_vpt<VEC, 2>(vpt, g, part, wide);
    case 3: return pick_vpt<VEC, 3>(vpt, g, part, wide);
    case 4: return pick_vpt<VEC, 4>(vpt, g, part, wide);
    case 5: return pick_vpt<VEC, 5>(vpt, g, part, wide);
    case 6: return pick_vpt<VEC, 6>(vpt, g, part, wide);
    case 7: return pick_vpt<VEC, 7>(vpt, g, part, wide);
    case 8: return pick_vpt<VEC, 8>(vpt, g, part, wide);
    default: return nullptr;
    }
}

// ---- all-to-all instantiations: VEC x W x VPT, 1 to 8 vectors per thread
// and chunk tile (two register sets of one tile each stay live)
template <int VEC, int W>
CopyFn pick_a2a_vpt(int vpt, bool wide)
{
    switch (vpt) {
    case 1: return wide ? ag_a2a_kernel<VEC, W, 1, true> : ag_a2a_kernel<VEC, W, 1, false>;
    case 2: return wide ? ag_a2a_kernel<VEC, W, 2, true> : ag_a2a_kernel<VEC, W, 2, false>;
    case 4: return wide ? ag_a2a_kernel<VEC, W, 4, true> : ag_a2a_kernel<VEC, W, 4, false>;
    case 8: return wide ? ag_a2a_kernel<VEC, W, 8, true> : ag_a2a_kernel<VEC, W, 8, false>;
    default: return nullptr;
    }
}

template <int VEC>
CopyFn pick_a2a_world(int w, int vpt, bool wide)
{
    switch (w) {
    case 1: return pick_a2a_vpt<VEC, 1>(vpt, wide);
    case 2: return pick_a2a_vpt<VEC, 2>(vpt, wide);
    case 3: return pick_a2a_vpt<VEC, 3>(vpt, wide);
    case 4: return pick_a2a_vpt<VEC, 4>(vpt, wide);
    case 5: return pick_a2a_vpt<VEC, 5>(vpt, wide);
    case 6: return pick_a2a_vpt<VEC, 6>(vpt, wide);
    case 7: return pick_a2a_vpt<VEC, 7>(vpt, wide);
    case 8: return pick_a2a_vpt<VEC, 8>(vpt, wide);
    default: return nullptr;
    }
}

// ---- ticket-order all-gather instantiations: 16-byte vectors, W = 1..8, one or two vectors per
// thread per tile, 4, 8 or 16 tiles per ticket, and 3 (one vector) or 2 (two) for full-chip launches
// (WIDE, DRAIN): WIDE from half the CUs; DRAIN from three quarters of the CUs' worth of vectors
// (programs x vectors per thread), with either store policy
template <int W, int VPT, int G>
CopyFn pick_ticket_policy(bool wide, bool drain)
{
    if (drain) return wide ? ag_copy_ticket_kernel<16, W, VPT, G, true, true> : ag_copy_ticket_kernel<16, W, VPT, G, false, true>;
    return wide ? ag_copy_ticket_kernel<16, W, VPT, G, true, false> : ag_copy_ticket_kernel<16, W, VPT, G, false, false>;
}

template <int W, int VPT>
CopyFn pick_ticket_g(int ticket, bool wide, bool drain)
{
    switch (ticket) {
    case 2:
        if constexpr (VPT == 2) return pick_ticket_policy<W, VPT, 2>(wide, drain);
        return nullptr;
    case 3:
        if constexpr (VPT == 1) return pick_ticket_policy<W, VPT, 3>(wide, drain);
        return nullptr;
    case 4: return pick_ticket_policy<W, VPT, 4>(wide, drain);
    case 8: return pick_ticket_policy<W, VPT, 8>(wide, drain);
    case 16:
        if constexpr (VPT == 1) return pick_ticket_policy<W, VPT, 16>(wide, drain);
        return nullptr;
    default: return nullptr;
    }
}

template <int W>
CopyFn pick_ticket_vpt(int vpt, int ticket, bool wide, bool drain)
{
    switch (vpt) {
    case 1: return pick_ticket_g<W, 1>(ticket, wide, drain);
    case 2: return ticket <= 8 ? pick_ticket_g<W, 2>(ticket, wide, drain) : nullptr;   // at most 16 vectors per batch
    default: return nullptr;
    }
}

CopyFn pick_ticket(int vec, int w, int vpt, int ticket, bool wide, bool drain)
{
    if (vec != 16) return nullptr;
    switch (w) {
    case 1: return pick_ticket_vpt<1>(vpt, ticket, wide, drain);
    case 2: return pick_ticket_vpt<2>(vpt, ticket, wide, drain);
    case 3: return pick_ticket_vpt<3>(vpt, ticket, wide, drain);
    case 4: return pick_ticket_vpt<4>(vpt, ticket, wide, drain);
    case 5: return pick_ticket_vpt<5>(vpt, ticket, wide, drain);
    case 6: return pick_ticket_vpt<6>(vpt, ticket, wide, drain);
    case 7: return pick_ticket_vpt<7>(vpt, ticket, wide, drain);
    case 8: return pick_ticket_vpt<8>(vpt, ticket, wide, drain);
    default: return nullptr;
    }
}

// ---- ticket-order all-to-all instantiations: 16-byte vectors, W = 1..8; a tile moves its bytes twice
// (one read, one write), so the planner's 96 KiB per ticket is 16 tiles of one vector per thread and 8
// of two, whatever the launch
template <int W, int VPT, int G>
CopyFn pick_a2a_ticket_policy(bool wide, bool drain)
{
    if (drain) return wide ? ag_a2a_ticket_kernel<W, VPT, G, true, true> : ag_a2a_ticket_kernel<W, VPT, G, false, true>;
    return wide ? ag_a2a_ticket_kernel<W, VPT, G, true, false> : ag_a2a_ticket_kernel<W, VPT, G, false, false>;
}

template <int W>
CopyFn pick_a2a_ticket_vpt(int vpt, int ticket, bool wide, bool drain)
{
    if (vpt == 1 && ticket == 16) return pick_a2a_ticket_policy<W, 1, 16>(wide, drain);
    if (vpt == 2 && ticket == 8) return pick_a2a_ticket_policy<W, 2, 8>(wide, drain);
    return nullptr;
}

CopyFn pick_a2a_ticket(int vec, int w, int vpt, int ticket, bool wide, bool drain)
{
    if (vec != 16) return nullptr;
    switch (w) {
    case 1: return pick_a2a_ticket_vpt<1>(vpt, ticket, wide, drain);
    case 2: return pick_a2a_ticket_vpt<2>(vpt, ticket, wide, drain);
    case 3: return pick_a2a_ticket_vpt<3>(vpt, ticket, wide, drain);
    case 4: return pick_a2a_ticket_vpt<4>(vpt, ticket, wide, drain);
    case 5: return pick_a2a_ticket_vpt<5>(vpt, ticket, wide, drain);
    case 6: return pick_a2a_ticket_vpt<6>(vpt, ticket, wide, drain);
    case 7: return pick_a2a_ticket_vpt<7>(vpt, ticket, wide, drain);
    case 8: return pick_a2a_ticket_vpt<8>(vpt, ticket, wide, drain);
    default: return nullptr;
    }
}

CopyFn pick_kernel(int kind, int vec, int w, int g, int vpt, bool part, bool wide)
{
    // the partitioned all-to-all runs the partitioned copy kernel (one destination per program)
    if (kind == kCopyAllToAll && !part) {
        if (g != 0) return nullptr;
        switch (vec) {
        case 16: return pick_a2a_world<16>(w, vpt, wide);
        case 8: return pick_a2a_world<8>(w, vpt, wide);
        case 4: return pick_a2a_world<4>(w, vpt, wide);
        case 2: return pick_a2a_world<2>(w, vpt, wide);
        default: return nullptr;
        }
    }
    switch (vec) {
    case 16: return pick_world<16>(w, vpt, g, part, wide);
    case 8: return pick_world<8>(w, vpt, g, part, wide);
    case 4: return pick_world<4>(w, vpt, g, part, wide);
    case 2: return pick_world<2>(w, vpt, g, part, wide);
    default: return nullptr;
    }
}

}  // namespace

bool copy_supported(int kind, int vec_bytes, int dests, int group, int vpt, bool partitioned)
{
    return pick_kernel(kind, vec_bytes, dests, group, vpt, partitioned, false) != nullptr;
}

bool copy_ticket_supported(int kind, int vec_bytes, int dests, int vpt, int ticket)
{
    if (kind == kCopyAllToAll) return pick_a2a_ticket(vec_bytes, dests, vpt, ticket, false, false) != nullptr;
    return pick_ticket(vec_bytes, dests, vpt, ticket, false, false) != nullptr;
}

// ---- tile counters of the allocation-free entry point: a fixed device array, one 64-byte block
// (16 words, two used) per rank index, zero-initialised when the code object is loaded.  Host code
// reaches it only through the address hipGetSymbolAddress reports for the current device (the
// array's name is a host-side stand-in, not a device address).
static __device__ __align__(256) uint32_t scratch[kNoAllocMaxRanks * 16];

namespace {
constexpr int kNoAllocMaxDevices = 64;

// Zeroes one rank's counter pair at the start of a call (a kernel, not a memset: the call may be
// captured into a graph, and replays must clear it too).
__global__ __launch_bounds__(64) void clear_tickets_kernel(uint32_t* counter)
{
    if (threadIdx.x < 2) counter[threadIdx.x] = 0u;
}
}  // namespace

hipError_t noalloc_tickets(int rank, hipStream_t stream, uint32_t** out)
{
    if (rank < 0 || rank >= kNoAllocMaxRanks) return hipErrorInvalidValue;
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kNoAllocMaxDevices) return hipErrorInvalidDevice;
    static std::mutex mu;
    static uint32_t* base[kNoAllocMaxDevices] = {};
    uint32_t* b = nullptr;
    {
        std::lock_guard<std::mutex> lock(mu);
        if (base[dev] == nullptr) {   // once per device, with that device current
            void* p = nullptr;
            e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (e != hipSuccess) return e;
            if (p == nullptr) return hipErrorInvalidSymbol;
            base[dev] = static_cast<uint32_t*>(p);
        }
        b = base[dev];
    }
    uint32_t* counter = b + 16 * static_cast<size_t>(rank);
    hipLaunchKernelGGL(clear_tickets_kernel, dim3(1), dim3(64), 0, stream, counter);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    *out = counter;
    return hipSuccess;
}

hipError_t launch_copy(const CopyLaunch& l, hipStream_t stream)
{
    if (l.ticket != 0) {
        CopyFn fn = nullptr;
        if (l.group == 0 && !l.args.partitioned && l.args.slices == 1) {
            if (l.kind == kCopyAllGather) fn = pick_ticket(l.vec_bytes, l.dests, l.vpt, l.ticket, l.wide != 0, l.drain != 0);
            if (l.kind == kCopyAllToAll)
                fn = pick_a2a_ticket(l.vec_bytes, l.dests, l.vpt, l.ticket, l.wide != 0, l.drain != 0);
        }
        if (fn == nullptr || l.grid < 1 || l.args.tickets == nullptr) return hipErrorInvalidValue;
        hipLaunchKernelGGL(fn, dim3(l.grid), dim3(256), 0, stream, l.args);
        return hipGetLastError();
    }
    CopyFn fn = pick_kernel(l.kind, l.vec_bytes, l.dests, l.group, l.vpt, l.args.partitioned != 0, l.wide != 0);
    const uint32_t max_slices = l.kind == kCopyAllToAll ? 1 : 4;
    if (fn == nullptr || l.args.slices < 1 || l.args.slices > max_slices || l.grid < 1 || l.args.world < 1)
        return hipErrorInvalidValue;
    if (l.args.partitioned && (l.args.slices != 1 || l.dests != 1 || l.grid % l.args.world != 0))
        return hipErrorInvalidValue;
    hipLaunchKernelGGL(fn, dim3(l.grid), dim3(256 * l.args.slices), 0, stream, l.args);
    return hipGetLastError();
}

}  // namespace ag
