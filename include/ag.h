/*
 * ag.h -- C ABI of libag: a symmetric heap of logical ranks on one MI355X
 * (gfx950), a persistent tiled multi-destination all-gather, and a tiled
 * GEMM whose epilogue performs the same multi-destination store.
 *
 * Sources (the three pages on the iris all-gather):
 *  - ROCm/iris #626, "Summary": the device-side all-gather loads the local
 *    and every peer heap base once, before the first store, keeps each peer
 *    as a pointer delta (peer_base - local_base), stores the local copy
 *    first and then the peers in rotated order (rank+1, rank+2, ...).
 *  - ROCm/iris #626, "Triton CCL all-gather": the persistent kernel walks
 *    tiles with a grid stride and translates the output base once per peer
 *    before the tile loop.
 *  - ROCm/iris #626, "Assembly" table: the fused matmul + all-gather kernel
 *    stores its 256x256 fp16 C tile to every rank, with the heap-base loads
 *    hoisted above the K loop.
 *  - ROCm/iris #594, "Multi-GPU CI" / "Local validation": the result is that
 *    of torch.distributed.all_gather_into_tensor; logical ranks may be
 *    independent regions of memory on one GPU.
 *  - ROCm/iris #591, "Hoist the peer heap bases": groups are described by
 *    (rank_start, rank_stride, world_size); heap_bases is a device array of
 *    every rank's heap base.
 *
 * Conventions shared by every entry point
 *  - All pointers named dev_* or passed as input/A/B are device addresses in
 *    the current HIP device's memory; host pointers are named out/plan/etc.
 *  - Every entry point returns ag_status_t.  On any status other than AG_OK
 *    nothing was launched and no output argument was written, and
 *    ag_last_error_message() gives a one-line reason (thread-local).
 *  - Launching entry points are asynchronous and ordered on the given
 *    hipStream_t (NULL = the null stream).  They never synchronise.  A launch
 *    failure reported by the runtime returns AG_ERR_HIP.  They launch on the
 *    current HIP device, which must be the device the heap was created or
 *    wrapped on (AG_ERR_INVALID_ARG otherwise).
 *  - Argument validation is done on the host before any HIP call; values are
 *    never remapped: 0 means "documented default", anything else is used as
 *    given or rejected.
 */
#ifndef AG_H
#define AG_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum ag_status {
    AG_OK = 0,
    AG_ERR_INVALID_ARG = 1,   /* an argument is out of range, misaligned, null or overlapping */
    AG_ERR_UNSUPPORTED = 2,   /* valid request this library does not implement (e.g. W > 8) */
    AG_ERR_OUT_OF_MEMORY = 3, /* device allocation failed or the symmetric heap is exhausted */
    AG_ERR_HIP = 4            /* a HIP runtime call failed (no device, launch error, ...) */
} ag_status_t;

typedef enum ag_dtype {
    AG_F16 = 0,   /* IEEE binary16, 2 bytes */
    AG_BF16 = 1,  /* bfloat16, 2 bytes */
    AG_F32 = 2    /* IEEE binary32, 4 bytes (the copies only, not the GEMM) */
} ag_dtype_t;

/* Largest group the kernels are instantiated for (destination loop is a static unroll). */
#define AG_MAX_WORLD 8
/* Alignment (and unit) of every region stride created by ag_heap_create. */
#define AG_REGION_ALIGN ((size_t)2 << 20)

typedef struct ag_heap ag_heap_t;  /* opaque */

/* Where a heap lives; filled by ag_heap_geometry, or by hand for planning only. */
typedef struct ag_heap_geometry {
    uint64_t slab_addr;       /* device address of region 0 (region r = slab_addr + r*bytes_per_rank) */
    uint64_t bytes_per_rank;  /* region stride in bytes, a multiple of 256 */
    int32_t n_ranks;          /* number of regions, >= 1 */
    int32_t rank;             /* calling rank of a view, or -1 for the root handle */
    int32_t num_cus;          /* compute units of the heap's device (default n_programs) */
    int32_t reserved;         /* must be 0 */
} ag_heap_geometry_t;

/* What a call will launch: filled by the ag_plan_* functions (pure host logic). */
typedef struct ag_plan {
    int32_t group_rank;          /* g = (rank - rank_start) / rank_stride */
    int32_t vec_bytes;           /* bytes per vector access of the copy kernel (16/8/4/2) */
    int32_t tile_m, tile_n, tile_k; /* effective tile (tile_k = 0 for the all-gather) */
    int32_t n_programs;          /* persistent workgroups launched */
    int32_t threads;             /* threads per workgroup */
    int32_t lds_bytes;           /* LDS per workgroup */
    int32_t vectors_per_thread;  /* copy kernel: vector accesses per thread per tile */
    int32_t variant;             /* library-internal kernel variant (informational) */
    int64_t tiles_m, tiles_n, total_tiles;
    uint64_t rank_block_offset;  /* byte offset of this rank's rows inside every region (out_offset + g*M_local*N*e) */
    uint64_t bytes_read;         /* algorithmic bytes read per call */
    uint64_t bytes_written;      /* algorithmic bytes written per call (W destinations) */
    double flops;                /* 2*M_local*N*K for the GEMM, 0 for the all-gather */
    int32_t dest_group;          /* copy kernels: destinations stored per wait (0 = all of them, no wait) */
    int32_t schedule;            /* copy kernels: ag_schedule_t of the launch */
    int32_t tile_order;          /* copy kernels: ag_tile_order_t applied (AG_ORDER_STRIDE or AG_ORDER_TICKETS) */
    int32_t tiles_per_ticket;    /* copy kernels with AG_ORDER_TICKETS: consecutive tiles per ticket (else 0) */
    int32_t ticket_wait;         /* AG_ORDER_TICKETS on wide launches: 1 when each program takes its next
                                    ticket after the stores of the batch in hand (its first wave waits for
                                    its own stores to complete, and the barrier that hands the ticket out
                                    holds the other waves until then), 0 when it takes it before them */
    int32_t reserved_plan;       /* 0 */
} ag_plan_t;

/* Tile schedules of the all-gather (ag_all_gather_ex) and the all-to-all (ag_all_to_all_ex). */
typedef enum ag_schedule {
    AG_SCHEDULE_TILES = 0,       /* each program walks tiles and stores every tile to all W destinations
                                    (the all-to-all: each chunk tile to its one destination) */
    AG_SCHEDULE_PARTITIONED = 1  /* each program owns one destination and walks the tiles for it alone */
} ag_schedule_t;

/* Order in which the persistent programs of AG_SCHEDULE_TILES take their tiles (the all-to-all's
 * tiles: the W chunk copies as one sequence, destination by destination).  The result does not
 * depend on it. */
typedef enum ag_tile_order {
    AG_ORDER_AUTO = 0,     /* the library's choice: AG_ORDER_TICKETS where a ticket kernel exists and,
                              for the all-gather, the call has at least 64 tiles per program; for the
                              all-to-all, at least 64 tiles per program and vector per thread with
                              programs x vectors per thread below twice the CU count.
                              AG_ORDER_STRIDE otherwise */
    AG_ORDER_STRIDE = 1,   /* fixed grid stride: program p takes tiles p, p + P, p + 2P, ... */
    AG_ORDER_TICKETS = 2   /* programs take G consecutive tiles at a time from a device counter of the
                              calling rank, in increasing tile order; 16-byte vectors, one or two per
                              thread and tile, no destination groups, every tile row of the block below
                              2 GiB.  G is one of 3, 4, 8, 16 (one vector per thread) or 2, 4, 8 (two):
                              the smallest whose tiles move at least 96 KiB of HBM traffic (the
                              all-gather's read once and written W times, the all-to-all's read and
                              written once; the largest where none does), and on launches with fewer
                              programs than CUs at least the largest of 16, 8 and 4 (within those
                              sizes) with G x programs <= 1024.  When programs x vectors per thread
                              reach three quarters of the CU count, each program takes its next ticket
                              after the stores of the batch in hand (plan.ticket_wait) */
} ag_tile_order_t;

/* Options of ag_all_gather_ex and ag_all_to_all_ex; all-zero (or a NULL pointer) is the plain call. */
typedef struct ag_copy_options {
    int32_t dest_group;   /* 0: one straight run of W destination stores per tile (default).
                             1, 2 or 4 (< W): store that many destinations, then wait until the
                             stores before them have completed, then the next group */
    int32_t schedule;     /* ag_schedule_t */
    int32_t tile_order;   /* ag_tile_order_t (AG_SCHEDULE_TILES only; else 0) */
    int32_t reserved[5];  /* must be 0 */
} ag_copy_options_t;

/* ------------------------------------------------------------------------
 * Symmetric heap (ROCm/iris #626 "Summary" and #591: one heap per rank,
 * tensors at the same offset in every heap, kernels read the device array
 * heap_bases).  Here the n_ranks heaps are disjoint regions of one device
 * allocation (ROCm/iris #594 "Local validation": logical ranks as separate
 * memory on one GPU), and heap_bases[r] = slab + r*bytes_per_rank lives in
 * a separate device array of n_ranks uint64_t.
 * ------------------------------------------------------------------------ */

/* The region stride ag_heap_create uses for bytes_per_rank (ROCm/iris #594
 * "Local validation": logical ranks as separate memory of one GPU; how the
 * regions sit in HBM is this library's choice).  bytes_per_rank rounded up
 * to AG_REGION_ALIGN, plus one AG_REGION_ALIGN when the result is a power of
 * two of 512 MiB or more: the W copies of a tile are stored at the same
 * offset of W regions at once, and strides of a large power of two alias
 * them in the HBM channel interleave (W=8, 16384x8192 fp16 per rank: 349-354
 * against 354-360 us per call).  Callers of ag_heap_wrap can lay out their
 * slab the same way.  Host-only.  AG_ERR_INVALID_ARG when region_bytes is
 * NULL or bytes_per_rank is 0 or above 1 TiB. */
ag_status_t ag_heap_region_bytes(size_t bytes_per_rank, size_t* region_bytes);

/* Allocate a slab of n_ranks regions of bytes_per_rank bytes (the region
 * stride is ag_heap_region_bytes(bytes_per_rank)) plus the device base
 * table, on the current device.  The
 * heap owns both.  n_ranks in [1, 1024], bytes_per_rank >= 1.  Contents of
 * the slab are undefined.  AG_ERR_OUT_OF_MEMORY if hipMalloc fails,
 * AG_ERR_HIP if no device is usable. */
ag_status_t ag_heap_create(int n_ranks, size_t bytes_per_rank, ag_heap_t** out);

/* Build a heap over caller-owned device memory of n_ranks*bytes_per_rank
 * bytes (e.g. a torch uint8 tensor).  dev_slab must be 256-byte aligned and
 * bytes_per_rank a non-zero multiple of 256.  dev_slab must be device (or
 * managed) memory of the current device, and its allocation must hold the
 * n_ranks*bytes_per_rank bytes from dev_slab on (AG_ERR_INVALID_ARG
 * otherwise: checked with hipPointerGetAttributes and, where the runtime
 * reports the allocation's extent, hipMemGetAddressRange).
 * The library allocates and owns only the base table; the caller keeps the
 * slab alive until every handle on it is destroyed. */
ag_status_t ag_heap_wrap(void* dev_slab, int n_ranks, size_t bytes_per_rank, ag_heap_t** out);

/* A handle for one calling rank ("the caller's rank", as the context object
 * of iris knows its rank).  Views share the slab, the table and the
 * allocator of the heap; the shared state lives until the last handle is
 * destroyed. */
ag_status_t ag_heap_view(const ag_heap_t* heap, int rank, ag_heap_t** view);

/* Release a handle.  The caller must have synchronised every stream that
 * uses the heap.  NULL is accepted and ignored. */
ag_status_t ag_heap_destroy(ag_heap_t* heap);

/* Symmetric bump allocation: returns a byte offset valid in every region.
 * align must be a power of two >= 256 (0 = 256).  AG_ERR_OUT_OF_MEMORY when
 * the region is exhausted.  Host-only; thread-safe per heap. */
ag_status_t ag_heap_alloc(ag_heap_t* heap, size_t bytes, size_t align, size_t* offset);

/* Forget every allocation (offsets restart at 0). */
ag_status_t ag_heap_reset(ag_heap_t* heap);

/* Zero every rank's tile counters (the ticket order's; see ag_all_gather) with a small kernel on stream
 * (hipStream_t; no memset, so the call can be captured in a graph).  The counters are zero between calls
 * and need no clearing in correct use; this restores them after calls of one rank overlapped in time,
 * which the all-gather and the all-to-all do not allow and which can leave a counter non-zero for the
 * rank's later calls.
 * Stream-ordered; no call of this heap may run concurrently with it. */
ag_status_t ag_heap_clear_tickets(const ag_heap_t* heap, void* stream);

/* Device address of offset in region rank.  offset <= bytes_per_rank. */
ag_status_t ag_heap_rank_ptr(const ag_heap_t* heap, int rank, size_t offset, void** dev_ptr);

/* Device address of the uint64_t[n_ranks] base table the kernels read. */
ag_status_t ag_heap_base_table(const ag_heap_t* heap, const uint64_t** dev_table);

/* Geometry of a handle (host copy, no device access). */
ag_status_t ag_heap_geometry(const ag_heap_t* heap, ag_heap_geometry_t* geom);

/* What a device kernel needs to reach every rank's heap (ROCm/iris #591,
 * "Hoist the peer heap bases": the context knows its rank and keeps the
 * heap bases of all ranks in one device array, heap_bases, which the kernels
 * read).  Host-only, no device access:
 *   *n_ranks         number of regions (ranks) of the heap;
 *   *rank            the calling rank of a view (ag_heap_view), -1 for the
 *                    root handle;
 *   *bytes_per_rank  region stride in bytes (region r starts at
 *                    heap_bases[r] = region 0 + r*bytes_per_rank);
 *   *dev_base_table  device address of heap_bases, uint64_t[n_ranks], owned
 *                    by the heap (valid until its last handle is destroyed;
 *                    the caller must not write or free it).
 * Each output pointer may be NULL, and that item is then not reported.
 * AG_ERR_INVALID_ARG when heap is NULL.  The same values as
 * ag_heap_geometry (n_ranks, rank, bytes_per_rank) and ag_heap_base_table. */
ag_status_t ag_heap_info(const ag_heap_t* heap, int* n_ranks, int* rank, size_t* bytes_per_rank,
                         const uint64_t** dev_base_table);

/* ------------------------------------------------------------------------
 * All-gather (ROCm/iris #626 "Summary" and "Triton CCL all-gather"; result
 * defined by ROCm/iris #594 "Multi-GPU CI").
 *
 * heap          a view (ag_heap_view) of the calling rank
 * W             group size, 1..AG_MAX_WORLD
 * rank_start,
 * rank_stride   group members are regions rank_start + j*rank_stride, j < W;
 *               the view's rank must be one of them; g is its group index
 * input         device pointer to M_local x N elements, row-major, ld = N
 * out_offset    byte offset (multiple of the element size) of the gathered
 *               W*M_local x N output inside every member region
 * tile_m,tile_n tile of the persistent loop; 0,0 = 8x256.  Powers of two with
 *               tile_n in [8, 4096], tile_m in [1, 256]; one tile must hold
 *               between 1 and 8 vector accesses per thread of a 256-thread
 *               workgroup at the vector width chosen (AG_ERR_UNSUPPORTED
 *               otherwise)
 * n_programs    persistent workgroups; 0 = number of CUs
 * stream        hipStream_t
 *
 * After the call completes on stream, rows [g*M_local, (g+1)*M_local) of the
 * output in every member region hold input; no other byte of the slab
 * changes.  The input tile is read once and stored to the local region
 * first, then to the peers in rotated group order (g+1, g+2, ... mod W).
 * Calls for different ranks of a group write disjoint rows and may run
 * concurrently on different streams.  Calls for the same rank must not
 * overlap in time (order them on one stream): a call in ticket order
 * (AG_ORDER_TICKETS, the library's choice for long calls) takes its tiles
 * from a counter the heap keeps for each rank, zero between calls; calls of
 * one rank that overlap give undefined output and may leave the counter
 * non-zero for that rank's later calls (ag_heap_clear_tickets restores it).
 * M_local = 0 is a no-op.  input must not overlap any member's output
 * block, except that it may be exactly this rank's own rows in its own
 * region (in-place).
 * ------------------------------------------------------------------------ */
ag_status_t ag_all_gather(const ag_heap_t* heap, int W, int rank_start, int rank_stride,
                          const void* input, size_t out_offset, int64_t M_local, int64_t N,
                          ag_dtype_t dtype, int tile_m, int tile_n, int n_programs, void* stream);

/* The validation and launch decisions of ag_all_gather for a heap
 * geometry, without touching any device (input_addr is the device address
 * as an integer).  Returns the status ag_all_gather would return before
 * launching; fills *plan on AG_OK. */
ag_status_t ag_plan_all_gather(const ag_heap_geometry_t* geom, int W, int rank_start, int rank_stride,
                               uint64_t input_addr, size_t out_offset, int64_t M_local, int64_t N,
                               ag_dtype_t dtype, int tile_m, int tile_n, int n_programs, ag_plan_t* plan);

/* ------------------------------------------------------------------------
 * All-gather variants (ROCm/iris #594, "Reviewer performance evaluation"
 * and "Compiler inspection and grouping"; ROCm/iris #591, "INLINE
 * grouping"; ROCm/iris #626, "Triton CCL all-gather").  Same arguments,
 * result and errors as ag_all_gather, plus:
 *
 * options->dest_group  peers stored per wait.  The pages leave open whether
 *               keeping every destination's stores in flight at once costs
 *               link efficiency; grouping stores G destinations, then waits
 *               for the memory counter to retire everything before them.
 *               Supported: 0 (no grouping), and 1, 2 or 4 when it is below
 *               W and the vector width is 16 or 8 bytes (AG_ERR_UNSUPPORTED
 *               otherwise).  G >= W is the same as 0.
 * options->schedule    AG_SCHEDULE_PARTITIONED: the persistent programs are
 *               split into W equal sets, set i storing only to destination
 *               i of the rotated order (i = 0 is the local region); each
 *               program walks its set's share of the tiles, so every input
 *               tile is read W times (once per destination).  n_programs is
 *               rounded down to a multiple of W (at least W); dest_group
 *               must be 0.
 * options->tile_order  ag_tile_order_t, for AG_SCHEDULE_TILES without
 *               destination groups: AG_ORDER_STRIDE or AG_ORDER_TICKETS force
 *               the order (AG_ERR_UNSUPPORTED where no ticket kernel fits the
 *               call: vectors other than 16 bytes or more than two per thread,
 *               destination groups).  Ticket order at 256 programs, W=8,
 *               16384x8192 fp16: 6.77 TB/s against 5.28 for the grid stride;
 *               below about 64 tiles per program the counter's round trips
 *               cost more than they save.
 * Plan: ag_plan_all_gather_ex reports dest_group, schedule and tile_order as
 * applied, and bytes_read of the schedule (W times the input when
 * partitioned).
 * ------------------------------------------------------------------------ */
ag_status_t ag_all_gather_ex(const ag_heap_t* heap, int W, int rank_start, int rank_stride,
                             const void* input, size_t out_offset, int64_t M_local, int64_t N,
                             ag_dtype_t dtype, int tile_m, int tile_n, int n_programs,
                             const ag_copy_options_t* options, void* stream);

ag_status_t ag_plan_all_gather_ex(const ag_heap_geometry_t* geom, int W, int rank_start, int rank_stride,
                                  uint64_t input_addr, size_t out_offset, int64_t M_local, int64_t N,
                                  ag_dtype_t dtype, int tile_m, int tile_n, int n_programs,
                                  const ag_copy_options_t* options, ag_plan_t* plan);

/* ------------------------------------------------------------------------
 * ag_all_gather_ex for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  Same arguments, result, errors and kernels as
 * ag_all_gather_ex; it calls no allocating routine.  The only device memory
 * it uses beyond the input and the heap is the ticket order's tile counter,
 * which here lives in a fixed device array of the library (one counter per
 * rank index, AG_NOALLOC_MAX_RANKS of them, 4 KiB per GPU, held until the
 * process ends) instead of in the heap; each call first zeroes the calling
 * rank's counter with a small kernel on stream.  Heaps of more than
 * AG_NOALLOC_MAX_RANKS ranks give AG_ERR_UNSUPPORTED.  Every call on a GPU
 * shares that GPU's array: calls that overlap in time and use the same
 * rank index race, whichever heaps they use.
 * ------------------------------------------------------------------------ */
#define AG_NOALLOC_MAX_RANKS 64
ag_status_t ag_all_gather_noalloc(const ag_heap_t* heap, int W, int rank_start, int rank_stride,
                                  const void* input, size_t out_offset, int64_t M_local, int64_t N,
                                  ag_dtype_t dtype, int tile_m, int tile_n, int n_programs,
                                  const ag_copy_options_t* options, void* stream);

/* ------------------------------------------------------------------------
 * All-to-all on the same heap and destination machinery (ROCm/iris #594,
 * "Compiler inspection and grouping", and ROCm/iris #591, "Hoist the peer
 * heap bases": the all_to_all collective has the same per-destination
 * heap-base pattern).  The result is that of
 * torch.distributed.all_to_all_single with equal splits:
 *
 * input         device, W chunks of M_chunk x N elements, row-major (ld = N),
 *               chunk c at input + c*M_chunk*N*e; chunk c is destined for
 *               group member c
 * out_offset    byte offset (multiple of the element size) of the W*M_chunk x N
 *               output inside every member region
 * After the call completes, rows [g*M_chunk, (g+1)*M_chunk) of member j's
 * output hold chunk j of this rank's input; no other byte of the slab
 * changes.  Every destination base is translated once before the tile loop.
 * The W chunk copies are walked as one sequence of W x (tiles per chunk)
 * tiles, destination by destination: the local region first, then the peers
 * in rotated order; each tile is loaded once and stored once.  Tiles as for
 * ag_all_gather (0,0 = 8x256): 1 to 8 vectors per thread of a 256-thread
 * workgroup (AG_ERR_UNSUPPORTED otherwise; 8x256 always fits); W x tiles per
 * chunk below 2^31.  Calls for different ranks may run concurrently on
 * different streams; calls for the same rank must not overlap in time (a
 * call in ticket order uses the rank's counter, as ag_all_gather does).
 * M_chunk = 0 is a no-op.  input must not overlap any member's output
 * block.
 * ------------------------------------------------------------------------ */
ag_status_t ag_all_to_all(const ag_heap_t* heap, int W, int rank_start, int rank_stride,
                          const void* input, size_t out_offset, int64_t M_chunk, int64_t N,
                          ag_dtype_t dtype, int tile_m, int tile_n, int n_programs, void* stream);

ag_status_t ag_plan_all_to_all(const ag_heap_geometry_t* geom, int W, int rank_start, int rank_stride,
                               uint64_t input_addr, size_t out_offset, int64_t M_chunk, int64_t N,
                               ag_dtype_t dtype, int tile_m, int tile_n, int n_programs, ag_plan_t* plan);

/* ag_all_to_all with options (NULL or all-zero = ag_all_to_all).  Same
 * result.  dest_group must be 0 (AG_ERR_INVALID_ARG otherwise).  tile_order
 * as for ag_all_gather_ex (AG_SCHEDULE_TILES only).  schedule
 * AG_SCHEDULE_PARTITIONED (the partitioned schedule of ag_all_gather_ex
 * applied to the exchange): program p owns destination i = p mod W of the
 * rotated order and copies chunk (g + i) mod W there, the programs of one
 * destination walking all tiles among themselves; every chunk is read once.
 * n_programs is rounded down to a multiple of W (at least W). */
ag_status_t ag_all_to_all_ex(const ag_heap_t* heap, int W, int rank_start, int rank_stride,
                             const void* input, size_t out_offset, int64_t M_chunk, int64_t N,
                             ag_dtype_t dtype, int tile_m, int tile_n, int n_programs,
                             const ag_copy_options_t* options, void* stream);

ag_status_t ag_plan_all_to_all_ex(const ag_heap_geometry_t* geom, int W, int rank_start, int rank_stride,
                                  uint64_t input_addr, size_t out_offset, int64_t M_chunk, int64_t N,
                                  ag_dtype_t dtype, int tile_m, int tile_n, int n_programs,
                                  const ag_copy_options_t* options, ag_plan_t* plan);

/* ------------------------------------------------------------------------
 * Fused GEMM + all-gather (ROCm/iris #626 "Assembly" table and "Benchmark").
 *
 * C = A . B with fp32 accumulation, rounded once (nearest-even) to dtype,
 * then stored exactly as ag_all_gather stores its input: rows
 * [g*M_local, (g+1)*M_local) of the W*M_local x N output at out_offset in
 * every member region, local region first, peers in rotated order.
 *
 * A             device, M_local x K, row-major, element (m,k) at A[m*lda + k], lda >= K
 * B             device, K-contiguous: element (k,n) at B[n*ldb + k], ldb >= K
 *               (the N x K row-major weight of a linear layer)
 * dtype         AG_F16 or AG_BF16 (A, B and C share it); AG_F32 -> AG_ERR_UNSUPPORTED
 * tile_m,tile_n,tile_k   0,0,0 = chosen by the library: the configuration
 *               with the fewest rounds-of-tiles x tile-area on the busiest
 *               program (ties to the larger tile); explicit values must be
 *               one of 256x256x64, 256x224x64, 128x128x64
 * n_programs    persistent workgroups; 0 = number of CUs (capped at the tile count)
 * Requirements: K a positive multiple of 64, lda/ldb multiples of 8, A, B
 * 16-byte aligned, N*2 and out_offset multiples of 16 bytes.  M_local and N
 * need not be tile multiples.  M_local = 0 is a no-op.  A and B must not
 * overlap any member's output block.
 * ------------------------------------------------------------------------ */
ag_status_t ag_gemm_all_gather(const ag_heap_t* heap, int W, int rank_start, int rank_stride,
                               const void* A, int64_t lda, const void* B, int64_t ldb,
                               size_t out_offset, int64_t M_local, int64_t N, int64_t K,
                               ag_dtype_t dtype, int tile_m, int tile_n, int tile_k,
                               int n_programs, void* stream);

/* Host-only validation and launch decisions of ag_gemm_all_gather. */
ag_status_t ag_plan_gemm_all_gather(const ag_heap_geometry_t* geom, int W, int rank_start, int rank_stride,
                                    uint64_t a_addr, int64_t lda, uint64_t b_addr, int64_t ldb,
                                    size_t out_offset, int64_t M_local, int64_t N, int64_t K,
                                    ag_dtype_t dtype, int tile_m, int tile_n, int tile_k,
                                    int n_programs, ag_plan_t* plan);

/* Storage of B for ag_gemm_all_gather_ex. */
typedef enum ag_b_layout {
    AG_B_K_CONTIGUOUS = 0,  /* element (k,n) at B[n*ldb + k], ldb >= K (as ag_gemm_all_gather) */
    AG_B_N_CONTIGUOUS = 1   /* element (k,n) at B[k*ldb + n], ldb >= N (a row-major K x N matrix) */
} ag_b_layout_t;

/* Options of ag_gemm_all_gather_ex; all-zero (or a NULL pointer) is ag_gemm_all_gather. */
typedef struct ag_gemm_options {
    int32_t b_layout;     /* ag_b_layout_t */
    int32_t reserved[7];  /* must be 0 */
} ag_gemm_options_t;

/* ag_gemm_all_gather with options: the same product and stores, with B in
 * either layout.  With AG_B_N_CONTIGUOUS, ldb >= N (multiple of 8), B
 * 16-byte aligned, and 64 rows of B plus a tile's columns
 * ((64*ldb + tile_n)*2 bytes) under 2 GiB (AG_ERR_UNSUPPORTED otherwise);
 * B itself may be larger.  The tiles are 256x224x64 or
 * 128x128x64 (0,0,0 chooses between them; 256x256x64 gives
 * AG_ERR_UNSUPPORTED).  The kernel reads the N-contiguous stage with LDS
 * transposing reads instead of a transpose pass. */
ag_status_t ag_gemm_all_gather_ex(const ag_heap_t* heap, int W, int rank_start, int rank_stride,
                                  const void* A, int64_t lda, const void* B, int64_t ldb,
                                  size_t out_offset, int64_t M_local, int64_t N, int64_t K,
                                  ag_dtype_t dtype, int tile_m, int tile_n, int tile_k,
                                  int n_programs, const ag_gemm_options_t* options, void* stream);

ag_status_t ag_plan_gemm_all_gather_ex(const ag_heap_geometry_t* geom, int W, int rank_start, int rank_stride,
                                       uint64_t a_addr, int64_t lda, uint64_t b_addr, int64_t ldb,
                                       size_t out_offset, int64_t M_local, int64_t N, int64_t K,
                                       ag_dtype_t dtype, int tile_m, int tile_n, int tile_k,
                                       int n_programs, const ag_gemm_options_t* options, ag_plan_t* plan);

/* ------------------------------------------------------------------------ */
const char* ag_status_string(ag_status_t status);  /* static string, never NULL */
const char* ag_last_error_message(void);           /* thread-local; "" after AG_OK */
const char* ag_version(void);                      /* static string */

#ifdef __cplusplus
}
#endif

#endif /* AG_H */
