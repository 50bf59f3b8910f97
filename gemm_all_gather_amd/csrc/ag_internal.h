// Internal interface between the host runtime (ag_host.cpp) and the kernel
// launchers (ag_copy.hip, ag_gemm.hip).  Not part of the public C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ag {

// Arguments of the persistent multi-destination copy kernels (by value).
struct CopyKernelArgs {
    const uint64_t* heap_bases;   // device uint64_t[n_ranks]
    const uint8_t* input;         // rank's M x N block (all-to-all: W such chunks), row-major
    uint64_t rank_block_offset;   // out_offset + g*M*N*e, same in every region
    uint64_t row_bytes;           // N*e
    uint64_t chunk_bytes;         // all-to-all: M*N*e between consecutive input chunks (all-gather: 0)
    uint32_t rows;                // M (M_local, or M_chunk for the all-to-all)
    uint32_t tile_m;              // rows per tile
    uint32_t tile_row_bytes;      // tile_n*e
    uint32_t vecs_per_row_log2;   // log2(tile_row_bytes / vec_bytes)
    uint32_t tiles_n;             // ceil(N / tile_n)
    uint32_t total_tiles;
    int32_t rank;                 // calling rank (region index)
    int32_t rank_start;
    int32_t rank_stride;
    int32_t group_rank;           // g
    uint32_t slices;              // 256-thread slices per workgroup (blockDim.x / 256)
    uint32_t world;               // group size W
    uint32_t partitioned;         // 1: program p stores only to destination p % W (the partitioned kernel)
    uint32_t reserved;
    uint32_t* tickets;            // ticket order: device uint32_t[2] = {next tile, programs finished}, zero at
                                  // launch; the last program to finish sets both back to zero (else unused)
};

enum CopyKind { kCopyAllGather = 0, kCopyAllToAll = 1 };

struct CopyLaunch {
    CopyKernelArgs args;
    int kind;          // CopyKind
    int vec_bytes;     // 16, 8, 4, 2
    int dests;         // destinations each program stores a tile to (W, or 1 when partitioned)
    int group;         // destinations per wait (0 = no waits between destinations)
    int vpt;           // vector accesses per thread per tile
    int grid;          // workgroups
    int wide;          // 1: the store policy of launches on at least half the CUs (no destination groups)
    int ticket;        // tiles per ticket of the ticket order (0: grid-stride order)
    int drain;         // ticket order: take each ticket after the stores of the batch before it
};

// Whether the launcher has a kernel for (kind, vec, dests, group, vpt, schedule) (host-only).
bool copy_supported(int kind, int vec_bytes, int dests, int group, int vpt, bool partitioned);
// Whether the ticket-order kernel of kind (all-gather or all-to-all) exists for (vec, dests, vpt, tiles per
// ticket) (host-only).
bool copy_ticket_supported(int kind, int vec_bytes, int dests, int vpt, int ticket);
hipError_t launch_copy(const CopyLaunch& l, hipStream_t stream);

// Tile counters of ag_all_gather_noalloc: rank indices below kNoAllocMaxRanks have a counter pair in a
// fixed device array of the library (no allocation).  noalloc_tickets returns the current device's
// counter of a rank, after enqueueing on stream a small kernel that zeroes it.
constexpr int kNoAllocMaxRanks = 64;
hipError_t noalloc_tickets(int rank, hipStream_t stream, uint32_t** out);
// Zeroes words [0, words) of a heap's tile counters with a kernel on stream (no memset: capturable).
hipError_t clear_counters(uint32_t* counters, uint32_t words, hipStream_t stream);

// Arguments of the fused GEMM + multi-destination store kernel.
struct GemmKernelArgs {
    const uint64_t* heap_bases;
    const uint16_t* A;            // M x K, element (m,k) at A[m*lda + k]
    const uint16_t* B;            // element (k,n) at B[n*ldb + k], or B[k*ldb + n] when N-contiguous
    uint64_t rank_block_offset;   // out_offset + g*M*N*2
    int64_t lda, ldb;
    int32_t M, N, K;
    int32_t tiles_m, tiles_n, total_tiles;
    int32_t rank, rank_start, rank_stride, group_rank;
};

// Tile configurations of the fused kernel (TM x TN, K step 64).
enum GemmTile { kGemmTile256x256 = 0, kGemmTile256x224 = 1, kGemmTile128x128 = 2 };

struct GemmLaunch {
    GemmKernelArgs args;
    int bf16;          // 0 = fp16, 1 = bf16
    int world;
    int cfg;           // GemmTile
    int grid;
    int b_n_contiguous;   // 1: B is stored N-contiguous (row-major K x N)
};

hipError_t launch_gemm(const GemmLaunch& l, hipStream_t stream);
// Threads per workgroup and LDS bytes of a tile configuration (host-only arithmetic).
void gemm_resources(int cfg, int* threads, int* lds_bytes);

}  // namespace ag
