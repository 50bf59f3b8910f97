// Internal interface between the host runtime (ag_host.cpp) and the kernel
// launchers (ag_copy.hip, ag_gemm.hip).  Not part of the public C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ag {

// Arguments of the persistent multi-destination copy kernel (by value).
struct CopyKernelArgs {
    const uint64_t* heap_bases;   // device uint64_t[n_ranks]
    const uint8_t* input;         // rank's M_local x N block, row-major
    uint64_t rank_block_offset;   // out_offset + g*M_local*N*e, same in every region
    uint64_t row_bytes;           // N*e
    uint32_t rows;                // M_local
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
    uint32_t reserved;
};

struct CopyLaunch {
    CopyKernelArgs args;
    int vec_bytes;     // 16, 8, 4, 2
    int world;         // W
    int vpt;           // vector accesses per thread per tile
    int grid;          // workgroups
};

hipError_t launch_copy(const CopyLaunch& l, hipStream_t stream);

// Arguments of the fused GEMM + multi-destination store kernel.
struct GemmKernelArgs {
    const uint64_t* heap_bases;
    const uint16_t* A;            // M x K, element (m,k) at A[m*lda + k]
    const uint16_t* B;            // element (k,n) at B[n*ldb + k]
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
};

hipError_t launch_gemm(const GemmLaunch& l, hipStream_t stream);
// Threads per workgroup and LDS bytes of a tile configuration (host-only arithmetic).
void gemm_resources(int cfg, int* threads, int* lds_bytes);

}  // namespace ag
