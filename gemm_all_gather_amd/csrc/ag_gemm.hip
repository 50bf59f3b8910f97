// Fused GEMM + multi-destination store for gfx950.
//
// Method (ROCm/iris #626, "Summary" and "Assembly" table): a persistent
// tiled matmul whose epilogue stores each C tile to every rank of the group;
// the heap-base loads that translate the destinations are done once, above
// the K loop and the tile loop, and the local copy is stored first, then the
// peers in rotated group order.
//
// gfx950 design:
//   * C = A . B with A row-major (M x K) and B K-contiguous (element (k,n) at
//     B[n*ldb + k]); both operands are therefore rows of 128-byte K slabs.
//   * 256 threads = 4 wave64s in a 2 x 2 grid; each wave owns a
//     (TM/2) x (TN/2) sub-tile made of 16 x 16 blocks computed with
//     v_mfma_f32_16x16x32_{f16,bf16} into fp32 accumulators.
//   * K advances 64 at a time through two LDS stages.  Each stage is filled
//     by buffer_load_dwordx4 ... lds (global to LDS without VGPRs): one wave
//     instruction moves 8 rows x 128 bytes.  The 16-byte chunks of a row are
//     XOR-swizzled by (row & 7), chosen through which global chunk each lane
//     fetches, so the ds_read_b128 fragment reads are free of bank conflicts.
//   * The MFMA takes B as its first operand and A as its second, so each
//     lane's accumulator holds four consecutive columns of one C row.
//   * Epilogue: convert to the 16-bit output type (round to nearest even),
//     stage the tile through LDS (reusing the two stages) so that every lane
//     then holds 16 contiguous bytes of a C row, and store the tile to the W
//     destinations with buffer_store_dwordx4: local region first, then the
//     rotated peers.  Rows past M and columns past N are dropped by the
//     buffer descriptors' bounds, never by branches.
//   * Tiles are walked by a persistent grid; consecutive workgroups land on
//     different XCDs, so the tile order gives each XCD a compact group of
//     tiles (8 tile rows at a time) that share A rows and B columns in its L2.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ag_internal.h"

#define AG_LDS __attribute__((address_space(3)))

namespace ag {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr int kRawBufferWord3 = 0x00020000;
constexpr uint32_t kOutOfRange = 0x80000000u;

__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(uint64_t base, uint64_t records)
{
    const uint32_t r = records < 0x7fffffffull ? static_cast<uint32_t>(records) : 0x7fffffffu;
    return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(base), static_cast<short>(0),
                                             static_cast<int>(r), kRawBufferWord3);
}

// s_waitcnt with only the vector-memory counter limited (gfx9 encoding).
template <int N>
__device__ inline void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}
__device__ inline void wait_lgkmcnt0() { __builtin_amdgcn_s_waitcnt(0xC07F); }

template <bool BF16> struct Mfma;
template <> struct Mfma<false> {
    using V = f16x8;
    static __device__ f32x4 run(V a, V b, f32x4 c) { return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0); }
    static __device__ uint32_t pack(float x, float y)
    {
        const _Float16 hx = static_cast<_Float16>(x), hy = static_cast<_Float16>(y);
        return static_cast<uint32_t>(__builtin_bit_cast(uint16_t, hx)) |
               (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, hy)) << 16);
    }
};
template <> struct Mfma<true> {
    using V = bf16x8;
    static __device__ f32x4 run(V a, V b, f32x4 c) { return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0); }
    static __device__ uint32_t pack(float x, float y)
    {
        const __bf16 hx = static_cast<__bf16>(x), hy = static_cast<__bf16>(y);
        return static_cast<uint32_t>(__builtin_bit_cast(uint16_t, hx)) |
               (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, hy)) << 16);
    }
};

}  // namespace

// Tile configuration.  Named namespace: a kernel template instantiated with a
// type of internal linkage gets no host-side launch handle.
namespace gemm_cfg {
template <int TM_, int TN_>
struct Cfg {
    static constexpr int TM = TM_, TN = TN_;
    static constexpr int WGM = 2, WGN = 2;                 // wave grid
    static constexpr int WTM = TM / WGM, WTN = TN / WGN;   // wave sub-tile
    static constexpr int BM = WTM / 16, BN = WTN / 16;     // 16x16 blocks per wave
    static constexpr int A_BYTES = TM * 128;               // one stage: TM rows x 64 K x 2 bytes
    static constexpr int B_BYTES = TN * 128;
    static constexpr int STAGE = A_BYTES + B_BYTES;
    static constexpr int A_LOADS = TM / 32;                // 1-KiB wave loads per wave per stage
    static constexpr int B_LOADS = TN / 32;
    static constexpr int CPR = TN / 8;                     // 16-byte chunks per C row
    static constexpr bool XOR_SWIZZLE = (CPR & (CPR - 1)) == 0 && CPR >= 16;
    static constexpr int C_PITCH = XOR_SWIZZLE ? TN * 2 : TN * 2 + 16;
    static constexpr int HALF_ROWS = TM / 2;               // C rows staged in each LDS stage
    static constexpr int CHUNKS_PER_THREAD = TM * CPR / 256;
    static_assert(WTM % 16 == 0 && WTN % 16 == 0, "wave tile must be made of 16x16 blocks");
    static_assert(TM % 32 == 0 && TN % 32 == 0, "stage loads move 8 rows per wave instruction");
    static_assert(HALF_ROWS * C_PITCH <= STAGE, "C staging must fit in one stage");
    static_assert((HALF_ROWS * CPR) % 256 == 0, "each LDS half must hold whole rounds of chunks");
    static_assert(2 * STAGE <= 160 * 1024, "gfx950 has 160 KiB of LDS");
};
}  // namespace gemm_cfg

namespace {
using gemm_cfg::Cfg;

// One K stage (64 wide) of the A and B tiles, global -> LDS: each wave
// instruction moves 8 rows x 128 bytes, lane l landing at byte 16*l of its
// 1-KiB LDS block.  (A free function: the LDS pointer conversion and the
// LDS-direct load are device-only.)
template <class C>
struct Stage {
    static __device__ __forceinline__ void load(uint64_t a_base, uint64_t a_records, uint64_t b_base,
                                                uint64_t b_records, uint8_t* buf, int kt, int wave,
                                                const uint32_t* a_voff, const uint32_t* b_voff)
    {
        const __amdgpu_buffer_rsrc_t ra = make_rsrc(a_base, a_records);
        const __amdgpu_buffer_rsrc_t rb = make_rsrc(b_base, b_records);
        const uint32_t soff = static_cast<uint32_t>(kt) * 128u;   // k0 * 2 bytes
#pragma unroll
        for (int q = 0; q < C::A_LOADS; ++q)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (AG_LDS void*)(buf + (q * 4 + wave) * 1024), 16, a_voff[q],
                                                     soff, 0, 0);
#pragma unroll
        for (int q = 0; q < C::B_LOADS; ++q)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (AG_LDS void*)(buf + C::A_BYTES + (q * 4 + wave) * 1024), 16,
                                                     b_voff[q], soff, 0, 0);
    }
};

template <bool BF16, int W, class C>
__global__ __launch_bounds__(256) void ag_gemm_kernel(GemmKernelArgs a)
{
    using M = Mfma<BF16>;
    using V = typename M::V;
    __shared__ __attribute__((aligned(1024))) uint8_t lds0[C::STAGE];
    __shared__ __attribute__((aligned(1024))) uint8_t lds1[C::STAGE];

    // ---- destinations, translated once above the tile and K loops
    uint64_t base[W];
#pragma unroll
    for (int i = 0; i < W; ++i) {
        int gi = a.group_rank + i;
        if (gi >= W) gi -= W;
        base[i] = __builtin_nontemporal_load(a.heap_bases + (a.rank_start + gi * a.rank_stride));
    }
    const uint64_t local_base = base[0];
    const uint64_t out_local = local_base + a.rank_block_offset;
    uint64_t dest[W];
#pragma unroll
    for (int i = 0; i < W; ++i) dest[i] = out_local + static_cast<uint64_t>(static_cast<int64_t>(base[i] - local_base));

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / C::WGN;
    const int wn = wave % C::WGN;

    // ---- tile-invariant lane offsets
    const uint32_t lda2 = static_cast<uint32_t>(a.lda) * 2u;
    const uint32_t ldb2 = static_cast<uint32_t>(a.ldb) * 2u;
    const uint32_t swz_chunk = static_cast<uint32_t>((lane & 7) ^ (lane >> 3));   // XOR-swizzled 16-B chunk
    uint32_t a_voff[C::A_LOADS], b_voff[C::B_LOADS];
#pragma unroll
    for (int q = 0; q < C::A_LOADS; ++q)
        a_voff[q] = static_cast<uint32_t>((q * 4 + wave) * 8 + (lane >> 3)) * lda2 + swz_chunk * 16u;
#pragma unroll
    for (int q = 0; q < C::B_LOADS; ++q)
        b_voff[q] = static_cast<uint32_t>((q * 4 + wave) * 8 + (lane >> 3)) * ldb2 + swz_chunk * 16u;
    uint32_t frag_off[2];   // row (lane & 15), logical chunk kk*4 + (lane >> 4), swizzled by row & 7
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
        frag_off[kk] = static_cast<uint32_t>((lane & 15) * 128 + ((((kk * 4) + (lane >> 4)) ^ (lane & 7)) << 4));

    const int kt_total = a.K / 64;
    const uint32_t out_row_bytes = static_cast<uint32_t>(a.N) * 2u;
    const int nprog = gridDim.x;
    const int p = blockIdx.x;
    // workgroup p runs on XCD p % 8; give each XCD a contiguous run of the tile order
    const int vp = (nprog % 8 == 0) ? (p % 8) * (nprog / 8) + p / 8 : p;

    for (int v = vp; v < a.total_tiles; v += nprog) {
        // grouped tile order: 8 tile rows at a time, column by column
        constexpr int GROUP_M = 8;
        const int group_tiles = GROUP_M * a.tiles_n;
        const int g = v / group_tiles;
        const int first_m = g * GROUP_M;
        const int gm = min(a.tiles_m - first_m, GROUP_M);
        const int r = v - g * group_tiles;
        const int tm = first_m + r % gm;
        const int tn = r / gm;
        const int m0 = tm * C::TM;
        const int n0 = tn * C::TN;

        const uint64_t a_base = reinterpret_cast<uint64_t>(a.A) + static_cast<uint64_t>(m0) * lda2;
        const uint64_t a_records = static_cast<uint64_t>(a.M - m0) * lda2;
        const uint64_t b_base = reinterpret_cast<uint64_t>(a.B) + static_cast<uint64_t>(n0) * ldb2;
        const uint64_t b_records = static_cast<uint64_t>(a.N - n0) * ldb2;

        f32x4 acc[C::BM][C::BN];
#pragma unroll
        for (int bm = 0; bm < C::BM; ++bm)
#pragma unroll
            for (int bn = 0; bn < C::BN; ++bn) acc[bm][bn] = f32x4{0.f, 0.f, 0.f, 0.f};

        auto compute = [&](const uint8_t* buf) {
            const uint8_t* abuf = buf + wm * C::WTM * 128;
            const uint8_t* bbuf = buf + C::A_BYTES + wn * C::WTN * 128;
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                V af[C::BM], bf[C::BN];
#pragma unroll
                for (int bm = 0; bm < C::BM; ++bm)
                    af[bm] = *reinterpret_cast<const V*>(abuf + bm * 16 * 128 + frag_off[kk]);
#pragma unroll
                for (int bn = 0; bn < C::BN; ++bn)
                    bf[bn] = *reinterpret_cast<const V*>(bbuf + bn * 16 * 128 + frag_off[kk]);
#pragma unroll
                for (int bm = 0; bm < C::BM; ++bm)
#pragma unroll
                    for (int bn = 0; bn < C::BN; ++bn) acc[bm][bn] = M::run(bf[bn], af[bm], acc[bm][bn]);
            }
        };

        // ---- K loop: two LDS stages used in turn
        Stage<C>::load(a_base, a_records, b_base, b_records, lds0, 0, wave, a_voff, b_voff);
        int kt = 0;
        for (; kt + 2 <= kt_total; kt += 2) {
            wait_vmcnt<0>();
            __builtin_amdgcn_s_barrier();
            Stage<C>::load(a_base, a_records, b_base, b_records, lds1, kt + 1, wave, a_voff, b_voff);
            compute(lds0);
            wait_vmcnt<0>();
            __builtin_amdgcn_s_barrier();
            if (kt + 2 < kt_total) Stage<C>::load(a_base, a_records, b_base, b_records, lds0, kt + 2, wave, a_voff, b_voff);
            compute(lds1);
        }
        if (kt < kt_total) {   // odd number of K steps
            wait_vmcnt<0>();
            __builtin_amdgcn_s_barrier();
            compute(lds0);
        }

        // ---- epilogue: round, stage C through LDS, store to every destination
        wait_lgkmcnt0();
        __builtin_amdgcn_s_barrier();   // every wave is done reading the stages
        {
            uint8_t* half = wm == 0 ? lds0 : lds1;   // wave rows lie in one half of the tile
#pragma unroll
            for (int bm = 0; bm < C::BM; ++bm) {
                const int row = bm * 16 + (lane & 15);
#pragma unroll
                for (int bn = 0; bn < C::BN; ++bn) {
                    const int byte_col = (wn * C::WTN + bn * 16) * 2 + (lane >> 4) * 8;
                    int chunk = byte_col >> 4;
                    if (C::XOR_SWIZZLE) chunk ^= (row & 15);
                    const f32x4 c = acc[bm][bn];
                    u32x2 packed;
                    packed.x = M::pack(c[0], c[1]);
                    packed.y = M::pack(c[2], c[3]);
                    *reinterpret_cast<u32x2*>(half + row * C::C_PITCH + chunk * 16 + (byte_col & 15)) = packed;
                }
            }
        }
        wait_lgkmcnt0();
        __builtin_amdgcn_s_barrier();
        {
            const uint64_t tile_off = (static_cast<uint64_t>(m0) * a.N + n0) * 2u;
            const uint64_t records = static_cast<uint64_t>(a.M - m0) * out_row_bytes - static_cast<uint64_t>(n0) * 2u;
            const int cols_left = a.N - n0;
            u32x4 vals[C::CHUNKS_PER_THREAD];
            uint32_t voff[C::CHUNKS_PER_THREAD];
#pragma unroll
            for (int j = 0; j < C::CHUNKS_PER_THREAD; ++j) {
                const int ci = tid + 256 * j;
                const int row = ci / C::CPR;
                const int c = ci - row * C::CPR;
                constexpr int kHalfChunks = C::HALF_ROWS * C::CPR;
                const uint8_t* half = (256 * j < kHalfChunks) ? lds0 : lds1;
                const int hrow = (256 * j < kHalfChunks) ? row : row - C::HALF_ROWS;
                const int pc = C::XOR_SWIZZLE ? (c ^ (hrow & 15)) : c;
                vals[j] = *reinterpret_cast<const u32x4*>(half + hrow * C::C_PITCH + pc * 16);
                voff[j] = (c * 8 < cols_left) ? static_cast<uint32_t>(row) * out_row_bytes + static_cast<uint32_t>(c) * 16u
                                              : kOutOfRange;
            }
#pragma unroll
            for (int i = 0; i < W; ++i) {   // local region first, then the rotated peers
                const __amdgpu_buffer_rsrc_t rd = make_rsrc(dest[i] + tile_off, records);
#pragma unroll
                for (int j = 0; j < C::CHUNKS_PER_THREAD; ++j)
                    __builtin_amdgcn_raw_buffer_store_b128(vals[j], rd, voff[j], 0, 0);
            }
        }
        wait_lgkmcnt0();
        __builtin_amdgcn_s_barrier();   // staging reads done before the next tile's loads land
    }
}

using GemmFn = void (*)(GemmKernelArgs);

template <bool BF16, class C>
GemmFn pick_world(int w)
{
    switch (w) {
    case 1: return ag_gemm_kernel<BF16, 1, C>;
    case 2: return ag_gemm_kernel<BF16, 2, C>;
    case 3: return ag_gemm_kernel<BF16, 3, C>;
    case 4: return ag_gemm_kernel<BF16, 4, C>;
    case 5: return ag_gemm_kernel<BF16, 5, C>;
    case 6: return ag_gemm_kernel<BF16, 6, C>;
    case 7: return ag_gemm_kernel<BF16, 7, C>;
    case 8: return ag_gemm_kernel<BF16, 8, C>;
    default: return nullptr;
    }
}

template <bool BF16>
GemmFn pick_cfg(int cfg, int w)
{
    switch (cfg) {
    case kGemmTile256x256: return pick_world<BF16, Cfg<256, 256>>(w);
    case kGemmTile256x224: return pick_world<BF16, Cfg<256, 224>>(w);
    case kGemmTile128x128: return pick_world<BF16, Cfg<128, 128>>(w);
    default: return nullptr;
    }
}

}  // namespace

hipError_t launch_gemm(const GemmLaunch& l, hipStream_t stream)
{
    GemmFn fn = l.bf16 ? pick_cfg<true>(l.cfg, l.world) : pick_cfg<false>(l.cfg, l.world);
    if (fn == nullptr || l.grid < 1) return hipErrorInvalidValue;
    hipLaunchKernelGGL(fn, dim3(l.grid), dim3(256), 0, stream, l.args);
    return hipGetLastError();
}

}  // namespace ag
