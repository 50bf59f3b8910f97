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
//   * 8 wave64s (two per SIMD) in a 4 x 2 wave grid; each wave owns a
//     (TM/4) x (TN/2) sub-tile made of 16 x 16 blocks computed with
//     v_mfma_f32_16x16x32_{f16,bf16} into fp32 accumulators.
//   * K advances 64 at a time through a ring of LDS stages (two for the
//     256-row tiles, four for 128 x 128).  Each stage is filled by
//     buffer_load_dwordx4 ... lds (global to LDS without VGPRs): one wave
//     instruction moves 8 rows x 128 bytes.  The 16-byte chunks of a row are
//     XOR-swizzled by (row & 7), chosen through which global chunk each lane
//     fetches, so the ds_read_b128 fragment reads are free of bank conflicts.
//   * A wave that issues a stage's loads is held at each load until the CU
//     accepts it (about one 1 KiB instruction per 22 cycles per CU).  With two
//     ring slots the loads are split between the two halves of the
//     workgroup and in time: stage k's A rows by half k % 2 right after the
//     barrier two stages ahead, its B rows by the other half one stage
//     ahead.  Waves are placed on SIMDs round-robin, so on every SIMD one
//     wave keeps issuing MFMAs while the other issues loads.  Fragments are
//     then single-buffered, which keeps the kernel within its registers.
//   * The MFMA takes B as its first operand and A as its second, so each
//     lane's accumulator holds four consecutive columns of one C row.
//   * Epilogue: convert to the 16-bit output type (round to nearest even),
//     stage the tile through LDS (reusing the ring) so that every lane then
//     holds 16 contiguous bytes of a C row, and store the tile to the W
//     destinations with non-temporal buffer_store_dwordx4: local region
//     first, then the rotated peers.  Rows past M and columns past N are
//     dropped by the buffer descriptors' bounds, never by branches.
//   * Tiles are walked by a persistent grid; consecutive workgroups land on
//     different XCDs, so the tile order gives each XCD a compact group of
//     tiles (8 tile rows at a time) that share A rows and B columns in its L2.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

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
// Wave rows of the 2-column wave grid (4: eight waves, two per SIMD).
#ifndef AG_GEMM_WGM
#define AG_GEMM_WGM 4
#endif
// Cache-policy bits of the epilogue stores (bit 1 = non-temporal).
#ifndef AG_GEMM_STORE_AUX
#define AG_GEMM_STORE_AUX 2
#endif
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
// s_waitcnt with only the LDS/scalar counter limited (at most N outstanding).
template <int N>
__device__ inline void wait_lgkmcnt()
{
    static_assert(N >= 0 && N < 16, "lgkmcnt is 4 bits");
    __builtin_amdgcn_s_waitcnt(0xF | (0x3 << 14) | (0x7 << 4) | (N << 8));
}

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
template <int TM_, int TN_, int WGM_, int WGN_, int BK_, int NS_, bool ALT_>
struct Cfg {
    static constexpr int TM = TM_, TN = TN_;
    static constexpr int WGM = WGM_, WGN = WGN_;           // wave grid
    static constexpr int NW = WGM * WGN;                   // waves per workgroup
    static constexpr int NT = 64 * NW;                     // threads per workgroup
    static constexpr int WTM = TM / WGM, WTN = TN / WGN;   // wave sub-tile
    static constexpr int BM = WTM / 16, BN = WTN / 16;     // 16x16 blocks per wave
    static constexpr int BK = BK_;                         // K per LDS stage (32 or 64)
    static constexpr int KSUB = BK / 32;                   // MFMA K-steps (32 wide) per stage
    static constexpr int NS = NS_;                         // LDS ring slots
    static constexpr bool ALT = ALT_;                      // stage loads by half the waves, alternating
    static constexpr int ROW_BYTES = BK * 2;               // bytes of one operand row in a stage
    static constexpr int LPR = ROW_BYTES / 16;             // lanes per row in a stage load
    static constexpr int RPI = 64 / LPR;                   // rows per 1-KiB wave load
    static constexpr int A_BYTES = TM * ROW_BYTES;
    static constexpr int STAGE = (TM + TN) * ROW_BYTES;
    static constexpr int A_INSTR = TM / RPI;
    static constexpr int B_INSTR = TN / RPI;
    static constexpr int INSTR = A_INSTR + B_INSTR;
    static constexpr int A_J = A_INSTR / NW;               // loads j < A_J of every wave are A rows
    static constexpr int MAXL = (INSTR + NW - 1) / NW;     // loads per wave per stage (waves 0..)
    static constexpr int CPR = TN / 8;                     // 16-byte chunks per C row
    static constexpr bool XOR_SWIZZLE = (CPR & (CPR - 1)) == 0 && CPR >= 16;
    static constexpr int C_PITCH = XOR_SWIZZLE ? TN * 2 : TN * 2 + 16;
    static constexpr int NSTG = (NS >= 4 && (TM / 4) * C_PITCH <= STAGE) ? 4 : 2;   // slots used to stage C
    static constexpr int QROWS = TM / NSTG;                // C rows staged in each of those slots
    static constexpr int SLOT_CHUNKS = QROWS * CPR;        // 16-byte C chunks per staging slot
    static constexpr int ROUNDS = (SLOT_CHUNKS + NT - 1) / NT;   // chunk rounds per slot per thread
    static constexpr int UNROLL = KSUB == 1 ? 2 * NS : NS; // stages per unrolled K-loop body
    static_assert(BK == 32 || BK == 64, "stages hold 32 or 64 K values");
    static_assert(WTM % 16 == 0 && WTN % 16 == 0, "wave tile must be made of 16x16 blocks");
    static_assert(TM % RPI == 0 && TN % RPI == 0, "stage loads move whole row groups");
    static_assert(QROWS * C_PITCH <= STAGE && NSTG <= NS, "C staging must fit in the ring");
    static_assert(QROWS % 16 == 0, "a 16-row accumulator block never straddles two staging slots");
    static_assert(A_INSTR % NW == 0, "every wave issues the same number of A loads");
    static_assert(BM + BN < 16, "one K-step's fragment reads fit the 4-bit LDS counter");
    static_assert(!ALT || (NS == 2 && A_INSTR % (NW / 2) == 0 && B_INSTR % (NW / 2) == 0),
                  "alternating loaders: two ring slots, an even split over half the waves");
    static_assert(NS >= 2 && NS * STAGE <= 160 * 1024, "gfx950 has 160 KiB of LDS");
};
}  // namespace gemm_cfg

namespace {
using gemm_cfg::Cfg;

// 16-byte chunk swizzle of an LDS stage row: chunks are XOR-ed with a few
// row bits so that the 8 lanes served together by a ds_read_b128 (8 rows at
// the same logical chunk) hit 8 different bank groups.
template <class C>
__device__ __forceinline__ uint32_t swz(uint32_t row)
{
    return C::BK == 64 ? (row & 7u) : ((row >> 1) & 3u);
}

// ds_read_b128 of one 16-row fragment block at a compile-time offset.
template <class C>
struct Frag {
    template <class V>
    static __device__ __forceinline__ void read(V& dst, uint32_t addr, int block)
    {
        switch (block) {   // the offset must be an immediate
#define AG_FRAG_CASE(b)                                                                                      \
    case b:                                                                                                  \
        asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(dst) : "v"(addr), "i"(b * 16 * C::ROW_BYTES)); \
        break;
            AG_FRAG_CASE(0) AG_FRAG_CASE(1) AG_FRAG_CASE(2) AG_FRAG_CASE(3)
            AG_FRAG_CASE(4) AG_FRAG_CASE(5) AG_FRAG_CASE(6) AG_FRAG_CASE(7)
#undef AG_FRAG_CASE
        default: break;
        }
    }
};

// B fragment of a 16-column block from an N-contiguous stage (rows of k,
// TN columns each): two transposing reads, k 0..3 then k 4..7 of the lane's
// 8-row group (the second 4 rows further: an immediate).  ds_read_b64_tr_b16
// gives lane i of each 16-lane group the (i & 3)-th 16-bit element of the
// 8-byte chunk addressed by lane 4*j + (i >> 2), for j = 0..3: with lane p
// addressing row (p >> 2) at columns 4*(p & 3) .. +3, lane i receives column
// i of rows 0..3.  A block is one 32-byte column pair of a row; rows with
// bit 3 set hold their pairs swapped (Stage::bt_off), so a lane of such a row
// finds an even logical pair one pair right and an odd one one pair left.
// lo_even / lo_odd are the lane's addresses for blocks whose logical pair is
// even / odd; the block's column offset is the immediate.
template <class C>
struct FragT {
    template <class V>
    static __device__ __forceinline__ void read(V& dst, uint32_t lo_even, uint32_t lo_odd, int block)
    {
        u32x2 a, b;
        switch (block) {   // the offsets must be immediates
#define AG_FRAGT_CASE(n)                                                                                  \
    case n:                                                                                               \
        asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2"                                                \
                     : "=v"(a) : "v"((n & 1) ? lo_odd : lo_even), "i"(n * 32));                           \
        asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2"                                                \
                     : "=v"(b) : "v"((n & 1) ? lo_odd : lo_even), "i"(n * 32 + 4 * C::TN * 2));           \
        break;
            AG_FRAGT_CASE(0) AG_FRAGT_CASE(1) AG_FRAGT_CASE(2) AG_FRAGT_CASE(3)
            AG_FRAGT_CASE(4) AG_FRAGT_CASE(5) AG_FRAGT_CASE(6) AG_FRAGT_CASE(7)
#undef AG_FRAGT_CASE
        default: a = u32x2{0u, 0u}; b = a; break;
        }
        dst = __builtin_bit_cast(V, u32x4{a.x, a.y, b.x, b.y});
    }
};

// One K stage of the A and B tiles, global -> LDS.  Wave instruction i of the
// stage moves RPI rows x ROW_BYTES (A rows for i < A_INSTR, then B rows) to
// LDS bytes [i*1024, i*1024 + 1024) of the slot; wave w issues instructions
// w, w+NW, ...  A descriptor of size 0 turns the loads of a stage past the
// end of K into no-ops that still count.  (Descriptors are passed as base +
// size: a template whose signature names the buffer-resource type fails to
// substitute in the host compilation pass.)
template <class C>
struct Stage {
    // Alternating loaders.  The stage's A_INSTR A-row and B_INSTR B-row wave
    // instructions are issued by one half of the workgroup's waves (wp =
    // index within the half): instruction i = wp + (NW/2)*j of each part.
    // la / lb are the lane's offsets inside a row group; the row group adds
    // a uniform term.  The operands are copied opaquely so that the
    // per-instruction offsets are not hoisted into registers held across the
    // K loop.
    static __device__ __forceinline__ void load_part(bool a_part, uint64_t base, uint64_t records, uint8_t* slot,
                                                     int kt, int wp, uint32_t lo, uint32_t ld2)
    {
        constexpr int H = C::NW / 2;
        const uint32_t soff = static_cast<uint32_t>(kt) * C::ROW_BYTES;
        asm volatile("" : "+v"(lo), "+s"(ld2));
        const __amdgpu_buffer_rsrc_t r = make_rsrc(base, records);
        if (a_part) {
#pragma unroll
            for (int j = 0; j < C::A_INSTR / H; ++j) {
                const int i = wp + H * j;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (AG_LDS void*)(slot + i * 1024), 16,
                                                         lo + static_cast<uint32_t>(i * C::RPI) * ld2, soff, 0, 0);
            }
        } else {
#pragma unroll
            for (int j = 0; j < C::B_INSTR / H; ++j) {
                const int i = wp + H * j;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (AG_LDS void*)(slot + (C::A_INSTR + i) * 1024), 16,
                                                         lo + static_cast<uint32_t>(i * C::RPI) * ld2, soff, 0, 0);
            }
        }
    }
    // N-contiguous B: the stage is BK rows of k with TN*2 bytes each, dense in
    // LDS; byte x of the stage region comes from row r = x / (TN*2) of the
    // stage, byte column x % (TN*2) of the tile's columns with bit 5 flipped
    // when bit 3 of r is set (32-byte pairs swapped; TN*2 is a multiple of
    // 64).  The transposing reads of lanes 0..31 touch rows 0..3 and 8..11 of
    // a K-step; with a row pitch that is a multiple of 64 bytes those rows
    // would start on the same banks, and the swap moves rows 8..11 onto the
    // banks rows 0..3 leave free.  lane16 = 16 * lane.
    static __device__ __forceinline__ uint32_t bt_off(int i, uint32_t lane16, uint32_t ld2)
    {
        constexpr uint32_t RB = C::TN * 2;
        static_assert(RB % 64 == 0, "pairs are swapped within a row");
        const uint32_t x = static_cast<uint32_t>(i) * 1024u + lane16;
        const uint32_t row = x / RB;
        return row * ld2 + ((x - row * RB) ^ (((row >> 3) & 1u) << 5));
    }
    // The descriptor of N-contiguous stage kt starts at its first row and
    // ends at the end of B: the stage offset goes into the base and the
    // extent, not into the SGPR offset, so the range check sees each lane's
    // whole offset from the stage and the columns past N of the last row of B
    // read as zero instead of past the end of B.
    static __device__ __forceinline__ __amdgpu_buffer_rsrc_t bt_rsrc(uint64_t base, uint64_t records, int kt,
                                                                     uint32_t ld2)
    {
        const uint64_t o = static_cast<uint64_t>(kt) * static_cast<uint64_t>(C::BK * ld2);
        return make_rsrc(base + o, records > o ? records - o : 0);
    }
    static __device__ __forceinline__ void load_part_bt(uint64_t base, uint64_t records, uint8_t* slot, int kt,
                                                        int wp, uint32_t lane16, uint32_t ld2)
    {
        constexpr int H = C::NW / 2;
        const __amdgpu_buffer_rsrc_t r = bt_rsrc(base, records, kt, ld2);
        asm volatile("" : "+v"(lane16), "+s"(ld2));
#pragma unroll
        for (int j = 0; j < C::B_INSTR / H; ++j) {
            const int i = wp + H * j;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (AG_LDS void*)(slot + (C::A_INSTR + i) * 1024), 16,
                                                     bt_off(i, lane16, ld2), 0, 0, 0);
        }
    }
    static __device__ __forceinline__ void load(uint64_t a_base, uint64_t a_records, uint64_t b_base,
                                                uint64_t b_records, uint8_t* slot, int kt, int wave,
                                                const uint32_t* voff, bool bt, uint32_t ldb2)
    {
        const __amdgpu_buffer_rsrc_t ra = make_rsrc(a_base, a_records);
        const uint32_t soff = static_cast<uint32_t>(kt) * C::ROW_BYTES;   // k0 * 2 bytes
        // K-contiguous B steps along its rows like A; N-contiguous B by whole rows of k
        const __amdgpu_buffer_rsrc_t rb = bt ? bt_rsrc(b_base, b_records, kt, ldb2) : make_rsrc(b_base, b_records);
        const uint32_t bsoff = bt ? 0u : soff;
#pragma unroll
        for (int j = 0; j < C::MAXL; ++j) {
            const int i = wave + C::NW * j;
            if (j < C::A_J) {
                __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (AG_LDS void*)(slot + i * 1024), 16, voff[j], soff, 0, 0);
            } else if (i < C::INSTR) {
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (AG_LDS void*)(slot + i * 1024), 16, voff[j], bsoff, 0, 0);
            }
        }
    }
};

// BT: B is N-contiguous (element (k,n) at B[k*ldb + n]); otherwise K-contiguous.
template <bool BF16, int W, class C, bool BT>
__global__ __launch_bounds__(C::NT) void ag_gemm_kernel(GemmKernelArgs a)
{
    static_assert(!BT || C::ALT || C::BM + 2 * C::BN < 16, "two B reads per block must fit the 4-bit LDS counter");
    using M = Mfma<BF16>;
    using V = typename M::V;
    __shared__ __attribute__((aligned(1024))) uint8_t ring[C::NS][C::STAGE];

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
    // loads per stage of this wave (MAXL or MAXL-1)
    const bool full_share = wave + C::NW * (C::MAXL - 1) < C::INSTR;

    // ---- tile-invariant lane offsets
    const uint32_t lda2 = static_cast<uint32_t>(a.lda) * 2u;
    const uint32_t ldb2 = static_cast<uint32_t>(a.ldb) * 2u;
    const uint32_t lrow = static_cast<uint32_t>(lane / C::LPR);                      // row in the load's row group
    const uint32_t lchunk = static_cast<uint32_t>(lane % C::LPR) ^ swz<C>(lrow);     // swizzled 16-byte chunk
    const uint32_t la = lrow * lda2 + lchunk * 16u;
    const uint32_t lb = lrow * ldb2 + lchunk * 16u;
    // alternating loaders: waves are assigned to SIMDs round-robin, so each
    // half has one wave on every SIMD
    const int half = wave / (C::NW / 2), wp = wave % (C::NW / 2);
    uint32_t voff[C::MAXL];
#pragma unroll
    for (int j = 0; j < C::MAXL; ++j) {
        const int i = wave + C::NW * j;
        if (BT && j >= C::A_J)
            voff[j] = Stage<C>::bt_off(i - C::A_INSTR, static_cast<uint32_t>(lane) * 16u, ldb2);
        else
            voff[j] = (j < C::A_J) ? (static_cast<uint32_t>(i * C::RPI) + lrow) * lda2 + lchunk * 16u
                                   : (static_cast<uint32_t>((i - C::A_INSTR) * C::RPI) + lrow) * ldb2 + lchunk * 16u;
    }
    // N-contiguous B fragments: lane (q = lane >> 4, p = lane & 15) addresses row 8q + (p >> 2) of its
    // K-step, columns 4*(p & 3) .. +3 of its wave's first block (logical pair wn*BN).  Rows of odd q
    // hold their pairs swapped: block b's data sits one pair right of its place if wn*BN + b is even,
    // one pair left if it is odd.
    const uint32_t bt_lane = static_cast<uint32_t>((8 * (lane >> 4) + ((lane & 15) >> 2)) * (C::TN * 2)) +
                             static_cast<uint32_t>(wn * C::WTN + 4 * (lane & 3)) * 2u;
    const int bt_shift = ((lane >> 4) & 1) * (((wn * C::BN) & 1) ? -32 : 32);   // for even b
    const uint32_t bt_even = bt_lane + static_cast<uint32_t>(bt_shift);
    const uint32_t bt_odd = bt_lane - static_cast<uint32_t>(bt_shift);
    // fragment of MFMA K-step kk: row (lane & 15) of a 16-row block, logical chunk kk*4 + (lane >> 4)
    uint32_t frag_off[C::KSUB];
#pragma unroll
    for (int kk = 0; kk < C::KSUB; ++kk)
        frag_off[kk] = static_cast<uint32_t>((lane & 15) * C::ROW_BYTES) +
                       ((static_cast<uint32_t>(kk * 4 + (lane >> 4)) ^ swz<C>(static_cast<uint32_t>(lane & 15))) << 4);
    const uint32_t a_row0 = static_cast<uint32_t>(wm * C::WTM * C::ROW_BYTES);
    const uint32_t b_row0 = static_cast<uint32_t>(C::A_BYTES + wn * C::WTN * C::ROW_BYTES);

    const int kt_total = a.K / C::BK;
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
        const uint64_t b_base = BT ? reinterpret_cast<uint64_t>(a.B) + static_cast<uint64_t>(n0) * 2u
                                   : reinterpret_cast<uint64_t>(a.B) + static_cast<uint64_t>(n0) * ldb2;
        const uint64_t b_records = BT ? static_cast<uint64_t>(a.K - 1) * ldb2 + static_cast<uint64_t>(a.N - n0) * 2u
                                      : static_cast<uint64_t>(a.N - n0) * ldb2;

        f32x4 acc[C::BM][C::BN];
#pragma unroll
        for (int bm = 0; bm < C::BM; ++bm)
#pragma unroll
            for (int bn = 0; bn < C::BN; ++bn) acc[bm][bn] = f32x4{0.f, 0.f, 0.f, 0.f};
        V fa[2][C::BM], fb[2][C::BN];

        // Loads of a whole stage kt into a ring slot (with alternating loaders:
        // by half kt % 2; used for the first NS stages of a tile).
        auto issue = [&](int slot, int kt) {
            const bool live = kt < kt_total;
            if constexpr (C::ALT) {
                if (half == (kt & 1)) {   // whole stage (prologue)
                    Stage<C>::load_part(true, a_base, live ? a_records : 0, &ring[slot][0], kt, wp, la, lda2);
                    if constexpr (BT)
                        Stage<C>::load_part_bt(b_base, live ? b_records : 0, &ring[slot][0], kt, wp,
                                               static_cast<uint32_t>(lane) * 16u, ldb2);
                    else
                        Stage<C>::load_part(false, b_base, live ? b_records : 0, &ring[slot][0], kt, wp, lb, ldb2);
                }
            } else {
                Stage<C>::load(a_base, live ? a_records : 0, b_base, live ? b_records : 0, &ring[slot][0], kt, wave,
                               voff, BT, ldb2);
            }
        };
        // Fragment reads are inline assembly: the compiler cannot tell these
        // LDS reads apart from LDS-direct loads still landing in other ring
        // slots and would otherwise wait for all of them.  Their completion is
        // awaited explicitly (lgkmcnt) before the data is used.
        auto read_frags = [&](int slot, int kk, int f) {
            const uint32_t sbase = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((AG_LDS uint8_t*)&ring[slot][0]));
            const uint32_t sa = sbase + a_row0 + frag_off[kk];
            const uint32_t sb = sbase + b_row0 + frag_off[kk];
#pragma unroll
            for (int bm = 0; bm < C::BM; ++bm) Frag<C>::read(fa[f][bm], sa, bm);
            if constexpr (BT) {
                const uint32_t kb = sbase + C::A_BYTES + static_cast<uint32_t>(kk * 32 * C::TN * 2);
                const uint32_t le = kb + bt_even, lo = kb + bt_odd;
#pragma unroll
                for (int bn = 0; bn < C::BN; ++bn) FragT<C>::read(fb[f][bn], le, lo, bn);
            } else {
#pragma unroll
                for (int bn = 0; bn < C::BN; ++bn) Frag<C>::read(fb[f][bn], sb, bn);
            }
        };
        auto mfmas = [&](int f) {
#pragma unroll
            for (int bm = 0; bm < C::BM; ++bm)
#pragma unroll
                for (int bn = 0; bn < C::BN; ++bn) acc[bm][bn] = M::run(fb[f][bn], fa[f][bm], acc[bm][bn]);
        };
        auto wait_stages = [&](auto n_stages) {   // all of this wave's loads but the last n stages' have landed
            constexpr int n = decltype(n_stages)::value;
            if constexpr (C::ALT) {
                // two slots: a wave's only loads in flight at a boundary are
                // those of the next stage, if it issued them (n == 0); in the
                // prologue half 0 holds stage 0 and half 1 only stage 1
                if (n == 0 || half == 0) wait_vmcnt<0>();
            } else if (full_share) {
                wait_vmcnt<n * C::MAXL>();
            } else {
                wait_vmcnt<n * (C::MAXL - 1)>();
            }
        };
        // Alternating loaders (two slots).  Stage s+2's A rows are loaded by
        // half s % 2 right after the boundary barrier of stage s, into the
        // slot stage s has just released; its B rows by the other half at the
        // start of stage s+1.  Each wave is thus held at loads about half as
        // long, at a different time from its SIMD partner, and at a boundary
        // its only loads in flight are those of the next stage: vmcnt(0).
        // Fragments are single-buffered: each K-step reads its own, waits,
        // then issues its MFMAs (the SIMD partner hides the read latency).
        auto stage_alt = [&](int s, int slot, int next_slot) {
#pragma unroll
            for (int kk = 0; kk < C::KSUB; ++kk) {
                if (kk == 0 && s >= 1 && half != ((s - 1) & 1)) {
                    const int kn = s + 1;
                    if constexpr (BT)
                        Stage<C>::load_part_bt(b_base, kn < kt_total ? b_records : 0, &ring[next_slot][0], kn, wp,
                                               static_cast<uint32_t>(lane) * 16u, ldb2);
                    else
                        Stage<C>::load_part(false, b_base, kn < kt_total ? b_records : 0, &ring[next_slot][0], kn,
                                            wp, lb, ldb2);
                }
                read_frags(slot, kk, 0);
                __builtin_amdgcn_sched_barrier(0);
                wait_lgkmcnt0();
                __builtin_amdgcn_sched_barrier(0);
                if (kk + 1 == C::KSUB) {
                    wait_vmcnt<0>();
                    __builtin_amdgcn_s_barrier();
                    __builtin_amdgcn_sched_barrier(0);
                    const int kn = s + C::NS;
                    if (half == (kn & 1))
                        Stage<C>::load_part(true, a_base, kn < kt_total ? a_records : 0, &ring[slot][0], kn, wp, la,
                                            lda2);
                }
                mfmas(0);
            }
        };
        // Stage s (in ring slot s % NS): its MFMA K-steps run on fragments read
        // one K-step ahead.  At the last K-step the next stage is made visible
        // (its own loads waited for, then a barrier), the slot of stage s is
        // refilled with stage s + NS, and stage s+1's first fragments are read.
        auto stage = [&](int s, int slot, int next_slot, int f0) {
#pragma unroll
            for (int kk = 0; kk < C::KSUB; ++kk) {
                const int f = f0 ^ (kk & 1);
                if (kk + 1 < C::KSUB) {
                    read_frags(slot, kk + 1, f ^ 1);
                    // the fragments of this K-step (read one step earlier,
                    // possibly at the stage boundary) have landed; the reads
                    // just issued may still be in flight
                    __builtin_amdgcn_sched_barrier(0);
                    // (alternating-loader tiles run stage_alt, never this path)
                    wait_lgkmcnt<C::ALT ? 0 : C::BM + (BT ? 2 : 1) * C::BN>();
                    __builtin_amdgcn_sched_barrier(0);
                } else {
                    __builtin_amdgcn_sched_barrier(0);
                    wait_stages(std::integral_constant<int, C::NS - 2>{});
                    wait_lgkmcnt0();              // this wave's reads of stage s are complete
                    __builtin_amdgcn_s_barrier();
                    __builtin_amdgcn_sched_barrier(0);
                    issue(slot, s + C::NS);
                    if (s + 1 < kt_total) read_frags(next_slot, 0, f ^ 1);
                }
                mfmas(f);
            }
        };

        // ---- prologue: stages 0..NS-1 in flight, stage 0's first fragments in registers
#pragma unroll
        for (int q = 0; q < C::NS; ++q) issue(q, q);
        wait_stages(std::integral_constant<int, C::NS - 1>{});
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (!C::ALT) read_frags(0, 0, 0);

        // ---- K loop, unrolled over the ring slots (and the fragment buffers)
        for (int s = 0; s < kt_total; s += C::UNROLL) {
#pragma unroll
            for (int u = 0; u < C::UNROLL; ++u) {
                if (u == 0 || s + u < kt_total) {
                    if constexpr (C::ALT) stage_alt(s + u, u % C::NS, (u + 1) % C::NS);
                    else stage(s + u, u % C::NS, (u + 1) % C::NS, C::KSUB == 1 ? (u & 1) : 0);
                }
            }
        }

        // ---- epilogue: round, stage C through the ring, store to every destination
        wait_vmcnt<0>();                // loads of stages past the end have landed too
        wait_lgkmcnt0();
        __builtin_amdgcn_s_barrier();
        {
#pragma unroll
            for (int bm = 0; bm < C::BM; ++bm) {
                const int trow = wm * C::WTM + bm * 16;          // first tile row of this block row
                const int q = trow / C::QROWS;                   // ring slot holding these rows
                uint8_t* slot = &ring[q][0];
                const int row = trow - q * C::QROWS + (lane & 15);
#pragma unroll
                for (int bn = 0; bn < C::BN; ++bn) {
                    const int byte_col = (wn * C::WTN + bn * 16) * 2 + (lane >> 4) * 8;
                    int chunk = byte_col >> 4;
                    if (C::XOR_SWIZZLE) chunk ^= (row & 15);
                    const f32x4 c = acc[bm][bn];
                    u32x2 packed;
                    packed.x = M::pack(c[0], c[1]);
                    packed.y = M::pack(c[2], c[3]);
                    *reinterpret_cast<u32x2*>(slot + row * C::C_PITCH + chunk * 16 + (byte_col & 15)) = packed;
                }
            }
        }
        wait_lgkmcnt0();
        __builtin_amdgcn_s_barrier();
        {
            // opaque copy of the thread index: keeps the epilogue's lane
            // arithmetic here instead of live (and spilled) across the K loop
            int etid = tid;
            asm volatile("" : "+v"(etid));
            const uint64_t tile_off = (static_cast<uint64_t>(m0) * a.N + n0) * 2u;
            const uint64_t records = static_cast<uint64_t>(a.M - m0) * out_row_bytes - static_cast<uint64_t>(n0) * 2u;
            const int cols_left = a.N - n0;
            constexpr int NCH = C::NSTG * C::ROUNDS;
            u32x4 vals[NCH];
            uint32_t ooff[NCH];
#pragma unroll
            for (int q = 0; q < C::NSTG; ++q) {
                const uint8_t* slot = &ring[q][0];
#pragma unroll
                for (int rr = 0; rr < C::ROUNDS; ++rr) {
                    const int ci = etid + C::NT * rr;             // chunk within this slot
                    const bool live = (C::SLOT_CHUNKS % C::NT == 0) || ci < C::SLOT_CHUNKS;
                    const int cic = live ? ci : 0;
                    const int qrow = cic / C::CPR;
                    const int c = cic - qrow * C::CPR;
                    const int row = q * C::QROWS + qrow;
                    const int pc = C::XOR_SWIZZLE ? (c ^ (qrow & 15)) : c;
                    vals[q * C::ROUNDS + rr] = *reinterpret_cast<const u32x4*>(slot + qrow * C::C_PITCH + pc * 16);
                    ooff[q * C::ROUNDS + rr] = (live && c * 8 < cols_left)
                                                   ? static_cast<uint32_t>(row) * out_row_bytes + static_cast<uint32_t>(c) * 16u
                                                   : kOutOfRange;
                }
            }
#pragma unroll
            for (int i = 0; i < W; ++i) {   // local region first, then the rotated peers
                const __amdgpu_buffer_rsrc_t rd = make_rsrc(dest[i] + tile_off, records);
#pragma unroll
                for (int j = 0; j < NCH; ++j)
                    __builtin_amdgcn_raw_buffer_store_b128(vals[j], rd, ooff[j], 0, AG_GEMM_STORE_AUX);
            }
        }
        wait_lgkmcnt0();
        __builtin_amdgcn_s_barrier();   // staging reads done before the next tile's loads land
    }
}

// Instantiated configurations: tile, wave grid, K per stage, ring slots,
// alternating loaders.  K = 64 per stage makes every operand row of a stage a
// full 128-byte line (measured 1.7x the L2 -> LDS throughput of 64-byte
// rows), at the price of only two ring slots for the 256-row tiles.
// Alternating loaders measured 5-7% faster at 256 x 224 (915 -> 850 us per
// W=8 call at M_local 16384) and 5-7% at 256 x 256 (928 -> 879 us in fp16,
// 900 -> 840 in bf16, 254 -> 206 VGPRs with single-buffered fragments).
#ifndef AG_GEMM_CFG_256x256
#define AG_GEMM_CFG_256x256 256, 256, AG_GEMM_WGM, 2, 64, 2, true
#endif
#ifndef AG_GEMM_CFG_256x224
#define AG_GEMM_CFG_256x224 256, 224, AG_GEMM_WGM, 2, 64, 2, true
#endif
#ifndef AG_GEMM_CFG_128x128
#define AG_GEMM_CFG_128x128 128, 128, AG_GEMM_WGM, 2, 64, 4, false
#endif
using CfgT256x256 = Cfg<AG_GEMM_CFG_256x256>;
using CfgT256x224 = Cfg<AG_GEMM_CFG_256x224>;
using CfgT128x128 = Cfg<AG_GEMM_CFG_128x128>;

using GemmFn = void (*)(GemmKernelArgs);

template <bool BF16, class C, bool BT>
GemmFn pick_world(int w)
{
    switch (w) {
    case 1: return ag_gemm_kernel<BF16, 1, C, BT>;
    case 2: return ag_gemm_kernel<BF16, 2, C, BT>;
    case 3: return ag_gemm_kernel<BF16, 3, C, BT>;
    case 4: return ag_gemm_kernel<BF16, 4, C, BT>;
    case 5: return ag_gemm_kernel<BF16, 5, C, BT>;
    case 6: return ag_gemm_kernel<BF16, 6, C, BT>;
    case 7: return ag_gemm_kernel<BF16, 7, C, BT>;
    case 8: return ag_gemm_kernel<BF16, 8, C, BT>;
    default: return nullptr;
    }
}

// N-contiguous B has kernels for the 256x224 and 128x128 tiles (256x256 would
// need more LDS reads per K-step than the 4-bit LDS counter tracks)
template <bool BF16>
GemmFn pick_cfg(int cfg, int w, bool bt)
{
    switch (cfg) {
    case kGemmTile256x256: return bt ? nullptr : pick_world<BF16, CfgT256x256, false>(w);
    case kGemmTile256x224: return bt ? pick_world<BF16, CfgT256x224, true>(w) : pick_world<BF16, CfgT256x224, false>(w);
    case kGemmTile128x128: return bt ? pick_world<BF16, CfgT128x128, true>(w) : pick_world<BF16, CfgT128x128, false>(w);
    default: return nullptr;
    }
}

}  // namespace

void gemm_resources(int cfg, int* threads, int* lds_bytes)
{
    switch (cfg) {
    case kGemmTile256x256: *threads = CfgT256x256::NT; *lds_bytes = CfgT256x256::NS * CfgT256x256::STAGE; break;
    case kGemmTile256x224: *threads = CfgT256x224::NT; *lds_bytes = CfgT256x224::NS * CfgT256x224::STAGE; break;
    default: *threads = CfgT128x128::NT; *lds_bytes = CfgT128x128::NS * CfgT128x128::STAGE; break;
    }
}

hipError_t launch_gemm(const GemmLaunch& l, hipStream_t stream)
{
    GemmFn fn = l.bf16 ? pick_cfg<true>(l.cfg, l.world, l.b_n_contiguous != 0)
                       : pick_cfg<false>(l.cfg, l.world, l.b_n_contiguous != 0);
    if (fn == nullptr || l.grid < 1) return hipErrorInvalidValue;
    int threads = 0, lds = 0;
    gemm_resources(l.cfg, &threads, &lds);
    hipLaunchKernelGGL(fn, dim3(l.grid), dim3(threads), 0, stream, l.args);
    return hipGetLastError();
}

}  // namespace ag
