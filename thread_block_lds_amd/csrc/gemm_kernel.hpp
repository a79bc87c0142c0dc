// The four-wave GEMM kernel template (64 x 64 and 128 x 128 tiles; launched from gemm.hip) and
// the helpers it shares with the eight-wave 256 x 256 kernel of gemm_pp_kernel.hpp: direct-to-LDS
// loads, wait counts, LDS swizzles, the MFMA wrappers and the epilogues (store_tile16, store_tile).
//
// Tiled GEMM C = A * B for gfx950 with a swizzled, optionally persistent tile schedule.
//
// What is computed follows the GEMM kernel of "CUDA Thread Block Swizzle" (leimao.github.io),
// section "CUDA Thread Block Swizzle Benchmark": workgroup p walks tile ids p, p + P, p + 2P, ...
// (P = workgroups launched), maps each id to an output tile (m, n) through the selected order, and
// accumulates that tile in fp32 over k before casting to the output type. The order decides only
// when a tile is computed, never its value.
//
// How it is computed on CDNA4:
//   * 256 threads = 4 wave64s arranged 2 x 2; each wave owns a (BM/2) x (BN/2) sub-tile made of
//     16 x 16 MFMA blocks (v_mfma_f32_16x16x32_{f16,bf16}) with fp32 accumulators in VGPRs, as the
//     eight-wave kernel (the 32 x 32 x 16 MFMA form remains in that kernel's layout variants).
//   * A workgroup's tiles form one stream of 32-deep k steps (tile after tile). Operands move
//     global -> LDS with direct-to-LDS 16-byte buffer loads (no registers in between) into five
//     LDS stages of (BM + BN) x 32 sixteen-bit values, issued four steps ahead of their use, also
//     across tile boundaries, so the next tile's first steps load during the current epilogue.
//   * A sits in LDS row-major (one 64-byte row of k per m); B sits k-major as loaded (one row of
//     BN values per k) and is read transposed by ds_read_b64_tr_b16, which hands each lane the
//     8 consecutive k of one column that the MFMA B operand wants; no register transposes.
//   * LDS swizzles (the chunk-XOR idea of "CUDA Swizzle & bank conflict", sections "Hopper TMA 的
//     swizzling" and "Triton - Shared Layout swizzling", applied to 16-byte chunks and sized to
//     gfx950's 64 x 4-byte banks), chosen for the 16 x 16 x 32 read patterns: A chunk c of row r at
//     c XOR ((r >> 1) mod 4); B chunk c of row k at c XOR swz_b_four_wave(k). The XOR is applied on
//     the global-address side of the direct loads, whose LDS destinations are fixed (lane l writes
//     bytes 16 l .. 16 l + 15 of its 1 KiB block).
//   * One barrier per 32-deep step; the step's MFMAs run on fragments read during the previous step,
//     while the next step's fragments are read and the loads four steps ahead issue in between.
//   * The MFMA is issued with B as its first operand, so each lane ends up holding 4 consecutive
//     output columns of one row; the epilogue stores 16 bytes per lane.
//   * At most 256 registers per wave (two waves per SIMD): the compiler then keeps the
//     accumulators in VGPRs, updated in place, instead of the AGPRs it would otherwise pick.
#pragma once

#include <stdint.h>

#include "internal.hpp"

namespace tbl {
namespace {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;
typedef __attribute__((address_space(3))) void lds_void_t;

constexpr int kThreads = 256;
constexpr int kBK = 32;          // k depth of one step / LDS stage
constexpr int kStages = 5;       // LDS stages in flight
constexpr int kARow = kBK * 2;   // bytes of one A row in LDS: 32 sixteen-bit values = 4 chunks
constexpr int kTraceInts = 8;    // int32 per tile in the optional schedule trace

template <bool kBf16>
__device__ __forceinline__ f32x16_t mfma32x32x16(uint4 a, uint4 b, f32x16_t c) {
  if constexpr (kBf16) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(half8_t, a),
                                                  __builtin_bit_cast(half8_t, b), c, 0, 0, 0);
  }
}

__device__ __forceinline__ uint16_t to_out16(float v, bool bf16) {
  if (bf16) return __builtin_bit_cast(uint16_t, static_cast<__bf16>(v));
  return __builtin_bit_cast(uint16_t, static_cast<_Float16>(v));
}

__device__ __forceinline__ int xcc_id() {
  // HW_REG_XCC_ID (hardware register 20), bits [3:0]: the XCD this wave runs on.
  return __builtin_amdgcn_s_getreg((3 << 11) | (0 << 6) | 20) & 0xF;
}

typedef int i32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) char lds_char_t;

// Raw buffer descriptor over [base, base + bytes): loads past ``bytes`` return zero.
__device__ __forceinline__ i32x4_t make_desc(const void* base, size_t bytes) {
  const uint64_t b = reinterpret_cast<uint64_t>(base);
  const unsigned n = bytes > 0xFFFFFFFFull ? 0xFFFFFFFFu : static_cast<unsigned>(bytes);
  // The values are wave-uniform; readfirstlane makes that explicit so they live in SGPRs.
  return i32x4_t{__builtin_amdgcn_readfirstlane(static_cast<int>(static_cast<unsigned>(b))),
                 __builtin_amdgcn_readfirstlane(static_cast<int>((b >> 32) & 0xFFFFu)),
                 __builtin_amdgcn_readfirstlane(static_cast<int>(n)), 0x00020000};
}

// 16 bytes per lane from desc + voffset straight into LDS: lane l writes lds_addr + 16 l.
// Issued as inline asm so that the compiler's wait-count pass, which would otherwise make every
// later LDS read wait for all direct loads in flight, leaves the waits to the explicit ones below.
// M0 carries the LDS address; nothing else in this kernel keeps a value in M0.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void load_to_lds(i32x4_t desc, unsigned lds_addr, int voffset) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :: "s"(__builtin_amdgcn_readfirstlane(lds_addr)), "v"(voffset), "s"(desc) : "memory", "m0");
}
#pragma clang diagnostic pop

#define TBL_WAIT_VMCNT(n) asm volatile("s_waitcnt vmcnt(" #n ")" ::: "memory")

// s_waitcnt vmcnt(N): wait until at most N vector-memory operations of this wave are in flight.
// They retire in issue order on this architecture, so every older one has then completed.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  if constexpr (N == 0) TBL_WAIT_VMCNT(0);
  else if constexpr (N == 1) TBL_WAIT_VMCNT(1);
  else if constexpr (N == 2) TBL_WAIT_VMCNT(2);
  else if constexpr (N == 3) TBL_WAIT_VMCNT(3);
  else if constexpr (N == 4) TBL_WAIT_VMCNT(4);
  else if constexpr (N == 5) TBL_WAIT_VMCNT(5);
  else if constexpr (N == 6) TBL_WAIT_VMCNT(6);
  else if constexpr (N == 8) TBL_WAIT_VMCNT(8);
  else if constexpr (N == 10) TBL_WAIT_VMCNT(10);
  else if constexpr (N == 12) TBL_WAIT_VMCNT(12);
  else if constexpr (N == 20) TBL_WAIT_VMCNT(20);
  else if constexpr (N == 24) TBL_WAIT_VMCNT(24);
  else static_assert(N < 0, "add this count");
}

// Workgroup barrier that is also a compiler memory barrier. It first waits for this wave's LDS
// reads (so no wave reads a stage that another wave refills after the barrier), but not for the
// direct loads in flight, which __syncthreads() would drain.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

__device__ __forceinline__ unsigned lds_address(const char* p) {
  return static_cast<unsigned>(reinterpret_cast<uintptr_t>((const lds_char_t*)p));   // generic -> LDS offset
}

// LDS swizzles, the chunk-XOR family of the Triton shared layouts ("CUDA Swizzle & bank conflict",
// section "Triton - Shared Layout swizzling"), on 16-byte chunks: row r of A stores logical chunk c
// at chunk c XOR ((r / kAPP) mod kAMP); row k of B stores chunk c at chunk
// c XOR ((((k / kBPP) mod kBMP) * kBV) mod chunks-per-row), i.e. the XOR unit is kBV chunks.
template <int kAPP, int kAMP>
__device__ __forceinline__ int swz_a(int r) {
  return (r / kAPP) % kAMP;
}
template <int kBV, int kBPP, int kBMP, int kChunks>
__device__ __forceinline__ int swz_b(int k) {
  return (((k / kBPP) % kBMP) * kBV) & (kChunks - 1);
}

// The 16 x 16 x 32 MFMA (v_mfma_f32_16x16x32_{f16,bf16}); its lane layout, checked on the device:
// first operand lane l holds row l mod 16, k 8 (l / 16) .. + 7; second operand lane l holds k
// 8 (l / 16) .. + 7 of column l mod 16; the result lane l holds rows 4 (l / 16) .. + 3 of column
// l mod 16. Issued with B as the first operand (as the 32 x 32 form), each lane ends up holding 4
// consecutive output columns of one row.
typedef float f32x4_t __attribute__((ext_vector_type(4)));
template <bool kBf16>
__device__ __forceinline__ f32x4_t mfma16x16x32(uint4 a, uint4 b, f32x4_t c) {
  if constexpr (kBf16) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, a),
                                                  __builtin_bit_cast(half8_t, b), c, 0, 0, 0);
  }
}

// B swizzle for the 16 x 16 x 32 operand reads: chunk c of row k at c XOR (4 (k mod 4) + 2 ((k / 8)
// mod 2)). One transposing read of a 32-lane phase touches 16 column bytes of rows k0 .. k0 + 3 and
// k0 + 8 .. k0 + 11; the first term spreads the four rows of each quad over the 256-byte bank window
// (as the 32 x 32 layout's XOR does), the second separates the two quads, so the phase's 32 pieces
// of 8 bytes land on 32 distinct bank pairs.
__device__ __forceinline__ int swz_b16(int k) { return (4 * (k & 3)) | (2 * ((k >> 3) & 1)); }

// The B chunk XOR a kernel instantiation uses: in the 16 x 16 x 32 form kBV = 0 selects swz_b16 (the
// default); any other (kBV, kBPP, kBMP) is that member of the chunk-XOR family.
template <bool kM16, int kBV, int kBPP, int kBMP, int kChunks>
__device__ __forceinline__ int swz_b_of(int k) {
  if constexpr (kM16 && kBV == 0) return swz_b16(k);
  else return swz_b<kBV, kBPP, kBMP, kChunks>(k);
}

// Store a wave's sub-tile of 16 x 16 accumulator blocks: lane l holds row (l mod 16) and columns
// 4 (l / 16) .. + 3 of block (i, j). fp32 output stores those 16 bytes per lane (64 contiguous
// bytes of each of 16 rows per store). 16-bit output packs each block's four values into 8 bytes
// and pairs blocks j and j + 1 with v_permlane16_swap (rows 1 and 3 of 16 lanes of the first operand
// trade places with rows 0 and 2 of the second): afterwards lane group g = l / 16 holds columns
// 8 (g / 2) .. + 7 of block j + (g mod 2), so each store writes 16 bytes per lane and 64 contiguous
// bytes of each of 16 rows, half as many stores of twice the width as 8-byte pieces.
template <int BM, int BN, int WM, int WN, int TM, int TN, bool kBf16, bool kF32Out>
__device__ __forceinline__ void store_tile16(f32x4_t (&acc)[TM][TN], void* __restrict__ Cv, int M, int N,
                                             int tile_m, int tile_n, int wm, int wn, int lane) {
  static_assert(kF32Out || TN % 2 == 0, "16-bit stores pair adjacent blocks");
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    const size_t row = static_cast<size_t>(tile_m) * BM + wm * WM + i * 16 + (lane & 15);
    if constexpr (kF32Out) {
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const size_t col = static_cast<size_t>(tile_n) * BN + wn * WN + j * 16 + 4 * (lane >> 4);
        if (row >= static_cast<size_t>(M) || col >= static_cast<size_t>(N)) continue;  // N % 8 == 0
        float* C = static_cast<float*>(Cv);
        *reinterpret_cast<float4*>(C + row * N + col) =
            make_float4(acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]);
      }
    } else {
      uint16_t* C = static_cast<uint16_t*>(Cv);
      const int g = lane >> 4;
#pragma unroll
      for (int j = 0; j < TN; j += 2) {
        uint32_t pk[2][2];
#pragma unroll
        for (int b = 0; b < 2; ++b) {
          pk[b][0] = to_out16(acc[i][j + b][0], kBf16) | (static_cast<uint32_t>(to_out16(acc[i][j + b][1], kBf16)) << 16);
          pk[b][1] = to_out16(acc[i][j + b][2], kBf16) | (static_cast<uint32_t>(to_out16(acc[i][j + b][3], kBf16)) << 16);
        }
        const auto lo = __builtin_amdgcn_permlane16_swap(pk[0][0], pk[1][0], false, false);
        const auto hi = __builtin_amdgcn_permlane16_swap(pk[0][1], pk[1][1], false, false);
        const size_t col = static_cast<size_t>(tile_n) * BN + wn * WN + (j + (g & 1)) * 16 + 8 * (g >> 1);
        if (row >= static_cast<size_t>(M) || col >= static_cast<size_t>(N)) continue;  // N % 8 == 0
        *reinterpret_cast<uint4*>(C + row * N + col) = make_uint4(lo[0], hi[0], lo[1], hi[1]);
      }
    }
  }
}

// Store a wave's sub-tile of the output tile (tile_m, tile_n); the wave sits at (wm, wn) in the
// workgroup's wave grid and holds TM x TN accumulator blocks of 32 x 32.
// Lane l holds, for MFMA block (i, j) and group g, row (l mod 32) and columns
// 8g + 4*(l div 32) .. +3 of that 32 x 32 block. Accumulators stay in AGPRs until their block is
// stored: fp32 stores take AGPR data directly (16 bytes per lane, 32 contiguous bytes per row and
// store). The 16-bit path copies one block at a time to VGPRs (an explicit v_accvgpr_read keeps
// the compiler from copying all of them up front), packs each group's four values into 8 bytes,
// and swaps halves of the wave between groups g and g + 1 (v_permlane32_swap: lanes 32..63 of
// the first operand trade places with lanes 0..31 of the second), after which lane l < 32 holds
// columns 16p .. 16p + 7 of its row and lane l + 32 columns 16p + 8 .. 16p + 15, for p = g / 2.
// Each store then writes 16 bytes per lane and 32 contiguous bytes per row, half as many
// stores of twice the width, which the memory system drains several times faster than 8-byte
// pieces when every workgroup stores its tile at once.
template <int BM, int BN, int WM, int WN, int TM, int TN, bool kBf16, bool kF32Out>
__device__ __forceinline__ void store_tile(f32x16_t (&acc)[TM][TN], void* __restrict__ Cv, int M, int N,
                                           int tile_m, int tile_n, int wm, int wn, int lane) {
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    const size_t row = static_cast<size_t>(tile_m) * BM + wm * WM + i * 32 + (lane & 31);
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const size_t col0 = static_cast<size_t>(tile_n) * BN + wn * WN + j * 32;
      if constexpr (kF32Out) {
        float* C = static_cast<float*>(Cv);
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const size_t col = col0 + 8 * g + 4 * (lane >> 5);
          if (row >= static_cast<size_t>(M) || col >= static_cast<size_t>(N)) continue;  // N % 8 == 0
          *reinterpret_cast<float4*>(C + row * N + col) =
              make_float4(acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]);
        }
      } else {
        float v[16];
#pragma unroll
        for (int r = 0; r < 16; ++r)
          asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(v[r]) : "a"(acc[i][j][r]) : "memory");
        uint32_t pk[4][2];
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          pk[g][0] = to_out16(v[4 * g], kBf16) | (static_cast<uint32_t>(to_out16(v[4 * g + 1], kBf16)) << 16);
          pk[g][1] = to_out16(v[4 * g + 2], kBf16) | (static_cast<uint32_t>(to_out16(v[4 * g + 3], kBf16)) << 16);
        }
        uint16_t* C = static_cast<uint16_t*>(Cv);
#pragma unroll
        for (int p = 0; p < 2; ++p) {
          const auto lo = __builtin_amdgcn_permlane32_swap(pk[2 * p][0], pk[2 * p + 1][0], false, false);
          const auto hi = __builtin_amdgcn_permlane32_swap(pk[2 * p][1], pk[2 * p + 1][1], false, false);
          const size_t col = col0 + 16 * p + 8 * (lane >> 5);
          if (row >= static_cast<size_t>(M) || col >= static_cast<size_t>(N)) continue;  // N % 8 == 0
          *reinterpret_cast<uint4*>(C + row * N + col) = make_uint4(lo[0], hi[0], lo[1], hi[1]);
        }
      }
      __builtin_amdgcn_sched_barrier(0);   // one 32 x 32 block at a time
    }
  }
}

// B chunk XOR of the four-wave kernel's 16 x 16 x 32 reads for its row width: 256-byte rows (128
// columns) take swz_b16; 128-byte rows (64 columns) hold two rows per 256-byte bank window, and one
// half-wave phase of the transposing read touches rows k0 .. k0 + 3 and k0 + 8 .. k0 + 11 (32 bytes
// of each): the rows of one parity must then sit at 4 distinct 32-byte positions of their half of
// the window, which 2 ((k / 2) mod 2) + 4 ((k / 8) mod 2) (in 16-byte chunks) gives. Both are
// conflict-free under the bank model of the oracle (64 banks, 32-lane phases).
template <int BN>
__device__ __forceinline__ int swz_b_four_wave(int k) {
  if constexpr (BN == 64) return 2 * ((k >> 1) & 1) + 4 * ((k >> 3) & 1);
  else return swz_b16(k);
}

template <int BM, int BN, bool kBf16, bool kF32Out>
__global__ __launch_bounds__(kThreads, 2) void gemm_kernel(const uint16_t* __restrict__ A,
                                                        const uint16_t* __restrict__ B,
                                                        void* __restrict__ Cv, int M, int N, int K,
                                                        TileOrder order, int num_programs,
                                                        int32_t* __restrict__ trace) {
  constexpr int WM = BM / 2, WN = BN / 2;          // wave sub-tile (2 x 2 waves)
  constexpr int TM = WM / 16, TN = WN / 16;        // 16 x 16 MFMA blocks per wave
  constexpr int kBRow = BN * 2;                    // bytes of one B row (one k) in LDS
  constexpr int kAStage = BM * kARow;
  constexpr int kBStage = kBK * kBRow;
  constexpr int kStage = kAStage + kBStage;
  constexpr int kAInst = kAStage / 1024 / 4;       // 1 KiB direct loads per wave per step
  constexpr int kBInst = kBStage / 1024 / 4;
  constexpr int kLoads = kAInst + kBInst;
  constexpr int kAPP = 2, kAMP = 4;                // A swizzle: chunk c of row r at c XOR ((r / 2) mod 4)
  static_assert(kAInst >= 1 && kBInst >= 1, "each wave loads at least one block of A and B");
  static_assert(kStages == 5, "the wait counts assume four steps in flight");
  static_assert(TN % 2 == 0, "the 16-bit epilogue pairs adjacent blocks");

  __shared__ __attribute__((aligned(1024))) char lds[kStages * kStage];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int nk = (K + kBK - 1) / kBK;
  const int P = num_programs;
  if (static_cast<int>(blockIdx.x) >= order.tiles) return;
  const int my_tiles = (order.tiles - 1 - static_cast<int>(blockIdx.x)) / P + 1;
  const int total = my_tiles * nk;

  // ---- per-lane constants ----
  // Direct loads. A block (16 rows of 64 bytes): lane l fills physical chunk l mod 4 of row l / 4,
  // which holds logical chunk (l mod 4) XOR swz_a(row). In the last k step of a K that is not a
  // multiple of 32, chunks at k >= K belong to the next row of A; a_voff_tail points those lanes
  // past the buffer range, so they read zero.
  constexpr int kOutOfRange = 0x7FFFFFF0;
  int a_voff[kAInst], a_voff_tail[kAInst];
#pragma unroll
  for (int j = 0; j < kAInst; ++j) {
    const int row = (wave * kAInst + j) * 16 + (lane >> 2);
    const int chunk = (lane & 3) ^ swz_a<kAPP, kAMP>(row);
    a_voff[j] = (row * K + chunk * 8) * 2;
    a_voff_tail[j] = chunk * 8 + 8 <= K % kBK ? a_voff[j] : kOutOfRange;
  }
  // B block (1 KiB of k-major rows of BN values): lane l fills bytes 16 l of the block.
  int b_voff[kBInst];
#pragma unroll
  for (int j = 0; j < kBInst; ++j) {
    const int o = (wave * kBInst + j) * 1024 + 16 * lane;
    const int k = o / kBRow;
    const int chunk = ((o % kBRow) >> 4) ^ swz_b_four_wave<BN>(k);
    b_voff[j] = (k * N + chunk * 8) * 2;
  }
  // MFMA operand reads (the 16 x 16 x 32 lane layouts, as in the eight-wave kernel): A lane l takes
  // row l mod 16 of a 16-row block at chunk l / 16; B lane L of 16-lane group G addresses the 8-byte
  // row piece k = 8 G + (L mod 16) / 4, columns 4 (L mod 4) .. + 3 of a 16-column block, which the
  // transposing read turns into 4 k of one column per lane (twice: k and k + 4)
  const int a_row = wm * WM + (lane & 15);
  const int a_rd = a_row * kARow + ((lane >> 4) ^ swz_a<kAPP, kAMP>(a_row)) * 16;
  int b_rd[TN];
  {
    const int r = lane & 15;
    const int k = 8 * (lane >> 4) + (r >> 2);
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int n = wn * WN + j * 16 + 4 * (r & 3);
      b_rd[j] = kAStage + k * kBRow + ((n >> 3) ^ swz_b_four_wave<BN>(k)) * 16 + (n & 7) * 2;
    }
  }

  // ---- load cursor: the next step whose operands go to LDS ----
  // Every step issues exactly kLoads direct loads; past the end of this workgroup's stream they
  // read a zero-length buffer (no memory access) into a stage nobody reads again, which keeps the
  // number of loads in flight, and so every wait count, the same at each step.
  int ld_t = blockIdx.x, ld_kt = 0, ld_issued = 0, ld_stage = 0;
  // Running (wave-uniform) positions of the next step's A and B blocks; set with multiplies only
  // when the cursor enters a new tile, then advanced by additions. Each step's buffer ranges end
  // at this tile's last row of A that exists (from k0 on) and at B's last row of this step that
  // exists (k < K); loads past them read zero instead of touching memory. Tile rows past M and
  // columns past N read values that only reach C elements that are never stored.
  uint64_t ld_a = 0, ld_b = 0;
  const unsigned a_step = kBK * 2;                                        // bytes per k step in A
  const uint64_t b_step = static_cast<uint64_t>(kBK) * static_cast<unsigned>(N) * 2;
  const unsigned b_row = static_cast<unsigned>(N) * 2;
  unsigned a_range = 0, b_lead = 0;   // b_lead: n0 * 2, the base's offset into its row
  auto enter_tile = [&]() {
    int m, n;
    order_tile(order, ld_t, m, n);
    m = __builtin_amdgcn_readfirstlane(m);
    n = __builtin_amdgcn_readfirstlane(n);
    const int rows = min(BM, M - m * BM);
    ld_a = reinterpret_cast<uint64_t>(A) +
           static_cast<uint64_t>(static_cast<unsigned>(m)) * BM * static_cast<unsigned>(K) * 2;
    ld_b = reinterpret_cast<uint64_t>(B) + static_cast<uint64_t>(static_cast<unsigned>(n)) * (BN * 2);
    a_range = static_cast<unsigned>(rows) * static_cast<unsigned>(K) * 2;
    b_lead = static_cast<unsigned>(n) * (BN * 2);
  };
  enter_tile();
  i32x4_t ld_da, ld_db;
  unsigned ld_lds = 0;
  bool ld_tail = false;   // the step being issued is a partial last k step
  auto prepare_step = [&]() {
    const bool real = ld_issued < total;
    const int k_left = K - ld_kt * kBK;
    const unsigned b_rows = static_cast<unsigned>(k_left < kBK ? k_left : kBK);
    ld_tail = k_left < kBK;
    ld_da = make_desc(reinterpret_cast<const void*>(ld_a), real ? a_range : 0u);
    ld_db = make_desc(reinterpret_cast<const void*>(ld_b), real ? b_rows * b_row - b_lead : 0u);
    ld_lds = lds_address(lds + ld_stage * kStage);
  };
  auto issue_load = [&](int q) {   // q-th of this wave's kLoads loads of the prepared step
    if (q < kAInst) load_to_lds(ld_da, ld_lds + (wave * kAInst + q) * 1024, ld_tail ? a_voff_tail[q] : a_voff[q]);
    else load_to_lds(ld_db, ld_lds + kAStage + (wave * kBInst + q - kAInst) * 1024, b_voff[q - kAInst]);
  };
  auto advance_load_cursor = [&]() {
    ++ld_issued;
    ld_stage = ld_stage == kStages - 1 ? 0 : ld_stage + 1;
    ld_a += a_step;
    ld_b += b_step;
    a_range -= a_step;   // stays positive: the last step starts before the end of K
    if (++ld_kt == nk) {
      ld_kt = 0;
      ld_t += P;
      if (ld_t < order.tiles) enter_tile();
    }
  };

  // ---- operand fragments, double-buffered by step parity ----
  // Read item q of a step from a stage: items 0 .. TM-1 are A blocks (one 16-byte read each),
  // items TM .. TM + 2 TN - 1 are halves (k and k + 4) of B blocks (one transposing read each).
  constexpr int kReads = TM + 2 * TN;
  uint4 af[2][TM], bf[2][TN];
  auto read_item = [&](int stage, int buf, int q) {
    const char* base = lds + stage * kStage;
    if (q < TM) {
      af[buf][q] = *reinterpret_cast<const uint4*>(base + a_rd + q * 16 * kARow);
    } else {
      const int j = (q - TM) >> 1, t = (q - TM) & 1;
      const uint2 h = __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                                    (lds_s16x4_t*)(base + b_rd[j] + t * 4 * kBRow)));
      if (t == 0) {
        bf[buf][j].x = h.x;
        bf[buf][j].y = h.y;
      } else {
        bf[buf][j].z = h.x;
        bf[buf][j].w = h.y;
      }
    }
  };

  // Accumulators are zeroed in place, each register through a tied asm operand: the compiler can
  // neither see the zero (a visible constant lets it peel the first k step, an MFMA with a zero
  // addend) nor give the zeroed value a register of its own (the tile-end merge inside the k loop
  // then needs no copies of the accumulators).
  f32x4_t acc[TM][TN] = {};
  auto zero_acc = [&]() {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) asm volatile("v_mov_b32 %0, 0" : "+v"(acc[i][j][r]));
  };

  // One 32-deep step: its TM x TN MFMAs (B fragments forward for even i, backward for odd i, so one
  // operand stays at every change of A), the operand reads of the next step and the loads of the
  // step four ahead spread over the MFMA slots; the scheduling barrier after each slot keeps the
  // interleaving, so the matrix pipe has an MFMA queued while loads and reads issue.
  constexpr int kSlots = TM * TN;
  static_assert(kSlots >= kLoads, "one load per slot at most");
  constexpr int kLoadEvery = kSlots / kLoads;
  constexpr int kReadsPerSlot = (kReads + kSlots - 1) / kSlots;
  auto step = [&](int buf, int next_stage) {
#pragma unroll
    for (int q = 0; q < kSlots; ++q) {
      const int i = q / TN, jj = q % TN;
      const int j = (i & 1) ? TN - 1 - jj : jj;
      acc[i][j] = mfma16x16x32<kBf16>(bf[buf][j], af[buf][i], acc[i][j]);
      if (q % kLoadEvery == 0 && q / kLoadEvery < kLoads) issue_load(q / kLoadEvery);
#pragma unroll
      for (int r = 0; r < kReadsPerSlot; ++r)
        if (q * kReadsPerSlot + r < kReads) read_item(next_stage, buf ^ 1, q * kReadsPerSlot + r);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // ---- compute cursor ----
  int c_t = blockIdx.x, c_iter = 0, c_m = 0, c_n = 0;
  order_tile(order, c_t, c_m, c_n);
  // Schedule trace (optional): per tile id, the program, its loop iteration, (m, n), the XCD, the
  // core-clock cycles and 100 MHz real-time ticks from the tile's start to its epilogue, and the
  // start itself (low 32 bits of the real-time counter). A program's first tile starts before its
  // prologue; a later one when its predecessor's epilogue ends.
  uint64_t clk0 = 0, rt0 = 0;
  auto record = [&]() {
    if (trace != nullptr) {
      if (tid == 0) {
        int32_t* rec = trace + kTraceInts * static_cast<size_t>(c_t);
        rec[0] = blockIdx.x;
        rec[1] = c_iter;
        rec[2] = c_m;
        rec[3] = c_n;
        rec[4] = xcc_id();
      }
      clk0 = __builtin_readcyclecounter();
      rt0 = __builtin_amdgcn_s_memrealtime();
    }
  };
  auto record_time = [&]() {
    if (trace != nullptr && tid == 0) {
      int32_t* rec = trace + kTraceInts * static_cast<size_t>(c_t);
      rec[5] = static_cast<int32_t>(__builtin_readcyclecounter() - clk0);
      rec[6] = static_cast<int32_t>(__builtin_amdgcn_s_memrealtime() - rt0);
      rec[7] = static_cast<int32_t>(rt0);
    }
  };
  record();

  // prologue: steps 0 .. 3 in flight; step 0 landed everywhere, then its fragments read
#pragma unroll
  for (int i = 0; i < kStages - 1; ++i) {
    prepare_step();
#pragma unroll
    for (int q = 0; q < kLoads; ++q) issue_load(q);
    advance_load_cursor();
  }
  wait_vm<3 * kLoads>();   // step 0 landed; steps 1..3 may still be in flight
  lds_barrier();
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int q = 0; q < kReads; ++q) read_item(0, 0, q);

  // Step s (global count g, fragments in buffer g mod 2): first this wave's loads of step s + 1 are
  // waited for (two steps of loads, issued later, may stay in flight; an epilogue's stores, issued
  // later still, only make the wait longer) and a barrier certifies step s + 1 in every wave's LDS
  // blocks and every wave's reads of step s done; then the MFMAs of step s run with the reads of step
  // s + 1 and the loads of step s + 4, into the stage of step s - 1, whose reads all finished before
  // the previous barrier.
  // The stream's steps run two per iteration, the first on fragment buffer 0 and the second on
  // buffer 1, so that every buffer index is a compile-time constant (a runtime parity would make the
  // compiler keep two copies of the accumulators and move them at every join); a tile's epilogue
  // follows whichever step ends it.
  int c_stage = 0, kt = 0;
  auto run_step = [&](int buf) {
    wait_vm<2 * kLoads>();
    lds_barrier();
    __builtin_amdgcn_sched_barrier(0);
    prepare_step();
    const int next_stage = c_stage == kStages - 1 ? 0 : c_stage + 1;
    step(buf, next_stage);
    advance_load_cursor();
    c_stage = next_stage;
    if (++kt == nk) {
      kt = 0;
      record_time();
      store_tile16<BM, BN, WM, WN, TM, TN, kBf16, kF32Out>(acc, Cv, M, N, c_m, c_n, wm, wn, lane);
      c_t += P;
      ++c_iter;
      if (c_t < order.tiles) {
        order_tile(order, c_t, c_m, c_n);
        record();
      }
      zero_acc();
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  zero_acc();
  for (int g = 0; g < total; g += 2) {
    run_step(0);
    if (g + 1 < total) run_step(1);
  }
  wait_vm<0>();   // no direct load may still be writing this workgroup's LDS
}

template <int BM, int BN>
const void* kernel_for(int dtype) {
  switch (dtype) {
    case 0: return reinterpret_cast<const void*>(&gemm_kernel<BM, BN, false, false>);
    case 1: return reinterpret_cast<const void*>(&gemm_kernel<BM, BN, true, false>);
    case 2: return reinterpret_cast<const void*>(&gemm_kernel<BM, BN, false, true>);
    case 3: return reinterpret_cast<const void*>(&gemm_kernel<BM, BN, true, true>);
    default: return nullptr;
  }
}

template <int BM, int BN>
hipError_t launch(int dtype, const GemmLaunch& a, hipStream_t s) {
  const dim3 grid(a.num_programs), block(kThreads);
  const uint16_t* A = static_cast<const uint16_t*>(a.A);
  const uint16_t* B = static_cast<const uint16_t*>(a.B);
  switch (dtype) {
    case 0:
      hipLaunchKernelGGL((gemm_kernel<BM, BN, false, false>), grid, block, 0, s, A, B, a.C, a.M, a.N,
                         a.K, a.order, a.num_programs, a.trace);
      break;
    case 1:
      hipLaunchKernelGGL((gemm_kernel<BM, BN, true, false>), grid, block, 0, s, A, B, a.C, a.M, a.N,
                         a.K, a.order, a.num_programs, a.trace);
      break;
    case 2:
      hipLaunchKernelGGL((gemm_kernel<BM, BN, false, true>), grid, block, 0, s, A, B, a.C, a.M, a.N,
                         a.K, a.order, a.num_programs, a.trace);
      break;
    case 3:
      hipLaunchKernelGGL((gemm_kernel<BM, BN, true, true>), grid, block, 0, s, A, B, a.C, a.M, a.N,
                         a.K, a.order, a.num_programs, a.trace);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace
}  // namespace tbl
