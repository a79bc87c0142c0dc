// Tiled GEMM C = A * B for gfx950 with a swizzled, optionally persistent tile schedule.
//
// What is computed follows the GEMM kernel of "CUDA Thread Block Swizzle" (leimao.github.io),
// section "CUDA Thread Block Swizzle Benchmark": every workgroup p walks tile ids p, p + P, p + 2P,
// ... (P = workgroups launched), maps each id to an output tile (m, n) through the selected order,
// and accumulates that tile in fp32 over k before casting to the output type. The order decides only
// when a tile is computed, never its value.
//
// How it is computed on CDNA4:
//   * 256 threads = 4 wave64s arranged 2 x 2; each wave owns a (BM/2) x (BN/2) sub-tile made of
//     32 x 32 MFMA blocks (v_mfma_f32_32x32x16_{f16,bf16}) with fp32 accumulators.
//   * Per 64-wide k step, A (BM x 64) and B (64 x BN) move global -> registers with 16-byte loads
//     and registers -> LDS. LDS holds A as BM rows of 64 k values and B transposed, as BN rows of
//     64 k values, so both MFMA operands read 8 consecutive k values (one 16-byte chunk) per lane.
//     B is transposed in registers, in 8 x 8 blocks, on its way into LDS.
//   * Each 128-byte LDS row is 8 chunks of 16 bytes; chunk c of row r is stored at chunk
//     c XOR ((r XOR (r >> 3)) mod 8). This is the chunk-XOR swizzle of "CUDA Swizzle & bank
//     conflict" (sections "Hopper TMA 的 swizzling" and "Triton - Shared Layout swizzling", vec = 8
//     halves) with a phase that mixes two row bit-fields: the low 3 bits spread the 32 rows an MFMA
//     operand read touches across all chunk columns, and bits 3..5 spread the rows 8 apart that the
//     transposed B store writes in one instruction.
//   * Two LDS stages: the loads of step k+1 are in flight while step k multiplies; one barrier per
//     step.
//   * The MFMA is issued with B as its first operand, so each lane ends up holding 4 consecutive
//     output columns of one row and stores them with one 8-byte (16-bit output) or 16-byte (fp32
//     output) store.
#include <stdint.h>

#include "internal.hpp"

namespace tbl {
namespace {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kThreads = 256;
constexpr int kBK = 64;          // k depth of one LDS stage
constexpr int kRowBytes = 128;   // one LDS row: 64 sixteen-bit values = 8 chunks of 16 bytes

__device__ __forceinline__ int swizzle_phase(int row) { return (row ^ (row >> 3)) & 7; }

// Byte offset of logical chunk ``chunk`` of LDS row ``row``.
__device__ __forceinline__ int lds_offset(int row, int chunk) {
  return row * kRowBytes + ((chunk ^ swizzle_phase(row)) << 4);
}

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

__device__ __forceinline__ uint32_t word(const uint4& v, int i) {
  return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

// rows[e] holds 8 sixteen-bit values of row e (columns 0..7); cols[q] receives column q (rows 0..7).
__device__ __forceinline__ void transpose_8x8_b16(const uint4 (&rows)[8], uint4 (&cols)[8]) {
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    uint32_t w[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t lo = word(rows[2 * e], q >> 1);
      const uint32_t hi = word(rows[2 * e + 1], q >> 1);
      w[e] = (q & 1) ? ((lo >> 16) | (hi & 0xFFFF0000u)) : ((lo & 0xFFFFu) | (hi << 16));
    }
    cols[q] = make_uint4(w[0], w[1], w[2], w[3]);
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

template <int BM, int BN, bool kBf16, bool kF32Out>
__global__ __launch_bounds__(kThreads) void gemm_kernel(const uint16_t* __restrict__ A,
                                                        const uint16_t* __restrict__ B,
                                                        void* __restrict__ Cv, int M, int N, int K,
                                                        TileOrder order, int num_programs,
                                                        int32_t* __restrict__ trace) {
  constexpr int WM = BM / 2, WN = BN / 2;          // wave sub-tile
  constexpr int TM = WM / 32, TN = WN / 32;        // 32 x 32 MFMA blocks per wave
  constexpr int kABytes = BM * kRowBytes;
  constexpr int kStage = (BM + BN) * kRowBytes;
  constexpr int kALoads = BM * (kBK / 8) / kThreads;            // 16-byte chunks of A per thread
  constexpr int kBBlocks = (BN / 8) * (kBK / 8);                // 8 x 8 blocks of B per stage
  constexpr int kBPerThread = (kBBlocks + kThreads - 1) / kThreads;
  static_assert(kALoads >= 1 && BM * (kBK / 8) % kThreads == 0, "A tile must split over the threads");
  static_assert(kBBlocks % 64 == 0, "B blocks must fill whole waves");

  __shared__ __attribute__((aligned(16))) char lds[2 * kStage];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int nk = K / kBK;
  (void)M;

  int iter = 0;
  for (int t = blockIdx.x; t < order.tiles; t += num_programs, ++iter) {
    int tile_m, tile_n;
    order_tile(order, t, tile_m, tile_n);
    if (trace != nullptr && tid == 0) {
      int32_t* rec = trace + 5 * static_cast<size_t>(t);
      rec[0] = blockIdx.x;
      rec[1] = iter;
      rec[2] = tile_m;
      rec[3] = tile_n;
      rec[4] = xcc_id();
    }
    const uint16_t* a_tile = A + static_cast<size_t>(tile_m) * BM * K;
    const uint16_t* b_tile = B + static_cast<size_t>(tile_n) * BN;

    uint4 a_reg[kALoads];
    uint4 b_reg[kBPerThread][8];

    auto global_load = [&](int k0) {
#pragma unroll
      for (int j = 0; j < kALoads; ++j) {
        const int q = tid + j * kThreads;
        const int row = q >> 3, chunk = q & 7;
        a_reg[j] = *reinterpret_cast<const uint4*>(a_tile + static_cast<size_t>(row) * K + k0 + chunk * 8);
      }
#pragma unroll
      for (int j = 0; j < kBPerThread; ++j) {
        const int blk = tid + j * kThreads;
        if (blk < kBBlocks) {
          const int nb = blk % (BN / 8), kb = blk / (BN / 8);
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            b_reg[j][e] = *reinterpret_cast<const uint4*>(
                b_tile + static_cast<size_t>(k0 + kb * 8 + e) * N + nb * 8);
          }
        }
      }
    };

    auto lds_store = [&](int stage) {
      char* sa = lds + stage * kStage;
      char* sb = sa + kABytes;
#pragma unroll
      for (int j = 0; j < kALoads; ++j) {
        const int q = tid + j * kThreads;
        *reinterpret_cast<uint4*>(sa + lds_offset(q >> 3, q & 7)) = a_reg[j];
      }
#pragma unroll
      for (int j = 0; j < kBPerThread; ++j) {
        const int blk = tid + j * kThreads;
        if (blk < kBBlocks) {
          const int nb = blk % (BN / 8), kb = blk / (BN / 8);
          uint4 cols[8];
          transpose_8x8_b16(b_reg[j], cols);
#pragma unroll
          for (int q = 0; q < 8; ++q) {
            *reinterpret_cast<uint4*>(sb + lds_offset(nb * 8 + q, kb)) = cols[q];
          }
        }
      }
    };

    f32x16_t acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) acc[i][j] = f32x16_t{};

    global_load(0);
    lds_store(0);
    __syncthreads();

    for (int kt = 0; kt < nk; ++kt) {
      const int cur = kt & 1;
      if (kt + 1 < nk) global_load((kt + 1) * kBK);
      const char* sa = lds + cur * kStage;
      const char* sb = sa + kABytes;
#pragma unroll
      for (int s = 0; s < kBK / 16; ++s) {
        const int chunk = 2 * s + (lane >> 5);
        uint4 af[TM], bf[TN];
#pragma unroll
        for (int i = 0; i < TM; ++i)
          af[i] = *reinterpret_cast<const uint4*>(sa + lds_offset(wm * WM + i * 32 + (lane & 31), chunk));
#pragma unroll
        for (int j = 0; j < TN; ++j)
          bf[j] = *reinterpret_cast<const uint4*>(sb + lds_offset(wn * WN + j * 32 + (lane & 31), chunk));
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j) acc[i][j] = mfma32x32x16<kBf16>(bf[j], af[i], acc[i][j]);
      }
      if (kt + 1 < nk) lds_store(cur ^ 1);
      __syncthreads();
    }

    // Lane l holds, for MFMA block (i, j) and group g, row (l mod 32) and columns
    // 8g + 4*(l div 32) .. +3 of that 32 x 32 block.
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const size_t row = static_cast<size_t>(tile_m) * BM + wm * WM + i * 32 + (lane & 31);
#pragma unroll
      for (int j = 0; j < TN; ++j) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int col = tile_n * BN + wn * WN + j * 32 + 8 * g + 4 * (lane >> 5);
          const float v0 = acc[i][j][4 * g + 0], v1 = acc[i][j][4 * g + 1];
          const float v2 = acc[i][j][4 * g + 2], v3 = acc[i][j][4 * g + 3];
          if constexpr (kF32Out) {
            float* C = static_cast<float*>(Cv);
            *reinterpret_cast<float4*>(C + row * N + col) = make_float4(v0, v1, v2, v3);
          } else {
            uint16_t* C = static_cast<uint16_t*>(Cv);
            const uint32_t lo = to_out16(v0, kBf16) | (static_cast<uint32_t>(to_out16(v1, kBf16)) << 16);
            const uint32_t hi = to_out16(v2, kBf16) | (static_cast<uint32_t>(to_out16(v3, kBf16)) << 16);
            *reinterpret_cast<uint2*>(C + row * N + col) = make_uint2(lo, hi);
          }
        }
      }
    }
  }
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

bool gemm_tile_supported(int bm, int bn, int bk) {
  return bk == kBK && bm == bn && (bm == 64 || bm == 128 || bm == 256);
}

hipError_t launch_gemm(int dtype, int bm, int bn, int bk, const GemmLaunch& a, hipStream_t s) {
  if (!gemm_tile_supported(bm, bn, bk)) return hipErrorInvalidValue;
  if (bm == 64) return launch<64, 64>(dtype, a, s);
  if (bm == 128) return launch<128, 128>(dtype, a, s);
  return launch<256, 256>(dtype, a, s);
}

hipError_t gemm_blocks_per_cu(int dtype, int bm, int bn, int bk, int* out) {
  if (!gemm_tile_supported(bm, bn, bk)) return hipErrorInvalidValue;
  const void* k = bm == 64 ? kernel_for<64, 64>(dtype)
                : bm == 128 ? kernel_for<128, 128>(dtype) : kernel_for<256, 256>(dtype);
  if (k == nullptr) return hipErrorInvalidValue;
  return hipOccupancyMaxActiveBlocksPerMultiprocessor(out, k, kThreads, 0);
}

}  // namespace tbl
