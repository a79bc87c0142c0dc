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

typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));

// Raw buffer resource over [base, base + bytes): loads past ``bytes`` return zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, size_t bytes) {
  const int n = bytes > 0xFFFFFFFFull ? -1 : static_cast<int>(static_cast<unsigned>(bytes));
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, n, 0x00020000);
}

__device__ __forceinline__ uint4 buffer_load16(__amdgpu_buffer_rsrc_t r, int voffset, int soffset) {
  const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, voffset, soffset, 0);
  return make_uint4(v.x, v.y, v.z, v.w);
}

template <int BM, int BN, bool kBf16, bool kF32Out>
__global__ __launch_bounds__(kThreads) void gemm_kernel(const uint16_t* __restrict__ A,
                                                        const uint16_t* __restrict__ B,
                                                        void* __restrict__ Cv, int M, int N, int K,
                                                        TileOrder order, int num_programs,
                                                        int32_t* __restrict__ trace) {
  constexpr int WM = BM / 2, WN = BN / 2;          // wave sub-tile
  constexpr int TM = WM / 32, TN = WN / 32;        // 32 x 32 MFMA blocks per wave
  constexpr int kABytes = BM * kRowBytes;          // one A stage
  constexpr int kBBytes = BN * kRowBytes;          // one B stage
  constexpr int kBBase = 2 * kABytes;              // LDS: A0 A1 B0 B1
  constexpr int kALoads = BM * (kBK / 8) / kThreads;            // 16-byte chunks of A per thread
  constexpr int kNBlk = BN / 8;                                 // 8-column blocks of B
  constexpr int kBBlocks = kNBlk * (kBK / 8);                   // 8 x 8 blocks of B per stage
  static_assert(kALoads >= 1 && BM * (kBK / 8) % kThreads == 0, "A tile must split over the threads");
  static_assert(kBBlocks <= kThreads && kBBlocks % 64 == 0, "B blocks must fill whole waves");

  __shared__ __attribute__((aligned(16))) char lds[2 * (kABytes + kBBytes)];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int nk = K / kBK;
  (void)M;

  // ---- per-thread constants (independent of the tile and of k) ----
  // A: chunk (tid & 7) of tile rows (tid >> 3) + 32 j.
  const int a_row0 = tid >> 3, a_chunk = tid & 7;
  const int a_voff = (a_row0 * K + a_chunk * 8) * 2;
  int a_st[kALoads];
#pragma unroll
  for (int j = 0; j < kALoads; ++j) a_st[j] = lds_offset(a_row0 + 32 * j, a_chunk);
  // B: 8 x 8 block (k block kb, column block nb); rows kb*8 + e, columns nb*8 .. nb*8+7.
  const bool b_active = tid < kBBlocks;
  const int nb = tid % kNBlk, kb = tid / kNBlk;
  const int b_voff = (kb * 8 * N + nb * 8) * 2;
  int b_st[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) b_st[q] = kBBase + lds_offset(nb * 8 + q, kb);
  // MFMA operand reads: lane reads row (lane mod 32) of a 32-row block, chunk 2s + lane/32.
  int a_rd[2][4], b_rd[2][4];
#pragma unroll
  for (int p = 0; p < 2; ++p)
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      a_rd[p][s] = lds_offset(wm * WM + p * 32 + (lane & 31), 2 * s + (lane >> 5));
      b_rd[p][s] = kBBase + lds_offset(wn * WN + p * 32 + (lane & 31), 2 * s + (lane >> 5));
    }

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
    const size_t m0 = static_cast<size_t>(tile_m) * BM;
    const size_t n0 = static_cast<size_t>(tile_n) * BN;

    uint4 a_reg[kALoads];
    uint4 b_reg[8];

    auto global_load = [&](int kt) {
      const size_t k0 = static_cast<size_t>(kt) * kBK;
      const uint16_t* a_base = A + m0 * K + k0;
      const uint16_t* b_base = B + k0 * N + n0;
      const __amdgpu_buffer_rsrc_t ra = make_rsrc(a_base, (static_cast<size_t>(M) - m0) * K * 2 - k0 * 2);
      const __amdgpu_buffer_rsrc_t rb = make_rsrc(b_base, (static_cast<size_t>(K) - k0) * N * 2 - n0 * 2);
#pragma unroll
      for (int j = 0; j < kALoads; ++j) a_reg[j] = buffer_load16(ra, a_voff, j * 32 * K * 2);
      if (b_active) {
#pragma unroll
        for (int e = 0; e < 8; ++e) b_reg[e] = buffer_load16(rb, b_voff, e * N * 2);
      }
    };

    auto lds_store = [&](int stage) {
#pragma unroll
      for (int j = 0; j < kALoads; ++j)
        *reinterpret_cast<uint4*>(lds + stage * kABytes + a_st[j]) = a_reg[j];
      if (b_active) {
        uint4 cols[8];
        transpose_8x8_b16(b_reg, cols);
#pragma unroll
        for (int q = 0; q < 8; ++q)
          *reinterpret_cast<uint4*>(lds + stage * kBBytes + b_st[q]) = cols[q];
      }
    };

    f32x16_t acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) acc[i][j] = f32x16_t{};

    auto read_frags = [&](int stage, int s, uint4 (&af)[TM], uint4 (&bf)[TN]) {
#pragma unroll
      for (int i = 0; i < TM; ++i)
        af[i] = *reinterpret_cast<const uint4*>(lds + stage * kABytes + a_rd[i & 1][s] + (i >> 1) * 64 * kRowBytes);
#pragma unroll
      for (int j = 0; j < TN; ++j)
        bf[j] = *reinterpret_cast<const uint4*>(lds + stage * kBBytes + b_rd[j & 1][s] + (j >> 1) * 64 * kRowBytes);
    };

    auto compute = [&](int stage) {
      uint4 af[2][TM], bf[2][TN];
      read_frags(stage, 0, af[0], bf[0]);
#pragma unroll
      for (int s = 0; s < kBK / 16; ++s) {
        if (s + 1 < kBK / 16) read_frags(stage, s + 1, af[(s + 1) & 1], bf[(s + 1) & 1]);
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j)
            acc[i][j] = mfma32x32x16<kBf16>(bf[s & 1][j], af[s & 1][i], acc[i][j]);
      }
    };

    // One k step: prefetch step kt+1 into registers, multiply from LDS stage ``stage``, then move
    // the prefetched step into the other stage. The scheduling barriers keep the prefetch loads
    // at the top, so their latency overlaps the whole multiply.
    auto k_step = [&](int kt, int stage) {
      const bool next = kt + 1 < nk;
      if (next) global_load(kt + 1);
      __builtin_amdgcn_sched_barrier(0);
      compute(stage);
      __builtin_amdgcn_sched_barrier(0);
      if (next) lds_store(stage ^ 1);
      __syncthreads();
    };

    global_load(0);
    lds_store(0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) k_step(kt, kt & 1);

    // Lane l holds, for MFMA block (i, j) and group g, row (l mod 32) and columns
    // 8g + 4*(l div 32) .. +3 of that 32 x 32 block.
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const size_t row = m0 + wm * WM + i * 32 + (lane & 31);
#pragma unroll
      for (int j = 0; j < TN; ++j) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const size_t col = n0 + wn * WN + j * 32 + 8 * g + 4 * (lane >> 5);
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
