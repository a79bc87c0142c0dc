// GEMM for shapes whose matrix rows are not whole 16-byte chunks: N or K not a multiple of 8.
//
// The GEMM kernel of "CUDA Thread Block Swizzle" (leimao.github.io), section "CUDA Thread Block
// Swizzle Benchmark", masks every operand load and every output store at the matrix edges, so any
// M, N and K is allowed. The fast kernels (gemm_kernel.hpp, gemm_pp_kernel.hpp) move operands with
// 16-byte direct-to-LDS loads, which need every row of A and B to start on a 16-byte boundary; when
// N or K is not a multiple of 8 they do not, and this kernel runs instead. It keeps what the orders
// are about -- the same tile grid, the same stride schedule over the same order_tile, the same
// optional trace -- and moves operands through registers with buffer loads whose ranges (and
// offsets past them) give zeros outside the matrices:
//   * A in 16-byte chunks along k in every full k step, at whatever 2-byte alignment the rows have
//     (gfx950 serves unaligned buffer loads; the odd-K parity tests depend on it); in a last,
//     partial k step, element pairs with k >= K masked;
//   * B in 16-byte chunks along n when N is a multiple of 8 (rows then stay 16-byte aligned), laid
//     out k-major in LDS and read with transposing reads as in the four-wave kernel; otherwise
//     element by element along k for each column (consecutive threads, consecutive columns), laid
//     out n-major. Unaligned 16-byte loads along B's rows measured slower than that (2048 x 2047 x
//     2049: 169 against 297 TFLOP/s), unlike A's;
//   * software-pipelined by one k step in registers: step s + 1's loads are issued right after step
//     s is written to LDS and land while step s's MFMAs run; the barriers wait for LDS accesses
//     only, never for those loads;
//   * A row-major in LDS, rows padded to 40 values; the operand fragments feed
//     v_mfma_f32_16x16x32 with B as the first operand (as in the fast kernels: each lane holds 4
//     consecutive output columns of one row) and fp32 accumulators, k ascending;
//   * every output element is stored on its own, guarded by row < M and column < N.
// Wave grid: 2 x 2 waves of 32 x 32 (64 tiles) or 64 x 64 (128 tiles), 2 x 4 waves of 128 x 64
// (256 tiles). This path trades speed for generality; the aligned shapes never reach it.
#include "gemm_kernel.hpp"

namespace tbl {
namespace {

template <int BM>
struct AnyShape {
  static constexpr int kWavesN = BM == 256 ? 4 : 2;
  static constexpr int kWaves = 2 * kWavesN;
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int WM = BM / 2;             // wave sub-tile rows
  static constexpr int WN = BM / kWavesN;       // and columns
  static constexpr int TM = WM / 16, TN = WN / 16;
  static constexpr int kPitch = 40;             // LDS row pitch in 16-bit values (80 bytes)
};

template <int BM, bool kBf16, bool kF32Out, bool kWideB>
__global__ __launch_bounds__(AnyShape<BM>::kThreads) void gemm_any_kernel(
    const uint16_t* __restrict__ A, const uint16_t* __restrict__ B, void* __restrict__ Cv, int M, int N,
    int K, TileOrder order, int num_programs, int32_t* __restrict__ trace) {
  using S = AnyShape<BM>;
  constexpr int BN = BM;
  constexpr int WM = S::WM, WN = S::WN, TM = S::TM, TN = S::TN, kPitch = S::kPitch;
  constexpr int kChunksA = BM * kBK / 8 / S::kThreads;  // 16-byte chunks of A per thread (full steps)
  constexpr int kPairsA = BM * kBK / 2 / S::kThreads;   // (row, 2 k) pairs of A per thread (last step)
  constexpr int kChunksB = kBK * BN / 8 / S::kThreads;  // 16-byte chunks of B per thread and step
  constexpr int kRunsB = kChunksB;                      // or (column, 8 k) runs (N not a multiple of 8)
  static_assert(kChunksA * S::kThreads == BM * kBK / 8 && kPairsA * S::kThreads == BM * kBK / 2 &&
                    kChunksB * S::kThreads == BN * kBK / 8,
                "whole chunks and pairs per thread");
  __shared__ __attribute__((aligned(16))) uint16_t lds_a[BM * kPitch];
  // B k-major (kWideB) or n-major with padded rows
  __shared__ __attribute__((aligned(16))) uint16_t lds_b[kWideB ? kBK * BN : BN * kPitch];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / S::kWavesN, wn = wave % S::kWavesN;
  int b_rd[TN];   // byte offsets of this lane's transposing B reads (row k, k + 4 at + 4 rows)
  {
    const int r = lane & 15, k = 8 * (lane >> 4) + (r >> 2);
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int n = wn * WN + j * 16 + 4 * (r & 3);
      b_rd[j] = k * BN * 2 + ((n >> 3) ^ swz_b_four_wave<BN>(k)) * 16 + (n & 7) * 2;
    }
  }
  const int P = num_programs;
  if (static_cast<int>(blockIdx.x) >= order.tiles) return;
  const int nk = (K + kBK - 1) / kBK;

  // One k step's operand elements as loaded. They come through buffer loads: a descriptor (in
  // scalar registers) per tile for A and per k step for B whose range ends after the last element
  // of the matrix that the tile or step may touch, so elements past it read as zero; an element
  // inside the range but outside the matrix (k >= K in A, a column >= N in B) gets an offset past
  // the range. Except in a tile's last k step when K is not a multiple of 32, nothing is waited
  // for until the values are written to LDS.
  constexpr int kOut = 0x7FFFFFF0;   // an offset past every range
  constexpr int kRsrcFlags = 0x00020000;
  typedef int i32x4v_t __attribute__((ext_vector_type(4)));
  // A in full k steps (k0 + 32 <= K): 16-byte chunks, chunk c of this thread row g / 4 of the tile,
  // k 8 (g mod 4) .. + 7 (g = c threads + tid; a wave reads 16 rows x 64 contiguous bytes per
  // instruction). A row of A starts on a 16-byte boundary only when K is a multiple of 8; the
  // loads take any 2-byte alignment (gfx950 runs them unaligned; the odd-K parity tests depend on
  // it), and each chunk lies inside its row, so none straddles the end of the range (the range
  // check zeroes whole dwords)
  i32x4v_t wa[kChunksA], wb[kWideB ? kChunksB : 1];
  uint16_t rb[kWideB ? 1 : 8 * kRunsB];
  auto fetch = [&](__amdgpu_buffer_rsrc_t rsrc_a, int n0, int k0) {
    if (k0 + kBK <= K) {
#pragma unroll
      for (int c = 0; c < kChunksA; ++c) {
        const int g = c * S::kThreads + tid;
        wa[c] = __builtin_amdgcn_raw_buffer_load_b128(rsrc_a, ((g >> 2) * K + k0 + 8 * (g & 3)) * 2, 0, 0);
      }
    }
    // The step's B descriptor starts at (k0, n0) and ends after element (min(k0 + 32, K) - 1, N - 1):
    // rows k >= K lie past it. Columns past N are zero (an offset past the range).
    const int rows_k = K - k0 < kBK ? K - k0 : kBK;
    const __amdgpu_buffer_rsrc_t rsrc_b = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(B + static_cast<size_t>(k0) * N + n0), 0, (rows_k * N - n0) * 2, kRsrcFlags);
    if constexpr (kWideB) {
      // N a multiple of 8: 16-byte chunks along n, chunk q of this thread row g / (BN / 8) of the
      // step, columns 8 (g mod (BN / 8)) .. + 7 (g = q threads + tid; a wave reads 512 contiguous
      // bytes of each of two rows per instruction at BN = 256); every chunk lies inside [0, N) or
      // wholly past it, and starts on a 16-byte boundary
#pragma unroll
      for (int q = 0; q < kChunksB; ++q) {
        const int g = q * S::kThreads + tid;
        const int kk = g / (BN / 8), n = 8 * (g % (BN / 8));
        wb[q] = __builtin_amdgcn_raw_buffer_load_b128(rsrc_b, n0 + n < N ? (kk * N + n) * 2 : kOut, 0, 0);
      }
    } else {
      // otherwise element by element, run q: column g mod BN of the tile (consecutive threads,
      // consecutive columns: 128 contiguous bytes per load instruction), k 8 (g / BN) .. + 7. 16-byte
      // loads at 2-byte alignment along B's rows measured slower here (the A chunks above gain)
#pragma unroll
      for (int q = 0; q < kRunsB; ++q) {
        const int g = q * S::kThreads + tid;
        const int c = g % BN, kc = (g / BN) * 8;
        const bool col_in = n0 + c < N;
#pragma unroll
        for (int e = 0; e < 8; ++e)
          rb[8 * q + e] = __builtin_amdgcn_raw_buffer_load_b16(rsrc_b, col_in ? ((kc + e) * N + c) * 2 : kOut, 0, 0);
      }
    }
  };
  // the fetched step into LDS: A row-major (k along a row), B n-major (k along a column's row)
  auto stash = [&](__amdgpu_buffer_rsrc_t rsrc_a, int k0) {
    if (k0 + kBK <= K) {
#pragma unroll
      for (int c = 0; c < kChunksA; ++c) {
        const int g = c * S::kThreads + tid;
        *reinterpret_cast<i32x4v_t*>(lds_a + (g >> 2) * kPitch + 8 * (g & 3)) = wa[c];
      }
    } else {
      // the last step of a K that is not a multiple of 32: element pairs, k >= K masked, loaded
      // and written here (pair p: row g / 16, k 2 (g mod 16) and the next; g = p threads + tid)
#pragma unroll
      for (int p = 0; p < kPairsA; ++p) {
        const int g = p * S::kThreads + tid;
        const int k = k0 + 2 * (g & 15);
        const int off = ((g >> 4) * K + k) * 2;
        const uint32_t lo = __builtin_amdgcn_raw_buffer_load_b16(rsrc_a, k < K ? off : kOut, 0, 0);
        const uint32_t hi = __builtin_amdgcn_raw_buffer_load_b16(rsrc_a, k + 1 < K ? off + 2 : kOut, 0, 0);
        *reinterpret_cast<uint32_t*>(lds_a + (g >> 4) * kPitch + 2 * (g & 15)) = lo | (hi << 16);
      }
    }
    if constexpr (kWideB) {
      // B k-major, one row of BN values per k, chunk c of row k at c XOR swz_b_four_wave(k) (the
      // four-wave kernel's layout, conflict-free for its transposing reads)
#pragma unroll
      for (int q = 0; q < kChunksB; ++q) {
        const int g = q * S::kThreads + tid;
        const int kk = g / (BN / 8), c = g % (BN / 8);
        *reinterpret_cast<i32x4v_t*>(lds_b + kk * BN + 8 * (c ^ swz_b_four_wave<BN>(kk))) = wb[q];
      }
    } else {
      // B n-major (k along a column's row). The values are packed by an asm statement, which
      // consumes the loaded registers here and no earlier: left to itself the compiler packs (and
      // so waits) right after the loads, before the MFMAs
      auto pack = [](uint16_t lo, uint16_t hi) {
        uint32_t r;
        asm volatile("v_lshl_or_b32 %0, %1, 16, %2" : "=v"(r) : "v"(uint32_t{hi}), "v"(uint32_t{lo}));
        return r;
      };
#pragma unroll
      for (int q = 0; q < kRunsB; ++q) {
        const int g = q * S::kThreads + tid;
        const uint16_t* v = rb + 8 * q;
        *reinterpret_cast<uint4*>(lds_b + (g % BN) * kPitch + (g / BN) * 8) =
            make_uint4(pack(v[0], v[1]), pack(v[2], v[3]), pack(v[4], v[5]), pack(v[6], v[7]));
      }
    }
  };

  int iter = 0;
  for (int t = blockIdx.x; t < order.tiles; t += P, ++iter) {
    int tm, tn;
    order_tile(order, t, tm, tn);
    const uint64_t clk0 = __builtin_readcyclecounter();
    const uint64_t rt0 = __builtin_amdgcn_s_memrealtime();
    if (trace != nullptr && tid == 0) {
      int32_t* rec = trace + kTraceInts * static_cast<size_t>(t);
      rec[0] = blockIdx.x;
      rec[1] = iter;
      rec[2] = tm;
      rec[3] = tn;
      rec[4] = xcc_id();
    }
    const int m0 = tm * BM, n0 = tn * BN;
    // A's rows of this tile: [m0, min(m0 + BM, M)), K elements each
    const int rows_a = M - m0 < BM ? M - m0 : BM;
    const __amdgpu_buffer_rsrc_t rsrc_a = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(A + static_cast<size_t>(m0) * K), 0, rows_a * K * 2, kRsrcFlags);
    f32x4_t acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    fetch(rsrc_a, n0, 0);
    for (int kt = 0; kt < nk; ++kt) {
      stash(rsrc_a, kt * kBK);
      lds_barrier();   // the step's operands are in LDS (and no load is waited for here)
      if (kt + 1 < nk) fetch(rsrc_a, n0, (kt + 1) * kBK);
      // fragments: A lane l takes row l mod 16 of a 16-row block, k 8 (l / 16) .. + 7; B (k-major)
      // lane L of 16-lane group G addresses the 8-byte row piece k = 8 G + (L mod 16) / 4, columns
      // 4 (L mod 4) .. + 3 of a 16-column block, which the transposing read turns into 4 k of one
      // column per lane (twice: k and k + 4, whose rows take the same chunk XOR). All of B's, then
      // A's one block row at a time.
      uint4 bf[TN];
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        if constexpr (kWideB) {
          const char* p = reinterpret_cast<const char*>(lds_b) + b_rd[j];
          const uint2 lo = __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)p));
          const uint2 hi = __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(p + 4 * BN * 2)));
          bf[j] = make_uint4(lo.x, lo.y, hi.x, hi.y);
        } else {   // n-major: lane l takes column l mod 16 of the block, k 8 (l / 16) .. + 7
          bf[j] = *reinterpret_cast<const uint4*>(lds_b + (wn * WN + j * 16 + (lane & 15)) * kPitch + 8 * (lane >> 4));
        }
      }
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const uint4 af = *reinterpret_cast<const uint4*>(lds_a + (wm * WM + i * 16 + (lane & 15)) * kPitch + 8 * (lane >> 4));
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = mfma16x16x32<kBf16>(bf[j], af, acc[i][j]);
      }
      lds_barrier();   // every wave has read the step before the next one is written
    }
    if (trace != nullptr && tid == 0) {
      int32_t* rec = trace + kTraceInts * static_cast<size_t>(t);
      rec[5] = static_cast<int32_t>(__builtin_readcyclecounter() - clk0);
      rec[6] = static_cast<int32_t>(__builtin_amdgcn_s_memrealtime() - rt0);
      rec[7] = static_cast<int32_t>(rt0);
    }
    // lane l holds row l mod 16 and columns 4 (l / 16) .. + 3 of block (i, j)
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int row = m0 + wm * WM + i * 16 + (lane & 15);
      if (row >= M) continue;
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int col0 = n0 + wn * WN + j * 16 + 4 * (lane >> 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if (col0 + e >= N) continue;
          const size_t at = static_cast<size_t>(row) * N + col0 + e;
          if constexpr (kF32Out) static_cast<float*>(Cv)[at] = acc[i][j][e];
          else static_cast<uint16_t*>(Cv)[at] = to_out16(acc[i][j][e], kBf16);
        }
      }
    }
  }
}

template <int BM, bool kWideB>
const void* any_kernel_for(int dtype) {
  switch (dtype) {
    case 0: return reinterpret_cast<const void*>(&gemm_any_kernel<BM, false, false, kWideB>);
    case 1: return reinterpret_cast<const void*>(&gemm_any_kernel<BM, true, false, kWideB>);
    case 2: return reinterpret_cast<const void*>(&gemm_any_kernel<BM, false, true, kWideB>);
    case 3: return reinterpret_cast<const void*>(&gemm_any_kernel<BM, true, true, kWideB>);
    default: return nullptr;
  }
}

template <int BM, bool kWideB>
hipError_t launch_any(int dtype, const GemmLaunch& a, hipStream_t s) {
  const uint16_t* A = static_cast<const uint16_t*>(a.A);
  const uint16_t* B = static_cast<const uint16_t*>(a.B);
  const dim3 grid(a.num_programs), block(AnyShape<BM>::kThreads);
  switch (dtype) {
    case 0: hipLaunchKernelGGL((gemm_any_kernel<BM, false, false, kWideB>), grid, block, 0, s, A, B, a.C, a.M,
                               a.N, a.K, a.order, a.num_programs, a.trace); break;
    case 1: hipLaunchKernelGGL((gemm_any_kernel<BM, true, false, kWideB>), grid, block, 0, s, A, B, a.C, a.M,
                               a.N, a.K, a.order, a.num_programs, a.trace); break;
    case 2: hipLaunchKernelGGL((gemm_any_kernel<BM, false, true, kWideB>), grid, block, 0, s, A, B, a.C, a.M,
                               a.N, a.K, a.order, a.num_programs, a.trace); break;
    case 3: hipLaunchKernelGGL((gemm_any_kernel<BM, true, true, kWideB>), grid, block, 0, s, A, B, a.C, a.M,
                               a.N, a.K, a.order, a.num_programs, a.trace); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int BM>
hipError_t launch_any_b(int dtype, const GemmLaunch& a, hipStream_t s) {
  return a.N % 8 == 0 ? launch_any<BM, true>(dtype, a, s) : launch_any<BM, false>(dtype, a, s);
}

template <int BM>
const void* any_kernel_for_b(int dtype, bool wide_b) {
  return wide_b ? any_kernel_for<BM, true>(dtype) : any_kernel_for<BM, false>(dtype);
}

}  // namespace

hipError_t launch_gemm_any(int dtype, int bm, const GemmLaunch& a, hipStream_t s) {
  if (bm == 64) return launch_any_b<64>(dtype, a, s);
  if (bm == 128) return launch_any_b<128>(dtype, a, s);
  if (bm == 256) return launch_any_b<256>(dtype, a, s);
  return hipErrorInvalidValue;
}

hipError_t gemm_any_blocks_per_cu(int dtype, int bm, int N, int* out) {
  const bool wide_b = N % 8 == 0;
  const void* k = bm == 64 ? any_kernel_for_b<64>(dtype, wide_b)
                : bm == 128 ? any_kernel_for_b<128>(dtype, wide_b)
                : bm == 256 ? any_kernel_for_b<256>(dtype, wide_b) : nullptr;
  if (k == nullptr) return hipErrorInvalidValue;
  const int threads = bm == 64 ? AnyShape<64>::kThreads : bm == 128 ? AnyShape<128>::kThreads
                                                                   : AnyShape<256>::kThreads;
  return hipOccupancyMaxActiveBlocksPerMultiprocessor(out, k, threads, 0);
}

}  // namespace tbl
