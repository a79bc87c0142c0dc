// GEMM for shapes whose matrix rows are not whole 16-byte chunks: N or K not a multiple of 8.
//
// The GEMM kernel of "CUDA Thread Block Swizzle" (leimao.github.io), section "CUDA Thread Block
// Swizzle Benchmark", masks every operand load and every output store at the matrix edges, so any
// M, N and K is allowed. The fast kernels (gemm_kernel.hpp, gemm_pp_kernel.hpp) move operands with
// 16-byte direct-to-LDS loads, which need every row of A and B to start on a 16-byte boundary; when
// N or K is not a multiple of 8 they do not, and this kernel runs instead. It keeps what the orders
// are about -- the same tile grid, the same stride schedule over the same order_tile, the same
// optional trace -- and moves operands element by element:
//   * one 32-deep k step at a time, single-buffered: every thread fetches 8-element runs of A (along
//     k, row-major in LDS) and of B (along k for one column, so B lands transposed, n-major), each
//     element with 2-byte loads guarded by m < M, n < N, k < K (zero otherwise), and writes a run
//     with one 16-byte LDS store; LDS rows are padded to 40 values so runs stay 16-byte aligned;
//   * both operand fragments are then plain 16-byte LDS reads, fed to v_mfma_f32_16x16x32 with B as
//     the first operand (as in the fast kernels: each lane holds 4 consecutive output columns of one
//     row) and fp32 accumulators, k ascending;
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

template <int BM, bool kBf16, bool kF32Out>
__global__ __launch_bounds__(AnyShape<BM>::kThreads) void gemm_any_kernel(
    const uint16_t* __restrict__ A, const uint16_t* __restrict__ B, void* __restrict__ Cv, int M, int N,
    int K, TileOrder order, int num_programs, int32_t* __restrict__ trace) {
  using S = AnyShape<BM>;
  constexpr int BN = BM;
  constexpr int WM = S::WM, WN = S::WN, TM = S::TM, TN = S::TN, kPitch = S::kPitch;
  constexpr int kRunsA = BM * kBK / 8;          // 8-element runs per step
  constexpr int kRunsB = BN * kBK / 8;
  static_assert(kRunsA % S::kThreads == 0 && kRunsB % S::kThreads == 0, "whole runs per thread");
  __shared__ __attribute__((aligned(16))) uint16_t lds_a[BM * kPitch];
  __shared__ __attribute__((aligned(16))) uint16_t lds_b[BN * kPitch];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / S::kWavesN, wn = wave % S::kWavesN;
  const int P = num_programs;
  if (static_cast<int>(blockIdx.x) >= order.tiles) return;
  const int nk = (K + kBK - 1) / kBK;

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
    f32x4_t acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    for (int kt = 0; kt < nk; ++kt) {
      const int k0 = kt * kBK;
      // A run q: row q / 4 of the tile, k offset 8 (q mod 4)
#pragma unroll
      for (int it = 0; it < kRunsA / S::kThreads; ++it) {
        const int q = tid + it * S::kThreads;
        const int r = q >> 2, kc = (q & 3) * 8;
        const int row = m0 + r;
        uint16_t v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int k = k0 + kc + e;
          v[e] = (row < M && k < K) ? A[static_cast<size_t>(row) * K + k] : uint16_t{0};
        }
        *reinterpret_cast<uint4*>(lds_a + r * kPitch + kc) =
            make_uint4(v[0] | (uint32_t{v[1]} << 16), v[2] | (uint32_t{v[3]} << 16),
                       v[4] | (uint32_t{v[5]} << 16), v[6] | (uint32_t{v[7]} << 16));
      }
      // B run q: column q mod BN of the tile (consecutive threads, consecutive columns), k offset
      // 8 (q / BN); stored n-major
#pragma unroll
      for (int it = 0; it < kRunsB / S::kThreads; ++it) {
        const int q = tid + it * S::kThreads;
        const int c = q % BN, kc = (q / BN) * 8;
        const int col = n0 + c;
        uint16_t v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int k = k0 + kc + e;
          v[e] = (col < N && k < K) ? B[static_cast<size_t>(k) * N + col] : uint16_t{0};
        }
        *reinterpret_cast<uint4*>(lds_b + c * kPitch + kc) =
            make_uint4(v[0] | (uint32_t{v[1]} << 16), v[2] | (uint32_t{v[3]} << 16),
                       v[4] | (uint32_t{v[5]} << 16), v[6] | (uint32_t{v[7]} << 16));
      }
      __syncthreads();
      // fragments: lane l takes row (col) l mod 16 of a 16-block, k 8 (l / 16) .. + 7
      uint4 af[TM], bf[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i)
        af[i] = *reinterpret_cast<const uint4*>(lds_a + (wm * WM + i * 16 + (lane & 15)) * kPitch + 8 * (lane >> 4));
#pragma unroll
      for (int j = 0; j < TN; ++j)
        bf[j] = *reinterpret_cast<const uint4*>(lds_b + (wn * WN + j * 16 + (lane & 15)) * kPitch + 8 * (lane >> 4));
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = mfma16x16x32<kBf16>(bf[j], af[i], acc[i][j]);
      __syncthreads();
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

template <int BM>
const void* any_kernel_for(int dtype) {
  switch (dtype) {
    case 0: return reinterpret_cast<const void*>(&gemm_any_kernel<BM, false, false>);
    case 1: return reinterpret_cast<const void*>(&gemm_any_kernel<BM, true, false>);
    case 2: return reinterpret_cast<const void*>(&gemm_any_kernel<BM, false, true>);
    case 3: return reinterpret_cast<const void*>(&gemm_any_kernel<BM, true, true>);
    default: return nullptr;
  }
}

template <int BM>
hipError_t launch_any(int dtype, const GemmLaunch& a, hipStream_t s) {
  const void* k = any_kernel_for<BM>(dtype);
  if (k == nullptr) return hipErrorInvalidValue;
  const uint16_t* A = static_cast<const uint16_t*>(a.A);
  const uint16_t* B = static_cast<const uint16_t*>(a.B);
  const dim3 grid(a.num_programs), block(AnyShape<BM>::kThreads);
  switch (dtype) {
    case 0: hipLaunchKernelGGL((gemm_any_kernel<BM, false, false>), grid, block, 0, s, A, B, a.C, a.M, a.N,
                               a.K, a.order, a.num_programs, a.trace); break;
    case 1: hipLaunchKernelGGL((gemm_any_kernel<BM, true, false>), grid, block, 0, s, A, B, a.C, a.M, a.N,
                               a.K, a.order, a.num_programs, a.trace); break;
    case 2: hipLaunchKernelGGL((gemm_any_kernel<BM, false, true>), grid, block, 0, s, A, B, a.C, a.M, a.N,
                               a.K, a.order, a.num_programs, a.trace); break;
    default: hipLaunchKernelGGL((gemm_any_kernel<BM, true, true>), grid, block, 0, s, A, B, a.C, a.M, a.N,
                                a.K, a.order, a.num_programs, a.trace); break;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_any(int dtype, int bm, const GemmLaunch& a, hipStream_t s) {
  if (bm == 64) return launch_any<64>(dtype, a, s);
  if (bm == 128) return launch_any<128>(dtype, a, s);
  if (bm == 256) return launch_any<256>(dtype, a, s);
  return hipErrorInvalidValue;
}

hipError_t gemm_any_blocks_per_cu(int dtype, int bm, int* out) {
  const void* k = bm == 64 ? any_kernel_for<64>(dtype)
                : bm == 128 ? any_kernel_for<128>(dtype)
                : bm == 256 ? any_kernel_for<256>(dtype) : nullptr;
  if (k == nullptr) return hipErrorInvalidValue;
  const int threads = bm == 64 ? AnyShape<64>::kThreads : bm == 128 ? AnyShape<128>::kThreads
                                                                   : AnyShape<256>::kThreads;
  return hipOccupancyMaxActiveBlocksPerMultiprocessor(out, k, threads, 0);
}

}  // namespace tbl
