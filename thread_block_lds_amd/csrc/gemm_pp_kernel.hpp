// The 256 x 256 GEMM kernel with eight waves in two alternating groups ("ping-pong").
//
// Same computation as gemm_kernel (gemm_kernel.hpp): workgroup p walks tile ids p, p + P, ... and
// accumulates each output tile in fp32 over k in ascending 16-deep MFMA steps, so the results are
// bit-identical to it. What differs is how the work is laid out over the CU:
//   * 512 threads = 8 wave64s, two per SIMD. Group 0 (waves 0-3) owns output rows 0-127 of the
//     tile, group 1 (waves 4-7) rows 128-255; inside a group wave w owns columns 64 (w mod 4) ..
//     + 63, a 128 x 64 sub-tile of 4 x 2 blocks of 32 x 32 (128 accumulator registers).
//   * Each group alternates a memory half-period M(s) -- read all operand fragments of k step s
//     from LDS into registers, issue this wave's four direct loads of step s + 4, wait until its
//     loads of step s + 1 have landed -- and a compute half-period C(s) -- the step's 16 MFMAs
//     back to back, then the epilogue if s ends a tile. Group 1 starts one half-period late, so
//     while one wave of a SIMD computes, the other issues its memory operations; a wave stalled on
//     a load or an LDS read no longer idles the matrix pipe.
//   * Every half-period ends with a workgroup barrier (which also waits for the wave's LDS reads).
//     Loads of step t are waited for by each wave before the barrier that closes its M(t - 1),
//     and step t is read only after both groups' M(t - 1) have closed; loads of step s + 4 go to
//     the stage of step s - 1, which both groups finished reading before the barrier preceding the
//     first M(s). Five 32 KiB stages hold the steps in flight.
// LDS layout, swizzles and direct loads are those of gemm_kernel.
#pragma once

#include "gemm_kernel.hpp"

namespace tbl {
namespace {

constexpr int kPPThreads = 512;

template <bool kBf16, bool kF32Out, int kAPP = 4, int kAMP = 4, int kBV = 4, int kBPP = 1, int kBMP = 4>
__global__ __launch_bounds__(kPPThreads) void gemm_pp_kernel(const uint16_t* __restrict__ A,
                                                             const uint16_t* __restrict__ B,
                                                             void* __restrict__ Cv, int M, int N, int K,
                                                             TileOrder order, int num_programs,
                                                             int32_t* __restrict__ trace) {
  constexpr int BM = 256, BN = 256;
  constexpr int WM = 128, WN = 64;                 // wave sub-tile
  constexpr int TM = WM / 32, TN = WN / 32;        // 4 x 2 MFMA blocks per wave
  constexpr int kBRow = BN * 2;                    // bytes of one B row (one k) in LDS
  constexpr int kAStage = BM * kARow;
  constexpr int kBStage = kBK * kBRow;
  constexpr int kStage = kAStage + kBStage;
  constexpr int kWaves = kPPThreads / 64;
  constexpr int kAInst = kAStage / 1024 / kWaves;  // 2 direct loads of A per wave per step
  constexpr int kBInst = kBStage / 1024 / kWaves;  // 2 of B
  constexpr int kLoads = kAInst + kBInst;
  constexpr int kBChunks = BN / 8;
  static_assert(kLoads == 4, "the wait counts assume four loads per wave and step");
  static_assert(kStages == 5, "loads run four steps ahead");
  static_assert(kAPP >= 1 && kAMP >= 1 && kAMP <= 4 && (32 / kAPP) % kAMP == 0 && 32 % kAPP == 0,
                "A swizzle must repeat every 32 rows");
  static_assert(kBPP >= 1 && kBMP >= 1 && 4 % kBPP == 0 && (4 / kBPP) % kBMP == 0,
                "B swizzle must repeat every 4 k rows");

  __shared__ __attribute__((aligned(1024))) char lds[kStages * kStage];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2, wn = wave & 3;
  const int nk = (K + kBK - 1) / kBK;
  const int P = num_programs;
  if (static_cast<int>(blockIdx.x) >= order.tiles) return;
  const int my_tiles = (order.tiles - 1 - static_cast<int>(blockIdx.x)) / P + 1;
  const int total = my_tiles * nk;

  // ---- per-lane constants of the direct loads (as gemm_kernel, eight waves) ----
  constexpr int kOutOfRange = 0x7FFFFFF0;
  int a_voff[kAInst], a_voff_tail[kAInst];
#pragma unroll
  for (int j = 0; j < kAInst; ++j) {
    const int row = (wave * kAInst + j) * 16 + (lane >> 2);
    const int chunk = (lane & 3) ^ swz_a<kAPP, kAMP>(row);
    a_voff[j] = (row * K + chunk * 8) * 2;
    a_voff_tail[j] = chunk * 8 + 8 <= K % kBK ? a_voff[j] : kOutOfRange;
  }
  int b_voff[kBInst];
#pragma unroll
  for (int j = 0; j < kBInst; ++j) {
    const int o = (wave * kBInst + j) * 1024 + 16 * lane;
    const int k = o / kBRow;
    const int chunk = ((o % kBRow) >> 4) ^ swz_b<kBV, kBPP, kBMP, kBChunks>(k);
    b_voff[j] = (k * N + chunk * 8) * 2;
  }
  // ---- per-lane constants of the operand reads ----
  int a_rd[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int row = grp * WM + (lane & 31);
    const int chunk = (2 * h + (lane >> 5)) ^ swz_a<kAPP, kAMP>(row);
    a_rd[h] = row * kARow + chunk * 16;
  }
  int b_rd[TN];
  {
    const int g = lane >> 4, r = lane & 15;
    const int k = 8 * (g >> 1) + (r >> 2);
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int n = wn * WN + j * 32 + 16 * (g & 1) + 4 * (r & 3);
      const int chunk = (n >> 3) ^ swz_b<kBV, kBPP, kBMP, kBChunks>(k);
      b_rd[j] = kAStage + k * kBRow + chunk * 16 + (n & 7) * 2;
    }
  }

  // ---- load cursor (as gemm_kernel) ----
  int ld_t = blockIdx.x, ld_kt = 0, ld_issued = 0, ld_stage = 0;
  uint64_t ld_a = 0, ld_b = 0;
  const unsigned a_step = kBK * 2;
  const uint64_t b_step = static_cast<uint64_t>(kBK) * static_cast<unsigned>(N) * 2;
  const unsigned b_row = static_cast<unsigned>(N) * 2;
  unsigned a_range = 0, b_lead = 0;
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
  // issue this wave's loads of the next step in the stream (zero-length ones past its end, which
  // keep the number of loads per step, and so every wait count, the same)
  auto load_step = [&]() {
    const bool real = ld_issued < total;
    const int k_left = K - ld_kt * kBK;
    const unsigned b_rows = static_cast<unsigned>(k_left < kBK ? k_left : kBK);
    const bool tail = k_left < kBK;
    const i32x4_t da = make_desc(reinterpret_cast<const void*>(ld_a), real ? a_range : 0u);
    const i32x4_t db = make_desc(reinterpret_cast<const void*>(ld_b), real ? b_rows * b_row - b_lead : 0u);
    const unsigned base = lds_address(lds + ld_stage * kStage);
#pragma unroll
    for (int q = 0; q < kAInst; ++q)
      load_to_lds(da, base + (wave * kAInst + q) * 1024, tail ? a_voff_tail[q] : a_voff[q]);
#pragma unroll
    for (int q = 0; q < kBInst; ++q)
      load_to_lds(db, base + kAStage + (wave * kBInst + q) * 1024, b_voff[q]);
    ++ld_issued;
    ld_stage = ld_stage == kStages - 1 ? 0 : ld_stage + 1;
    ld_a += a_step;
    ld_b += b_step;
    a_range -= a_step;
    if (++ld_kt == nk) {
      ld_kt = 0;
      ld_t += P;
      if (ld_t < order.tiles) enter_tile();
    }
  };

  // ---- operand fragments of one step: [k half][block] ----
  uint4 af[2][TM], bf[2][TN];
  auto read_step = [&](int stage) {
    const char* base = lds + stage * kStage;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
      for (int i = 0; i < TM; ++i)
        af[h][i] = *reinterpret_cast<const uint4*>(base + a_rd[h] + i * 32 * kARow);
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const char* p = base + b_rd[j] + h * 16 * kBRow;
        const uint2 lo = __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)p));
        const uint2 hi = __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                                       (lds_s16x4_t*)(p + 4 * kBRow)));
        bf[h][j] = make_uint4(lo.x, lo.y, hi.x, hi.y);
      }
    }
  };

  f32x16_t acc[TM][TN];
  auto zero_acc = [&]() {
    float z;
    asm volatile("v_mov_b32 %0, 0" : "=v"(z));
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = z;
  };

  // ---- compute cursor and optional schedule trace (as gemm_kernel) ----
  int c_t = blockIdx.x, c_iter = 0, c_m = 0, c_n = 0;
  order_tile(order, c_t, c_m, c_n);
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

  // prologue: steps 0 .. 3 in flight, step 0 landed everywhere
#pragma unroll
  for (int i = 0; i < kStages - 1; ++i) load_step();
  wait_vm<3 * kLoads>();
  lds_barrier();
  if (grp == 1) lds_barrier();   // group 1 runs one half-period behind group 0
  __builtin_amdgcn_sched_barrier(0);

  int c_stage = 0;
  // M(s): this step's fragments into registers, the loads of step s + 4, then the wait for this
  // wave's loads of step s + 1; the barrier closes the half-period
  auto memory_half = [&]() {
    read_step(c_stage);
    load_step();
    wait_vm<3 * kLoads>();
    __builtin_amdgcn_sched_barrier(0);
    lds_barrier();
    __builtin_amdgcn_sched_barrier(0);
  };
  // C(s): the step's 16 MFMAs
  auto compute_half = [&]() {
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = mfma32x32x16<kBf16>(bf[h][j], af[h][i], acc[i][j]);
    c_stage = c_stage == kStages - 1 ? 0 : c_stage + 1;
    __builtin_amdgcn_sched_barrier(0);
  };
  for (int tile = 0; tile < my_tiles; ++tile) {
    zero_acc();
    for (int kt = 0; kt < nk; ++kt) {
      memory_half();
      compute_half();
      lds_barrier();
      __builtin_amdgcn_sched_barrier(0);
    }
    // the epilogue overlaps the other group's last compute half-period
    record_time();
    store_tile<BM, BN, WM, WN, TM, TN, kBf16, kF32Out>(acc, Cv, M, N, c_m, c_n, grp, wn, lane);
    c_t += P;
    ++c_iter;
    if (c_t < order.tiles) {
      order_tile(order, c_t, c_m, c_n);
      record();
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  if (grp == 0) lds_barrier();   // match group 1's extra barrier
  wait_vm<0>();                  // no direct load may still be writing this workgroup's LDS
}

template <bool kBf16, bool kF32Out>
const void* pp_kernel_ptr() {
  return reinterpret_cast<const void*>(&gemm_pp_kernel<kBf16, kF32Out>);
}

const void* pp_kernel_for(int dtype) {
  switch (dtype) {
    case 0: return pp_kernel_ptr<false, false>();
    case 1: return pp_kernel_ptr<true, false>();
    case 2: return pp_kernel_ptr<false, true>();
    case 3: return pp_kernel_ptr<true, true>();
    default: return nullptr;
  }
}

template <bool kBf16, bool kF32Out, int kAPP = 4, int kAMP = 4, int kBV = 4, int kBPP = 1, int kBMP = 4>
hipError_t launch_pp_typed(const GemmLaunch& a, hipStream_t s) {
  hipLaunchKernelGGL((gemm_pp_kernel<kBf16, kF32Out, kAPP, kAMP, kBV, kBPP, kBMP>), dim3(a.num_programs),
                     dim3(kPPThreads), 0, s, static_cast<const uint16_t*>(a.A),
                     static_cast<const uint16_t*>(a.B), a.C, a.M, a.N, a.K, a.order, a.num_programs,
                     a.trace);
  return hipGetLastError();
}

hipError_t launch_pp(int dtype, const GemmLaunch& a, hipStream_t s) {
  switch (dtype) {
    case 0: return launch_pp_typed<false, false>(a, s);
    case 1: return launch_pp_typed<true, false>(a, s);
    case 2: return launch_pp_typed<false, true>(a, s);
    case 3: return launch_pp_typed<true, true>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace
}  // namespace tbl
