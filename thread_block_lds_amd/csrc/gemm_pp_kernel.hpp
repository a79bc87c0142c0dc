// The 256 x 256 GEMM kernel with eight waves in two alternating groups ("ping-pong").
//
// Same computation as gemm_kernel (gemm_kernel.hpp): workgroup p walks tile ids p, p + P, ... and
// accumulates each output tile in fp32 over k in ascending MFMA steps. In the 32 x 32 x 16 form
// (kM16 = false) the steps are 16 deep, exactly as gemm_kernel's, so the results are bit-identical
// to it; the 16 x 16 x 32 form (kM16, the default kernel) takes 32-deep steps, and on gfx950 one
// 32-deep step leaves the same fp32 bits as two 16-deep ones (checked on the device on random fp16
// and bf16 operands, and by the layout-variant tests, which compare the two forms bit for bit).
// With kDyn the tiles come instead from claim counters (the dynamic schedule
// that "CUDA Thread Block Swizzle", section "CUDA Thread Block Swizzle Benchmark", notes its
// persistent loop lacks); only the schedule changes, never a tile's arithmetic. What differs from
// gemm_kernel is how the work is laid out over the CU:
//   * 512 threads = 8 wave64s, two per SIMD. Group 0 (waves 0-3) owns output rows 0-127 of the
//     tile, group 1 (waves 4-7) rows 128-255; inside a group wave w owns columns 64 (w mod 4) ..
//     + 63, a 128 x 64 sub-tile (128 accumulator registers): 4 x 2 blocks of 32 x 32, or with kM16
//     8 x 4 blocks of 16 x 16.
//   * Each group alternates a memory half-period M(s) -- read all operand fragments of k step s
//     from LDS into registers and issue this wave's four direct loads of step s + 4 (in the kM16
//     form interleaved with the reads), wait until its loads of step s + 1 have landed -- and a
//     compute half-period C(s) -- the step's 16 MFMAs of
//     32 x 32 x 16 (or 32 of 16 x 16 x 32) back to back, then the epilogue if s ends a tile. Group 1 starts one half-period late, so
//     while one wave of a SIMD computes, the other issues its memory operations; a wave stalled on
//     a load or an LDS read no longer idles the matrix pipe.
//   * Every half-period ends with a workgroup barrier (which also waits for the wave's LDS reads).
//     Loads of step t are waited for by each wave before the barrier that closes its M(t - 1),
//     and step t is read only after both groups' M(t - 1) have closed; loads of step s + 4 go to
//     the stage of step s - 1, which both groups finished reading before the barrier preceding the
//     first M(s). Five 32 KiB stages hold the steps in flight.
// LDS layout, swizzles and direct loads are those of gemm_kernel, except that the kM16 form reads
// its operands in other lane patterns and so takes other chunk XORs: A by (row / 2) mod 4 and B by
// swz_b16 (both conflict-free for its reads, measured with the LDS bank-conflict counter).
#pragma once

#include "gemm_kernel.hpp"

namespace tbl {
namespace {

constexpr int kPPThreads = 512;

// Vector-memory accesses of the dynamic schedule (claim counters, mailboxes). Those returning a value
// wait for it inside the asm (vmcnt(0): also for every load in flight), so the compiler never sees
// a pending result it would have to track through the pipeline's steps -- it would then wait for
// all loads in every step. The cache-policy bits are the ones the compiler itself emits for these
// scopes on gfx950: atomics return with sc0 and are device-coherent; sc0 marks workgroup-scope
// loads and stores, sc1 device-scope loads.
__device__ __forceinline__ unsigned dyn_atomic_add(unsigned* p, unsigned v) {   // device scope
  unsigned r;
  asm volatile("global_atomic_add %0, %1, %2, off sc0\n\ts_waitcnt vmcnt(0)" : "=v"(r) : "v"(p), "v"(v) : "memory");
  return r;
}
__device__ __forceinline__ void dyn_store_wg(uint64_t* p, uint64_t v) {   // workgroup scope
  asm volatile("global_store_dwordx2 %0, %1, off sc0" : : "v"(p), "v"(v) : "memory");
}
// A uniform 64-bit read through the scalar path with glc (the scalar cache is bypassed, the value
// comes from L2). Scalar loads count on lgkmcnt, not vmcnt, so waiting for this one leaves the
// wave's direct loads in flight. Reads only: the scalar path is never used to write.
__device__ __forceinline__ uint64_t dyn_load_scalar(const uint64_t* p) {
  uint64_t r;
  asm volatile("s_load_dwordx2 %0, %1, 0x0 glc\n\ts_waitcnt lgkmcnt(0)" : "=s"(r) : "s"(p) : "memory");
  return r;
}
__device__ __forceinline__ unsigned dyn_load_device(const unsigned* p) {   // device scope
  unsigned r;
  asm volatile("global_load_dword %0, %1, off sc1\n\ts_waitcnt vmcnt(0)" : "=v"(r) : "v"(p) : "memory");
  return r;
}

template <bool kBf16, bool kF32Out, int kAPP = 4, int kAMP = 4, int kBV = 4, int kBPP = 1, int kBMP = 4,
          bool kDyn = false, bool kM16 = false>
__global__ __launch_bounds__(kPPThreads) void gemm_pp_kernel(const uint16_t* __restrict__ A,
                                                             const uint16_t* __restrict__ B,
                                                             void* __restrict__ Cv, int M, int N, int K,
                                                             TileOrder order, int num_programs,
                                                             int32_t* __restrict__ trace,
                                                             int32_t* __restrict__ work, int xcd_aware) {
  constexpr int BM = 256, BN = 256;
  constexpr int WM = 128, WN = 64;                 // wave sub-tile
  constexpr int TM = WM / 32, TN = WN / 32;        // 4 x 2 MFMA blocks of 32 x 32 per wave
  constexpr int TM16 = WM / 16, TN16 = WN / 16;    // or 8 x 4 blocks of 16 x 16 (kM16)
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
  static_assert((kM16 && kBV == 0) || (kBPP >= 1 && kBMP >= 1 && 4 % kBPP == 0 && (4 / kBPP) % kBMP == 0),
                "B swizzle must repeat every 4 k rows");
  // the 16 x 16 x 32 reads address A blocks 16 rows apart from one base
  static_assert(!kM16 || (16 / kAPP) % kAMP == 0, "A swizzle must repeat every 16 rows");

  __shared__ __attribute__((aligned(1024))) char lds[kStages * kStage];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2, wn = wave & 3;
  const int nk = (K + kBK - 1) / kBK;
  const int P = num_programs;
  // static schedule: this workgroup's tiles are blockIdx.x + i P; the dynamic one takes every tile,
  // the first included, from the claim counters, so every workgroup runs its prologue claim
  if (!kDyn && static_cast<int>(blockIdx.x) >= order.tiles) return;
  const int my_tiles = kDyn ? 0 : (order.tiles - 1 - static_cast<int>(blockIdx.x)) / P + 1;
  const int total = my_tiles * nk;

  // ---- dynamic schedule: claims of order positions (wave 0) and their hand-over to the others ----
  // work[0..7]: claim counters, zeroed by dyn_reset_kernel before the launch -- one queue over all
  // positions, or (xcd_aware) one per XCD over the block floor(q T / 8) .. floor((q + 1) T / 8) - 1;
  // work[9]: hand-over faults (stays 0); work[32 + 32 p ..]: workgroup p's two mailbox slots, each a
  // 64-bit (claim number << 32 | position). A position < 0 means no work is left.
  // The first claims of all workgroups (made together at the start, in workgroup order) are settled
  // without atomics: workgroup p takes position p of the one queue, or (xcd_aware; round-robin
  // dispatch puts p on XCD p mod 8) the (p / 8)-th position of block p mod 8 while that block has
  // one; the counters then hand out the positions after these first ones.
  const unsigned T = static_cast<unsigned>(order.tiles);
  const int own_q = kDyn && xcd_aware ? xcc_id() : 0;
  int cur_q = own_q;
  uint64_t* mailbox = kDyn ? reinterpret_cast<uint64_t*>(work + 32 + 32 * static_cast<size_t>(blockIdx.x))
                           : nullptr;
  auto queue_lo = [&](int q) -> unsigned {
    return xcd_aware ? static_cast<unsigned>(static_cast<uint64_t>(q) * T / kNumXcds) : 0u;
  };
  auto queue_size = [&](int q) -> unsigned {
    return xcd_aware ? static_cast<unsigned>(static_cast<uint64_t>(q + 1) * T / kNumXcds) - queue_lo(q) : T;
  };
  auto queue_first = [&](int q) -> unsigned {   // positions of queue q taken in the first round
    const unsigned n = xcd_aware ? (P > q ? static_cast<unsigned>(P - 1 - q) / kNumXcds + 1 : 0u)
                                 : static_cast<unsigned>(P);
    return min(n, queue_size(q));
  };
  auto claim_one = [&]() -> unsigned {   // wave 0: one claim on the current queue, waited for
    unsigned r = 0;
    if (lane == 0) r = dyn_atomic_add(reinterpret_cast<unsigned*>(work) + cur_q, 1u);
    return __builtin_amdgcn_readfirstlane(r);
  };
  // wave 0, XCD-aware, once the current queue is empty: read all eight counters at once and claim
  // from the queue with the most positions left (ties: the nearest after the own XCD); -1 when
  // none has any. A claim that loses a race for a queue's last positions reads again.
  auto steal = [&]() -> int {
    for (;;) {
      const int q = lane & (kNumXcds - 1);
      unsigned cnt = 0;
      if (lane < kNumXcds) cnt = dyn_load_device(reinterpret_cast<unsigned*>(work) + q);
      const unsigned avail = queue_size(q) - queue_first(q);
      const unsigned left = lane < kNumXcds && cnt < avail ? avail - cnt : 0u;
      const unsigned key = left ? (left << 3) | (7u - ((q - own_q) & (kNumXcds - 1))) : 0u;
      unsigned best = 0;
#pragma unroll
      for (int l = 0; l < kNumXcds; ++l) best = max(best, __builtin_amdgcn_readlane(key, l));
      if (best == 0) return -1;
      cur_q = (own_q + 7 - static_cast<int>(best & 7u)) & (kNumXcds - 1);
      const unsigned i = queue_first(cur_q) + claim_one();
      if (i < queue_size(cur_q)) return static_cast<int>(queue_lo(cur_q) + i);
    }
  };
  auto claim = [&]() -> int {   // wave 0, waited for: the next position, or -1
    const unsigned i = queue_first(cur_q) + claim_one();
    if (i < queue_size(cur_q)) return static_cast<int>(queue_lo(cur_q) + i);
    return xcd_aware ? steal() : -1;
  };
  auto mailbox_put = [&](int k, int pos) {   // wave 0
    if (lane == 0)
      dyn_store_wg(mailbox + (k & 1),
                   (static_cast<uint64_t>(static_cast<unsigned>(k)) << 32) | static_cast<unsigned>(pos));
  };
  auto mailbox_take = [&](int k) -> int {   // other waves: read the slot, check its claim number
    for (int tries = 0; tries < 1024; ++tries) {
      const uint64_t v = dyn_load_scalar(mailbox + (k & 1));
      if (static_cast<unsigned>(__builtin_amdgcn_readfirstlane(static_cast<unsigned>(v >> 32))) ==
          static_cast<unsigned>(k)) {
        const int pos = static_cast<int>(__builtin_amdgcn_readfirstlane(static_cast<unsigned>(v)));
        if (pos < static_cast<int>(T)) return pos;   // -1 (no work) or a position of this grid
        break;
      }
    }
    // never expected: the slot was written, and its store completed, before a barrier. Counted,
    // and no tile is taken, so no address outside the operands is formed.
    if (lane == 0) dyn_atomic_add(reinterpret_cast<unsigned*>(work) + 9, 1u);
    return -1;
  };

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
    const int chunk = ((o % kBRow) >> 4) ^ swz_b_of<kM16, kBV, kBPP, kBMP, kBChunks>(k);
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
  int b_rd[TN] = {};
  if constexpr (!kM16) {
    const int g = lane >> 4, r = lane & 15;
    const int k = 8 * (g >> 1) + (r >> 2);
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int n = wn * WN + j * 32 + 16 * (g & 1) + 4 * (r & 3);
      const int chunk = (n >> 3) ^ swz_b<kBV, kBPP, kBMP, kBChunks>(k);
      b_rd[j] = kAStage + k * kBRow + chunk * 16 + (n & 7) * 2;
    }
  }
  // 16 x 16 x 32 reads: A lane l takes row (l mod 16) of a 16-row block, chunk l / 16 (k 8 (l / 16)
  // .. + 7); B lane L of 16-lane group G addresses the 8-byte row piece k = 8 G + (L mod 16) / 4,
  // columns 4 (L mod 4) .. + 3 of a 16-column block, which the transposing read turns into 4 k of
  // one column per lane (twice: k and k + 4)
  int a_rd16 = 0, b_rd16[TN16];
  if constexpr (kM16) {
    const int row = grp * WM + (lane & 15);
    a_rd16 = row * kARow + ((lane >> 4) ^ swz_a<kAPP, kAMP>(row)) * 16;
    const int r = lane & 15;
    const int k = 8 * (lane >> 4) + (r >> 2);
#pragma unroll
    for (int j = 0; j < TN16; ++j) {
      const int n = wn * WN + j * 16 + 4 * (r & 3);
      b_rd16[j] = kAStage + k * kBRow + ((n >> 3) ^ swz_b_of<kM16, kBV, kBPP, kBMP, kBChunks>(k)) * 16 + (n & 7) * 2;
    }
  }

  // the first tile: blockIdx.x; dynamic: the first-round position, else claimed by wave 0 and
  // handed over through the mailbox
  int first = static_cast<int>(blockIdx.x);
  int nxt = -1;   // dynamic: position of the tile after the current one, known from k step 4 on
  if constexpr (kDyn) {
    const int p = static_cast<int>(blockIdx.x);
    const int fq = xcd_aware ? (p & (kNumXcds - 1)) : 0;
    const unsigned fi = xcd_aware ? static_cast<unsigned>(p) / kNumXcds : static_cast<unsigned>(p);
    if (fi < queue_size(fq)) {
      first = static_cast<int>(queue_lo(fq) + fi);
    } else {   // uniform over the workgroup
      if (wave == 0) {
        first = claim();
        mailbox_put(0, first);
        wait_vm<0>();   // the mailbox store has landed before the barrier
      }
      lds_barrier();
      if (wave != 0) first = mailbox_take(0);
      if (first < 0) return;   // every wave of the workgroup alike
    }
  }

  // ---- load cursor (as gemm_kernel) ----
  // the claimed positions are uniform over the workgroup (each is read through readfirstlane), but
  // the compiler cannot see it through the claim code's lane-0 branches: said here, so the load
  // cursor and its addresses stay scalar (in vector registers they cost every step ~25 VALU ops)
  int ld_t = __builtin_amdgcn_readfirstlane(first), ld_kt = 0, ld_issued = 0, ld_stage = 0;
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
  // this wave's loads of the next step in the stream (zero-length ones past its end, which keep the
  // number of loads per step, and so every wait count, the same): prepare_step sets up the step's
  // buffer descriptors, issue_load(q) issues load q (A blocks first, then B blocks),
  // advance_load_cursor moves to the step after it
  i32x4_t ld_da, ld_db;
  unsigned ld_lds = 0;
  bool ld_tail = false;
  auto prepare_step = [&]() {
    const bool real = kDyn ? ld_t >= 0 : ld_issued < total;
    const int k_left = K - ld_kt * kBK;
    const unsigned b_rows = static_cast<unsigned>(k_left < kBK ? k_left : kBK);
    ld_tail = k_left < kBK;
    ld_da = make_desc(reinterpret_cast<const void*>(ld_a), real ? a_range : 0u);
    ld_db = make_desc(reinterpret_cast<const void*>(ld_b), real ? b_rows * b_row - b_lead : 0u);
    ld_lds = lds_address(lds + ld_stage * kStage);
  };
  auto issue_load = [&](int q) {
    if (q < kAInst)
      load_to_lds(ld_da, ld_lds + (wave * kAInst + q) * 1024, ld_tail ? a_voff_tail[q] : a_voff[q]);
    else
      load_to_lds(ld_db, ld_lds + kAStage + (wave * kBInst + q - kAInst) * 1024, b_voff[q - kAInst]);
  };
  auto advance_load_cursor = [&]() {
    ++ld_issued;
    ld_stage = ld_stage == kStages - 1 ? 0 : ld_stage + 1;
    ld_a += a_step;
    ld_b += b_step;
    a_range -= a_step;
    if (++ld_kt == nk) {
      ld_kt = 0;
      if constexpr (kDyn) {
        ld_t = __builtin_amdgcn_readfirstlane(nxt);
        if (ld_t >= 0) enter_tile();
      } else {
        ld_t += P;
        if (ld_t < order.tiles) enter_tile();
      }
    }
  };
  auto load_step = [&]() {
    prepare_step();
#pragma unroll
    for (int q = 0; q < kLoads; ++q) issue_load(q);
    advance_load_cursor();
  };

  // ---- operand fragments of one step: [k half][block] ----
  uint4 af[2][TM], bf[2][TN];
  uint4 af16[TM16], bf16f[TN16];
  // 16 x 16 x 32 form: A block i (one 16-byte read), B block j (two transposing 8-byte reads)
  auto read_a16 = [&](int stage, int i) {
    af16[i] = *reinterpret_cast<const uint4*>(lds + stage * kStage + a_rd16 + i * 16 * kARow);
  };
  auto read_b16 = [&](int stage, int j) {
    const char* p = lds + stage * kStage + b_rd16[j];
    const uint2 lo = __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)p));
    const uint2 hi = __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                                   (lds_s16x4_t*)(p + 4 * kBRow)));
    bf16f[j] = make_uint4(lo.x, lo.y, hi.x, hi.y);
  };
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
  f32x4_t acc16[TM16][TN16];
  auto zero_acc = [&]() {
    float z;
    asm volatile("v_mov_b32 %0, 0" : "=v"(z));
    if constexpr (kM16) {
#pragma unroll
      for (int i = 0; i < TM16; ++i)
#pragma unroll
        for (int j = 0; j < TN16; ++j)
#pragma unroll
          for (int r = 0; r < 4; ++r) acc16[i][j][r] = z;
      return;
    }
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = z;
  };

  // ---- compute cursor and optional schedule trace (as gemm_kernel) ----
  int c_t = first, c_iter = 0, c_m = 0, c_n = 0;
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
  // wave's loads of step s + 1; the barrier closes the half-period.
  // In the 16 x 16 x 32 form the four loads are interleaved with the operand reads. Issuing a direct
  // load stalls the wave until the CU's address unit takes it (about 1 KiB per 16 cycles, shared by
  // the group's four waves: some 260 cycles for the group's 16 loads), while the reads keep the LDS
  // busy for about 300 cycles; issued one after the other the two made the memory half-period
  // longer than the MFMA one (cycle stamps on the device), interleaved they overlap (1240 -> 1165
  // cycles per step).
  auto memory_half = [&]() {
    if constexpr (kM16) {
      static_assert(kLoads == 4 && TM16 == 8 && TN16 == 4, "interleave written for this wave tile");
      prepare_step();
      issue_load(0);
      read_b16(c_stage, 0);
      read_a16(c_stage, 0);
      issue_load(1);
      read_b16(c_stage, 1);
      read_a16(c_stage, 1);
      read_a16(c_stage, 2);
      issue_load(2);
      read_b16(c_stage, 2);
      read_a16(c_stage, 3);
      read_a16(c_stage, 4);
      issue_load(3);
      read_b16(c_stage, 3);
      read_a16(c_stage, 5);
      read_a16(c_stage, 6);
      read_a16(c_stage, 7);
      advance_load_cursor();
    } else {
      read_step(c_stage);
      load_step();
    }
    wait_vm<3 * kLoads>();
    __builtin_amdgcn_sched_barrier(0);
    lds_barrier();
    __builtin_amdgcn_sched_barrier(0);
  };
  // C(s): the step's MFMAs (16 of 32 x 32 x 16, or 32 of 16 x 16 x 32)
  auto compute_half = [&]() {
    if constexpr (kM16) {   // 32 MFMAs of 16 x 16 x 32
      // The B fragments run forward for even i and backward for odd i, so at every change of A the
      // B operand stays: fewer operand bits switch per MFMA, which lets the board hold a higher
      // clock (the MFMA-only loop runs 2-3 % faster in this order).
#pragma unroll
      for (int i = 0; i < TM16; ++i)
#pragma unroll
        for (int jj = 0; jj < TN16; ++jj) {
          const int j = (i & 1) ? TN16 - 1 - jj : jj;
          acc16[i][j] = mfma16x16x32<kBf16>(bf16f[j], af16[i], acc16[i][j]);
        }
    } else {
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = mfma32x32x16<kBf16>(bf[h][j], af[h][i], acc[i][j]);
    }
    c_stage = c_stage == kStages - 1 ? 0 : c_stage + 1;
    __builtin_amdgcn_sched_barrier(0);
  };
  // dynamic: at the start of tile j's k step 0, wave 0 claims tile j + 1 and posts it in the
  // mailbox; the other waves read it at the start of step 4 (the post, issued before step 0's loads,
  // has landed by wave 0's wait at the end of step 2); the load cursor moves to tile j + 1 at the
  // end of step nk - 5's loads, so nk >= 9. The claim waits for its result at once, and with it for
  // wave 0's loads in flight (about one load latency per tile); the other waves read the mailbox
  // through the scalar path, whose wait leaves their loads in flight. The claim number in each
  // slot catches a stale read.
  auto dyn_hook = [&](int kt) {
    const int k = c_iter + 1;
    if (wave == 0) {
      if (kt == 0) {
        nxt = claim();
        mailbox_put(k, nxt);
      }
    } else if (kt == 4) {
      nxt = mailbox_take(k);
    }
  };
  for (int tile = 0; kDyn || tile < my_tiles; ++tile) {
    zero_acc();
    int kt = 0;
    if constexpr (kDyn) {
      // steps 0 .. 4 carry the claim hook in a loop of their own, so the steady-state loop below
      // is the static kernel's, with no per-step test
      for (; kt < 5; ++kt) {
        dyn_hook(kt);
        memory_half();
        compute_half();
        lds_barrier();
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    for (; kt < nk; ++kt) {
      memory_half();
      compute_half();
      lds_barrier();
      __builtin_amdgcn_sched_barrier(0);
    }
    // the epilogue overlaps the other group's last compute half-period
    record_time();
    if constexpr (kM16)
      store_tile16<BM, BN, WM, WN, TM16, TN16, kBf16, kF32Out>(acc16, Cv, M, N, c_m, c_n, grp, wn, lane);
    else
      store_tile<BM, BN, WM, WN, TM, TN, kBf16, kF32Out>(acc, Cv, M, N, c_m, c_n, grp, wn, lane);
    if constexpr (kDyn) {
      c_t = __builtin_amdgcn_readfirstlane(nxt);
      ++c_iter;
      if (c_t < 0) break;
      order_tile(order, c_t, c_m, c_n);
      record();
    } else {
      c_t += P;
      ++c_iter;
      if (c_t < order.tiles) {
        order_tile(order, c_t, c_m, c_n);
        record();
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  if (grp == 0) lds_barrier();   // match group 1's extra barrier
  wait_vm<0>();                  // no direct load may still be writing this workgroup's LDS
}

// The default 256 x 256 kernel: 16 x 16 x 32 MFMAs with A swizzled by (row / 2) mod 4 (the
// (perPhase 2, maxPhase 4) member of the chunk-XOR family: conflict-free for 16 rows x 2 chunks
// per half-wave, where (row / 4) mod 4 costs twice the cycles) and B by swz_b16. The 32 x 32 x 16
// form (kM16 = false) serves the LDS-layout variants of gemm_layouts.hip.
constexpr int kM16APP = 2, kM16AMP = 4;

template <bool kBf16, bool kF32Out>
const void* pp_kernel_ptr() {
  return reinterpret_cast<const void*>(
      &gemm_pp_kernel<kBf16, kF32Out, kM16APP, kM16AMP, 0, 0, 0, false, true>);
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

template <bool kBf16, bool kF32Out, int kAPP = 4, int kAMP = 4, int kBV = 4, int kBPP = 1, int kBMP = 4,
          bool kDyn = false, bool kM16 = false>
hipError_t launch_pp_typed(const GemmLaunch& a, hipStream_t s) {
  hipLaunchKernelGGL((gemm_pp_kernel<kBf16, kF32Out, kAPP, kAMP, kBV, kBPP, kBMP, kDyn, kM16>), dim3(a.num_programs),
                     dim3(kPPThreads), 0, s, static_cast<const uint16_t*>(a.A),
                     static_cast<const uint16_t*>(a.B), a.C, a.M, a.N, a.K, a.order, a.num_programs,
                     a.trace, a.work, a.xcd_aware);
  return hipGetLastError();
}

hipError_t launch_pp(int dtype, const GemmLaunch& a, hipStream_t s) {
  switch (dtype) {
    case 0: return launch_pp_typed<false, false, kM16APP, kM16AMP, 0, 0, 0, false, true>(a, s);
    case 1: return launch_pp_typed<true, false, kM16APP, kM16AMP, 0, 0, 0, false, true>(a, s);
    case 2: return launch_pp_typed<false, true, kM16APP, kM16AMP, 0, 0, 0, false, true>(a, s);
    case 3: return launch_pp_typed<true, true, kM16APP, kM16AMP, 0, 0, 0, false, true>(a, s);
    default: return hipErrorInvalidValue;
  }
}

// Zeroes the dynamic schedule's claim counters (vector stores), run on the GEMM's stream before it.
__global__ __launch_bounds__(64) void dyn_reset_kernel(int32_t* __restrict__ work) {
  if (threadIdx.x < 9) work[threadIdx.x] = 0;
}

// The dynamic schedule (claim counters and mailboxes in a.work).
hipError_t launch_pp_dynamic(int dtype, const GemmLaunch& a, hipStream_t s) {
  hipLaunchKernelGGL(dyn_reset_kernel, dim3(1), dim3(64), 0, s, a.work);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  switch (dtype) {
    case 0: return launch_pp_typed<false, false, kM16APP, kM16AMP, 0, 0, 0, true, true>(a, s);
    case 1: return launch_pp_typed<true, false, kM16APP, kM16AMP, 0, 0, 0, true, true>(a, s);
    case 2: return launch_pp_typed<false, true, kM16APP, kM16AMP, 0, 0, 0, true, true>(a, s);
    case 3: return launch_pp_typed<true, true, kM16APP, kM16AMP, 0, 0, 0, true, true>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace
}  // namespace tbl
