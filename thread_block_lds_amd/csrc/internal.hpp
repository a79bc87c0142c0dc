// Internal interface between the C-ABI layer (api.hip) and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tile_order.hpp"

namespace tbl {

struct GemmLaunch {
  const void* A;
  const void* B;
  void* C;
  int M, N, K;
  TileOrder order;
  int num_programs;
  int32_t* trace;   // nullable
  int32_t* work = nullptr;   // dynamic schedule: claim counters and mailboxes
  int xcd_aware = 0;         // dynamic schedule: one claim queue per XCD
};

// dtype: TBL_F16 .. TBL_BF16_F32OUT. Returns hipSuccess or the launch error.
hipError_t launch_gemm(int dtype, int bm, int bn, int bk, const GemmLaunch& a, hipStream_t s);
// Resident workgroups per CU of the kernel for (dtype, tile), from the HIP occupancy query.
hipError_t gemm_blocks_per_cu(int dtype, int bm, int bn, int bk, int* out);
bool gemm_tile_supported(int bm, int bn, int bk);
// Shapes whose rows are not whole 16-byte chunks (N or K not a multiple of 8): the element-wise
// load path of gemm_any.hip, for the tile shapes gemm_tile_supported accepts (bm == bn).
hipError_t launch_gemm_any(int dtype, int bm, const GemmLaunch& a, hipStream_t s);
// Its two forms: B moved in 16-byte chunks when N is a multiple of 8, element by element otherwise.
hipError_t gemm_any_blocks_per_cu(int dtype, int bm, int N, int* out);
// C = 0 for K = 0 (the empty sum): zeroes ``bytes`` bytes of C (16-byte aligned, an even count).
hipError_t launch_gemm_zero(void* C, int64_t bytes, hipStream_t s);
// The 256 x 256 x 32 kernel with the dynamic (work-queue) schedule; a.work and a.xcd_aware set.
hipError_t launch_gemm_dynamic(int dtype, const GemmLaunch& a, hipStream_t s);

// The 256 x 256 x 32 fp16 -> fp16 kernel with the LDS swizzles (A: perPhase, maxPhase; B: vec in
// 16-byte chunks, perPhase, maxPhase) of one compiled variant; gemm_layout_supported lists them.
// m16: the 16 x 16 x 32 MFMA form (b_vec 0 = its default B layout) instead of the 32 x 32 x 16 one.
bool gemm_layout_supported(bool m16, int a_pp, int a_mp, int b_vec, int b_pp, int b_mp);
hipError_t launch_gemm_layout(bool m16, int a_pp, int a_mp, int b_vec, int b_pp, int b_mp,
                              const GemmLaunch& a, hipStream_t s);

hipError_t launch_tile_map(const TileOrder& o, int32_t* tile_m, int32_t* tile_n, hipStream_t s);

// Offline L2 replay of the order's operand-block reads (host only; arguments already validated):
// writes the hits and accesses summed over num_caches byte-capacity LRU caches.
void predict_l2(const TileOrder& o, int grid_k, int64_t a_bytes, int64_t b_bytes, int64_t capacity,
                int num_caches, int num_programs, int resident, int64_t* hits, int64_t* accesses);

// The GEMM's operand reads as byte ranges: A (M x K) at a_base and B (K x N) at b_base, row-major,
// elem_bytes per element, bm x bn x bk tiles.
struct GemmReadShape {
  int64_t M, N, K;
  int elem_bytes, bm, bn, bk;
  uint64_t a_base, b_base;
};
// Set-associative caches: sets x ways lines of line_bytes; line L in set
// (L xor ((L >> fold_from) mod 2^fold_width)) mod sets.
struct L2Geometry {
  int64_t sets;
  int ways;
  int64_t line_bytes;
  int fold_from, fold_width;
};
// Line-granular replay with predict_l2's grouping and read order (host only; validated arguments).
void predict_l2_lines(const TileOrder& o, const GemmReadShape& r, const L2Geometry& g, int num_caches,
                      int64_t num_programs, int resident, int64_t* hits, int64_t* accesses);

// The matrix-pipe rate kernel (mfma_rate.hip); arguments already validated.
hipError_t launch_mfma_rate(const void* A, const void* B, int64_t elems, bool bf16, int workgroups,
                            int iters, float* out, int64_t* cycles, hipStream_t s);

hipError_t launch_transpose_i32(const int32_t* in, int32_t* out, int rows, int cols, int layout,
                                hipStream_t s);

// The plain 16-byte-per-lane copy (copy.hip); bytes a positive multiple of 16, arguments validated.
hipError_t launch_copy16(const void* src, void* dst, int64_t bytes, bool nontemporal, hipStream_t s);

}  // namespace tbl
