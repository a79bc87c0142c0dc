// C ABI of libtbl.so (declared and documented in include/tbl.h): argument validation, the tile
// shape rule, default program counts, device properties, and dispatch to the kernels.
//
// Every argument is checked before the first HIP call, so the error paths run without a GPU.
// The checks mirror the benchmark script of "CUDA Thread Block Swizzle" (leimao.github.io):
// positive sizes and group sizes, and Morton / XOR used only on square power-of-two tile grids
// (elsewhere those orders drop some tiles and repeat others).
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include <mutex>

#include "../../include/tbl.h"
#include "internal.hpp"

namespace {

constexpr int64_t kMaxDim = int64_t{1} << 20;
constexpr int kMaxDynamicPrograms = 1 << 16;
constexpr int kMinDynamicKSteps = 9;
constexpr int kMaxDevices = 64;
constexpr int64_t kMaxCopyBytes = int64_t{1} << 40;

struct DeviceInfo {
  bool valid = false;
  int cus = 0;
  int lds = 0;
  int l2 = 0;
  char arch[64] = {0};
};

std::mutex g_info_mutex;
DeviceInfo g_info[kMaxDevices];

int device_info(DeviceInfo* out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return TBL_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_info_mutex);
  DeviceInfo& d = g_info[dev];
  if (!d.valid) {
    hipDeviceProp_t p;
    if (hipGetDeviceProperties(&p, dev) != hipSuccess) return TBL_ERR_HIP;
    d.cus = p.multiProcessorCount;
    d.lds = static_cast<int>(p.sharedMemPerBlock);
    d.l2 = p.l2CacheSize;
    strncpy(d.arch, p.gcnArchName, sizeof(d.arch) - 1);
    d.valid = true;
  }
  *out = d;
  return TBL_OK;
}

bool is_pow2(int64_t v) { return v > 0 && (v & (v - 1)) == 0; }
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Whether the byte ranges [p, p + pn) and [q, q + qn) share a byte (sizes > 0; an empty range or a
// null pointer overlaps nothing).
bool overlaps(const void* p, int64_t pn, const void* q, int64_t qn) {
  if (p == nullptr || q == nullptr || pn <= 0 || qn <= 0) return false;
  const uintptr_t a = reinterpret_cast<uintptr_t>(p), b = reinterpret_cast<uintptr_t>(q);
  return a < b ? b - a < static_cast<uintptr_t>(pn) : a - b < static_cast<uintptr_t>(qn);
}

int64_t out_elem_bytes(int dtype) { return dtype == TBL_F16_F32OUT || dtype == TBL_BF16_F32OUT ? 4 : 2; }

// Whether C shares a byte with A or B (A and B, which are only read, may overlap each other).
// Sizes come from validated arguments (M, N, K <= 2^20: no overflow).
bool c_overlaps_operands(const void* A, const void* B, const void* C, int64_t M, int64_t N, int64_t K,
                         int dtype) {
  const int64_t cn = M * N * out_elem_bytes(dtype);
  return overlaps(C, cn, A, M * K * 2) || overlaps(C, cn, B, K * N * 2);
}

// Whether another buffer the GEMM writes (a trace or a workspace, [w, w + wn)) shares a byte with
// A, B or C.
bool extra_overlaps(const void* w, int64_t wn, const void* A, const void* B, const void* C, int64_t M,
                    int64_t N, int64_t K, int dtype) {
  return overlaps(w, wn, A, M * K * 2) || overlaps(w, wn, B, K * N * 2) ||
         overlaps(w, wn, C, M * N * out_elem_bytes(dtype));
}

// Cluster dimensions encoded in bits 16..19 (cm - 1) and 20..23 (cn - 1) of a swizzle mode.
int cluster_m(int swizzle_mode) { return ((swizzle_mode >> 16) & 15) + 1; }
int cluster_n(int swizzle_mode) { return ((swizzle_mode >> 20) & 15) + 1; }

// The checks of an order that do not depend on the grid.
int check_mode(int swizzle_mode, int group) {
  const int mode = swizzle_mode & 0xFF;
  if ((swizzle_mode & ~(0xFF | TBL_XCD_REMAP | 0xFF0000)) != 0) return TBL_ERR_INVALID_ARG;
  if (mode < TBL_ROW || mode > TBL_SERPENTINE) return TBL_ERR_INVALID_ARG;
  if ((mode == TBL_PANEL || mode == TBL_SERPENTINE) && group < 1) return TBL_ERR_INVALID_ARG;
  return TBL_OK;
}

int check_order(int swizzle_mode, int64_t gm, int64_t gn, int group) {
  const int rc = check_mode(swizzle_mode, group);
  if (rc != TBL_OK) return rc;
  if (gm < 1 || gn < 1 || gm > kMaxDim || gn > kMaxDim || gm * gn > INT32_MAX) return TBL_ERR_SHAPE;
  // a cluster of cm x cn tiles must tile the grid exactly
  if (gm % cluster_m(swizzle_mode) || gn % cluster_n(swizzle_mode)) return TBL_ERR_SHAPE;
  return TBL_OK;
}

// Morton and XOR are bijections only on square power-of-two grids (of cluster tiles, when
// clustered).
bool bijective_grid(int swizzle_mode, int64_t gm, int64_t gn) {
  const int mode = swizzle_mode & 0xFF;
  if (mode != TBL_MORTON && mode != TBL_XOR) return true;
  gm /= cluster_m(swizzle_mode);
  gn /= cluster_n(swizzle_mode);
  return gm == gn && is_pow2(gm);
}

tbl::TileOrder make_order(int swizzle_mode, int gm, int gn, int group) {
  const int mode = swizzle_mode & 0xFF;
  const int cm = cluster_m(swizzle_mode), cn = cluster_n(swizzle_mode);
  const int cgm = gm / cm, cgn = gn / cn;   // the grid the order walks
  // A panel group taller than that grid, or a serpentine strip wider than it, orders the tiles
  // exactly as one of the grid's own height / width does; clamping keeps the device arithmetic in
  // 32 bits.
  int g = 1;
  if (mode == TBL_PANEL) g = group < cgm ? group : cgm;
  else if (mode == TBL_SERPENTINE) g = group < cgn ? group : cgn;
  return tbl::make_tile_order(mode, (swizzle_mode & TBL_XCD_REMAP) ? 1 : 0, cgm, cgn, g, cm, cn);
}

// The largest square tile whose grid has at least kFillTiles tiles, else 64: a grid of fewer tiles
// than half of gfx950's 256 CUs leaves most of the chip idle, and below that the smaller tile's
// extra parallelism outweighs its lower per-CU rate (measured over square and rectangular shapes
// from 768 to 16384: the 256 tile wins from 128 tiles up, the 128 tile from 128 of its own).
constexpr int64_t kFillTiles = 128;

void tile_rule(int64_t M, int64_t N, int* bm, int* bn, int* bk) {
  auto tiles = [&](int64_t t) { return ((M + t - 1) / t) * ((N + t - 1) / t); };
  const int t = tiles(256) >= kFillTiles ? 256 : tiles(128) >= kFillTiles ? 128 : 64;
  *bm = t;
  *bn = t;
  *bk = 32;
}

// Rows of A and B are whole 16-byte chunks: the fast kernels' direct loads apply; otherwise the
// general path (gemm_any.hip) runs.
bool chunk_rows(int64_t N, int64_t K) { return N % 8 == 0 && K % 8 == 0; }

// general: the entry points for any shape (tbl_gemm, tbl_gemm_tiled): N and K need not be
// multiples of 8, and sizes may be 0 (an operand with no elements may then be NULL). The dynamic
// schedule and the LDS-layout variants run only the fast kernel and keep both requirements.
int validate_gemm(const void* A, const void* B, void* C, int64_t M, int64_t N, int64_t K, int dtype,
                  int swizzle_mode, int group, int persistent, int num_programs, int bm, int bn,
                  int bk, bool general = false) {
  if (M < 0 || N < 0 || K < 0) return TBL_ERR_INVALID_ARG;
  if (!general && (M == 0 || N == 0 || K == 0)) return TBL_ERR_INVALID_ARG;
  if (M > kMaxDim || N > kMaxDim || K > kMaxDim) return TBL_ERR_SHAPE;
  if ((A == nullptr && M * K > 0) || (B == nullptr && K * N > 0) || (C == nullptr && M * N > 0))
    return TBL_ERR_INVALID_ARG;
  if (dtype < TBL_F16 || dtype > TBL_BF16_F32OUT) return TBL_ERR_DTYPE;
  if (persistent != 0 && persistent != 1) return TBL_ERR_INVALID_ARG;
  if (num_programs < 0) return TBL_ERR_INVALID_ARG;
  if (!tbl::gemm_tile_supported(bm, bn, bk)) return TBL_ERR_SHAPE;
  // partial tiles at the M, N and K edges are masked; outside the general entry points rows of B
  // and A must be whole 16-byte chunks
  if (!general && !chunk_rows(N, K)) return TBL_ERR_SHAPE;
  // no output element, an empty tile grid: only what does not depend on the grid can be checked
  if (M == 0 || N == 0) return check_mode(swizzle_mode, group);
  const int64_t gm = (M + bm - 1) / bm, gn = (N + bn - 1) / bn;
  int rc = check_order(swizzle_mode, gm, gn, group);
  if (rc != TBL_OK) return rc;
  if (!bijective_grid(swizzle_mode, gm, gn)) return TBL_ERR_NOT_BIJECTIVE;
  if (!aligned16(A) || !aligned16(B) || !aligned16(C)) return TBL_ERR_ALIGN;
  if (c_overlaps_operands(A, B, C, M, N, K, dtype)) return TBL_ERR_INVALID_ARG;
  return TBL_OK;
}

int resolve_programs(int dtype, int bm, int bn, int bk, int64_t tiles, int persistent,
                     int num_programs, int* out, bool chunked = true, int64_t N = 0) {
  if (num_programs > 0) {
    *out = num_programs;
    return TBL_OK;
  }
  if (!persistent) {
    *out = static_cast<int>(tiles);
    return TBL_OK;
  }
  DeviceInfo d;
  int rc = device_info(&d);
  if (rc != TBL_OK) return rc;
  int per_cu = 0;
  const hipError_t e = chunked ? tbl::gemm_blocks_per_cu(dtype, bm, bn, bk, &per_cu)
                               : tbl::gemm_any_blocks_per_cu(dtype, bm, static_cast<int>(N), &per_cu);
  if (e != hipSuccess) return TBL_ERR_HIP;
  if (per_cu < 1) per_cu = 1;
  const int64_t cap = static_cast<int64_t>(d.cus) * per_cu;
  *out = static_cast<int>(tiles < cap ? tiles : cap);
  return TBL_OK;
}

}  // namespace

extern "C" {

int tbl_version(void) { return 107; }

const char* tbl_status_string(int status) {
  switch (status) {
    case TBL_OK: return "ok";
    case TBL_ERR_INVALID_ARG: return "invalid argument";
    case TBL_ERR_DTYPE: return "unknown dtype";
    case TBL_ERR_SHAPE: return "unsupported shape (not a tile multiple, too large, or unsupported tile)";
    case TBL_ERR_NOT_BIJECTIVE: return "order is not a bijection on this tile grid (Morton/XOR need a square power-of-two grid)";
    case TBL_ERR_HIP: return "HIP runtime error";
    case TBL_ERR_ALIGN: return "pointer not 16-byte aligned";
    case TBL_ERR_SCRATCH: return "more workgroups than the allocation-free entry point's scratch holds";
    case TBL_WARN_NOT_BIJECTIVE: return "warning: table written, but the order is not a bijection on this grid";
    default: return "unknown status";
  }
}

int tbl_gemm_tile_shape(int64_t M, int64_t N, int64_t K, int* block_m, int* block_n, int* block_k) {
  if (block_m == nullptr || block_n == nullptr || block_k == nullptr) return TBL_ERR_INVALID_ARG;
  if (M < 0 || N < 0 || K < 0) return TBL_ERR_INVALID_ARG;
  tile_rule(M, N, block_m, block_n, block_k);
  return TBL_OK;
}

int tbl_gemm_tiled(const void* A, const void* B, void* C, int64_t M, int64_t N, int64_t K, int dtype,
                   int swizzle_mode, int group_size, int persistent, int num_programs, int block_m,
                   int block_n, int block_k, int32_t* trace, void* stream) {
  int rc = validate_gemm(A, B, C, M, N, K, dtype, swizzle_mode, group_size, persistent, num_programs,
                         block_m, block_n, block_k, true);
  if (rc != TBL_OK) return rc;
  if (M == 0 || N == 0) return TBL_OK;   // C has no element: nothing to compute
  const int gm = static_cast<int>((M + block_m - 1) / block_m);
  const int gn = static_cast<int>((N + block_n - 1) / block_n);
  if (extra_overlaps(trace, int64_t{32} * gm * gn, A, B, C, M, N, K, dtype)) return TBL_ERR_INVALID_ARG;
  // K = 0: every element of C is the empty sum; no tile runs, so a trace is left as it is
  if (K == 0)
    return tbl::launch_gemm_zero(C, M * N * out_elem_bytes(dtype), static_cast<hipStream_t>(stream)) == hipSuccess
               ? TBL_OK
               : TBL_ERR_HIP;
  const bool chunked = chunk_rows(N, K);
  int programs = 0;
  rc = resolve_programs(dtype, block_m, block_n, block_k, static_cast<int64_t>(gm) * gn, persistent,
                        num_programs, &programs, chunked, N);
  if (rc != TBL_OK) return rc;
  tbl::GemmLaunch a;
  a.A = A;
  a.B = B;
  a.C = C;
  a.M = static_cast<int>(M);
  a.N = static_cast<int>(N);
  a.K = static_cast<int>(K);
  a.order = make_order(swizzle_mode, gm, gn, group_size);
  a.num_programs = programs;
  a.trace = trace;
  const hipError_t e = chunked ? tbl::launch_gemm(dtype, block_m, block_n, block_k, a, static_cast<hipStream_t>(stream))
                               : tbl::launch_gemm_any(dtype, block_m, a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return TBL_ERR_HIP;
  return TBL_OK;
}

}  // extern "C"

namespace {

int gemm_lds_layout_impl(bool m16, const void* A, const void* B, void* C, int64_t M, int64_t N,
                         int64_t K, int dtype, int swizzle_mode, int group_size, int persistent,
                         int num_programs, int a_per_phase, int a_max_phase, int b_vec,
                         int b_per_phase, int b_max_phase, void* stream) {
  int rc = validate_gemm(A, B, C, M, N, K, dtype, swizzle_mode, group_size, persistent, num_programs,
                         256, 256, 32);
  if (rc != TBL_OK) return rc;
  if (dtype != TBL_F16) return TBL_ERR_DTYPE;
  if (!tbl::gemm_layout_supported(m16, a_per_phase, a_max_phase, b_vec, b_per_phase, b_max_phase))
    return TBL_ERR_INVALID_ARG;
  const int gm = static_cast<int>((M + 255) / 256), gn = static_cast<int>((N + 255) / 256);
  int programs = 0;
  rc = resolve_programs(dtype, 256, 256, 32, static_cast<int64_t>(gm) * gn, persistent, num_programs,
                        &programs);
  if (rc != TBL_OK) return rc;
  tbl::GemmLaunch a;
  a.A = A;
  a.B = B;
  a.C = C;
  a.M = static_cast<int>(M);
  a.N = static_cast<int>(N);
  a.K = static_cast<int>(K);
  a.order = make_order(swizzle_mode, gm, gn, group_size);
  a.num_programs = programs;
  a.trace = nullptr;
  if (tbl::launch_gemm_layout(m16, a_per_phase, a_max_phase, b_vec, b_per_phase, b_max_phase, a,
                              static_cast<hipStream_t>(stream)) != hipSuccess)
    return TBL_ERR_HIP;
  return TBL_OK;
}

}  // namespace

extern "C" {

int tbl_gemm_lds_layout(const void* A, const void* B, void* C, int64_t M, int64_t N, int64_t K,
                        int dtype, int swizzle_mode, int group_size, int persistent, int num_programs,
                        int a_per_phase, int a_max_phase, int b_vec, int b_per_phase,
                        int b_max_phase, void* stream) {
  return gemm_lds_layout_impl(false, A, B, C, M, N, K, dtype, swizzle_mode, group_size, persistent,
                              num_programs, a_per_phase, a_max_phase, b_vec, b_per_phase, b_max_phase,
                              stream);
}

int tbl_gemm_lds_layout16(const void* A, const void* B, void* C, int64_t M, int64_t N, int64_t K,
                          int dtype, int swizzle_mode, int group_size, int persistent, int num_programs,
                          int a_per_phase, int a_max_phase, int b_vec, int b_per_phase,
                          int b_max_phase, void* stream) {
  return gemm_lds_layout_impl(true, A, B, C, M, N, K, dtype, swizzle_mode, group_size, persistent,
                              num_programs, a_per_phase, a_max_phase, b_vec, b_per_phase, b_max_phase,
                              stream);
}

int64_t tbl_gemm_dynamic_workspace(int num_programs) {
  if (num_programs < 1 || num_programs > kMaxDynamicPrograms) return -1;
  return 32 + 32 * static_cast<int64_t>(num_programs);
}

}  // extern "C"

namespace {

// Bytes of a dynamic-schedule trace: 8 ints per 256 x 256 tile.
int64_t dynamic_trace_bytes(int64_t M, int64_t N) { return int64_t{32} * ((M + 255) / 256) * ((N + 255) / 256); }

// Checks the arguments of a dynamic-schedule GEMM and resolves its workgroup count; the workspace
// is checked by the caller. Returns TBL_OK with *programs set, or the error.

int prepare_dynamic(const void* A, const void* B, void* C, int64_t M, int64_t N, int64_t K, int dtype,
                    int swizzle_mode, int group_size, int num_programs, const int32_t* trace, int* programs) {
  int rc = validate_gemm(A, B, C, M, N, K, dtype, swizzle_mode, group_size, 1, num_programs, 256, 256, 32);
  if (rc != TBL_OK) return rc;
  // wave 0 posts the next tile at k step 0 and the others read it at step 4; the load cursor
  // moves to the next tile at the end of step nk - 5's loads
  if ((K + 31) / 32 < kMinDynamicKSteps) return TBL_ERR_SHAPE;
  const int gm = static_cast<int>((M + 255) / 256), gn = static_cast<int>((N + 255) / 256);
  if (static_cast<int64_t>(gm) * gn > (int64_t{1} << 30)) return TBL_ERR_SHAPE;
  if (extra_overlaps(trace, dynamic_trace_bytes(M, N), A, B, C, M, N, K, dtype)) return TBL_ERR_INVALID_ARG;
  rc = resolve_programs(dtype, 256, 256, 32, static_cast<int64_t>(gm) * gn, 1, num_programs, programs);
  if (rc != TBL_OK) return rc;
  if (*programs > kMaxDynamicPrograms) return TBL_ERR_INVALID_ARG;
  return TBL_OK;
}

int launch_dynamic(const void* A, const void* B, void* C, int64_t M, int64_t N, int64_t K, int dtype,
                   int swizzle_mode, int group_size, int programs, int32_t* workspace, int32_t* trace,
                   void* stream) {
  const int gm = static_cast<int>((M + 255) / 256), gn = static_cast<int>((N + 255) / 256);
  tbl::GemmLaunch a;
  a.A = A;
  a.B = B;
  a.C = C;
  a.M = static_cast<int>(M);
  a.N = static_cast<int>(N);
  a.K = static_cast<int>(K);
  // the claim queues take the remap's place: positions are the order's own ids
  a.order = make_order(swizzle_mode & ~TBL_XCD_REMAP, gm, gn, group_size);
  a.num_programs = programs;
  a.trace = trace;
  a.work = workspace;
  a.xcd_aware = (swizzle_mode & TBL_XCD_REMAP) ? 1 : 0;
  if (tbl::launch_gemm_dynamic(dtype, a, static_cast<hipStream_t>(stream)) != hipSuccess) return TBL_ERR_HIP;
  return TBL_OK;
}

}  // namespace

// The allocation-free variant's workspace: a device array of the library, one copy per GPU, for at
// most TBL_NOALLOC_MAX_PROGRAMS workgroups (the workspace layout of tbl_gemm_dynamic). In host code
// ``scratch`` names a host-side stand-in, so its device address is looked up once per device
// (hipGetSymbolAddress with that device current) and only that address is passed on.
constexpr int kNoAllocScratchInts = 32 + 32 * TBL_NOALLOC_MAX_PROGRAMS;
static __device__ __align__(256) int32_t scratch[kNoAllocScratchInts];

namespace {

std::mutex g_scratch_mutex;
int32_t* g_scratch_ptr[kMaxDevices] = {};

// The current device's copy of ``scratch`` (nullptr with TBL_ERR_HIP in *rc if the lookup fails).
int32_t* device_scratch(int* rc) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    *rc = TBL_ERR_HIP;
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) {
      *rc = TBL_ERR_HIP;
      return nullptr;
    }
    g_scratch_ptr[dev] = static_cast<int32_t*>(p);
  }
  *rc = TBL_OK;
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

int tbl_gemm_dynamic(const void* A, const void* B, void* C, int64_t M, int64_t N, int64_t K, int dtype,
                     int swizzle_mode, int group_size, int num_programs, int32_t* workspace,
                     int64_t workspace_ints, int32_t* trace, void* stream) {
  int programs = 0;
  int rc = prepare_dynamic(A, B, C, M, N, K, dtype, swizzle_mode, group_size, num_programs, trace, &programs);
  if (rc != TBL_OK) return rc;
  if (workspace == nullptr || !aligned16(workspace)) return workspace == nullptr ? TBL_ERR_INVALID_ARG
                                                                                 : TBL_ERR_ALIGN;
  if (workspace_ints < tbl_gemm_dynamic_workspace(programs)) return TBL_ERR_INVALID_ARG;
  // the part of the workspace the kernels touch
  const int64_t ws_bytes = 4 * tbl_gemm_dynamic_workspace(programs);
  if (extra_overlaps(workspace, ws_bytes, A, B, C, M, N, K, dtype)) return TBL_ERR_INVALID_ARG;
  if (overlaps(trace, dynamic_trace_bytes(M, N), workspace, ws_bytes)) return TBL_ERR_INVALID_ARG;
  return launch_dynamic(A, B, C, M, N, K, dtype, swizzle_mode, group_size, programs, workspace, trace,
                        stream);
}

int tbl_gemm_dynamic_noalloc(const void* A, const void* B, void* C, int64_t M, int64_t N, int64_t K,
                             int dtype, int swizzle_mode, int group_size, int num_programs,
                             int32_t* trace, void* stream) {
  int programs = 0;
  int rc = prepare_dynamic(A, B, C, M, N, K, dtype, swizzle_mode, group_size, num_programs, trace, &programs);
  if (rc != TBL_OK) return rc;
  if (programs > TBL_NOALLOC_MAX_PROGRAMS) return TBL_ERR_SCRATCH;
  int32_t* ws = device_scratch(&rc);
  if (ws == nullptr) return rc;
  return launch_dynamic(A, B, C, M, N, K, dtype, swizzle_mode, group_size, programs, ws, trace, stream);
}

int tbl_gemm(const void* A, const void* B, void* C, int64_t M, int64_t N, int64_t K, int dtype,
             int swizzle_mode, int group_size, int persistent, int num_programs, void* stream) {
  if (M < 0 || N < 0 || K < 0) return TBL_ERR_INVALID_ARG;
  int bm, bn, bk;
  tile_rule(M, N, &bm, &bn, &bk);
  return tbl_gemm_tiled(A, B, C, M, N, K, dtype, swizzle_mode, group_size, persistent, num_programs,
                        bm, bn, bk, nullptr, stream);
}

int tbl_default_num_programs(int64_t M, int64_t N, int64_t K, int dtype, int persistent,
                             int* num_programs) {
  if (num_programs == nullptr || M <= 0 || N <= 0 || K <= 0) return TBL_ERR_INVALID_ARG;
  if (dtype < TBL_F16 || dtype > TBL_BF16_F32OUT) return TBL_ERR_DTYPE;
  if (persistent != 0 && persistent != 1) return TBL_ERR_INVALID_ARG;
  int bm, bn, bk;
  tile_rule(M, N, &bm, &bn, &bk);
  if (M > kMaxDim || N > kMaxDim || K > kMaxDim) return TBL_ERR_SHAPE;
  return resolve_programs(dtype, bm, bn, bk, ((M + bm - 1) / bm) * ((N + bn - 1) / bn), persistent, 0,
                          num_programs, chunk_rows(N, K), N);
}

int tbl_tile_map(int swizzle_mode, int grid_m, int grid_n, int group_size, int32_t* tile_m,
                 int32_t* tile_n, void* stream) {
  if (grid_m < 0 || grid_n < 0) return TBL_ERR_SHAPE;
  if (grid_m == 0 || grid_n == 0) return check_mode(swizzle_mode, group_size);   // an empty table
  if (tile_m == nullptr || tile_n == nullptr) return TBL_ERR_INVALID_ARG;
  int rc = check_order(swizzle_mode, grid_m, grid_n, group_size);
  if (rc != TBL_OK) return rc;
  const tbl::TileOrder o = make_order(swizzle_mode, grid_m, grid_n, group_size);
  if (tbl::launch_tile_map(o, tile_m, tile_n, static_cast<hipStream_t>(stream)) != hipSuccess)
    return TBL_ERR_HIP;
  return bijective_grid(swizzle_mode, grid_m, grid_n) ? TBL_OK : TBL_WARN_NOT_BIJECTIVE;
}

int tbl_predict_l2(int swizzle_mode, int grid_m, int grid_n, int grid_k, int group_size,
                   int64_t a_block_bytes, int64_t b_block_bytes, int64_t capacity_bytes,
                   int num_caches, int num_programs, int resident, int64_t* hits,
                   int64_t* accesses) {
  if (hits == nullptr || accesses == nullptr) return TBL_ERR_INVALID_ARG;
  if (a_block_bytes < 1 || b_block_bytes < 1 || capacity_bytes < 0) return TBL_ERR_INVALID_ARG;
  if (num_caches < 1 || num_caches > 64 || num_programs < 0 || resident < 1) return TBL_ERR_INVALID_ARG;
  int rc = check_order(swizzle_mode, grid_m, grid_n, group_size);
  if (rc != TBL_OK) return rc;
  if (grid_k < 1 || grid_k > kMaxDim) return TBL_ERR_SHAPE;
  const int64_t tiles = static_cast<int64_t>(grid_m) * grid_n;
  // bounded work and memory: at most 2^33 block reads, 2^26 distinct blocks (16 bytes each)
  if (2 * tiles * grid_k > (int64_t{1} << 33)) return TBL_ERR_SHAPE;
  if ((static_cast<int64_t>(grid_m) + grid_n) * grid_k > (int64_t{1} << 26)) return TBL_ERR_SHAPE;
  const tbl::TileOrder o = make_order(swizzle_mode, grid_m, grid_n, group_size);
  tbl::predict_l2(o, grid_k, a_block_bytes, b_block_bytes, capacity_bytes, num_caches,
                  num_programs == 0 ? static_cast<int>(tiles) : num_programs, resident, hits,
                  accesses);
  return bijective_grid(swizzle_mode, grid_m, grid_n) ? TBL_OK : TBL_WARN_NOT_BIJECTIVE;
}

int tbl_predict_l2_lines(int swizzle_mode, int64_t M, int64_t N, int64_t K, int elem_bytes,
                         int block_m, int block_n, int block_k, int group_size, int num_caches,
                         int num_programs, int resident, int64_t sets, int ways, int64_t line_bytes,
                         int fold_from, int fold_width, uint64_t a_base, uint64_t b_base,
                         int64_t* hits, int64_t* accesses, int64_t* misses) {
  if (hits == nullptr || accesses == nullptr || misses == nullptr) return TBL_ERR_INVALID_ARG;
  if (elem_bytes != 1 && elem_bytes != 2 && elem_bytes != 4) return TBL_ERR_INVALID_ARG;
  if (block_m < 1 || block_n < 1 || block_k < 1 || block_m > 4096 || block_n > 4096 || block_k > 4096)
    return TBL_ERR_INVALID_ARG;
  if (num_caches < 1 || num_caches > 64 || num_programs < 0 || resident < 1) return TBL_ERR_INVALID_ARG;
  if (sets < 1 || ways < 1 || ways > 64 || sets * ways > (int64_t{1} << 24)) return TBL_ERR_INVALID_ARG;
  if (line_bytes < 1 || line_bytes > (1 << 20)) return TBL_ERR_INVALID_ARG;
  if (fold_from < 0 || fold_from > 63 || fold_width < 0 || fold_width > 32) return TBL_ERR_INVALID_ARG;
  if (M < 1 || N < 1 || K < 1 || M > kMaxDim || N > kMaxDim || K > kMaxDim) return TBL_ERR_SHAPE;
  const int64_t gm = (M + block_m - 1) / block_m, gn = (N + block_n - 1) / block_n;
  if (gm > kMaxDim || gn > kMaxDim) return TBL_ERR_SHAPE;
  int rc = check_order(swizzle_mode, static_cast<int>(gm), static_cast<int>(gn), group_size);
  if (rc != TBL_OK) return rc;
  // bounded work: at most 2^33 line reads (each tile row and k row reads at least one line)
  const int64_t nk = (K + block_k - 1) / block_k;
  const double lines_a = static_cast<double>(block_m) * (1.0 + static_cast<double>(block_k) * elem_bytes / line_bytes);
  const double lines_b = static_cast<double>(block_k) * (1.0 + static_cast<double>(block_n) * elem_bytes / line_bytes);
  if (static_cast<double>(gm) * gn * nk * (lines_a + lines_b) > 8589934592.0) return TBL_ERR_SHAPE;
  // the last byte of either operand must be addressable
  const double span = static_cast<double>(M) * K * elem_bytes + static_cast<double>(K) * N * elem_bytes;
  if (static_cast<double>(a_base) + span > 1.8e19 || static_cast<double>(b_base) + span > 1.8e19)
    return TBL_ERR_INVALID_ARG;
  const tbl::TileOrder o = make_order(swizzle_mode, static_cast<int>(gm), static_cast<int>(gn), group_size);
  const tbl::GemmReadShape r{M, N, K, elem_bytes, block_m, block_n, block_k, a_base, b_base};
  const tbl::L2Geometry g{sets, ways, line_bytes, fold_from, fold_width};
  tbl::predict_l2_lines(o, r, g, num_caches, num_programs == 0 ? gm * gn : num_programs, resident,
                        hits, accesses);
  *misses = *accesses - *hits;
  return bijective_grid(swizzle_mode, static_cast<int>(gm), static_cast<int>(gn)) ? TBL_OK
                                                                                : TBL_WARN_NOT_BIJECTIVE;
}

int tbl_transpose_i32(const int32_t* in, int32_t* out, int64_t rows, int64_t cols, int layout,
                      void* stream) {
  if (rows < 0 || cols < 0) return TBL_ERR_INVALID_ARG;
  if ((in == nullptr || out == nullptr) && rows * cols > 0) return TBL_ERR_INVALID_ARG;
  if (layout < TBL_T_NAIVE || layout > TBL_T_XOR) return TBL_ERR_INVALID_ARG;
  if (rows % 64 || cols % 64 || rows > kMaxDim || cols > kMaxDim) return TBL_ERR_SHAPE;
  if (rows == 0 || cols == 0) return TBL_OK;   // no element
  if (!aligned16(in) || !aligned16(out)) return TBL_ERR_ALIGN;
  if (overlaps(in, rows * cols * 4, out, rows * cols * 4)) return TBL_ERR_INVALID_ARG;
  if (tbl::launch_transpose_i32(in, out, static_cast<int>(rows), static_cast<int>(cols), layout,
                                static_cast<hipStream_t>(stream)) != hipSuccess)
    return TBL_ERR_HIP;
  return TBL_OK;
}

int tbl_copy16(const void* src, void* dst, int64_t bytes, int nontemporal, void* stream) {
  if (bytes < 0 || ((src == nullptr || dst == nullptr) && bytes > 0)) return TBL_ERR_INVALID_ARG;
  if (nontemporal != 0 && nontemporal != 1) return TBL_ERR_INVALID_ARG;
  if (bytes % 16 != 0 || bytes > kMaxCopyBytes) return TBL_ERR_SHAPE;
  if (bytes == 0) return TBL_OK;
  if (!aligned16(src) || !aligned16(dst)) return TBL_ERR_ALIGN;
  if (overlaps(src, bytes, dst, bytes)) return TBL_ERR_INVALID_ARG;
  if (tbl::launch_copy16(src, dst, bytes, nontemporal == 1, static_cast<hipStream_t>(stream)) != hipSuccess)
    return TBL_ERR_HIP;
  return TBL_OK;
}

int tbl_mfma_rate(const void* A, const void* B, int64_t elems, int dtype, int workgroups, int iters,
                  float* out, int64_t* cycles, void* stream) {
  if (A == nullptr || B == nullptr || out == nullptr || cycles == nullptr) return TBL_ERR_INVALID_ARG;
  if (dtype < TBL_F16 || dtype > TBL_BF16_F32OUT) return TBL_ERR_DTYPE;
  if (elems < 8 || workgroups < 1 || workgroups > 65536 || iters < 1 || iters > (1 << 24))
    return TBL_ERR_INVALID_ARG;
  if (!aligned16(A) || !aligned16(B)) return TBL_ERR_ALIGN;
  const bool bf16 = dtype == TBL_BF16 || dtype == TBL_BF16_F32OUT;
  if (tbl::launch_mfma_rate(A, B, elems, bf16, workgroups, iters, out, cycles,
                            static_cast<hipStream_t>(stream)) != hipSuccess)
    return TBL_ERR_HIP;
  return TBL_OK;
}

int tbl_device_info(int* num_cus, int* num_xcds, int* lds_bytes, int* l2_bytes, char* arch,
                    int arch_len) {
  DeviceInfo d;
  int rc = device_info(&d);
  if (rc != TBL_OK) return rc;
  if (num_cus) *num_cus = d.cus;
  if (num_xcds) *num_xcds = tbl::kNumXcds;
  if (lds_bytes) *lds_bytes = d.lds;
  if (l2_bytes) *l2_bytes = d.l2;
  if (arch != nullptr && arch_len > 0) {
    strncpy(arch, d.arch, static_cast<size_t>(arch_len) - 1);
    arch[arch_len - 1] = '\0';
  }
  return TBL_OK;
}

}  // extern "C"
