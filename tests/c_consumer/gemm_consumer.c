/*
 * A plain C11 consumer of libtbl.so (test infrastructure): device memory from the HIP runtime's C
 * API, the GEMM and the transpose through the C ABI of include/tbl.h, no Python and no torch.
 *
 *   gemm_consumer gemm M N K dtype mode group persistent A.bin B.bin C.bin
 *     A.bin, B.bin: the operands' 16-bit patterns, row-major; writes C (fp32 for the *_F32OUT
 *     dtypes, else 16-bit patterns) to C.bin.
 *   gemm_consumer transpose rows cols layout in.bin out.bin
 *     int32, row-major.
 * Exit status 0 on success; on any error it prints the failing call and exits 1.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "tbl.h"

static int fail(const char* what, const char* detail) {
  fprintf(stderr, "gemm_consumer: %s failed: %s\n", what, detail);
  return 1;
}

static void* read_file(const char* path, size_t bytes) {
  FILE* f = fopen(path, "rb");
  if (f == NULL) return NULL;
  void* p = malloc(bytes > 0 ? bytes : 1);
  if (p != NULL && fread(p, 1, bytes, f) != bytes) {
    free(p);
    p = NULL;
  }
  fclose(f);
  return p;
}

static int write_file(const char* path, const void* p, size_t bytes) {
  FILE* f = fopen(path, "wb");
  if (f == NULL) return -1;
  const size_t n = fwrite(p, 1, bytes, f);
  fclose(f);
  return n == bytes ? 0 : -1;
}

#define HIP_OK(call)                                               \
  do {                                                             \
    hipError_t e_ = (call);                                        \
    if (e_ != hipSuccess) return fail(#call, hipGetErrorString(e_)); \
  } while (0)

static int run_gemm(int argc, char** argv) {
  if (argc != 12) return fail("arguments", "gemm M N K dtype mode group persistent A B C");
  const int64_t M = atoll(argv[2]), N = atoll(argv[3]), K = atoll(argv[4]);
  const int dtype = atoi(argv[5]), mode = atoi(argv[6]), group = atoi(argv[7]), pers = atoi(argv[8]);
  const size_t out_elem = (dtype == TBL_F16_F32OUT || dtype == TBL_BF16_F32OUT) ? 4 : 2;
  const size_t a_bytes = (size_t)(M * K) * 2, b_bytes = (size_t)(K * N) * 2, c_bytes = (size_t)(M * N) * out_elem;
  void* ha = read_file(argv[9], a_bytes);
  void* hb = read_file(argv[10], b_bytes);
  void* hc = malloc(c_bytes);
  if (ha == NULL || hb == NULL || hc == NULL) return fail("reading the operands", argv[9]);
  void *da = NULL, *db = NULL, *dc = NULL;
  HIP_OK(hipMalloc(&da, a_bytes));
  HIP_OK(hipMalloc(&db, b_bytes));
  HIP_OK(hipMalloc(&dc, c_bytes));
  HIP_OK(hipMemcpy(da, ha, a_bytes, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(db, hb, b_bytes, hipMemcpyHostToDevice));
  const int rc = tbl_gemm(da, db, dc, M, N, K, dtype, mode, group, pers, 0, NULL);
  if (rc != TBL_OK) return fail("tbl_gemm", tbl_status_string(rc));
  HIP_OK(hipDeviceSynchronize());
  HIP_OK(hipMemcpy(hc, dc, c_bytes, hipMemcpyDeviceToHost));
  if (write_file(argv[11], hc, c_bytes) != 0) return fail("writing C", argv[11]);
  HIP_OK(hipFree(da));
  HIP_OK(hipFree(db));
  HIP_OK(hipFree(dc));
  free(ha);
  free(hb);
  free(hc);
  return 0;
}

static int run_transpose(int argc, char** argv) {
  if (argc != 7) return fail("arguments", "transpose rows cols layout in out");
  const int64_t rows = atoll(argv[2]), cols = atoll(argv[3]);
  const int layout = atoi(argv[4]);
  const size_t bytes = (size_t)(rows * cols) * 4;
  void* hx = read_file(argv[5], bytes);
  void* hy = malloc(bytes);
  if (hx == NULL || hy == NULL) return fail("reading the input", argv[5]);
  void *dx = NULL, *dy = NULL;
  HIP_OK(hipMalloc(&dx, bytes));
  HIP_OK(hipMalloc(&dy, bytes));
  HIP_OK(hipMemcpy(dx, hx, bytes, hipMemcpyHostToDevice));
  const int rc = tbl_transpose_i32((const int32_t*)dx, (int32_t*)dy, rows, cols, layout, NULL);
  if (rc != TBL_OK) return fail("tbl_transpose_i32", tbl_status_string(rc));
  HIP_OK(hipDeviceSynchronize());
  HIP_OK(hipMemcpy(hy, dy, bytes, hipMemcpyDeviceToHost));
  if (write_file(argv[6], hy, bytes) != 0) return fail("writing the output", argv[6]);
  HIP_OK(hipFree(dx));
  HIP_OK(hipFree(dy));
  free(hx);
  free(hy);
  return 0;
}

int main(int argc, char** argv) {
  if (argc >= 2 && strcmp(argv[1], "gemm") == 0) return run_gemm(argc, argv);
  if (argc >= 2 && strcmp(argv[1], "transpose") == 0) return run_transpose(argc, argv);
  return fail("arguments", "gemm ... | transpose ...");
}
