/*
 * tbl.h -- C ABI of the MI355X (gfx950) swizzled-GEMM / LDS-transpose library (libtbl.so).
 *
 * Operations and where they are defined:
 *   - tbl_gemm / tbl_gemm_tiled: the tiled dense GEMM C = A * B whose program-id -> output-tile
 *     mapping is swizzled ("CUDA Thread Block Swizzle", leimao.github.io: sections "Linear Swizzle",
 *     "Grouped 2D Panel Swizzle", "Morton / Z-order Swizzle", "Bitwise XOR Swizzle", and the GEMM
 *     kernel with its persistent tile loop in section "CUDA Thread Block Swizzle Benchmark"), plus the
 *     group-major and serpentine orders of the tvm_tirx ClusterPersistentScheduler2D page
 *     (tvm.apache.org: "Tile Ordering", "Serpentine Mode", "Example 1").
 *   - tbl_gemm_dynamic: the same GEMM with a dynamic persistent schedule, tiles handed out at run
 *     time by counters -- what the persistent tile loop of "CUDA Thread Block Swizzle" (section
 *     "CUDA Thread Block Swizzle Benchmark", its "Known limitations") notes it does not have.
 *   - tbl_gemm_lds_layout, tbl_gemm_lds_layout16: the same GEMM (32x32x16- or 16x16x32-MFMA form)
 *     with the operands' LDS swizzles taken from the chunk-XOR
 *     family of "CUDA Swizzle & bank conflict" (section "Triton - Shared Layout swizzling").
 *   - tbl_tile_map: the program-id -> (m, n) table of any order, computed by the same device code
 *     the GEMM uses.
 *   - tbl_transpose_i32: the int32 shared-memory transpose with naive, padded and XOR-swizzled LDS
 *     layouts ("CUDA Swizzle & bank conflict", whc-imageprocess.github.io: section
 *     "Case Study / Matrix Transpose").
 *   - tbl_mfma_rate: a measurement aid, the GEMM's inner MFMA stream on its own operand data with no
 *     memory traffic, which gives the matrix-pipe rate the chip sustains for that data.
 *   - tbl_copy16: a measurement aid, a plain device copy that gives the HBM rate of the transpose's
 *     read-once, write-once traffic.
 *   - tbl_predict_l2: the offline LRU prediction of an order's L2 hit rate ("CUDA Thread Block
 *     Swizzle", section "CUDA Thread Block Swizzle Benchmark"), generalised to several private
 *     caches; host code only. tbl_predict_l2_lines: the same replay per cache line through
 *     set-associative caches indexed by address.
 *
 * Conventions shared by every entry point:
 *   - Matrices are dense and row-major with no padding: A is M x K, B is K x N, C is M x N.
 *   - Every pointer is device memory owned by the caller. The library never allocates or frees
 *     device memory in these calls and keeps no pointer after a call returns. A buffer a call writes
 *     must share no byte with the buffers it reads or its other outputs; the GEMM, transpose and copy
 *     entry points check this from the sizes and return TBL_ERR_INVALID_ARG. GEMM and transpose
 *     base pointers must be 16-byte aligned.
 *   - ``stream`` is a hipStream_t (NULL = the null stream). Calls enqueue work and return; only
 *     launch-time errors are reported, device-side faults surface at the caller's next
 *     synchronisation.
 *   - Every argument is validated before any HIP call, so invalid arguments return an error with
 *     nothing enqueued, also on a machine without a GPU.
 *   - Return value: TBL_OK (0) on success, a negative TBL_ERR_* on error, a positive TBL_WARN_* on
 *     success with a warning. tbl_status_string() gives text for any code.
 *   - Thread safety: the only global state is a per-device cache of device properties and of the
 *     scratch array's address (tbl_gemm_dynamic_noalloc), filled on first use; calls from several
 *     host threads are safe, except tbl_gemm_dynamic_noalloc calls that overlap on one GPU (they share
 *     its scratch array). Calls that write the same output race.
 *   - Every entry point allocates nothing; tbl_gemm_dynamic_noalloc uses a device array of the
 *     library instead of a workspace argument.
 */
#ifndef TBL_H_
#define TBL_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ---------------------------------------------------------------------------- */
enum {
  TBL_OK = 0,
  TBL_ERR_INVALID_ARG = -1,   /* null pointer, non-positive size, unknown mode/layout, bad group, overlapping buffers */
  TBL_ERR_DTYPE = -2,         /* unknown dtype code */
  TBL_ERR_SHAPE = -3,         /* sizes out of range, unsupported tile, or a cluster that does not tile the grid */
  TBL_ERR_NOT_BIJECTIVE = -4, /* GEMM with Morton/XOR on a (cluster) grid that is not a square power of two */
  TBL_ERR_HIP = -5,           /* a HIP runtime call failed (no device, launch failure, ...) */
  TBL_ERR_ALIGN = -6,         /* a GEMM or transpose pointer is not 16-byte aligned */
  TBL_ERR_SCRATCH = -7,       /* tbl_gemm_dynamic_noalloc: more workgroups than its scratch holds */
  TBL_WARN_NOT_BIJECTIVE = 1  /* tbl_tile_map wrote the table, but it is not a bijection */
};

/* ---- element types of a GEMM: A and B share the input type; C is the output type -------------- */
enum {
  TBL_F16 = 0,          /* A, B, C fp16 (IEEE binary16); fp32 accumulation; C rounded to nearest even */
  TBL_BF16 = 1,         /* A, B, C bfloat16; fp32 accumulation; C rounded to nearest even */
  TBL_F16_F32OUT = 2,   /* A, B fp16; C fp32 (the accumulator itself) */
  TBL_BF16_F32OUT = 3   /* A, B bf16; C fp32 */
};

/* ---- tile orders (swizzle modes) --------------------------------------------------------------
 * A tile id t in [0, T), T = grid_m * grid_n, is mapped to output tile (m, n):
 *   TBL_ROW        m = t / grid_n, n = t % grid_n                                 (linear, row-major)
 *   TBL_COL        m = t % grid_m, n = t / grid_m                                 (linear, column-major)
 *   TBL_PANEL      groups of ``group`` tile rows taken in row order; inside a group ids run down a
 *                  column of the group, then along the columns; the last group keeps the rows that
 *                  remain, and the row inside it is t modulo its height (grouped 2D panel; also the
 *                  group-major order of the tvm page)
 *   TBL_MORTON     bit 2i of t -> bit i of m, bit 2i+1 -> bit i of n (16 bit pairs), then modulo
 *                  the grid (Z-order; a bijection only on square power-of-two grids)
 *   TBL_XOR        x = t % grid_n, y = t / grid_n; m = (x ^ y) % grid_m, n = y % grid_n
 *                  (a bijection only on square power-of-two grids)
 *   TBL_SERPENTINE column strips ``group`` tiles wide, left to right; even strips walked top to
 *                  bottom, odd strips bottom to top, columns ascending along each strip row; the last
 *                  strip keeps the columns that remain (the reading of the tvm page's serpentine mode
 *                  that reproduces its 4x4 table)
 * TBL_XCD_REMAP may be OR-ed into any mode: before the order is applied, t is replaced by
 *   t' = (t % 8) * (T8 / 8) + t / 8 for t < T8 = 8 * floor(T / 8) (t' = t otherwise), so that the
 *   workgroups that round-robin dispatch places on one of the 8 XCDs (each with a private L2) walk one
 *   contiguous eighth of the order.
 * TBL_CLUSTER(cm, cn) may be OR-ed into any mode (1 <= cm, cn <= 16; TBL_CLUSTER(1, 1) is 0): the
 *   two-level schedule of the tvm_tirx page ("Example 2"). The order walks the (grid_m / cm) x
 *   (grid_n / cn) grid of cluster tiles: the (remapped) id t has cluster id c = t / (cm cn), which the
 *   order maps to cluster tile (m_c, n_c) (group / strip width counted in cluster tiles), and rank
 *   r = t % (cm cn), which picks tile (m_c cm + r % cm, n_c cn + r / cm). cm and cn must divide the
 *   tile grid (TBL_ERR_SHAPE otherwise); Morton and XOR need a square power-of-two cluster grid.
 *   With TBL_XCD_REMAP the ids of one cluster are consecutive on one XCD.
 */
enum {
  TBL_ROW = 0,
  TBL_COL = 1,
  TBL_PANEL = 2,
  TBL_MORTON = 3,
  TBL_XOR = 4,
  TBL_SERPENTINE = 5,
  TBL_XCD_REMAP = 0x100
};
#define TBL_CLUSTER(cm, cn) (((((cm) - 1) & 15) << 16) | ((((cn) - 1) & 15) << 20))

/* ---- LDS layouts of the transpose ---------------------------------------------------------- */
enum {
  TBL_T_NAIVE = 0,   /* 64 x 64 int32 tile, element (r, c) at r*64 + c */
  TBL_T_PADDED = 1,  /* 64 x 65 array, element (r, c) at r*65 + c */
  TBL_T_XOR = 2      /* element (r, c) at r*64 + (c XOR r) */
};

/*
 * tbl_gemm -- C = A * B with a swizzled, optionally persistent tile schedule.
 *   A, B, C       device pointers (row-major M x K, K x N, M x N), 16-byte aligned (TBL_ERR_ALIGN).
 *                 C shares no byte with A or B (TBL_ERR_INVALID_ARG); A and B may overlap.
 *   M, N, K       sizes, >= 0 (TBL_ERR_INVALID_ARG otherwise), each <= 2^20 (TBL_ERR_SHAPE
 *                 otherwise); any values. M = 0 or N = 0: C has no element and nothing is enqueued.
 *                 K = 0 (M, N > 0): C is set to +0, the empty sum, by a fill kernel. A buffer with
 *                 no element may be NULL. The tile shape is
 *                 fixed by a rule (tbl_gemm_tile_shape): 256x256x32 when that grid has at least 128
 *                 tiles (half of gfx950's 256 CUs), else 128x128x32 when its grid does, else 64x64x32
 *                 (k advances through LDS 32 deep). The tile grid is ceil(M/BM) x
 *                 ceil(N/BN); loads and stores are masked at every edge, as the page's kernel masks
 *                 them. When N and K are multiples of 8 (rows of A and B are whole 16-byte chunks)
 *                 the fast kernels run, moving operands with 16-byte direct-to-LDS loads; otherwise
 *                 a general path with the same tile grid, schedule and trace, which moves
 *                 operands through registers (A in unaligned 16-byte chunks, B in 16-byte chunks
 *                 when N is a multiple of 8, else element by element) and runs at roughly 40-65 %
 *                 of the fast kernels' rate at 4096-sized shapes.
 *   dtype         TBL_F16, TBL_BF16, TBL_F16_F32OUT or TBL_BF16_F32OUT.
 *   swizzle_mode  a TBL_* order, optionally | TBL_XCD_REMAP and | TBL_CLUSTER(cm, cn). Morton and
 *                 XOR need a square power-of-two grid of (cluster) tiles (TBL_ERR_NOT_BIJECTIVE
 *                 otherwise).
 *   group_size    group (TBL_PANEL) or strip width (TBL_SERPENTINE), >= 1; ignored by other modes.
 *   persistent    0: one workgroup per tile (num_programs defaults to T). 1: num_programs defaults
 *                 to min(T, CUs x resident workgroups per CU).
 *   num_programs  0 = the default above; > 0 = exactly this many workgroups. Workgroup p computes
 *                 tiles p, p + num_programs, p + 2 num_programs, ... < T (the static stride
 *                 schedule of the swizzle page's persistent loop); < 0 is TBL_ERR_INVALID_ARG.
 *   stream        hipStream_t or NULL.
 * Every output element is computed by exactly one workgroup with fp32 accumulation over k in
 * ascending 32-deep 16x16x32 MFMA steps (every tile shape and the general path; the 32x32x16
 * form of tbl_gemm_lds_layout takes two 16-deep steps instead, which on gfx950 leave the same
 * bits), so the result does not depend on the order, the remap flag, persistence, num_programs or
 * the tile shape.
 */
int tbl_gemm(const void* A, const void* B, void* C, int64_t M, int64_t N, int64_t K, int dtype,
             int swizzle_mode, int group_size, int persistent, int num_programs, void* stream);

/*
 * tbl_gemm_tiled -- tbl_gemm with an explicit tile shape and an optional schedule trace.
 *   block_m, block_n, block_k  one of the compiled shapes: 64x64x32, 128x128x32, 256x256x32
 *                 (TBL_ERR_SHAPE otherwise).
 *   trace         NULL, or device int32[8 * T]: for every tile id t the workgroup that ran it writes
 *                 {program id, iteration of its tile loop, m, n, XCC id, core-clock cycles and
 *                 100 MHz real-time ticks from the tile's start to its epilogue, the start as the
 *                 low 32 bits of the 100 MHz real-time counter}. A program's first tile starts
 *                 before its prologue loads, a later tile where the previous tile's epilogue ends
 *                 (its operands are already loading then). Times are those of the workgroup's
 *                 first wave.
 *                 Caller-owned; shares no byte with A, B or C (TBL_ERR_INVALID_ARG). Tracing adds a
 *                 few instructions per tile.
 *   All other arguments as tbl_gemm. With K = 0 no tile runs and the trace is left as it is.
 */
int tbl_gemm_tiled(const void* A, const void* B, void* C, int64_t M, int64_t N, int64_t K, int dtype,
                   int swizzle_mode, int group_size, int persistent, int num_programs, int block_m,
                   int block_n, int block_k, int32_t* trace, void* stream);

/*
 * tbl_gemm_dynamic -- tbl_gemm on 256x256x32 tiles with a dynamic persistent schedule ("CUDA Thread
 * Block Swizzle", section "CUDA Thread Block Swizzle Benchmark": its persistent loop hands tile ids
 * out statically, p, p + P, ...; its "Known limitations" name counter-based assignment as the
 * missing alternative). The positions 0 .. T-1 of the tile order (swizzle_mode, group_size,
 * clusters as tbl_gemm) are handed out in increasing order by claim counters; a workgroup claims
 * its next tile when it starts its current one. Without TBL_XCD_REMAP one counter serves all
 * positions and workgroup p's first tile is position p. With TBL_XCD_REMAP (which here replaces the
 * remap) there is one counter per XCD over the block floor(x T / 8) .. floor((x + 1) T / 8) - 1:
 * workgroup p's first tile is the (p / 8)-th position of block p mod 8 (the XCD round-robin
 * dispatch puts it on), and a workgroup on XCD x (the hardware's XCC id) claims from block x, then,
 * once it is empty, from the block with the most positions left. With equal tile times this
 * reproduces the stride schedule (resp. the XCD-remapped one); otherwise faster workgroups take
 * more tiles. The result bits equal tbl_gemm_tiled's with 256x256x32 tiles.
 *   num_programs  workgroups; 0 = CUs x the kernel's occupancy; at most 65536.
 *   workspace     device int32[workspace_ints], 16-byte aligned, caller-owned, with
 *                 workspace_ints >= tbl_gemm_dynamic_workspace(num_programs as resolved). Each call
 *                 first enqueues a one-workgroup kernel that zeroes the claim counters (ints 0..8),
 *                 so no initial contents are needed; calls that share a workspace must not overlap
 *                 in time (same stream, or synchronised). int 9 counts hand-over faults between a
 *                 workgroup's waves: never expected, never reset; zero it to watch it. The ints the
 *                 kernels touch share no byte with A, B, C or the trace (TBL_ERR_INVALID_ARG).
 *   trace         NULL or device int32[8 * T], as tbl_gemm_tiled (no byte shared with A, B or C),
 *                 indexed by order position.
 *   K             at least 257 (nine 32-deep k steps per tile: a tile's successor is claimed and
 *                 handed to all waves in its first five, before the loads run into it);
 *                 TBL_ERR_SHAPE otherwise. The tile grid may have at most 2^30 tiles.
 *   N, K          multiples of 8 (this schedule runs only the fast kernel, whose direct loads move
 *                 row chunks of 16 bytes); TBL_ERR_SHAPE otherwise.
 *   M, N          >= 1 (TBL_ERR_INVALID_ARG otherwise).
 *   All other arguments as tbl_gemm. Errors: as tbl_gemm_tiled, plus TBL_ERR_INVALID_ARG for a NULL
 *   or short workspace, TBL_ERR_ALIGN for a misaligned one.
 */
int tbl_gemm_dynamic(const void* A, const void* B, void* C, int64_t M, int64_t N, int64_t K, int dtype,
                     int swizzle_mode, int group_size, int num_programs, int32_t* workspace,
                     int64_t workspace_ints, int32_t* trace, void* stream);

/* int32 elements of the workspace tbl_gemm_dynamic needs for num_programs workgroups (>= 1), or -1
 * if num_programs is out of range. */
int64_t tbl_gemm_dynamic_workspace(int num_programs);

/*
 * tbl_gemm_dynamic_noalloc -- tbl_gemm_dynamic without a workspace argument, for callers that
 * cannot allocate device memory (code under HIP graph capture, serving loops, harnesses that forbid
 * hipMalloc). The claim counters and mailboxes live in a device array of the library (one per GPU,
 * 4 * (32 + 32 * TBL_NOALLOC_MAX_PROGRAMS) bytes = 512 KiB, held until the process ends), whose
 * address is looked up once per device. The call allocates nothing and calls no allocating routine.
 *   num_programs  as tbl_gemm_dynamic (0 = CUs x occupancy); a count above
 *                 TBL_NOALLOC_MAX_PROGRAMS returns TBL_ERR_SCRATCH before any HIP call when given,
 *                 after the occupancy query when resolved.
 *   Every other argument, the result bits and the errors are those of tbl_gemm_dynamic. Each call
 *   first zeroes the claim counters with a one-workgroup kernel (no memset), so the array needs no
 *   initial contents; all calls on one GPU share its array, so calls that overlap in time on one GPU
 *   (different streams, several host threads) race and must be serialised by the caller.
 */
#define TBL_NOALLOC_MAX_PROGRAMS 4096
int tbl_gemm_dynamic_noalloc(const void* A, const void* B, void* C, int64_t M, int64_t N, int64_t K,
                             int dtype, int swizzle_mode, int group_size, int num_programs,
                             int32_t* trace, void* stream);

/*
 * tbl_gemm_lds_layout -- tbl_gemm on 256x256x32 tiles with chosen LDS swizzles for the operands,
 * members of the chunk-XOR family of "CUDA Swizzle & bank conflict" (section "Triton - Shared
 * Layout swizzling"), on 16-byte chunks. A sits in LDS as rows of 32 k (4 chunks): row r stores
 * logical chunk c at c XOR ((r / a_per_phase) mod a_max_phase). B sits k-major as rows of 256 n
 * (32 chunks): row k stores chunk c at c XOR ((((k / b_per_phase) mod b_max_phase) * b_vec) mod 32).
 * The variants run the 256x256 kernel in its 32x32x16-MFMA form, whose operand reads these
 * layouts were chosen for (tbl_gemm itself runs the 16x16x32 form, with A at (2,4) and its own B
 * layout). The layout changes which LDS banks the operand reads hit, never the result: every
 * variant returns the same bits as tbl_gemm_tiled with 256x256x32 tiles.
 *   dtype         TBL_F16 only (TBL_ERR_DTYPE otherwise).
 *   (a_per_phase, a_max_phase, b_vec, b_per_phase, b_max_phase) one of the compiled variants:
 *                 (4,4,4,1,4) conflict-free for the 32x32x16 reads; A varied with B at its default:
 *                 (1,1,...) no swizzle, (1,4), (2,4), (4,2), (8,4); B varied with A at its default:
 *                 (...,1,1,1) no swizzle, (1,1,4), (2,1,4), (4,1,2), (4,2,2), (8,1,4).
 *                 TBL_ERR_INVALID_ARG for any other combination.
 *   N, K          multiples of 8, as for tbl_gemm_dynamic (TBL_ERR_SHAPE otherwise).
 *   M, N, K       >= 1 (TBL_ERR_INVALID_ARG otherwise).
 *   All other arguments as tbl_gemm (num_programs = 0 resolves as for the 256x256 kernel).
 */
int tbl_gemm_lds_layout(const void* A, const void* B, void* C, int64_t M, int64_t N, int64_t K,
                        int dtype, int swizzle_mode, int group_size, int persistent, int num_programs,
                        int a_per_phase, int a_max_phase, int b_vec, int b_per_phase,
                        int b_max_phase, void* stream);

/*
 * tbl_gemm_lds_layout16 -- tbl_gemm_lds_layout in the 16x16x32-MFMA form that tbl_gemm runs (the
 * same source, same section of "CUDA Swizzle & bank conflict"), whose operand reads take other lane
 * patterns (A: 16 rows x 2 chunks per half-wave; B: transposing reads of k rows k0..k0+3 and
 * k0+8..k0+11). b_vec = 0 (with b_per_phase = b_max_phase = 0) selects its default B layout, chunk c
 * of row k at c XOR (4 (k mod 4) + 2 ((k / 8) mod 2)); other B triples are family members as above.
 * Every variant returns the same bits as tbl_gemm_tiled with 256x256x32 tiles.
 *   (a_per_phase, a_max_phase, b_vec, b_per_phase, b_max_phase) one of the compiled variants:
 *                 (2,4,0,0,0) the default kernel's layouts; (4,4,0,0,0), (1,1,0,0,0) and (4,2,0,0,0)
 *                 vary A; (2,4,4,1,4) and (2,4,1,1,1) vary B. TBL_ERR_INVALID_ARG otherwise.
 *   All other arguments and errors as tbl_gemm_lds_layout.
 */
int tbl_gemm_lds_layout16(const void* A, const void* B, void* C, int64_t M, int64_t N, int64_t K,
                          int dtype, int swizzle_mode, int group_size, int persistent, int num_programs,
                          int a_per_phase, int a_max_phase, int b_vec, int b_per_phase,
                          int b_max_phase, void* stream);

/*
 * tbl_tile_map -- write the forward table of an order: tile_m[t], tile_n[t] for t in [0, T).
 *   swizzle_mode  as tbl_gemm (TBL_XCD_REMAP and TBL_CLUSTER allowed).
 *   grid_m, grid_n  the tile grid, each in [0, 2^20], with grid_m * grid_n < 2^31. An empty grid
 *                 (either 0) has an empty table: nothing is written (the pointers may be NULL).
 *   group_size    as tbl_gemm (>= 1 for TBL_PANEL / TBL_SERPENTINE).
 *   tile_m, tile_n  device int32[T], caller-owned.
 * Returns TBL_WARN_NOT_BIJECTIVE (after enqueueing) for Morton/XOR on a grid that is not a square
 * power of two: the table is still written, exactly as the formulas give it.
 */
int tbl_tile_map(int swizzle_mode, int grid_m, int grid_n, int group_size, int32_t* tile_m,
                 int32_t* tile_n, void* stream);

/*
 * tbl_transpose_i32 -- out (cols x rows) = transpose of in (rows x cols), int32, bit-exact,
 * staged through a 64 x 64 LDS tile in the given layout.
 *   in, out       device pointers, 16-byte aligned (TBL_ERR_ALIGN), sharing no byte
 *                 (TBL_ERR_INVALID_ARG).
 *   rows, cols    >= 0 (TBL_ERR_INVALID_ARG otherwise), multiples of 64, each <= 2^20
 *                 (TBL_ERR_SHAPE otherwise). Either 0: nothing to do, the pointers may be NULL.
 *   layout        TBL_T_NAIVE, TBL_T_PADDED or TBL_T_XOR.
 */
int tbl_transpose_i32(const int32_t* in, int32_t* out, int64_t rows, int64_t cols, int layout,
                      void* stream);

/*
 * tbl_predict_l2 -- offline L2 hit-rate prediction for an order (host only, no HIP call; runs on a
 * machine without a GPU). "CUDA Thread Block Swizzle", section "CUDA Thread Block Swizzle
 * Benchmark": operand blocks are replayed through a byte-capacity LRU cache. Running tiles are
 * taken together, and k block by k block each reads its A block (m, k) then its B block (k, n); a
 * miss inserts the block, then least-recently-used blocks are evicted while the cache holds more
 * than capacity_bytes and more than one block. Generalised to private caches: program p (tile ids
 * p, p + P, ..., as the persistent GEMM runs them; one id each when P >= T) replays on cache
 * p mod num_caches, `resident` programs of a cache at a time, in program order. The page's own
 * model is num_caches = 1, num_programs = T, resident = its wave size; gfx950's XCD L2s are
 * num_caches = 8, resident = CUs per XCD x workgroups per CU.
 *   swizzle_mode, grid_m, grid_n, group_size  as tbl_tile_map (the GEMM's executed order).
 *   grid_k          k blocks per tile, in [1, 2^20].
 *   a_block_bytes   bytes of one A block (block_m x block_k elements), >= 1; b_block_bytes likewise.
 *   capacity_bytes  per cache, >= 0.
 *   num_caches      in [1, 64].  num_programs  >= 0 (0 = T).  resident  >= 1.
 *   hits, accesses  host int64 outputs: hits and block reads summed over the caches
 *                   (accesses = 2 x T x grid_k).
 * TBL_ERR_SHAPE when 2 x T x grid_k > 2^33 or (grid_m + grid_n) x grid_k > 2^26 (work and host
 * memory bounds; the call allocates and frees 16 bytes per distinct block). Returns
 * TBL_WARN_NOT_BIJECTIVE, with results, where tbl_tile_map would.
 */
int tbl_predict_l2(int swizzle_mode, int grid_m, int grid_n, int grid_k, int group_size,
                   int64_t a_block_bytes, int64_t b_block_bytes, int64_t capacity_bytes,
                   int num_caches, int num_programs, int resident, int64_t* hits,
                   int64_t* accesses);

/*
 * tbl_predict_l2_lines -- the same offline replay counted per cache line through set-associative
 * caches indexed by address (host only, no HIP call). "CUDA Thread Block Swizzle", section "CUDA
 * Thread Block Swizzle Benchmark", replays operand blocks; this keeps its read order and program
 * grouping (as tbl_predict_l2: program p on cache p mod num_caches, tile ids p, p + P, ...,
 * `resident` programs of a cache at a time, each loop iteration of a group read k block by k
 * block, tiles in program order, A then B) and changes the unit read:
 *   - at k block j a tile reads, for each of its A rows (< M), the bytes of k in
 *     [j block_k, (j+1) block_k) (k < K), then for each B row k of the block its columns' bytes
 *     (< N); each contiguous range counts one access per line it touches;
 *   - each cache has `sets` sets of `ways` lines of `line_bytes`, least-recently-used within a
 *     set; line L (byte address / line_bytes) lives in set
 *     (L xor ((L >> fold_from) mod 2^fold_width)) mod sets (fold_width 0: plain modulo).
 * The gfx950 reading: 8 caches, 2048 sets, 16 ways, 128-byte lines, fold_from 11, fold_width 4
 * (address bits 18-21 folded onto bits 7-10); the fold is a fit to measured TCC counters.
 *   swizzle_mode, group_size  as tbl_tile_map, on the ceil(M/block_m) x ceil(N/block_n) grid.
 *   M, N, K         in [1, 2^20].   elem_bytes  1, 2 or 4.   block_*  in [1, 4096].
 *   num_caches      in [1, 64].  num_programs  >= 0 (0 = the tile count).  resident  >= 1.
 *   sets, ways      sets >= 1, ways in [1, 64], sets x ways <= 2^24.   line_bytes  in [1, 2^20].
 *   fold_from       in [0, 63].  fold_width  in [0, 32].
 *   a_base, b_base  byte addresses of A (M x K) and B (K x N), row-major (for example the device
 *                   pointers the GEMM will read).
 *   hits, accesses, misses  host int64 outputs summed over the caches; each miss fills one line,
 *                   so misses x line_bytes is the predicted fetch.
 * TBL_ERR_INVALID_ARG for arguments out of range, TBL_ERR_SHAPE when the replay would exceed 2^33
 * line reads. Host memory: 16 bytes per line of one cache, allocated and freed inside the call.
 * Returns TBL_WARN_NOT_BIJECTIVE, with results, where tbl_tile_map would.
 */
int tbl_predict_l2_lines(int swizzle_mode, int64_t M, int64_t N, int64_t K, int elem_bytes,
                         int block_m, int block_n, int block_k, int group_size, int num_caches,
                         int num_programs, int resident, int64_t sets, int ways, int64_t line_bytes,
                         int fold_from, int fold_width, uint64_t a_base, uint64_t b_base,
                         int64_t* hits, int64_t* accesses, int64_t* misses);

/*
 * tbl_mfma_rate -- the dense matrix-pipe rate the device sustains on given operand data (a
 * measurement aid for the GEMM's roofline, not part of the method). Each of the 4 waves of each of
 * ``workgroups`` 256-thread workgroups loads four 16-byte fragments of A and four of B (wave w,
 * fragment q, lane l takes the 8 values starting at element 8 x (((4 w + q) x 64 + l) mod (elems / 8)))
 * and then runs ``iters`` rounds of 32 independent 16x16x32 MFMAs (fp32 accumulate, accumulators
 * in VGPRs) in the GEMM's issue order, with no other memory traffic. The MFMA count is
 * 32 x iters x 4 x workgroups, each 2 x 16 x 16 x 32 flops. The chip lowers its core clock as the operands' switching activity
 * rises, so this rate, not the clock-only figure, bounds what the GEMM can reach on the same data.
 *   A, B        device pointers to at least ``elems`` 16-bit values each, 16-byte aligned.
 *   elems       >= 8.
 *   dtype       TBL_F16 / TBL_F16_F32OUT (fp16 operands) or TBL_BF16 / TBL_BF16_F32OUT (bf16).
 *   workgroups  in [1, 65536]; iters in [1, 2^24] (TBL_ERR_INVALID_ARG otherwise).
 *   out         device float[256 x workgroups]: per-lane sums of the accumulators (keeps the work
 *               observable; the values carry no meaning). Caller-owned.
 *   cycles      device int64[2]: core-clock cycles and 100 MHz real-time ticks of workgroup 0's
 *               first wave over its MFMA loop (their ratio is the core clock). Caller-owned.
 */
int tbl_mfma_rate(const void* A, const void* B, int64_t elems, int dtype, int workgroups, int iters,
                  float* out, int64_t* cycles, void* stream);

/*
 * tbl_copy16 -- dst = src, ``bytes`` bytes, 16 per lane (a measurement aid for the transpose's
 * roofline, not part of the method): the rate one read stream and one write stream of the same bytes
 * reach on this device, the traffic of tbl_transpose_i32 ("CUDA Swizzle & bank conflict", section
 * "Case Study / Matrix Transpose", reads and writes every element once).
 *   src, dst      device pointers, 16-byte aligned (TBL_ERR_ALIGN), ranges not overlapping
 *                 (TBL_ERR_INVALID_ARG).
 *   bytes         >= 0 (TBL_ERR_INVALID_ARG), a multiple of 16 and at most 2^40 (TBL_ERR_SHAPE);
 *                 0 copies nothing (the pointers may then be NULL).
 *   nontemporal   0: ordinary loads and stores; 1: non-temporal ones (streaming hints to the caches).
 */
int tbl_copy16(const void* src, void* dst, int64_t bytes, int nontemporal, void* stream);

/* tbl_gemm_tile_shape -- the tile shape tbl_gemm uses for these sizes (>= 0; host only, no HIP
 * call). */
int tbl_gemm_tile_shape(int64_t M, int64_t N, int64_t K, int* block_m, int* block_n, int* block_k);

/*
 * tbl_default_num_programs -- the num_programs tbl_gemm launches for num_programs = 0:
 * T when persistent = 0, else min(T, CUs x resident workgroups per CU of the chosen kernel, from
 * the HIP occupancy query). Writes *num_programs. Needs a device unless persistent = 0.
 */
int tbl_default_num_programs(int64_t M, int64_t N, int64_t K, int dtype, int persistent,
                             int* num_programs);

/*
 * tbl_device_info -- properties of the current device: compute units, XCDs (assumed 8 on gfx950),
 * LDS bytes per workgroup, L2 bytes (as reported by HIP), and the architecture name (written into
 * ``arch`` with at most arch_len bytes including the terminator; ``arch`` may be NULL).
 */
int tbl_device_info(int* num_cus, int* num_xcds, int* lds_bytes, int* l2_bytes, char* arch,
                    int arch_len);

/* tbl_status_string -- static text for a status code (never NULL). */
const char* tbl_status_string(int status);

/* tbl_version -- ABI version of this header (major * 100 + minor). */
int tbl_version(void);

#ifdef __cplusplus
}
#endif

#endif /* TBL_H_ */
