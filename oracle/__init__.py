"""CPU oracle for the swizzled-GEMM / LDS-transpose path.

TEST INFRASTRUCTURE. Only tests/, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
bench.py may import this package. The library (thread_block_lds_amd) never imports it, shares no
code with it, and does not fall back to it.

Everything here is plain and slow on purpose: each function restates, in its own words, the
definition or the steps given on one of the source pages, cited by page title and section:

  * "CUDA Thread Block Swizzle" (leimao.github.io)                 -- tile orders, the persistent
    stride schedule, the GEMM that the swizzle feeds, the offline L2 model.
  * "CUDA Swizzle & bank conflict" (whc-imageprocess.github.io)   -- shared-memory (LDS) bank model,
    padding and XOR layouts, the int32 shared-memory transpose.
  * "tvm_tirx ... ClusterPersistentScheduler2D" (tvm.apache.org)  -- group-major and serpentine
    orders, the per-cluster persistent work lists.

Floating point is fp64. Integer results (tile maps, transposes, layout maps) are exact.

Modules:
  tile_maps   pid -> (m, n) orders, XCD remap (a reading), persistent schedule
  gemm        fp16/bf16 decoding and the fp64 GEMM definition
  transpose   int32 transpose definition
  lds         LDS layout maps (naive / padded / XOR / chunk-XOR) and the bank-conflict model
  l2_model    byte-granular LRU L2 model and Spearman rank check (the offline predictor of "CUDA
              Thread Block Swizzle")
  l2_lines    the same replay counted per cache line through set-associative per-XCD caches (a
              reading for gfx950), in plain C (l2_lines.c) compiled with gcc on first use
  schedule    the static stride schedule and the dynamic (work-queue) schedule that "CUDA Thread
              Block Swizzle" names as missing: event simulation and the checks every GPU trace of
              it must pass
"""

from . import tile_maps, gemm, transpose, lds, l2_model, l2_lines, schedule  # noqa: F401
