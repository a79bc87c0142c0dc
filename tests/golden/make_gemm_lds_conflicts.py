"""Writes gemm_lds_conflicts_4096.txt: the oracle's predicted LDS bank-conflict cycles of one
4096^3 fp16 GEMM launch (256x256x32 tiles, eight waves in a 2 x 4 grid) for every compiled
operand-layout variant.

Calls only oracle/. Run from the repository root: python tests/golden/make_gemm_lds_conflicts.py
"""

import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

from oracle import lds  # noqa: E402

LAYOUTS = [(4, 4, 4, 1, 4), (1, 1, 4, 1, 4), (1, 4, 4, 1, 4), (2, 4, 4, 1, 4), (4, 2, 4, 1, 4),
           (8, 4, 4, 1, 4), (4, 4, 1, 1, 1), (4, 4, 1, 1, 4), (4, 4, 2, 1, 4), (4, 4, 4, 1, 2),
           (4, 4, 4, 2, 2), (4, 4, 8, 1, 4)]


def main():
    out = os.path.join(os.path.dirname(os.path.abspath(__file__)), "gemm_lds_conflicts_4096.txt")
    with open(out, "w") as f:
        f.write("# Predicted LDS bank-conflict cycles (extra passes) of one 4096^3 fp16 GEMM launch with\n"
                "# 256x256x32 tiles and eight waves (2 x 4, 128 x 64 each), per operand layout, from\n"
                "# oracle.lds.gemm_lds_conflicts: the chunk-XOR\n"
                "# family of \"CUDA Swizzle & bank conflict\" (section \"Triton - Shared Layout swizzling\") and\n"
                "# that page's bank model with gfx950's geometry (64 banks x 4 bytes; 16- and 8-byte reads\n"
                "# served in 32-lane phases). Written by make_gemm_lds_conflicts.py.\n"
                "# a_per_phase a_max_phase b_vec b_per_phase b_max_phase extra_a_per_step extra_b_per_step launch_total\n")
        for v in LAYOUTS:
            a, b = lds.gemm_operand_read_passes(*v, waves=(2, 4))
            f.write(" ".join(str(x) for x in v) + f" {a} {b} {lds.gemm_lds_conflicts(4096, 4096, 4096, v, waves=(2, 4))}\n")
    print(out)


if __name__ == "__main__":
    main()
