"""Writes gemm16_lds_conflicts_4096.txt: the oracle's predicted LDS bank-conflict cycles of one
4096^3 fp16 GEMM launch in the 16x16x32 MFMA form (256x256x32 tiles, eight waves in a 2 x 4 grid)
for every compiled operand-layout variant of that form. Written before those variants were
measured on the device.

b_vec = 0 names the kernel's default B layout (chunk XOR 4 (k mod 4) + 2 ((k / 8) mod 2)); other
(b_vec, b_per_phase, b_max_phase) are members of the Triton chunk-XOR family.

Calls only oracle/. Run from the repository root: python tests/golden/make_gemm16_lds_conflicts.py
"""

import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

from oracle import lds  # noqa: E402

# (a_per_phase, a_max_phase, b_vec, b_per_phase, b_max_phase) -> the oracle's B layout name
LAYOUTS = [((2, 4, 0, 0, 0), "kstep8"), ((4, 4, 0, 0, 0), "kstep8"), ((1, 1, 0, 0, 0), "kstep8"),
           ((4, 2, 0, 0, 0), "kstep8"), ((2, 4, 4, 1, 4), "vec4"), ((2, 4, 1, 1, 1), "none")]


def main():
    out = os.path.join(os.path.dirname(os.path.abspath(__file__)), "gemm16_lds_conflicts_4096.txt")
    with open(out, "w") as f:
        f.write("# Predicted LDS bank-conflict cycles (extra passes) of one 4096^3 fp16 GEMM launch in the\n"
                "# 16x16x32 MFMA form, 256x256x32 tiles, eight waves (2 x 4, 128 x 64 each), per operand\n"
                "# layout, from oracle.lds.gemm16_lds_conflicts: the chunk-XOR family of \"CUDA Swizzle &\n"
                "# bank conflict\" (section \"Triton - Shared Layout swizzling\") and that page's bank model with\n"
                "# gfx950's geometry (64 banks x 4 bytes; 16- and 8-byte reads in 32-lane phases), applied to\n"
                "# this form's read patterns. b_vec 0 = the kernel's default B layout. Written by\n"
                "# make_gemm16_lds_conflicts.py before the variants were measured.\n"
                "# a_per_phase a_max_phase b_vec b_per_phase b_max_phase extra_a_per_step extra_b_per_step launch_total\n")
        for v, b in LAYOUTS:
            a_x, b_x = lds.gemm16_operand_read_passes(v[0], v[1], lds.GEMM16_B_LAYOUTS[b])
            total = lds.gemm16_lds_conflicts(4096, 4096, 4096, v[0], v[1], b)
            f.write(" ".join(str(x) for x in v) + f" {a_x} {b_x} {total}\n")
    print(out)


if __name__ == "__main__":
    main()
