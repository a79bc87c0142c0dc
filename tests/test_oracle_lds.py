"""Pins of the LDS layout maps and the bank model. CPU only.

Pins: the five Triton shared-layout grids and the transpose case study's row-1 order printed on
"CUDA Swizzle & bank conflict"; the page's TMA chunk formula, which must give the same map as the
Triton family at vec = 16 bytes / element size, per_phase 1, max_phase 8; the three swizzle-map
properties the page lists (one-to-one, range kept, distinct within a column); the page's stride
claims (stride s gives an s-way conflict) and its closed-form conflict count for the naive
1024 x 2048 transpose (2048 blocks x 32 warps x 31 extra passes, 2048 x 32 x 32 passes), with zero
for the padded and XOR layouts.
"""

import numpy as np
import pytest

from conftest import golden_lines, golden_sections
from oracle import lds


def test_triton_grids():
    sec = golden_sections("p2_triton_shared_layouts.txt")
    assert len(sec) == 5
    for name, (hdr, lines) in sec.items():
        vec, pp, mp, W = (int(v) for v in hdr)
        grid = np.array([[int(v) for v in ln.split()] for ln in lines])
        for r in range(grid.shape[0]):
            for c in range(W):
                assert lds.chunk_xor(r, c, W, vec, pp, mp) == grid[r, c], (name, r, c)


def test_transpose_xor_row1():
    lines = golden_lines("p2_transpose_xor_row1.txt")
    prefix = [int(v) for v in lines[0].split(":")[1].split()]
    suffix = [int(v) for v in lines[1].split(":")[1].split()]
    order = [lds.xor_element(1, c, 32) - 32 for c in range(32)]
    assert order[:len(prefix)] == prefix and order[-len(suffix):] == suffix


@pytest.mark.parametrize("elem_bytes", [1, 2, 4])
def test_tma_formula_equals_triton_family(elem_bytes):
    NX = 128 // elem_bytes
    vec = 16 // elem_bytes
    for y in range(24):
        for x in range(NX):
            yy, xs = lds.tma_swizzle(y, x, NX, elem_bytes)
            assert yy == y
            assert y * NX + xs == lds.chunk_xor(y, x, NX, vec, 1, 8)


@pytest.mark.parametrize("W,vec,pp,mp", [(32, 1, 1, 32), (64, 8, 1, 8), (64, 8, 2, 8), (64, 4, 1, 16),
                                          (8, 1, 2, 4), (128, 8, 1, 8)])
def test_swizzle_properties(W, vec, pp, mp):
    rows = 64
    phys = np.array([[lds.chunk_xor(r, c, W, vec, pp, mp) for c in range(W)] for r in range(rows)])
    # one-to-one and range kept: every row is a permutation of its own W slots
    for r in range(rows):
        assert sorted(phys[r] - r * W) == list(range(W))
    # distinct within a column for rows of one full phase cycle (pp*mp rows share no column slot
    # when vec == 1); for vec > 1 the chunk index is what differs
    if vec == 1 and mp == W:
        for c in range(W):
            cols = [phys[r, c] - r * W for r in range(min(rows, pp * mp)) if r % pp == 0]
            assert len(set(cols)) == len(cols)


def test_xor_element_properties():
    W = 64
    phys = np.array([[lds.xor_element(r, c, W) - r * W for c in range(W)] for r in range(W)])
    for r in range(W):
        assert sorted(phys[r]) == list(range(W))
    for c in range(W):
        assert len(set(phys[:, c])) == W


@pytest.mark.parametrize("stride", [1, 2, 4, 8, 16, 32])
def test_stride_conflict_degree(stride):
    passes, phases = lds.instruction_passes([4 * stride * lane for lane in range(32)], 4)
    assert phases == 1 and passes == stride


def test_broadcast_and_vector_phases():
    assert lds.instruction_passes([0] * 32, 4) == (1, 1)
    assert lds.instruction_passes([16 * lane for lane in range(32)], 16) == (4, 4)
    assert lds.instruction_passes([8 * lane for lane in range(32)], 8) == (2, 2)
    # 8 lanes of a 128-bit phase reading the same 16-byte column of 8 rows of 128 bytes: 8 passes
    assert lds.instruction_passes([128 * lane for lane in range(8)], 16) == (8, 1)
    # explicit phase size: 16-byte reads of 64 lanes in two 32-lane phases on 64 banks need at least
    # 2 passes each; all lanes of a phase in one bank group need one pass per lane
    assert lds.instruction_passes([16 * lane for lane in range(64)], 16, 64, lanes_per_phase=32) == (4, 4)
    assert lds.instruction_passes([256 * lane for lane in range(64)], 16, 64, lanes_per_phase=32) == (64, 4)
    # two lanes per bank group in each phase (rows of 64 bytes, every row at its own chunk offset)
    rows = [64 * r + 16 * ((r // 4) % 4) for r in range(64)]
    assert lds.instruction_passes(rows, 16, 64, lanes_per_phase=32) == (4, 4)


def test_page_closed_form_naive_transpose():
    want = {k: int(v) for k, v in (ln.split() for ln in golden_lines("p2_bank_conflict_counts.txt"))}
    passes, extra = lds.transpose_store_passes(1024, 2048, 32, "naive")
    assert passes == want["store_wavefronts_naive"]
    assert extra == want["store_conflicts_naive"]
    assert lds.transpose_store_passes(1024, 2048, 32, "padded")[1] == want["store_conflicts_padded"]
    assert lds.transpose_store_passes(1024, 2048, 32, "xor")[1] == want["store_conflicts_xor"]


# ---- the GEMM's operand reads under the chunk-XOR family (gfx950 geometry: 64 banks x 4 bytes,
# 16-byte and 8-byte reads both served in phases of 32 lanes) ----
#
# Hand counts per read instruction, derived from the row pitches alone:
#   A rows are 64 bytes, so a 256-byte bank window holds 4 rows, and its 16 sixteen-byte bank
#   groups are group 4 (r mod 4) + (physical chunk). A 32-lane phase reads 32 consecutive rows at
#   one logical chunk; conflict-free it puts 2 lanes on each group (2 passes). Unswizzled, or with a
#   phase value that is a function of r mod 4 (perPhase 1, maxPhase 4), only 4 groups are used,
#   8 lanes each: 8 passes, 6 extra per phase, 12 per instruction (2 phases). A phase value that adds
#   one bit of information beyond r mod 4 (perPhase 2 or maxPhase 2) uses 8 groups, 4 lanes each:
#   2 extra per phase, 4 per instruction. Two more bits (perPhase 4 or 8 with maxPhase 4, i.e. bits
#   2-3 or 3-4 of r): all 16 groups, conflict-free.
#   B rows are 512 bytes, all in the same window position. A 32-lane phase of the transposing read
#   covers 4 k rows x 64 contiguous bytes: unswizzled, 4 rows on the same 16 banks -> 4 passes per
#   phase, 3 extra, 6 per instruction (2 phases); 2 distinct 64-byte positions -> 2 per instruction.
HAND = [
    ((4, 4, 4, 1, 4), (0, 0)),
    ((1, 1, 4, 1, 4), (12, 0)), ((1, 4, 4, 1, 4), (12, 0)),
    ((2, 4, 4, 1, 4), (4, 0)), ((4, 2, 4, 1, 4), (4, 0)), ((8, 4, 4, 1, 4), (0, 0)),
    ((4, 4, 1, 1, 1), (0, 6)), ((4, 4, 1, 1, 4), (0, 6)),
    ((4, 4, 2, 1, 4), (0, 2)), ((4, 4, 4, 1, 2), (0, 2)), ((4, 4, 4, 2, 2), (0, 2)),
    ((4, 4, 8, 1, 4), (0, 2)),
]


@pytest.mark.parametrize("waves,reads", [((2, 2), (32, 64)), ((2, 4), (64, 64))])
@pytest.mark.parametrize("layout,per_inst", HAND)
def test_gemm_operand_read_passes_hand_counts(layout, per_inst, waves, reads):
    want = (reads[0] * per_inst[0], reads[1] * per_inst[1])
    assert lds.gemm_operand_read_passes(*layout, waves=waves) == want


def test_gemm_lds_conflicts_scales_with_tiles_and_steps():
    per_step = sum(lds.gemm_operand_read_passes(1, 1, 1, 1, 1))
    assert per_step == 64 * 12 + 64 * 6
    assert lds.gemm_lds_conflicts(4096, 4096, 4096, (1, 1, 1, 1, 1)) == 256 * 128 * per_step
    # partial tiles and a partial k step count as whole ones
    assert lds.gemm_lds_conflicts(300, 520, 40, (1, 1, 1, 1, 1)) == 2 * 3 * 2 * per_step
    assert lds.gemm_lds_conflicts(4096, 4096, 4096, (4, 4, 4, 1, 4)) == 0
    with pytest.raises(ValueError):
        lds.gemm_operand_read_passes(4, 4, 4, 1, 4, waves=(2, 16))


# ---- the 16x16x32 form's operand reads (same geometry) ----
#
# Hand counts per read instruction:
#   A: a 32-lane phase reads 16 consecutive rows at 2 logical chunks (lanes 0-31: chunks 0, 1;
#   lanes 32-63: chunks 2, 3). Bank group = 4 (r mod 4) + physical chunk. Unswizzled, or with a
#   phase value that takes one bit from the rows (perPhase 4, maxPhase 2: bit 2), only the chunk
#   pair's two groups per r mod 4 are used: 8 groups, 4 lanes each -> 4 passes against 2: 2 extra
#   per phase, 4 per instruction. A phase value with two bits above bit 1 of the row (perPhase 2 or
#   4 with maxPhase 4) spreads each r mod 4 over all 4 groups of its quarter: conflict-free.
#   B: a phase reads k rows k0 .. k0 + 3 and k0 + 8 .. k0 + 11 (512-byte pitch: the same window
#   position) at 4 eight-byte column offsets of one 32-byte span. Unswizzled all 8 rows land on the
#   same 4 bank pairs: 8 passes against 1, 7 extra per phase, 14 per instruction. The family member
#   4 (k mod 4) (in chunks) separates k mod 4 but not the rows 8 apart: 2 passes, 2 extra per
#   instruction. The kernel's layout adds 2 ((k / 8) mod 2): conflict-free.
HAND16 = [((2, 4, "kstep8"), (0, 0)), ((4, 4, "kstep8"), (0, 0)), ((1, 1, "kstep8"), (4, 0)),
          ((4, 2, "kstep8"), (4, 0)), ((2, 4, "vec4"), (0, 2)), ((2, 4, "none"), (0, 14))]


@pytest.mark.parametrize("layout,per_inst", HAND16)
def test_gemm16_operand_read_passes_hand_counts(layout, per_inst):
    # per workgroup and 32-deep step: A 2 row groups x 8 blocks x 4 waves reading each; B 4 column
    # groups x 4 blocks x 2 reads x 2 waves reading each
    a_pp, a_mp, b = layout
    assert lds.gemm16_operand_read_passes(a_pp, a_mp, lds.GEMM16_B_LAYOUTS[b]) == (64 * per_inst[0],
                                                                                  64 * per_inst[1])


def test_gemm16_kernel_b_layout_is_the_family_member_plus_the_kstep8_term():
    for k in range(64):
        assert lds.swz_b_kstep8(k) == lds.GEMM16_B_LAYOUTS["vec4"](k) ^ (2 * ((k // 8) % 2))
    # XOR by a value constant over a row keeps each row's chunks a permutation
    for k in range(32):
        assert sorted((c ^ lds.swz_b_kstep8(k)) for c in range(32)) == list(range(32))


def test_gemm16_fixture_matches_the_oracle():
    from conftest import golden_lines
    names = {(0, 0, 0): "kstep8", (4, 1, 4): "vec4", (1, 1, 1): "none"}
    for ln in golden_lines("gemm16_lds_conflicts_4096.txt"):
        v = [int(x) for x in ln.split()]
        b = names[tuple(v[2:5])]
        assert lds.gemm16_operand_read_passes(v[0], v[1], lds.GEMM16_B_LAYOUTS[b]) == (v[5], v[6])
        assert lds.gemm16_lds_conflicts(4096, 4096, 4096, v[0], v[1], b) == v[7]
