"""Oracle: shared-memory (LDS) layout maps and the bank-conflict model.

TEST INFRASTRUCTURE (see the package docstring): not imported by the library.

Source: "CUDA Swizzle & bank conflict" (whc-imageprocess.github.io):
  * section "Bank Conflict" and the hardware background before it: memory is split into banks that
    work in parallel; an access instruction costs one pass per phase of lanes, plus one more pass
    for every extra distinct word that the phase needs from an already-busy bank; lanes reading the
    same word share it (broadcast). 128-bit and 64-bit accesses are served in phases of 8 and 16
    lanes of a 32-lane warp (section "memory coalesce").
  * sections "Padding" / "Padding Row-Major Layout": row-major with one extra element per row.
  * section "Case Study / Matrix Transpose", swizzling variant: physical column = column XOR row.
  * section "Hopper TMA 的 swizzling": the 16-byte-chunk swizzle of a 128-byte row.
  * section "Triton - Shared Layout swizzling": the vec / perPhase / maxPhase chunk XOR family.

Layout maps return the physical element index of logical element (r, c) of a tile whose logical
rows hold W elements.
"""

import numpy as np


# ----------------------------------------------------------------------------- layout maps

def naive(r, c, W):
    """Row-major: element (r, c) at r*W + c."""
    return r * W + c


def padded(r, c, W, pad=1):
    """Row-major with ``pad`` unused elements after every row: r*(W+pad) + c."""
    return r * (W + pad) + c


def xor_element(r, c, W):
    """Element-wise XOR swizzle of the transpose case study: (r, c) stored at column c XOR r.

    Defined for a square power-of-two tile (r, c < W), where c XOR r stays inside the row."""
    return r * W + (c ^ r)


def chunk_xor(r, c, W, vec, per_phase, max_phase):
    """Triton shared-layout swizzle: chunks of ``vec`` elements are permuted inside a row.

    Chunk c // vec of row r is stored at chunk (c // vec) XOR ((r // per_phase) mod max_phase);
    the position inside a chunk is kept. XOR with a fixed value is its own inverse, so the same
    formula also gives, for a physical position, the logical column stored there.
    """
    chunk = (c // vec) ^ ((r // per_phase) % max_phase)
    return r * W + chunk * vec + c % vec


def tma_swizzle(y, x, NX, elem_bytes, swizzle_bytes=128):
    """The 16-byte-chunk swizzle the page describes for a ``T array[][NX]`` with NX*sizeof(T) equal
    to the swizzle size: the flat byte offset of (y, x) is cut into 16-byte chunks; the chunk's row
    (chunk index div 8) is kept and its column (chunk index mod 8) is XOR-ed with that row; the
    element keeps its place inside the chunk. Returns the physical (y, x_swz)."""
    if NX * elem_bytes != swizzle_bytes:
        raise ValueError("row must be exactly one swizzle span")
    per_chunk = 16 // elem_bytes
    i16 = (y * NX + x) * elem_bytes // 16
    y16 = i16 // 8
    x16 = i16 % 8
    x16_swz = y16 ^ x16
    x_swz = (x16_swz * per_chunk) % NX + x % per_chunk
    return y, x_swz


# ----------------------------------------------------------------------------- bank model

def instruction_passes(byte_addrs, access_bytes, num_banks=32, bank_bytes=4, lanes=None,
                       lanes_per_phase=None):
    """Passes (wavefronts) one shared-memory instruction needs under the page's bank model.

    ``byte_addrs``: start byte address of each active lane, in lane order. Every lane touches
    ``access_bytes`` consecutive bytes, i.e. access_bytes/bank_bytes consecutive words; word w sits
    in bank w mod num_banks. The lanes are served in phases of as many lanes as fill the banks once
    (num_banks*bank_bytes/access_bytes lanes, at most the lane count), or of ``lanes_per_phase``
    lanes when given. Within a phase, each bank delivers one distinct word per pass and lanes asking
    for the same word share it, so the phase needs as many passes as the busiest bank has distinct
    words; without conflicts a phase needs ceil(lanes x words per lane / num_banks) passes (one,
    when the phase fills the banks once).
    Returns (passes, ideal passes); their difference is the number of extra (conflict) passes.
    """
    addrs = np.asarray(byte_addrs, dtype=np.int64)
    if lanes is None:
        lanes = len(addrs)
    words_per_lane = max(1, access_bytes // bank_bytes)
    if lanes_per_phase is None:
        lanes_per_phase = (num_banks * bank_bytes) // access_bytes
    lanes_per_phase = max(1, min(lanes, lanes_per_phase))
    passes = 0
    ideal = 0
    for start in range(0, len(addrs), lanes_per_phase):
        phase = addrs[start:start + lanes_per_phase]
        words = set()
        for a in phase:
            first = int(a) // bank_bytes
            for w in range(words_per_lane):
                words.add(first + w)
        per_bank = {}
        for w in words:
            per_bank[w % num_banks] = per_bank.get(w % num_banks, 0) + 1
        passes += max(per_bank.values())
        ideal += max(1, -(-len(phase) * words_per_lane // num_banks))
    return passes, ideal


def transpose_store_passes(M, N, tile, layout, elem_bytes=4, num_banks=32, bank_bytes=4,
                           warp=32, pad=1):
    """Shared-store passes of the transpose case study's kernels, over the whole launch.

    The kernel runs (N/tile) x (M/tile) blocks of tile x tile threads, one element each; thread
    (tx, ty) stores its element at logical shared position [tx][ty] (the transposed store) of a
    tile x tile array laid out by ``layout`` ("naive", "padded" or "xor"). Warps are formed from
    consecutive threads in x-fastest order. Shared addresses do not depend on the block index, so
    one block is simulated and the counts are multiplied by the number of blocks.
    Returns (total passes, total extra passes).
    """
    if M % tile or N % tile:
        raise ValueError("the case study's sizes are tile multiples")
    blocks = (M // tile) * (N // tile)
    threads = [(tx, ty) for ty in range(tile) for tx in range(tile)]   # x fastest
    passes = extra = 0
    for w0 in range(0, len(threads), warp):
        addrs = []
        for tx, ty in threads[w0:w0 + warp]:
            r, c = tx, ty                                  # transposed store: s[tx][ty]
            if layout == "naive":
                e = naive(r, c, tile)
            elif layout == "padded":
                e = padded(r, c, tile, pad)
            elif layout == "xor":
                e = xor_element(r, c, tile)
            else:
                raise ValueError(layout)
            addrs.append(e * elem_bytes)
        p, ph = instruction_passes(addrs, elem_bytes, num_banks, bank_bytes)
        passes += p
        extra += p - ph
    return passes * blocks, extra * blocks


# ----------------------------------------------------------------------------- the GEMM's operand reads

def gemm_operand_read_passes(a_per_phase, a_max_phase, b_vec, b_per_phase, b_max_phase,
                             tile=256, waves=(2, 4), num_banks=64, bank_bytes=4):
    """Extra LDS passes of one workgroup's operand reads in one 32-deep k step of the GEMM.

    Layouts: the Triton chunk-XOR family of "CUDA Swizzle & bank conflict" (section "Triton -
    Shared Layout swizzling") on fp16 data. A is held as rows of 32 k (one per m), swizzled with
    vec = 8 elements (16 bytes) and (a_per_phase, a_max_phase); B is held k-major as rows of
    ``tile`` n values, swizzled with vec = 8 * b_vec elements and (b_per_phase, b_max_phase).

    The workgroup's waves form a waves[0] x waves[1] grid over the tile; wave (wm, wn) owns rows
    wm * tile / waves[0] .. and columns wn * tile / waves[1] .. of it.
    Read instructions (a reading of the hardware, not of the pages; see the bank geometry below):
      * A: a 16-byte read per lane; for MFMA block q of a wave's rows and k half s, lane l reads
        row r0 + 32 q + (l mod 32) at k = 16 s + 8 (l div 32), the operand layout of the 32x32x16
        MFMA;
      * B: a transposing 8-byte read per lane; for block j of a wave's columns, k half s and
        quarter t, lane r of 16-lane group g reads row k = 16 s + 4 t + 8 (g div 2) + r div 4 at
        columns n0 + 32 j + 16 (g mod 2) + 4 (r mod 4) .. + 3.
    Bank geometry (gfx950, measured with SQ_LDS_BANK_CONFLICT on the GEMM itself): 64 banks of 4
    bytes; both the 8-byte and the 16-byte reads are served in phases of 32 lanes (half a wave),
    which need 1 and 2 passes without conflicts (the page's model with those constants).
    Returns (extra passes of all A reads, extra passes of all B reads) per workgroup and k step.
    """
    wave_m, wave_n = tile // waves[0], tile // waves[1]
    if wave_m % 32 or wave_n % 32:
        raise ValueError("wave sub-tiles must be whole 32 x 32 MFMA blocks")
    b_stage = tile * 32 * 2            # bytes of A in a stage, where B starts
    extra_a = extra_b = 0
    for wm in range(waves[0]):
        for s in range(2):
            for q in range(wave_m // 32):
                addrs = []
                for l in range(64):
                    row = wave_m * wm + 32 * q + (l % 32)
                    k0 = 16 * s + 8 * (l // 32)
                    addrs.append(2 * chunk_xor(row, k0, 32, 8, a_per_phase, a_max_phase))
                p, ideal = instruction_passes(addrs, 16, num_banks, bank_bytes, lanes_per_phase=32)
                extra_a += (p - ideal) * waves[1]     # every wave of this row reads the same A
    for wn in range(waves[1]):
        for s in range(2):
            for j in range(wave_n // 32):
                for t in range(2):
                    addrs = []
                    for l in range(64):
                        g, r = l // 16, l % 16
                        k = 16 * s + 4 * t + 8 * (g // 2) + r // 4
                        n = wave_n * wn + 32 * j + 16 * (g % 2) + 4 * (r % 4)
                        addrs.append(b_stage + 2 * chunk_xor(k, n, tile, 8 * b_vec, b_per_phase,
                                                             b_max_phase))
                    p, ideal = instruction_passes(addrs, 8, num_banks, bank_bytes, lanes_per_phase=32)
                    extra_b += (p - ideal) * waves[0]
    return extra_a, extra_b


def gemm_lds_conflicts(M, N, K, layout, tile=256, waves=(2, 4)):
    """Predicted LDS bank-conflict cycles (extra passes) of one GEMM launch: every workgroup runs
    every 32-deep k step of its tiles, with the per-step extra passes of gemm_operand_read_passes."""
    tiles = -(-M // tile) * -(-N // tile)
    steps = -(-K // 32)
    a, b = gemm_operand_read_passes(*layout, tile=tile, waves=waves)
    return tiles * steps * (a + b)


def swz_b_kstep8(k):
    """The 16x16x32 kernel's B chunk XOR, as a function of the k row: 4 (k mod 4) + 2 ((k / 8) mod 2).
    The first term is the (vec 4 chunks, perPhase 1, maxPhase 4) member of the Triton family; the
    second separates rows 8 apart, which one transposing read of this MFMA form pairs up."""
    return 4 * (k % 4) + 2 * ((k // 8) % 2)


def gemm16_operand_read_passes(a_per_phase, a_max_phase, b_xor, tile=256, waves=(2, 4), num_banks=64,
                               bank_bytes=4):
    """Extra LDS passes of one workgroup's operand reads in one 32-deep k step of the 16x16x32 form.

    Layouts as gemm_operand_read_passes: A rows of 32 k (4 chunks of 16 bytes) swizzled by the
    Triton chunk XOR (vec 8 elements, a_per_phase, a_max_phase); B k-major rows of ``tile`` n
    values whose 16-byte chunk c of row k is stored at chunk c XOR b_xor(k) (b_xor: a function of k,
    e.g. the family member lambda k: 4 * (k % 4), or swz_b_kstep8).
    Read instructions of the 16x16x32 MFMA operands (the kernel's lane patterns):
      * A: one 16-byte read per lane and 16-row block i of a wave's rows: lane l reads row
        r0 + 16 i + (l mod 16) at k = 8 (l div 16), so a 32-lane half-wave reads 16 rows x 2 chunks;
      * B: two transposing 8-byte reads per 16-column block j of a wave's columns (h = 0, 1): lane
        r of 16-lane group g reads row k = 8 g + 4 h + r div 4 at columns n0 + 16 j + 4 (r mod 4)
        .. + 3, so a half-wave reads 4 rows and the 4 rows 8 further on.
    Bank geometry as gemm_operand_read_passes (64 banks of 4 bytes, 32-lane phases).
    Returns (extra passes of all A reads, extra passes of all B reads) per workgroup and k step.
    """
    wave_m, wave_n = tile // waves[0], tile // waves[1]
    if wave_m % 16 or wave_n % 16:
        raise ValueError("wave sub-tiles must be whole 16 x 16 MFMA blocks")
    b_stage = tile * 32 * 2
    extra_a = extra_b = 0
    for wm in range(waves[0]):
        for i in range(wave_m // 16):
            addrs = [2 * chunk_xor(wave_m * wm + 16 * i + (l % 16), 8 * (l // 16), 32, 8, a_per_phase,
                                   a_max_phase) for l in range(64)]
            p, ideal = instruction_passes(addrs, 16, num_banks, bank_bytes, lanes_per_phase=32)
            extra_a += (p - ideal) * waves[1]
    for wn in range(waves[1]):
        for j in range(wave_n // 16):
            for h in range(2):
                addrs = []
                for l in range(64):
                    g, r = l // 16, l % 16
                    k = 8 * g + 4 * h + r // 4
                    n = wave_n * wn + 16 * j + 4 * (r % 4)
                    chunk = (n // 8) ^ b_xor(k)
                    addrs.append(b_stage + 2 * (k * tile + chunk * 8 + n % 8))
                p, ideal = instruction_passes(addrs, 8, num_banks, bank_bytes, lanes_per_phase=32)
                extra_b += (p - ideal) * waves[0]
    return extra_a, extra_b


# B layouts of the 16x16x32 form by name: the kernel's default, the 32x32x16 form's (vec 4 chunks,
# perPhase 1, maxPhase 4) family member, and no swizzle
GEMM16_B_LAYOUTS = {"kstep8": swz_b_kstep8, "vec4": lambda k: 4 * (k % 4), "none": lambda k: 0}


def gemm16_lds_conflicts(M, N, K, a_per_phase, a_max_phase, b_layout, tile=256, waves=(2, 4)):
    """Predicted LDS bank-conflict cycles of one 16x16x32 GEMM launch (every workgroup, every 32-deep
    k step of its tiles, gemm16_operand_read_passes per step)."""
    tiles = -(-M // tile) * -(-N // tile)
    steps = -(-K // 32)
    a, b = gemm16_operand_read_passes(a_per_phase, a_max_phase, GEMM16_B_LAYOUTS[b_layout], tile, waves)
    return tiles * steps * (a + b)
