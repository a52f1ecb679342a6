"""Host check of the LDS / copy addressing used by the head_dim-128 kernels
(`csrc/attn_fwd.hip`, `csrc/svg_ear.hip`, `csrc/attn_bwd.hip`,
`csrc/linear_attn.hip`, `csrc/common.h`).

The kernels stage 64-row (forward and compensated attention, backward) or
32-row (fused route probe) tiles of K and V (row = 128 bf16 = 16 chunks of
16 B) with a per-row chunk permutation, and compute every per-lane address as
one lane base XOR / plus a compile-time immediate.  These tests restate the direct
definitions (swizzle of a row, MFMA operand layouts, accumulator rows) and check
the closed forms against them for every lane, exhaustively.  No GPU involved.
"""

import itertools


def swz_k(row):
    return row & 15


def swz_v(row):
    return 4 * (row & 3) + ((row >> 2) & 3)


def phys(row, col, swz):
    """Element offset of logical (row, col) in a swizzled 64 x 128 bf16 stage."""
    return row * 128 + 8 * ((col // 8) ^ swz(row)) + col % 8


def test_swizzles_are_permutations_of_the_chunks():
    for row in range(64):
        assert sorted(c ^ swz_k(row) for c in range(16)) == list(range(16))
        assert sorted(c ^ swz_v(row) for c in range(16)) == list(range(16))


def test_copy_offsets_xor_form():
    """Copy role: wave w, instruction j, lane l stages tile row 16w + 4j + l/16 at
    physical chunk l % 16, i.e. logical chunk (l % 16) ^ swizzle(row); the byte
    offset in the source row is base ^ immediate(j)."""
    for w, j, lane in itertools.product(range(4), range(4), range(64)):
        row = 16 * w + 4 * j + lane // 16
        p = lane % 16
        kbase = ((lane & 15) ^ (lane >> 4)) * 16
        vbase = ((lane & 15) ^ (4 * (lane >> 4))) * 16
        assert 16 * (p ^ swz_k(row)) == kbase ^ (64 * j)
        assert 16 * (p ^ swz_v(row)) == vbase ^ (16 * j)


def test_k_fragment_reads_xor_form():
    """A operand of S^T = K Q^T (32x32x16): lane l holds key row 32 kt + l % 32,
    head dims 16 t + 8 (l / 32) + 0..7, i.e. logical chunk 2t + l / 32."""
    for kt, t, lane in itertools.product(range(2), range(8), range(64)):
        l32, hi = lane % 32, lane // 32
        row = 32 * kt + l32
        direct = phys(row, 16 * t + 8 * hi, swz_k)
        kaddr = l32 * 128 + 16 * ((l32 & 15) >> 1) + 8 * (hi ^ (l32 & 1))
        assert direct == 4096 * kt + (kaddr ^ (16 * t))


def test_v_transpose_read_xor_form():
    """ds_read_b64_tr_b16 of the PV operand: in each 16-lane group, lane j16 points
    at 4 consecutive elements of row 16 ks + 4 (l / 32) + j16 / 4 (+ 8 for the
    second read), columns 32 dt + 16 ((l / 16) & 1) + 4 (j16 & 3)."""
    for ks, dt, lane in itertools.product(range(4), range(4), range(64)):
        hi, g16, j16 = lane // 32, lane // 16, lane % 16
        row = 16 * ks + 4 * hi + j16 // 4
        col = 32 * dt + 16 * (g16 & 1) + 4 * (j16 & 3)
        vq = j16 >> 2
        vc1 = (2 * (g16 & 1) + ((j16 >> 1) & 1)) ^ hi
        vaddr = (4 * hi + vq) * 128 + 32 * vq + 8 * vc1 + (j16 & 1) * 4
        vdelta = 1024 + 8 * ((vc1 ^ 2) - vc1)
        va = 2048 * ks + (vaddr ^ (32 * dt))
        assert phys(row, col, swz_v) == va
        assert phys(row + 8, col, swz_v) == va + vdelta
        # the 4 elements a lane names stay inside one 16-byte chunk
        assert col % 8 in (0, 4)


def tile_row_mask(n, hi):
    m = 0
    for kt in range(2):
        for g in range(4):
            c = min(max(n - (32 * kt + 8 * g + 4 * hi), 0), 4)
            m |= ((1 << c) - 1) << (16 * kt + 4 * g)
    return m


def test_tail_row_mask_matches_accumulator_rows():
    """Bit 16 kt + r of the mask covers s[kt][r], whose key row in the sub-tile is
    32 kt + 8 (r / 4) + 4 hi + r % 4; it is set exactly when that row is < n."""
    for n in range(0, 65):
        for hi in range(2):
            m = tile_row_mask(n, hi)
            for kt in range(2):
                for r in range(16):
                    key = 32 * kt + 8 * (r // 4) + 4 * hi + r % 4
                    assert bool((m >> (16 * kt + r)) & 1) == (key < n)


def test_causal_state_fragment_swap():
    """Causal linear kernel (`csrc/linear_attn.hip`): wave w keeps
    acc[t][r] = S[32 t + 8 (r / 4) + 4 hi + r % 4][32 w + l32].  For k-step
    f = 2 t + ks the lane packs x = group g0 = 2 ks and y = group g1 = g0 + 1 of
    acc[t] and swaps x of the upper 32 lanes with y of the lower 32 (a
    permlane32 swap).  Then the operand of lane (l32, hi), {x'[0], x'[1],
    y'[0], y'[1]}, holds d1 = 16 f + 8 hi + 0..7 in order, as the row fragment
    of phi(Q) does."""
    def held(t, g, hi):        # the 4 d1 values of group g of acc[t] in a lane of half hi
        return [32 * t + 8 * g + 4 * hi + j for j in range(4)]

    for f in range(8):
        t, ks = divmod(f, 2)
        g0, g1 = 2 * ks, 2 * ks + 1
        x = {hi: held(t, g0, hi) for hi in range(2)}
        y = {hi: held(t, g1, hi) for hi in range(2)}
        # swap(vdst = x, vsrc = y): vdst' = [x_lo, y_lo], vsrc' = [x_hi, y_hi]
        x_new = {0: x[0], 1: y[0]}
        y_new = {0: x[1], 1: y[1]}
        for hi in range(2):
            assert x_new[hi] + y_new[hi] == [16 * f + 8 * hi + e for e in range(8)]


def test_backward_dkdv_offsets_xor_form():
    """Fused dK / dV backward kernel (`csrc/attn_bwd.hip`): stages are row-major
    swz_v-swizzled [rows][128] bf16 (32-row Q / dO stages, the 128-row K stage);
    offsets in bytes.  Row fragment of lane l at k-step t: row r, head dims
    16 t + 8 (l / 32) + 0..7, with r = l % 32 (Q, dO) or 32 w + l % 32 (K of
    wave w): rq ^ 32 t, rk ^ 32 t.  Transpose read (ks, dt): rows
    16 ks + 4 (l / 32) + j16 / 4 and + 8, columns 32 dt + 16 ((l / 16) & 1) +
    4 (j16 & 3): 4096 ks + (tq ^ 64 dt) and 4096 ks + 2048 + (tq ^ 32 ^ 64 dt).
    Every offset stays inside its stage."""
    for w, t, lane in itertools.product(range(4), range(8), range(64)):
        l32, hi = lane % 32, lane // 32
        rq = 2 * (l32 * 128 + 8 * (hi ^ swz_v(l32)))
        rk = rq + 64 * 128 * w
        assert 2 * phys(l32, 16 * t + 8 * hi, swz_v) == rq ^ (32 * t)
        assert (rq ^ (32 * t)) + 16 <= 2 * 32 * 128
        assert 2 * phys(32 * w + l32, 16 * t + 8 * hi, swz_v) == rk ^ (32 * t)
        assert (rk ^ (32 * t)) + 16 <= 2 * 128 * 128
    for ks, dt, lane in itertools.product(range(2), range(4), range(64)):
        hi, g16, j16 = lane // 32, lane // 16, lane % 16
        row = 16 * ks + 4 * hi + j16 // 4
        col = 32 * dt + 16 * (g16 & 1) + 4 * (j16 & 3)
        tc1 = 2 * (g16 & 1) + ((j16 & 3) >> 1)
        tq = 2 * ((4 * hi + (j16 >> 2)) * 128 + ((tc1 ^ (4 * (j16 >> 2) + hi)) << 3) + (j16 & 1) * 4)
        assert 2 * phys(row, col, swz_v) == 4096 * ks + (tq ^ (64 * dt))
        assert 2 * phys(row + 8, col, swz_v) == 4096 * ks + 2048 + (tq ^ 32 ^ (64 * dt))
        assert 4096 * ks + 2048 + (tq ^ 32 ^ (64 * dt)) + 8 <= 2 * 32 * 128


def test_backward_dq_offsets_xor_form():
    """dQ backward kernel (`csrc/attn_bwd.hip`): 64-row swz_v-swizzled K and V
    stages, byte offsets.  Row fragment (A operand of S^T = K Q^T and
    dP^T = V dO^T) of lane l in half kt at k-step t: row 32 kt + l % 32, head
    dims 16 t + 8 (l / 32) + 0..7: 8192 kt + (rb ^ 32 t).  Transpose read of K
    (ks = 0..3, dt): rows 16 ks + 4 (l / 32) + j16 / 4 and + 8, columns
    32 dt + 16 ((l / 16) & 1) + 4 (j16 & 3): 4096 ks + (tb ^ 64 dt) and
    4096 ks + 2048 + (tb ^ 32 ^ 64 dt).  Every offset stays inside the stage."""
    stage = 2 * 64 * 128
    for kt, t, lane in itertools.product(range(2), range(8), range(64)):
        l32, hi = lane % 32, lane // 32
        rb = l32 * 256 + ((hi ^ swz_v(l32)) << 4)
        o = 8192 * kt + (rb ^ (32 * t))
        assert 2 * phys(32 * kt + l32, 16 * t + 8 * hi, swz_v) == o
        assert o + 16 <= stage
    for ks, dt, lane in itertools.product(range(4), range(4), range(64)):
        hi, g16, j16 = lane // 32, lane // 16, lane % 16
        row = 16 * ks + 4 * hi + j16 // 4
        col = 32 * dt + 16 * (g16 & 1) + 4 * (j16 & 3)
        a4, c4 = j16 >> 2, 2 * (g16 & 1) + ((j16 & 3) >> 1)
        tb = (4 * hi + a4) * 256 + 64 * a4 + 16 * (c4 ^ hi) + 8 * (j16 & 1)
        assert 2 * phys(row, col, swz_v) == 4096 * ks + (tb ^ (64 * dt))
        assert 2 * phys(row + 8, col, swz_v) == 4096 * ks + 2048 + (tb ^ 32 ^ (64 * dt))
        assert 4096 * ks + 2048 + (tb ^ 32 ^ (64 * dt)) + 8 <= stage


def test_backward_copy_offsets_scalar_form():
    """Copies of a whole sub-tile in the backward kernels: the source offset of
    lane l for stage row `row` (logical chunk (l % 16) ^ swz_v(row)) is a fixed
    per-lane part plus the sub-tile's first row times the row pitch, which the
    kernels pass as the scalar offset.  dQ (64-row K / V stages, wave w,
    instruction j < 4, row 16 w + 4 j + l / 16): rbase + 4 j pitch +
    (cbase ^ 16 j).  dK / dV (32-row Q / dO stages, row 8 w + 4 j + l / 16,
    j < 2): the per-lane part formed once from that row."""
    pitch = 128 * 2 * 3  # bytes between rows (e.g. a [B, N, H, D] layout with H = 3)
    for key0 in (0, 64, 4096):
        for w, j, lane in itertools.product(range(4), range(4), range(64)):
            row = 16 * w + 4 * j + lane // 16
            direct = (key0 + row) * pitch + 16 * ((lane % 16) ^ swz_v(row))
            rbase = (16 * w + lane // 16) * pitch
            cbase = ((lane & 15) ^ (4 * (lane >> 4))) * 16
            assert direct == rbase + 4 * j * pitch + (cbase ^ (16 * j)) + key0 * pitch
        for w, j, lane in itertools.product(range(4), range(2), range(64)):
            row = 8 * w + 4 * j + lane // 16
            direct = (key0 + row) * pitch + 16 * ((lane % 16) ^ swz_v(row))
            fixed = row * pitch + 16 * ((lane & 15) ^ swz_v(row))
            assert direct == fixed + key0 * pitch


def test_backward_dkdv_copy_rows_in_stage():
    """Copies of the fused kernel: instruction base row r0 (wave-uniform), lane l
    lands at r0 * 128 + 8 * (l % 16) + 64 * (l / 16) elements, i.e. row
    r0 + l / 16, physical chunk l % 16; the source is logical chunk
    (l % 16) ^ swz_v(row).  32-row stages take r0 = 8 w + 4 j (j < 2), the K
    stage r0 = 32 w + 4 j (j < 8): every row is written exactly once."""
    for rows, bases in ((32, [8 * w + 4 * j for w in range(4) for j in range(2)]),
                        (128, [32 * w + 4 * j for w in range(4) for j in range(8)])):
        seen = set()
        for r0, lane in itertools.product(bases, range(64)):
            row, p = r0 + lane // 16, lane % 16
            dst = r0 * 128 + 8 * lane
            logical = p ^ swz_v(row)
            assert dst == phys(row, 8 * logical, swz_v)
            seen.add(dst)
        assert seen == set(range(0, rows * 128, 8))


def test_fused_probe_offsets_xor_form():
    """Fused route probe (`csrc/svg_ear.hip`): 32-row K and V stages (K rows
    swz_k, V rows swz_v), byte offsets.  K row fragment of lane l at k-step t:
    row l % 32, head dims 16 t + 8 (l / 32) + 0..7: kb2 ^ 32 t.  Transposed
    reads (ks, dt) of V: va2 ^ (4096 ks + 64 dt), and ^ 2080 more for the rows
    8 further; this wave's V column sums (wave w) are the dt = w reads,
    vw2 = va2 ^ 64 w.  Transposed reads of K for the column sums of wave w
    (columns 32 w + ...): kt2 ^ 4096 ks, and ^ 2176 more for the rows 8
    further.  Each immediate's bits are disjoint from the others it is
    combined with, so ^ and + agree there, and every offset stays inside its
    8 KiB stage."""
    def rowfrag(r, hi):
        return r * 128 + 16 * ((r & 15) >> 1) + 8 * (hi ^ (r & 1))

    stage = 32 * 128 * 2
    for t, lane in itertools.product(range(8), range(64)):
        l32, hi = lane % 32, lane // 32
        kb2 = 2 * rowfrag(l32, hi)
        assert 2 * phys(l32, 16 * t + 8 * hi, swz_k) == kb2 ^ (32 * t)
        assert (kb2 ^ (32 * t)) + 16 <= stage
    for ks, dt, w, lane in itertools.product(range(2), range(4), range(4), range(64)):
        hi, g16, j16 = lane // 32, lane // 16, lane % 16
        row = 16 * ks + 4 * hi + j16 // 4
        q, c0 = j16 >> 2, 2 * (g16 & 1) + ((j16 >> 1) & 1)
        half = (j16 & 1) * 4
        # V (swz_v)
        col = 32 * dt + 16 * (g16 & 1) + 4 * (j16 & 3)
        va2 = 2 * ((4 * hi + q) * 128 + 32 * q + 8 * (c0 ^ hi) + half)
        o = 4096 * ks + 64 * dt
        assert o + 2080 == o ^ 2080
        assert 2 * phys(row, col, swz_v) == va2 ^ o
        assert 2 * phys(row + 8, col, swz_v) == va2 ^ (o + 2080)
        assert max(va2 ^ o, va2 ^ (o + 2080)) + 8 <= stage
        if dt == w:
            vw2 = va2 ^ (64 * w)
            assert vw2 ^ (4096 * ks) == va2 ^ o
        # K (swz_k), columns of wave w
        colk = 32 * w + 16 * (g16 & 1) + 4 * (j16 & 3)
        kt2 = 2 * ((4 * hi + q) * 128 + 8 * (4 * (w ^ hi) + (c0 ^ q)) + half)
        assert 4096 * ks + 2176 == (4096 * ks) ^ 2176
        assert 2 * phys(row, colk, swz_k) == kt2 ^ (4096 * ks)
        assert 2 * phys(row + 8, colk, swz_k) == kt2 ^ (4096 * ks + 2176)
        assert (kt2 ^ (4096 * ks + 2176)) + 8 <= stage

