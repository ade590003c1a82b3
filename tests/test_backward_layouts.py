"""Host-side checks of the backward kernels' LDS tile layout (the index maps that
attention_sink_softmax_amd/csrc/backward.hip implements in tile_off, src_of_slot and LaneOff,
and the load assignment of bwd_dkdv_kernel and bwd_dq_kernel).

A tile of W-element rows keeps row r at r * S (S = 448 bytes for W = 192, 320 for W = 128) and
its 16-byte chunk c at c ^ ((r >> 2) & 3).  Each load instruction moves 64 lanes x 16 bytes into
one 1 KB block of the tile.  The properties checked:
  * the lane-register-plus-constant addresses the kernels use equal the plain formula for every
    lane and every read they issue;
  * the loads fill every slot of every tile exactly once, each data slot with its own chunk;
  * with banks serving 256 bytes per cycle (16 lanes of a 16-byte read, 32 lanes of an 8-byte
    transposing read), no read meets a bank conflict.
"""
import itertools

import pytest


def stride(W):
    return 448 if W == 192 else 320


def tile_off(W, r, c):
    return r * stride(W) + ((c ^ ((r >> 2) & 3)) << 4)


def lane_off(W, lane):
    """row[p], col[h] of LaneOff<W>."""
    S = stride(W)
    g, gl, i = lane >> 5, (lane >> 4) & 1, lane & 15
    c4, r = i & 3, lane & 31
    row = [r * S + (((2 * p + g) ^ ((r >> 2) & 3)) << 4) for p in range(2)]
    col = [(4 * g + (i >> 2)) * S + (((2 * gl + (c4 >> 1)) ^ ((2 * h + g) & 3)) << 4) + 8 * (c4 & 1) for h in range(2)]
    return row, col


def src_of_slot(W, slot):
    ks, nch = stride(W) // 16, W // 8
    r, pc = slot // ks, slot % ks
    return r * (W * 2) + ((pc % nch) ^ ((r >> 2) & 3)) * 16


def row_read(W, rbase, kk):
    """Byte addresses of row_operand's 64 lanes: row rbase + (lane & 31), chunk 2 kk + g."""
    return [tile_off(W, rbase + (l & 31), 2 * kk + (l >> 5)) for l in range(64)]


def col_reads(W, rbase, col0):
    """The two transposing reads of col_operand (rows rbase + 8h + 4g + (i >> 2))."""
    out = []
    for h in range(2):
        a = []
        for l in range(64):
            g, gl, i = l >> 5, (l >> 4) & 1, l & 15
            col = col0 + 16 * gl + 4 * (i & 3)
            a.append(tile_off(W, rbase + 8 * h + 4 * g + (i >> 2), col >> 3) + 8 * ((col >> 2) & 1))
        out.append(a)
    return out


def bank_cycles(addrs, nbytes, group):
    """Cycles of one read: lanes in groups of `group`, 64 banks of 4 bytes; a bank that must
    serve k distinct words serialises k cycles."""
    cyc = 0
    for g0 in range(0, 64, group):
        words = {}
        for a in addrs[g0:g0 + group]:
            for wd in range(a // 4, (a + nbytes) // 4):
                words.setdefault(wd % 64, set()).add(wd)
        cyc += max(len(v) for v in words.values())
    return cyc


READS = [(W, rows) for W, rows in ((192, 32), (128, 32), (192, 64), (128, 64))]


@pytest.mark.parametrize("W,rows", READS)
def test_lane_parts_equal_the_formula(W, rows):
    for lane in range(64):
        row, col = lane_off(W, lane)
        for rbase in range(0, rows - 31, 16):      # row reads cover 32 rows
            for kk in range(W // 16):
                assert row_read(W, rbase, kk)[lane] == rbase * stride(W) + (kk >> 1) * 64 + row[kk & 1]
        for rbase in range(0, rows - 15, 16):      # transposing reads cover 16 rows
            for col0 in range(0, W, 32):
                for h in range(2):
                    assert col_reads(W, rbase, col0)[h][lane] == rbase * stride(W) + 2 * col0 + 8 * h * stride(W) + col[h]


@pytest.mark.parametrize("W,rows", READS)
def test_no_bank_conflicts(W, rows):
    for rbase in range(0, rows - 31, 16):
        for kk in range(W // 16):
            assert bank_cycles(row_read(W, rbase, kk), 16, 16) == 4
    for rbase in range(0, rows - 15, 16):
        for col0 in range(0, W, 32):
            for a in col_reads(W, rbase, col0):
                assert bank_cycles(a, 8, 32) == 2


@pytest.mark.parametrize("W,rows,assign", [
    (192, 32, lambda w: [w] + ([w + 8] if w < 6 else [])),                   # dK/dV: Q tile, 14 blocks
    (128, 32, lambda w: [w] + ([w + 8] if w < 2 else [])),                   # dK/dV: dO tile, 10 blocks
    (192, 64, lambda w: [w, w + 8, w + 16] + ([w + 24] if w < 4 else [])),  # dQ: K tile, 28 blocks
    (128, 64, lambda w: [w, w + 8] + ([w + 16] if w < 4 else [])),          # dQ: V tile, 20 blocks
])
def test_loads_fill_every_slot_once(W, rows, assign):
    nslots = rows * stride(W) // 16
    assert nslots % 64 == 0
    blocks = sorted(itertools.chain.from_iterable(assign(w) for w in range(8)))
    assert blocks == list(range(nslots // 64))
    # every data slot receives its own chunk; the unused slots receive some chunk of their row
    data = {tile_off(W, r, c) // 16: r * W * 2 + c * 16 for r in range(rows) for c in range(W // 8)}
    assert len(data) == rows * (W // 8)
    for slot in range(nslots):
        src = src_of_slot(W, slot)
        if slot in data:
            assert src == data[slot]
        else:
            r = slot // (stride(W) // 16)
            assert r * W * 2 <= src < (r + 1) * W * 2 and src % 16 == 0


def test_load_counts_match_the_waits():
    """vmcnt before each barrier = the loads a wave issues per item (dK/dV) or per tile (dQ)."""
    dkdv = [1 + (w < 6) + 1 + (w < 2) + (w == 6) + (w == 7) for w in range(8)]
    dq = [3 + (w < 4) + 2 + (w < 4) for w in range(8)]
    assert dkdv == [4, 4, 3, 3, 3, 3, 3, 3]   # vmcnt(4) on waves 0-1, vmcnt(3) on the others
    assert dq == [7, 7, 7, 7, 5, 5, 5, 5]     # vmcnt(7) on waves 0-3, vmcnt(5) on the others
