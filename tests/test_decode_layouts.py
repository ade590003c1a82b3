"""Host-side checks of the decode kernels' K layouts in LDS (the index maps that
attention_sink_softmax_amd/csrc/decode.hip implements in kswz/klane, k8_lane_chunk and k8_off).

Each load instruction moves 64 lanes x 16 bytes; lane l's bytes land at slot l of the
instruction's 1 KB block.  The properties checked: every (key, chunk) of a 16-key block is
loaded exactly once, each instruction reads whole 128-byte cache lines, and the 16 keys of one
operand read (one chunk) fall in 16 distinct 16-byte slots of a 256-byte bank phase.
"""


def bf16_slot(k, m):
    """bf16 K: key k (0..15) of a 16-key block, chunk m (0..23) of its 384-byte row ->
    (instruction, slot).  Instruction 3 kh + c holds keys 8 kh .. +7, line c of their rows;
    chunk m of the line at slot 8 (k & 7) + (m ^ kswz(k)), kswz(k) = (k >> 1) & 7."""
    kh, c, mi = k >> 3, m >> 3, m & 7
    return 3 * kh + c, 8 * (k & 7) + (mi ^ ((k >> 1) & 7))


def fp8_lane_chunk(i, lane):
    r, t = lane & 15, lane >> 4
    if i == 0:
        c = 2 * t + (r & 1)
    elif i == 1:
        c = 8 + 2 * t + (r & 1) if t < 2 else 2 * (t - 2) + ((r + 1) & 1)
    else:
        c = 4 + 2 * t + ((r + 1) & 1)
    return (r - c) & 15, c


def fp8_off(k, c):
    r = (k + c) & 15
    if k % 2 == 0:
        i, t = (0, c >> 1) if c < 8 else (1, (c - 8) >> 1)
    else:
        i, t = (1, 2 + (c >> 1)) if c < 4 else (2, (c - 4) >> 1)
    return i * 1024 + (r + 16 * t) * 16


def test_bf16_k_layout():
    seen = {}
    for k in range(16):
        for m in range(24):
            inst, slot = bf16_slot(k, m)
            assert 0 <= inst < 6 and 0 <= slot < 64
            assert (inst, slot) not in seen
            seen[(inst, slot)] = (k, m)
    for inst in range(6):  # whole lines: 8 keys x one 128-byte line each
        lines = {(seen[(inst, s)][0] * 384 + seen[(inst, s)][1] * 16) // 128 for s in range(64)}
        assert len(lines) == 8
    for m in range(24):  # an operand read: keys 0..15, one chunk
        assert len({(1024 * bf16_slot(k, m)[0] + 16 * bf16_slot(k, m)[1]) // 16 % 16 for k in range(16)}) == 16


def test_fp8_k_layout():
    seen = set()
    for i in range(3):
        lines = set()
        for lane in range(64):
            k, c = fp8_lane_chunk(i, lane)
            assert 0 <= k < 16 and 0 <= c < 12 and (k, c) not in seen
            seen.add((k, c))
            assert fp8_off(k, c) == i * 1024 + lane * 16  # the read address inverts the load map
            lines.add((k * 192 + c * 16) // 128)
        assert len(lines) == 8  # 8 whole lines per instruction
    assert len(seen) == 192
    for c in range(12):
        assert len({fp8_off(k, c) // 16 % 16 for k in range(16)}) == 16


def bank_cycles(addrs, nbytes, group):
    """Cycles of one LDS read: lanes served `group` at a time by 64 banks of 4 bytes (256
    bytes per cycle); a bank that must serve k distinct words serialises k cycles."""
    cyc = 0
    for g0 in range(0, len(addrs), group):
        words = {}
        for a in addrs[g0:g0 + group]:
            for wd in range(a // 4, (a + nbytes) // 4):
                words.setdefault(wd % 64, set()).add(wd)
        cyc += max(len(v) for v in words.values())
    return cyc


def bf16_v_slot(key, c):
    """bf16 V: key (0..31) of a slice, 16-byte chunk c (0..15) of its 256-byte row ->
    byte offset: block m = key / 4, row r = key % 4, slot c ^ 2r ^ 8 (m & 1)."""
    m, r = key >> 2, key & 3
    return m * 1024 + r * 256 + ((c ^ (2 * r) ^ (8 * (m & 1))) << 4)


def test_bf16_v_layout():
    # the load of block m: lane 16 r + s fetches chunk s ^ 2r ^ 8 (m & 1) of key 4m + r
    seen = set()
    for m in range(8):
        for lane in range(64):
            r, s = lane >> 4, lane & 15
            c = s ^ (2 * r) ^ (8 * (m & 1))
            assert bf16_v_slot(4 * m + r, c) == m * 1024 + lane * 16
            seen.add((4 * m + r, c))
    assert len(seen) == 32 * 16
    # the transposing reads (two per dv block db): lane group q reads rows of block q (then
    # 4 + q), row r = (lane & 15) >> 2 at chunk 2 db + ((lane & 3) >> 1), half lane & 1
    for db in range(8):
        for hi in (0, 1):
            addrs = []
            for lane in range(64):
                q, hl = lane >> 4, lane & 15
                r, c4 = hl >> 2, lane & 3
                addrs.append(bf16_v_slot(4 * (4 * hi + q) + r, 2 * db + (c4 >> 1)) + 8 * (c4 & 1))
            assert bank_cycles(addrs, 8, 32) == 2


def test_wave_merge_records():
    """The merge writes lane (hl, q)'s 4 floats of dv 16 db + 4 q to column hl's record:
    with records of 132 floats the 16 lanes of one write cycle hit 16 distinct slots."""
    for db in range(8):
        addrs = [((lane & 15) * 132 + 16 * db + 4 * (lane >> 4)) * 4 for lane in range(64)]
        assert bank_cycles(addrs, 16, 16) == 4
        unpadded = [((lane & 15) * 128 + 16 * db + 4 * (lane >> 4)) * 4 for lane in range(64)]
        assert bank_cycles(unpadded, 16, 16) == 64
