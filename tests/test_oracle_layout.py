"""CPU pins of the oracle's matrix-core operand layout (orc_to_mfma_layout).

The layout is this library's own placement of MX blocks for the gfx950
16x16x128 block-scaled matrix-core instruction (include/mxq.h, MXQ_LAYOUT_MFMA):
a pure byte permutation of the row layout, no arithmetic.  The oracle writes it
as a forward loop over (line, block).  These tests pin it against things other
than that loop:

  * the inverse map written out here from the header's description, for every
    destination slot: slot (step s, tile t, lane l = 16 g + r) holds block
    4 s + g of line 16 t + r; scale word (group q, tile t, lane l) holds in
    byte j the scale of step 4 q + j;
  * a bijection check with blocks that carry their own (line, block) number;
  * padding lines and absent steps of a last partial group left untouched;
  * hand-worked positions for lines = 17, k = 640 (two tiles, the second with
    one line; five steps, a second scale group with one step).
"""
import numpy as np
import pytest

FILL = 0xA5


def _tagged(lines, k, bb):
    """Row-layout codes whose block (line, jb) holds line in bytes 0-3 and jb
    in bytes 4-7 (little endian), the rest a byte pattern of both; scales
    the low byte of 7 line + 3 jb + 1."""
    nbk = k // 32
    codes = np.zeros((lines, nbk * bb), np.uint8)
    scales = np.zeros((lines, nbk), np.uint8)
    for line in range(lines):
        for jb in range(nbk):
            blk = np.zeros(bb, np.uint8)
            blk[0:4] = np.frombuffer(np.uint32(line).tobytes(), np.uint8)
            blk[4:8] = np.frombuffer(np.uint32(jb).tobytes(), np.uint8)
            blk[8:] = (np.arange(8, bb) * 31 + line * 5 + jb * 11) & 0xFF
            codes[line, jb * bb:(jb + 1) * bb] = blk
            scales[line, jb] = (7 * line + 3 * jb + 1) & 0xFF
    return codes, scales


def _inverse_map(lines, k, bb, tcodes, tscales, codes, scales):
    """Walk every destination slot of the header's layout and compare it with
    the source block the header assigns to it."""
    nbk, T, steps = k // 32, (lines + 15) // 16, k // 128
    groups = (steps + 3) // 4
    tc = tcodes.reshape(steps, T, 64, bb)
    ts = tscales.reshape(groups, T, 64, 4)
    untouched_codes = 0
    for s in range(steps):
        for t in range(T):
            for lane in range(64):
                g, r = lane // 16, lane % 16
                line, jb = 16 * t + r, 4 * s + g
                if line >= lines:
                    assert np.all(tc[s, t, lane] == FILL), (s, t, lane)
                    untouched_codes += 1
                    continue
                assert np.array_equal(tc[s, t, lane], codes[line, jb * bb:(jb + 1) * bb]), \
                    (s, t, lane)
    for q in range(groups):
        for t in range(T):
            for lane in range(64):
                g, r = lane // 16, lane % 16
                line = 16 * t + r
                for j in range(4):
                    s = 4 * q + j
                    if line >= lines or s >= steps:
                        assert ts[q, t, lane, j] == FILL, (q, t, lane, j)
                    else:
                        assert ts[q, t, lane, j] == scales[line, 4 * s + g], (q, t, lane, j)
    return untouched_codes


@pytest.mark.parametrize("lines,k", [(17, 640), (16, 128), (1, 128), (40, 512), (33, 1152)])
@pytest.mark.parametrize("fmt", [0, 1])
def test_layout_is_the_headers_permutation(orc, lines, k, fmt):
    bb = orc.block_bytes(fmt)
    codes, scales = _tagged(lines, k, bb)
    tc, ts = orc.to_mfma_layout(codes, scales, fmt, fill=FILL)
    T = (lines + 15) // 16
    assert tc.size == (k // 128) * T * 64 * bb
    assert ts.size == ((k // 128 + 3) // 4) * T * 256
    untouched = _inverse_map(lines, k, bb, tc, ts, codes, scales)
    assert untouched == (k // 128) * (16 * T - lines) * 4      # padding lines' slots only


@pytest.mark.parametrize("fmt", [0, 1])
def test_layout_is_a_bijection_onto_the_data_slots(orc, fmt):
    # every (line, block) appears exactly once, recovered from its own tag
    lines, k = 17, 640
    bb = orc.block_bytes(fmt)
    codes, scales = _tagged(lines, k, bb)
    tc, _ = orc.to_mfma_layout(codes, scales, fmt, fill=FILL)
    slots = tc.reshape(-1, bb)
    seen = set()
    for sl in slots:
        if np.all(sl == FILL):
            continue
        line = int(np.frombuffer(sl[0:4].tobytes(), np.uint32)[0])
        jb = int(np.frombuffer(sl[4:8].tobytes(), np.uint32)[0])
        assert (line, jb) not in seen
        seen.add((line, jb))
    assert seen == {(l, j) for l in range(lines) for j in range(k // 32)}


def test_layout_hand_worked_positions(orc):
    # lines = 17, k = 640: T = 2 tiles, 5 steps of 128, 2 scale groups.
    # FP4 blocks of 16 bytes.  Worked by hand from the header's description:
    #   block (line 0, jb 0):  s 0, g 0, t 0, r 0  -> lane 0,  slot 0         -> byte 0
    #   block (line 15, jb 3): s 0, g 3, t 0, r 15 -> lane 63, slot 63        -> byte 1008
    #   block (line 16, jb 0): s 0, g 0, t 1, r 0  -> lane 0,  slot 64        -> byte 1024
    #   block (line 16, jb 5): s 1, g 1, t 1, r 0  -> lane 16, slot 3*64+16   -> byte 3328
    #   block (line 3, jb 19): s 4, g 3, t 0, r 3  -> lane 51, slot 8*64+51   -> byte 9008
    #   scale (line 16, jb 5): q 0, t 1, lane 16, byte s%4 = 1 -> (64+16)*4+1 = 321
    #   scale (line 3, jb 19): q 1, t 0, lane 51, byte 0       -> (128+51)*4   = 716
    #   scale word (q 1, t 0, lane 51) bytes 1..3: steps 5..7 do not exist -> untouched
    lines, k, bb = 17, 640, 16
    codes, scales = _tagged(lines, k, bb)
    tc, ts = orc.to_mfma_layout(codes, scales, 0, fill=FILL)
    for (line, jb), off in (((0, 0), 0), ((15, 3), 1008), ((16, 0), 1024), ((16, 5), 3328),
                            ((3, 19), 9008)):
        assert np.array_equal(tc[off:off + 16], codes[line, jb * 16:(jb + 1) * 16]), (line, jb)
    assert ts[321] == scales[16, 5]
    assert ts[716] == scales[3, 19]
    assert list(ts[717:720]) == [FILL] * 3
    # line 17 does not exist: tile 1, lane r = 1 of every step stays at the fill
    assert np.all(tc[(64 + 1) * 16:(64 + 2) * 16] == FILL)


def test_layout_rejects_k_not_a_multiple_of_128(orc):
    codes = np.zeros((4, 3 * 16), np.uint8)
    scales = np.zeros((4, 3), np.uint8)
    with pytest.raises(ValueError):
        orc.to_mfma_layout(codes, scales, 0)
