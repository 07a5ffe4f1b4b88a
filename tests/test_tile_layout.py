"""CPU model of the swizzled 64 x 128 bf16 LDS tile shared by the forward
(K, V tiles) and the dK/dV pass (Q, dout tiles), written from the index
formulas of device_common.hpp: the DMA placement of a tile copy, the row reads
of an MFMA operand, and the transposing ds_read_b64_tr_b16 reads.  Checks that
every read returns the intended element and that no read pattern has LDS bank
conflicts (64 banks of 4 bytes; 16-byte reads served 16 lanes at a time,
8-byte reads 32 lanes at a time)."""
import pytest


def tile_swz(r):
    return ((r & 3) << 2) | ((r >> 2) & 3)


def perm_row(m):
    return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1)


def build_tile(nw):
    """LDS byte -> (row, column) after the copy by nw wavefronts."""
    tile = {}
    for w in range(nw):
        for m in range(16 // nw):
            for i in range(64):
                drow = 4 * w + (i >> 4)
                lchunk = (i & 15) ^ tile_swz(drow)
                row = drow + 4 * nw * m
                dst = 1024 * (w + nw * m) + 16 * i
                for e in range(8):
                    tile[dst + 2 * e] = (row, 8 * lchunk + e)
    return tile


def max_lanes_per_bank(addrs, width):
    cnt = {}
    for a in addrs:
        for w in range(width // 4):
            b = (a // 4 + w) % 64
            cnt[b] = cnt.get(b, 0) + 1
    return max(cnt.values())


@pytest.mark.parametrize("nw", [4, 8])
def test_copy_fills_every_element_once(nw):
    tile = build_tile(nw)
    assert len(tile) == 64 * 128 and max(tile) < 16384
    assert set(tile.values()) == {(r, c) for r in range(64) for c in range(128)}


def nat_offsets(lane):
    half, pr = lane >> 5, perm_row(lane & 31)
    return [pr * 256 + 16 * ((2 * kc + half) ^ tile_swz(pr)) for kc in range(8)]


def tr_offsets(lane):
    g, i = lane >> 4, lane & 15
    out = {}
    for db in range(4):
        for sub in range(2):
            r = 8 * (g >> 1) + 4 * sub + (i >> 2)
            col = 32 * db + 16 * (g & 1) + 4 * (i & 3)
            out[(db, sub)] = r * 256 + 16 * ((col >> 3) ^ tile_swz(r)) + 2 * (col & 7)
    return out


def test_row_reads_return_the_operand_and_do_not_conflict():
    tile = build_tile(4)
    for row0 in (0, 32):
        for kc in range(8):
            for lane in range(64):
                a = row0 * 256 + nat_offsets(lane)[kc]
                want = [(row0 + perm_row(lane & 31), 16 * kc + 8 * (lane >> 5) + e) for e in range(8)]
                assert [tile[a + 2 * e] for e in range(8)] == want
            for g in range(4):
                addrs = [row0 * 256 + nat_offsets(l)[kc] for l in range(16 * g, 16 * g + 16)]
                assert max_lanes_per_bank(addrs, 16) == 1


def test_transposed_reads_return_the_operand_and_do_not_conflict():
    tile = build_tile(4)
    for base_row in (0, 16, 32, 48):
        for db in range(4):
            for sub in range(2):
                piece = {}
                for lane in range(64):
                    a = base_row * 256 + tr_offsets(lane)[(db, sub)]
                    p = [tile[a + 2 * e] for e in range(4)]
                    assert len({x[0] for x in p}) == 1  # 8 bytes of one row
                    piece[lane] = p
                # ds_read_b64_tr_b16: lane j of a 16-lane group gets element j % 4
                # of the piece supplied by lane 4 e + j / 4
                for lane in range(64):
                    g, j = lane >> 4, lane & 15
                    got = [piece[16 * g + 4 * e + (j >> 2)][j & 3] for e in range(4)]
                    want = [(base_row + 8 * (lane >> 5) + 4 * sub + e, 32 * db + (lane & 31))
                            for e in range(4)]
                    assert got == want
                for p in range(2):
                    addrs = [base_row * 256 + tr_offsets(l)[(db, sub)] for l in range(32 * p, 32 * p + 32)]
                    assert max_lanes_per_bank(addrs, 8) == 1


def test_swizzle_properties():
    # bijection of r mod 16; top two bits distinct over any 4 aligned rows
    assert sorted(tile_swz(r) for r in range(16)) == list(range(16))
    for r0 in range(0, 64, 4):
        assert len({tile_swz(r) >> 2 for r in range(r0, r0 + 4)}) == 4
