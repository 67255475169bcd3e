"""Host model of the backward kernels' LDS tile layout (the streamed 32-row tiles of
streamkl_kernels.hip: `bwd_swz`, `BwdDma::init`, `swz_a_frag`, `tr_bases`, `swz_tr_frag`).

Checked on the CPU for d = 128 and d = 64:
* the loads that write LDS (each lane's 16 bytes at 16 * lane of a 1 KB piece) place every
  16-byte chunk of the tile exactly once;
* the S recomputation's row reads return row (l & 31), head_dim values kk*16 + h*8 .. + 7;
* the two transposing reads (ds_read_b64_tr_b16) of a gradient-product operand return, for lane
  l, the tile rows acc_row(8 cc + i, h), i = 0..7, of column nb*32 + (l & 31): the rows that the
  dS accumulator's registers 8 cc .. 8 cc + 7 hold;
* no two lanes of one LDS pass touch the same bank (64 banks of 4 bytes; 16 lanes per pass for
  16-byte reads, 32 for 8-byte reads).

The transposing read is modelled as measured on gfx950 with a probe kernel: in each group of 16
lanes, lane j receives element j % 4 of the 8 bytes read by lane 4 e + j // 4 as its element e.
"""
import pytest


def swz(d, r):
    if d == 128:
        return ((r & 3) << 2) | ((r >> 2) & 3)
    return (((r >> 1) & 1) << 2) | ((r >> 2) & 3)


def acc_row(r, h):
    return (r >> 2) * 8 + h * 4 + (r & 3)


def tile_lds(d):
    """LDS byte -> (row, column) of one tensor's tile, as the 1 KB loads place it."""
    rb, lds = 2 * d, {}
    for piece in range(32 * rb // 1024):
        for lane in range(64):
            o = piece * 1024 + 16 * lane
            row, pos = o // rb, (o % rb) // 16
            c = pos ^ swz(d, row)
            assert 0 <= c < d // 8
            for k in range(8):
                assert o + 2 * k not in lds
                lds[o + 2 * k] = (row, 8 * c + k)
    return lds


def banks(byte, nbytes):
    return [((byte // 4) + i) % 64 for i in range(nbytes // 4)]


@pytest.mark.parametrize("d", [128, 64])
def test_loads_place_every_chunk_once(d):
    lds = tile_lds(d)
    assert sorted(lds.values()) == sorted((r, c) for r in range(32) for c in range(d))


@pytest.mark.parametrize("d", [128, 64])
def test_row_reads(d):
    lds = tile_lds(d)
    for kk in range(d // 16):
        passes = {}
        for l in range(64):
            h, col = l >> 5, l & 31
            a_base = col * 2 * d + 16 * (h ^ swz(d, col))
            byte = a_base ^ (32 * kk)
            assert [lds[byte + 2 * k] for k in range(8)] == [(col, kk * 16 + h * 8 + k) for k in range(8)]
            passes.setdefault(l // 16, []).extend(banks(byte, 16))
        for b in passes.values():
            assert len(set(b)) == len(b)


def tr_read(lds, addr):
    """ds_read_b64_tr_b16 over 64 lanes: addr[l] = byte address of lane l."""
    fetched = [[lds[addr[l] + 2 * k] for k in range(4)] for l in range(64)]
    return [[fetched[16 * (l >> 4) + 4 * e + (l & 15) // 4][(l & 15) % 4] for e in range(4)]
            for l in range(64)]


@pytest.mark.parametrize("d", [128, 64])
def test_transposing_reads(d):
    lds = tile_lds(d)
    rb = 2 * d
    tb = {}
    for l in range(64):
        h, e, m = l >> 5, (l >> 2) & 3, l & 3
        low = 2 * ((l >> 4) & 1) + (m >> 1)
        for r in range(2):
            row = 8 * r + 4 * h + e
            tb[l, r] = row * rb + 8 * (m & 1) + 16 * (low ^ swz(d, row))
    for cc in range(2):
        for nb in range(d // 32):
            halves = []
            for r in range(2):
                addr = [cc * 16 * rb + (tb[l, r] ^ (64 * nb)) for l in range(64)]
                for p in range(2):
                    b = [x for l in range(32 * p, 32 * p + 32) for x in banks(addr[l], 8)]
                    assert len(set(b)) == len(b)
                halves.append(tr_read(lds, addr))
            for l in range(64):
                h = l >> 5
                got = halves[0][l] + halves[1][l]
                assert got == [(acc_row(8 * cc + i, h), nb * 32 + (l & 31)) for i in range(8)]


def test_mutated_swizzle_is_caught():
    """A plain layout (no swizzle) keeps the row reads correct but puts the transposing reads on
    the same banks: the bank check above would fail for it."""
    d, rb = 128, 256
    addr = []
    for l in range(32):
        h, e, m = l >> 5, (l >> 2) & 3, l & 3
        low = 2 * ((l >> 4) & 1) + (m >> 1)
        addr.append((4 * h + e) * rb + 8 * (m & 1) + 16 * low)
    b = [x for a in addr for x in banks(a, 8)]
    assert len(set(b)) < len(b)


@pytest.mark.parametrize("d", [128, 64])
@pytest.mark.parametrize("ntens", [1, 2])
def test_pieces_are_shared_out_once(d, ntens):
    """Piece i of a stage (1 KB, tensor i // pieces-per-tensor) is loaded by wave i % 8 as its
    load i // 8; every piece once, at most two loads per wave (what the wait before a barrier
    allows for), and a wave's wait counts exactly the loads it issued."""
    waves, tb = 8, 32 * 2 * d
    ppt = tb // 1024
    pieces = ntens * ppt
    n = (pieces + waves - 1) // waves
    assert n <= 2
    seen = []
    for w in range(waves):
        cnt = 0
        for j in range(n):
            idx = w + j * waves
            if idx < pieces:
                seen.append((idx // ppt, idx % ppt))
                cnt += 1
        assert cnt == sum(1 for i in range(pieces) if i % waves == w)
    assert sorted(seen) == [(te, p) for te in range(ntens) for p in range(ppt)]
