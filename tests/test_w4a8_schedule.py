"""CPU model of the W4A8 GEMM launch (no GPU): the grouped block ranges, the
XCD-grouped tile order inside each problem, the LDS staging and fragment
addresses of the 128 x 128-byte code tile, and the weight-word and code-byte
positions each MFMA step reads, mirrored from the kernel's index arithmetic
and checked for coverage, bounds and agreement with the packed format."""
import numpy as np
import pytest

ROWS, KT, PIECES = 128, 128, 8
MB, NB = 8, 2
SMALL_TILE_MAX_M = 256                   # 4-wave workgroups (128 x 128 tiles) up to this M


def waves_for(M):
    return 4 if M <= SMALL_TILE_MAX_M else 8


def xcd_grouped(b, total):
    xcd, slot = b & 7, b >> 3
    per, rem = total >> 3, total & 7
    return xcd * per + min(xcd, rem) + slot


def plan(problems, M):
    """Kernel-side view of a grouped launch: problems sorted by K (deepest
    first, stable), each a range of blocks starting at a multiple of 8."""
    order = sorted(range(len(problems)), key=lambda i: -problems[i][1])
    blocks_per_tile = waves_for(M) * NB
    mt = (M + ROWS - 1) // ROWS
    begin, tiles, blocks = [], [], 0
    for i in order:
        N, K = problems[i]
        ncb = (N + 15) // 16
        t = mt * ((ncb + blocks_per_tile - 1) // blocks_per_tile)
        begin.append(blocks)
        tiles.append(t)
        blocks += (t + 7) // 8 * 8
    return order, mt, begin, tiles, blocks


def block_to_tile(b, begin, tiles):
    p = 0
    for i in range(1, len(begin)):
        if b >= begin[i]:
            p = i
    local = b - begin[p]
    if local >= tiles[p]:
        return None
    return p, xcd_grouped(local, tiles[p])


@pytest.mark.parametrize("total", list(range(1, 70)) + [136, 1088, 1632, 4096 + 5])
def test_xcd_grouped_is_a_bijection(total):
    seen = sorted(xcd_grouped(b, total) for b in range(total))
    assert seen == list(range(total))


@pytest.mark.parametrize("M,problems", [
    (1024, [(7168, 5120), (5120, 6144), (34816, 5120), (5120, 17408)]),
    (256, [(7168, 5120), (5120, 6144), (34816, 5120), (5120, 17408)]),
    (130, [(300, 640), (1000, 1152), (48, 2048), (520, 256)]),
    (1, [(16, 64)]),
    (4096, [(5120, 17408)] * 8),
])
def test_grouped_blocks_cover_every_tile_once(M, problems):
    order, mt, begin, tiles, blocks = plan(problems, M)
    assert all(b % 8 == 0 for b in begin)
    ks = [problems[i][1] for i in order]
    assert ks == sorted(ks, reverse=True)
    seen = set()
    for b in range(blocks):
        r = block_to_tile(b, begin, tiles)
        if r is None:
            continue
        p, tile = r
        # the hardware's XCD of block b is also the XCD of the problem-local index
        assert (b - begin[p]) % 8 == b % 8
        assert (p, tile) not in seen and 0 <= tile < tiles[p]
        seen.add((p, tile))
    assert len(seen) == sum(tiles)


def slot(piece, row):
    return piece ^ (row & 7) ^ ((row >> 3) & 1)


@pytest.mark.parametrize("waves", [4, 8])
def test_staging_writes_fill_the_tile_and_reads_find_them(waves):
    """Every (row, piece) of a k-tile is staged exactly once, at a distinct
    16-byte slot inside the buffer; a fragment read of (row, piece) finds it."""
    THREADS = 64 * waves
    written = {}
    for tid in range(THREADS):
        spiece, srow0 = tid % PIECES, tid // PIECES
        for i in range(ROWS * PIECES // THREADS):
            row = srow0 + i * (THREADS // PIECES)
            addr = row * KT + slot(spiece, row) * 16
            assert 0 <= addr and addr + 16 <= ROWS * KT
            assert addr not in written.values()
            written[(row, spiece)] = addr
    assert len(written) == ROWS * PIECES
    for row in range(ROWS):
        arow = row & 15
        for piece in range(PIECES):
            assert row * KT + slot(piece, arow) * 16 == written[(row, piece)]


def test_lds_access_is_free_of_bank_conflicts():
    """Fragment reads: 16 lanes (rows 0..15 of one piece) cover 16 distinct
    16-byte slots of a 256-byte bank line pair, and any 8 of them distinct
    slots of one 128-byte line; staging writes of 8 lanes (one row, eight
    pieces) hit 8 distinct slots."""
    for piece in range(PIECES):
        addrs = [(r * KT + slot(piece, r) * 16) // 16 % 16 for r in range(16)]
        assert len(set(addrs)) == 16
        for lo in (0, 8):
            assert len({(r * KT + slot(piece, r) * 16) // 16 % 8 for r in range(lo, lo + 8)}) == 8
    for row in range(16):
        assert len({slot(p, row) for p in range(PIECES)}) == PIECES


# k offsets, within a block of 16, of the bytes of one MFMA operand register quad
STEP_ORDER = [0, 4, 1, 5, 2, 6, 3, 7, 8, 12, 9, 13, 10, 14, 11, 15]


def operand_codes(w0, w1):
    """The kernel's int8 operand from two packed words: (w << 4) & 0xF0F0F0F0
    and w & 0xF0F0F0F0, as signed bytes 16 q, in register order."""
    regs = [(w0 << 4) & 0xF0F0F0F0, w0 & 0xF0F0F0F0, (w1 << 4) & 0xF0F0F0F0, w1 & 0xF0F0F0F0]
    out = []
    for r in regs:
        for byte in range(4):
            v = (r >> (8 * byte)) & 0xFF
            out.append((v - 256 if v >= 128 else v))
    return out


@pytest.mark.parametrize("g", [64, 128])
def test_operand_bytes_match_the_arranged_codes(g):
    """For every lane group and step of a group, the 16 operand bytes from the
    lane's packed words are 16 q of the k positions that the arranged
    activation piece the lane reads holds, in the same byte order (column 0
    of a 16-column block; the packed words come from the oracle's pack)."""
    import oracle
    rng = np.random.default_rng(31)
    K = 2 * g
    q = np.zeros((16, K), np.int8)
    q[0] = rng.integers(-8, 8, size=K)
    s = np.full((16, K // g), 0x3C00, np.uint16)
    qw, _ = oracle.pack(q, s, g)
    codes_k = (np.arange(K) % 128).astype(np.int8)[None, :]
    arranged = oracle.arrange_xq(codes_k, 16)[0][0]
    wpl = g // 32
    for grp in range(K // g):
        tile = qw[grp * 64 * wpl:(grp + 1) * 64 * wpl].reshape(64, wpl)
        for lg in range(4):
            lane = 16 * lg  # column 0, lane group lg
            for st in range(g // 64):
                codes = operand_codes(int(tile[lane, 2 * st]), int(tile[lane, 2 * st + 1]))
                piece = grp * (g // 16) + lg * (g // 64) + st   # the kernel's piece index
                ks = [16 * piece + STEP_ORDER[j] for j in range(16)]
                assert codes == [16 * int(q[0, k]) for k in ks]
                assert [int(v) for v in arranged[16 * piece:16 * piece + 16]] == [k % 128 for k in ks]
