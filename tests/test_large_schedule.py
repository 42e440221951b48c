"""CPU model of the large-M kernel's indexing (w4a16_large.hip), checked over
many shapes for the facts its memory safety and coverage rest on:

* the XCD-grouped numbering maps workgroups one to one onto output tiles;
* every activation, weight and scale load, every LDS access and every store
  the kernel forms lies inside its buffer;
* every (row, column) of the output is stored exactly once.

It mirrors the kernel's integer formulas, so a change to either must keep this
test in step; it runs no device code.
"""
import pytest

ROWS, BLOCKS, KT, THREADS, MB, NB, WN = 128, 16, 128, 512, 8, 2, 8
PIECES = KT // 8
LOADS = ROWS * PIECES // THREADS
ABYTES = ROWS * KT * 2


def cfg(g):
    T = KT // g
    return dict(T=T, WPL=g // 32, LPG=g // 8, buf=ABYTES + T * ROWS * 4,
                lds=2 * (ABYTES + T * ROWS * 4))


def tile_of(bid, total):
    xcd, slot = bid & 7, bid >> 3
    per, rem = total >> 3, total & 7
    return xcd * per + min(xcd, rem) + slot


@pytest.mark.parametrize("total", list(range(1, 70)) + [159, 160, 161, 224, 1088, 4097])
def test_tile_numbering_is_a_bijection(total):
    assert sorted(tile_of(b, total) for b in range(total)) == list(range(total))


def check_shape(M, N, K, g):
    c = cfg(g)
    G, NCB = K // g, (N + 15) // 16
    MT, NT = (M + ROWS - 1) // ROWS, (NCB + BLOCKS - 1) // BLOCKS
    ntiles = (G + c["T"] - 1) // c["T"]
    assert c["lds"] <= 160 * 1024
    stored = {}
    for mt in range(MT):
        for nt in range(NT):
            m0 = mt * ROWS
            # staging through a buffer resource based at (row m0, k = 128 t) whose
            # range ends at the end of x: in-range pieces lie inside x, and rows
            # beyond M fall outside the range (read as zero)
            records0 = (M - m0) * K * 2
            assert 0 < records0 < 2 ** 32
            for t in range(ntiles):
                base = m0 * K * 2 + t * KT * 2
                records = records0 - t * KT * 2
                assert records > 0
                for tid in range(THREADS):
                    spiece, srow0 = tid % PIECES, tid // PIECES
                    for i in range(LOADS):
                        lrow = srow0 + i * (THREADS // PIECES)
                        voff = (lrow * K + spiece * 8) * 2
                        if voff + 16 <= records:
                            assert base + voff + 16 <= M * K * 2
                        else:
                            assert m0 + lrow >= M or t * KT + spiece * 8 >= K
                        sl = spiece ^ (lrow & 15)
                        assert lrow * KT * 2 + sl * 16 + 16 <= ABYTES
                        assert (spiece // c["LPG"]) * ROWS + lrow < c["T"] * ROWS
            for wave in range(8):
                wn = wave
                for lane in (0, 15, 16, 47, 63):
                    blks = [min(nt * BLOCKS + wn * NB + nb, NCB - 1) for nb in range(NB)]
                    for t in range(ntiles):
                        for gi in range(c["T"]):
                            grp = min(t * c["T"] + gi, G - 1)
                            for b in blks:
                                tile = b * G + grp
                                assert (tile * 64 + lane) * c["WPL"] + c["WPL"] <= NCB * 16 * K // 8
                                assert tile * 16 + (lane & 14) + 2 <= NCB * 16 * G
                            for mb in range(MB):
                                s0 = gi * ROWS + mb * 16 + 4 * (lane >> 4)
                                assert s0 % 4 == 0 and s0 + 4 <= c["T"] * ROWS
                        for st in range(4):
                            gi, w = st // c["WPL"], st % c["WPL"]
                            piece = gi * c["LPG"] + (lane >> 4) * c["WPL"] + w
                            assert piece < PIECES
                            for mb in range(MB):
                                row = (lane & 15) + mb * 16
                                assert row * KT * 2 + (piece ^ (lane & 15)) * 16 + 16 <= ABYTES
            # stores of the tile (every lane)
            for wave in range(8):
                wn = wave
                for lane in range(64):
                    for nb in range(NB):
                        col = (nt * BLOCKS + wn * NB + nb) * 16 + (lane & 15)
                        if col >= N:
                            continue
                        for mb in range(MB):
                            for r in range(4):
                                row = m0 + mb * 16 + 4 * (lane >> 4) + r
                                if row < M:
                                    key = (row, col)
                                    assert key not in stored
                                    stored[key] = 1
    assert len(stored) == M * N


@pytest.mark.parametrize("shape", [
    (1, 16, 32, 32), (3, 80, 256, 64), (65, 130, 768, 64), (129, 272, 384, 128),
    (200, 40, 96, 32), (256, 512, 1152, 128), (130, 257, 160, 32), (17, 4112, 192, 64),
])
def test_shapes_in_bounds_and_covered(shape):
    check_shape(*shape)
