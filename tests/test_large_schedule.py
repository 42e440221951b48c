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


def lds_slot(piece, row):
    """LDS slot of 16-byte piece `piece` of activation-tile row `row`
    (w4a16_large.hip, lg_slot)."""
    r = row & 15
    return piece ^ r ^ ((r & 4) << 1)


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
                        sl = lds_slot(spiece, lrow)
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
                                assert row * KT * 2 + lds_slot(piece, lane & 15) * 16 + 16 <= ABYTES
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


# ---------------------------------------------------------------- stream-K grid
# Mirrors large_streamk_kernel and its launcher: units are (problem, tile,
# k-tile), tiles row-tile fastest; workgroup w of NW owns units
# [U*w/NW, U*(w+1)/NW); a tile cut between workgroups is published by each of
# them into (workgroup, slot) and summed by the last to arrive.

MAX_WG = 320
MAXP = 8


def sk_rows(M):
    return 32 if M <= 32 else (64 if M <= 64 else 128)


def sk_plan(problems, M, g, cus=256):
    rows = sk_rows(M)
    T = max(1, KT // g)
    table, units, tiles = [], 0, 0
    for (N, K) in problems:
        G, NCB = K // g, (N + 15) // 16
        MT, NT, KTL = (M + rows - 1) // rows, (NCB + 15) // 16, (G + T - 1) // T
        table.append(dict(N=N, K=K, G=G, NCB=NCB, MT=MT, NT=NT, KT=KTL, u_begin=units,
                          t_begin=tiles))
        units += MT * NT * KTL
        tiles += MT * NT
    nw = min(cus, MAX_WG, units)
    return table, units, nw, tiles, rows


def sk_counter_ints(M, cols):
    rows = sk_rows(M)
    return ((M + rows - 1) // rows) * (MAXP + (cols + 255) // 256)


def sk_simulate(problems, M, g, cus=256):
    table, U, NW, tiles, rows = sk_plan(problems, M, g, cus)
    regs = rows // 16 * 2 * 4
    assert tiles <= sk_counter_ints(M, sum(N for N, _ in problems))
    assert sorted(xcd_b for xcd_b in (tile_of(b, NW) for b in range(NW))) == list(range(NW))
    first = lambda w: U * w // NW
    owner = lambda u: ((u + 1) * NW - 1) // U
    covered, counters, finals, stored, writers = set(), {}, {}, {}, {}
    for w in range(NW):
        u0, u1 = first(w), first(w + 1)
        assert u1 > u0
        u = u0
        while u < u1:
            p = max(i for i, t in enumerate(table) if u >= t["u_begin"])
            pr = table[p]
            v = u - pr["u_begin"]
            tile, k0 = v // pr["KT"], v % pr["KT"]
            assert tile < pr["MT"] * pr["NT"]
            tu0 = pr["u_begin"] + tile * pr["KT"]
            seg_end = min(tu0 + pr["KT"], u1)
            k1 = k0 + (seg_end - u)
            for uu in range(u, seg_end):
                assert uu not in covered
                covered.add(uu)
            key = pr["t_begin"] + tile
            if k0 == 0 and k1 == pr["KT"]:
                stored[key] = stored.get(key, 0) + 1
            else:
                slot = 0 if u0 >= tu0 else 1
                assert (w, slot) not in writers
                writers[(w, slot)] = key
                # last float of this wave's part region, wave 7, register regs-1, lane 63
                last = (((w * 2 + slot) * 8 + 7) * regs + regs - 1) * 64 + 63
                assert last < MAX_WG * 2 * 8 * regs * 64
                nseg = owner(tu0 + pr["KT"] - 1) - owner(tu0) + 1
                assert nseg >= 2 and owner(tu0) <= w <= owner(tu0 + pr["KT"] - 1)
                counters[key] = counters.get(key, 0) + 1
                if counters[key] == nseg:
                    finals[key] = finals.get(key, 0) + 1
                    for ww in range(owner(tu0), owner(tu0 + pr["KT"] - 1) + 1):
                        s2 = 0 if first(ww) >= tu0 else 1
                        assert writers.get((ww, s2)) == key
            u = seg_end
    assert covered == set(range(U))
    for key in range(tiles):
        assert stored.get(key, 0) + finals.get(key, 0) == 1, key
    return dict(U=U, NW=NW, tiles=tiles, rows=rows)


LAYER = [(7168, 5120), (5120, 6144), (34816, 5120), (5120, 17408)]


@pytest.mark.parametrize("M", [17, 32, 33, 64, 65, 128, 200, 256, 1024])
def test_streamk_layer_set(M):
    info = sk_simulate(LAYER, M, 128)
    assert info["NW"] == 256


@pytest.mark.parametrize("case", [
    ([(272, 384)], 129, 128), ([(40, 96)], 200, 32), ([(4112, 192)], 300, 64), ([(16, 32)], 17, 32),
    ([(512, 1152), (300, 640), (48, 128)], 70, 64), ([(5000, 4096)] * 8, 40, 128),
])
@pytest.mark.parametrize("cus", [1, 7, 80, 256, 400])
def test_streamk_small_and_ragged(case, cus):
    problems, M, g = case
    sk_simulate(problems, M, g, cus)


# ------------------------------------------------------- LDS bank behaviour
# A 128-bit LDS access of a wave is served in four passes of 16 lanes; the
# lanes of one pass are those with equal (l5, l2 ^ l3 ^ l4), and within a
# pass two lanes conflict when they touch the same 16-byte slot of the 64
# four-byte banks (address mod 256) at different addresses. Each extra
# distinct address on a slot costs one cycle. This model was fitted to
# SQ_LDS_BANK_CONFLICT counts of 128-bit reads over address patterns on an
# MI355X; MEASURED holds some of those counts (cycles per instruction), which
# the model must reproduce.

def _parity(v):
    return bin(v).count("1") & 1


def pass_conflicts(addr):
    """Conflict cycles of one 128-bit access of 64 lanes at byte addresses addr[l]."""
    passes = {}
    for lane in range(64):
        passes.setdefault((lane >> 5, _parity(lane & 0b11100)), []).append(lane)
    extra = 0
    for lanes in passes.values():
        by_slot = {}
        for lane in lanes:
            by_slot.setdefault(addr[lane] % 256 // 16, set()).add(addr[lane] // 16)
        extra += max(len(s) for s in by_slot.values()) - 1
    return extra


MEASURED = {  # pattern(lane) -> measured conflict cycles per ds_read_b128
    "contiguous": (lambda l: 16 * l, 0),
    "plain xor, group 128": (lambda l: (l & 15) * 256 + ((4 * (l >> 4)) ^ (l & 15)) * 16, 4),
    "same slot, 16 rows": (lambda l: (l & 15) * 256, 60),
    "plain xor, group 32": (lambda l: (l & 15) * 256 + (((l >> 4)) ^ (l & 15)) * 16, 0),
    "plain xor, group 64": (lambda l: (l & 15) * 256 + ((2 * (l >> 4)) ^ (l & 15)) * 16, 0),
    "padded rows": (lambda l: (l & 15) * 272 + 64 * (l >> 4), 4),
    "8 lanes per line": (lambda l: (l & 7) * 16 + (l >> 3) * 256, 4),
    "16 lanes per line": (lambda l: (l & 15) * 16 + (l >> 4) * 256, 0),
}


@pytest.mark.parametrize("name", sorted(MEASURED))
def test_bank_model_reproduces_measured_counts(name):
    f, cycles = MEASURED[name]
    assert pass_conflicts([f(lane) for lane in range(64)]) == cycles


@pytest.mark.parametrize("g", [32, 64, 128])
def test_fragment_reads_are_conflict_free(g):
    c = cfg(g)
    for st in range(4):
        gi, w = st // c["WPL"], st % c["WPL"]
        for mb in range(MB):
            addr = []
            for lane in range(64):
                piece = gi * c["LPG"] + (lane >> 4) * c["WPL"] + w
                addr.append(((lane & 15) + mb * 16) * KT * 2 + lds_slot(piece, lane & 15) * 16)
            assert pass_conflicts(addr) == 0


def test_staging_writes_are_conflict_free_and_read_back():
    written = {}
    for wave in range(THREADS // 64):
        for i in range(LOADS):
            addr = []
            for lane in range(64):
                tid = wave * 64 + lane
                spiece, row = tid % PIECES, tid // PIECES + i * (THREADS // PIECES)
                a = row * KT * 2 + lds_slot(spiece, row) * 16
                assert a not in written
                written[a] = (row, spiece)
                addr.append(a)
            assert pass_conflicts(addr) == 0
    assert len(written) == ROWS * PIECES
    # every fragment read finds the piece it asks for
    for row in range(ROWS):
        for piece in range(PIECES):
            assert written[row * KT * 2 + lds_slot(piece, row & 15) * 16] == (row, piece)
