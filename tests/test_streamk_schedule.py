"""CPU model of the stream-K kernel's schedule (w4a16_skinny.hip), checked for
the invariants its correctness rests on, over many shapes and grid sizes:

* the units (problem, column block, group) are split into contiguous,
  non-empty, disjoint runs, one per wave, covering everything exactly once;
* every super-block (NBW consecutive column blocks: 1 with activations staged
  in LDS, 4 otherwise) is either stored whole by one wave, or cut into parts by
  consecutive waves whose (wave, slot) partial buffers are distinct, and the
  per-super-block counter reaches exactly the number of parts (so exactly one
  wave finalizes it, and it finds every part);
* every weight, scale, activation, output, partial, counter and LDS index the
  kernel forms lies inside its buffer.

It mirrors the kernel's integer formulas (wave ranges, unit owners, slots) and
the launcher's grid and LDS sizing, so a change to either must keep this test
in step; it runs no device code.
"""
import itertools

import pytest

WAVES = 8
MAX_WAVES = 8192
LDS_BUDGET = 64 * 1024


def first_unit(w, U, NW):
    return U * w // NW


def owner(u, U, NW):
    return ((u + 1) * NW - 1) // U


WIDE = 4


WIDE_WG_PER_CU = 1
WIDE_MAX_WAVES = 4096


def plan(problems, M, group, cus=256, wg_per_cu=2, nbw=None):
    """The launcher's grid: (problem table, units, NW, workgroups, lds bytes,
    column blocks, nbw). With nbw None, the launcher's choice: 1 when the
    activations fit the LDS budget, WIDE otherwise (with WIDE_WG_PER_CU
    workgroups per compute unit)."""
    def grid(nbw):
        table, units, sbs, cbs = [], 0, 0, 0
        for (N, K) in problems:
            G, NCB = K // group, (N + 15) // 16
            NSB = (NCB + nbw - 1) // nbw
            table.append(dict(N=N, K=K, G=G, NCB=NCB, NSB=NSB, u_begin=units, sb_begin=sbs))
            units += NSB * G
            sbs += NSB
            cbs += NCB
        wgs = cus * (wg_per_cu if nbw == 1 else WIDE_WG_PER_CU)
        max_waves = MAX_WAVES if nbw == 1 else WIDE_MAX_WAVES
        if wgs * WAVES > max_waves:
            wgs = max_waves // WAVES
        nw = min(wgs * WAVES, units)
        wgs = (nw + WAVES - 1) // WAVES
        return table, units, nw, wgs, cbs
    table, units, nw, wgs, cbs = grid(1)
    Mr = min(M, 16)
    need = 0
    for b in range(wgs):
        wb0, wb1 = b * WAVES, min(b * WAVES + WAVES, nw)
        wu0, wu1 = units * wb0 // nw, units * wb1 // nw
        if wu1 <= wu0:
            continue
        e = sum(Mr * (p["K"] + 8) for p in table
                if p["u_begin"] + p["NSB"] * p["G"] > wu0 and p["u_begin"] < wu1)
        need = max(need, e)
    if nbw is None:
        nbw = 1 if need * 2 <= LDS_BUDGET else WIDE
    if nbw != 1:
        table, units, nw, wgs, cbs = grid(nbw)
    return table, units, nw, wgs, need * 2, cbs, nbw


def problem_of(table, u):
    p = 0
    for i in range(1, len(table)):
        if u >= table[i]["u_begin"]:
            p = i
    return p


def simulate(problems, M, group, cus=256, wg_per_cu=2, nbw=None):
    table, U, NW, wgs, lds, total_cbs, nbw = plan(problems, M, group, cus, wg_per_cu, nbw)
    Mr = min(M, 16)
    wpl = group // 32
    xlds = nbw == 1 and lds <= LDS_BUDGET
    total_sbs = sum(p["NSB"] for p in table)
    assert total_sbs <= 8 + total_cbs          # counters the host reserves
    covered = {}
    counters = [0] * total_sbs
    finalized = [0] * total_sbs
    part_writers = {}
    stored_whole = [0] * total_sbs
    for b in range(wgs):
        # LDS staging of the workgroup (problems touched by its waves)
        if xlds:
            wu0 = first_unit(b * WAVES, U, NW)
            wu1 = first_unit(min((b + 1) * WAVES, NW), U, NW)
            off = 0
            if wu1 > wu0:
                for i in range(problem_of(table, wu0), problem_of(table, wu1 - 1) + 1):
                    stride = table[i]["K"] + 8
                    # last 16-byte write: row Mr-1, chunk K/8-1
                    last = off + (Mr - 1) * stride + 8 * (table[i]["K"] // 8 - 1) + 8
                    assert last * 2 <= lds, (b, i)
                    off += Mr * stride
        for wave in range(WAVES):
            wg = b * WAVES + wave
            if wg >= NW:
                continue
            u0, u1 = first_unit(wg, U, NW), first_unit(wg + 1, U, NW)
            assert u1 > u0, "empty wave"
            seg_g0 = None
            for u in range(u0, u1):
                assert u not in covered
                covered[u] = wg
                p = problem_of(table, u)
                pr = table[p]
                v = u - pr["u_begin"]
                sb, g = v // pr["G"], v % pr["G"]
                assert sb < pr["NSB"]
                # weight / scale / activation indices of this unit
                for j in range(nbw):
                    tile = min(sb * nbw + j, pr["NCB"] - 1) * pr["G"] + g
                    assert (tile * 64 + 63) * wpl + wpl - 1 < pr["NCB"] * 16 * pr["K"] // 8
                    assert tile * 16 + 15 < pr["NCB"] * 16 * pr["G"]
                row = min(15, M - 1)
                assert row * pr["K"] + g * group + 3 * wpl * 8 + 8 * (wpl - 1) + 7 < M * pr["K"]
                if seg_g0 is None:
                    seg_g0 = g
                if g == pr["G"] - 1 or u == u1 - 1:
                    gsb = pr["sb_begin"] + sb
                    if seg_g0 == 0 and g == pr["G"] - 1:
                        stored_whole[gsb] += 1
                    else:
                        usb0 = pr["u_begin"] + sb * pr["G"]
                        wfirst, wlast = owner(usb0, U, NW), owner(usb0 + pr["G"] - 1, U, NW)
                        nseg = wlast - wfirst + 1
                        assert nseg >= 2
                        assert wfirst <= wg <= wlast
                        slot = 0 if u0 >= usb0 else 1
                        key = (wg, slot)
                        assert key not in part_writers, key
                        part_writers[key] = gsb
                        # last float of this wave's part, against the workspace size
                        part_floats = max(MAX_WAVES * 2, WIDE_MAX_WAVES * 2 * WIDE) * Mr * 16
                        assert ((wg * 2 + slot) * nbw + nbw) * Mr * 16 <= part_floats
                        counters[gsb] += 1
                        if counters[gsb] == nseg:
                            finalized[gsb] += 1
                            # the finalizer reads the part of every wave in [wfirst, wlast]
                            for w in range(wfirst, wlast + 1):
                                ws = 0 if first_unit(w, U, NW) >= usb0 else 1
                                assert part_writers.get((w, ws)) == gsb, (w, ws, gsb)
                    seg_g0 = 0
    assert len(covered) == U and sorted(covered) == list(range(U))
    for gsb in range(total_sbs):
        assert stored_whole[gsb] + finalized[gsb] == 1, gsb
        assert finalized[gsb] == 0 or counters[gsb] >= 2
    # every column block is in exactly one super-block
    for pr in table:
        assert pr["NSB"] * nbw >= pr["NCB"] > (pr["NSB"] - 1) * nbw
    return dict(U=U, NW=NW, wgs=wgs, lds=lds, xlds=xlds, nbw=nbw)


LAYER = [(7168, 5120), (5120, 6144), (34816, 5120), (5120, 17408)]


@pytest.mark.parametrize("M", [1, 2, 16])
def test_layer_set_grouped(M):
    info = simulate(LAYER, M, 128)
    assert info["NW"] == (4096 if info["nbw"] == 1 else 2048)
    if M == 1:
        assert info["xlds"] and info["lds"] <= LDS_BUDGET and info["nbw"] == 1
    if M == 16:
        assert not info["xlds"] and info["nbw"] == WIDE


@pytest.mark.parametrize("nbw", [1, WIDE])
@pytest.mark.parametrize("case", [([(200, 384)], 16, 64), ([(33, 512)], 7, 128),
                                  ([(100, 64), (300, 128), (17, 96)], 9, 32), (LAYER[:2], 16, 128)])
def test_forced_block_widths(case, nbw):
    problems, M, g = case
    simulate(problems, M, g, nbw=nbw)


@pytest.mark.parametrize("proj", LAYER)
@pytest.mark.parametrize("M", [1, 16])
def test_single_projection(proj, M):
    simulate([proj], M, 128)


@pytest.mark.parametrize("case", [
    ([(512, 256)], 1, 64), ([(16, 128)], 3, 32), ([(200, 384)], 1, 64), ([(1, 256)], 5, 64),
    ([(520, 1024)], 2, 128), ([(33, 512)], 7, 128), ([(48, 2048), (16, 512)], 16, 256),
    ([(100, 64), (300, 128), (17, 96)], 9, 32), ([(5000, 4096)] * 8, 1, 128),
])
def test_small_and_ragged(case):
    problems, M, g = case
    simulate(problems, M, g)


@pytest.mark.parametrize("cus,wg", itertools.product([1, 3, 80, 256, 304], [1, 2, 4]))
def test_grid_sizes(cus, wg):
    simulate(LAYER[:2], 1, 128, cus=cus, wg_per_cu=wg)
    simulate([(40, 256)], 4, 64, cus=cus, wg_per_cu=wg)
