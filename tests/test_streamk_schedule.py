"""CPU model of the stream-K kernel's schedule (w4a16_skinny.hip), checked for
the invariants its correctness rests on, over many shapes and grid sizes:

* the units (problem, column block, group) are split into contiguous,
  non-empty, disjoint runs, one per wave, covering everything exactly once;
* every super-block (NBW consecutive column blocks: 1 with activations staged
  in LDS, 4 otherwise) is stored exactly once: whole by one wave during its
  stream, or cut, in which case the waves keep their parts in LDS slots
  (wave, slot) that are distinct, the workgroup's leading wave sums exactly
  the slots written for that super-block, and either stores the result (the
  workgroup holds it whole) or hands one part per workgroup on: when exactly
  two workgroups share it, both swap their parts into the super-block's own
  slots (so each slot sees exactly two exchanges); otherwise it publishes the
  part in distinct workspace slots (workgroup, slot), with a counter that
  reaches exactly the number of those parts, so exactly one workgroup
  finalizes it and it finds every part;
* every weight, scale, activation, output, partial, counter and LDS index the
  kernel forms lies inside its buffer.

It mirrors the kernel's integer formulas (wave ranges, unit owners, slots,
leading waves) and the launcher's grid and LDS sizing, so a change to either
must keep this test in step; it runs no device code.
"""
import itertools

import pytest

WAVES = 8
MAX_WAVES = 8192
LDS_BUDGET = 78 * 1024


def sum_stride(M):
    """Floats per group of staged row sums: 16 rows, or 8 with at most 4 rows."""
    return 8 if M <= 4 else 16


def first_unit(w, U, NW):
    return U * w // NW


def owner(u, U, NW):
    return ((u + 1) * NW - 1) // U


WIDE_MAX = 6


def wide(group):
    """Column blocks per unit when each wave reads its activations."""
    return 3 if group == 256 else 6


WIDE_WG_PER_CU = 1
WIDE_MAX_WAVES = 4096


def lds_part_bytes(M, nbw):
    return WAVES * 2 * nbw * min(M, 16) * 16 * 4


def plan(problems, M, group, cus=256, wg_per_cu=2, nbw=None):
    """The launcher's grid: (problem table, units, NW, workgroups, staged
    activation bytes, column blocks, nbw). With nbw None, the launcher's
    choice: 1 when the staged activations and the LDS parts fit the LDS
    budget, wide(group) otherwise (with WIDE_WG_PER_CU workgroups per compute unit)."""
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
        # activation rows and their group sums (G x sum_stride fp32)
        e = sum(Mr * (p["K"] + 8) * 2 + p["G"] * sum_stride(M) * 4 for p in table
                if p["u_begin"] + p["NSB"] * p["G"] > wu0 and p["u_begin"] < wu1)
        need = max(need, e)
    x_bytes = (need + 15) // 16 * 16
    if nbw is None:
        nbw = 1 if x_bytes + lds_part_bytes(M, 1) <= LDS_BUDGET else wide(group)
    if nbw != 1:
        table, units, nw, wgs, cbs = grid(nbw)
    return table, units, nw, wgs, x_bytes, cbs, nbw


def problem_of(table, u):
    p = 0
    for i in range(1, len(table)):
        if u >= table[i]["u_begin"]:
            p = i
    return p


def simulate(problems, M, group, cus=256, wg_per_cu=2, nbw=None):
    table, U, NW, wgs, x_bytes, total_cbs, nbw = plan(problems, M, group, cus, wg_per_cu, nbw)
    Mr = min(M, 16)
    wpl = group // 32
    xlds = nbw == 1 and x_bytes + lds_part_bytes(M, 1) <= LDS_BUDGET
    # LDS layout: staged activations (XLDS only), then the waves' parts
    part_off = x_bytes if xlds else 0
    lds = part_off + lds_part_bytes(M, nbw)
    part_floats = nbw * Mr * 16
    total_sbs = sum(p["NSB"] for p in table)
    assert total_sbs <= 8 + total_cbs          # counters the host reserves
    ws_part_floats = max(MAX_WAVES // WAVES * 2, WIDE_MAX_WAVES // WAVES * 2 * WIDE_MAX) * Mr * 16
    total_cols = sum(N for (N, K) in problems)
    slot_values = ((total_cols + 15) // 16 + 8 * (1 + WIDE_MAX)) * 16 * Mr
    swaps = {}

    def sb_of(u):
        pr = table[problem_of(table, u)]
        sb = (u - pr["u_begin"]) // pr["G"]
        s0 = pr["u_begin"] + sb * pr["G"]
        return pr["sb_begin"] + sb, s0, s0 + pr["G"]

    def wg_of(u):
        return owner(u, U, NW) // WAVES

    covered = {}
    counters = [0] * total_sbs
    nseg_of = {}
    emitted = [0] * total_sbs
    ws_parts = {}
    for b in range(wgs):
        W0 = first_unit(min(b * WAVES, NW), U, NW)
        W1 = first_unit(min((b + 1) * WAVES, NW), U, NW)
        # LDS staging of the workgroup (problems touched by its waves): the
        # activation rows, then the group sums of each touched problem
        xs_base = {}
        if xlds:
            off = 0
            if W1 > W0:
                touched = range(problem_of(table, W0), problem_of(table, W1 - 1) + 1)
                for i in touched:
                    stride = table[i]["K"] + 8
                    # last 16-byte write: row Mr-1, chunk K/8-1
                    last = off + (Mr - 1) * stride + 8 * (table[i]["K"] // 8 - 1) + 8
                    assert last * 2 <= x_bytes, (b, i)
                    off += Mr * stride
                xoff = off // 2
                for i in touched:
                    xs_base[i] = xoff
                    xoff += table[i]["G"] * sum_stride(M)
                assert xoff * 4 <= x_bytes
        lds_parts = {}                      # (local wave, slot) -> super-block
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
                if xlds:  # this unit's group sums (4 floats at 4 * lg, lg <= 3, or <= 1 when compact)
                    ss = sum_stride(M)
                    assert (xs_base[p] + g * ss + (12 if ss == 16 else 4) + 4) * 4 <= part_off
                if seg_g0 is None:
                    seg_g0 = g
                if g == pr["G"] - 1 or u == u1 - 1:
                    gsb = pr["sb_begin"] + sb
                    if seg_g0 == 0 and g == pr["G"] - 1:
                        emitted[gsb] += 1
                    else:
                        usb0 = pr["u_begin"] + sb * pr["G"]
                        slot = 0 if u0 >= usb0 else 1
                        assert (wave, slot) not in lds_parts, (b, wave, slot)
                        lds_parts[(wave, slot)] = gsb
                        # last float of this slot in LDS
                        assert part_off + ((wave * 2 + slot) + 1) * part_floats * 4 <= lds
                    seg_g0 = 0
        # hand-off after the stream: each wave's led super-blocks
        read = set()
        for wave in range(WAVES):
            wg = b * WAVES + wave
            if wg >= NW:
                continue
            u0, u1 = first_unit(wg, U, NW), first_unit(wg + 1, U, NW)
            for k in range(2):
                u = u0 if k == 0 else u1 - 1
                gsb, s0, s1 = sb_of(u)
                if k == 1 and s0 <= u0:
                    break
                if k == 0 and s0 < u0 and wave > 0:
                    continue
                if s0 >= u0 and s1 <= u1:
                    continue
                vlast = owner(min(s1, W1) - 1, U, NW)
                assert wg <= vlast < min((b + 1) * WAVES, NW)
                for v in range(wg, vlast + 1):
                    slot = 0 if first_unit(v, U, NW) >= s0 else 1
                    key = (v - b * WAVES, slot)
                    assert lds_parts.get(key) == gsb, (b, key, gsb)
                    assert key not in read
                    read.add(key)
                if s0 >= W0 and s1 <= W1:
                    emitted[gsb] += 1
                    continue
                nseg = wg_of(s1 - 1) - wg_of(s0) + 1
                assert nseg >= 2
                if nseg == 2:
                    # swap: this super-block's slots, inside the slot region
                    assert (gsb + 1) * part_floats <= slot_values
                    swaps[gsb] = swaps.get(gsb, 0) + 1
                    if swaps[gsb] == 2:
                        emitted[gsb] += 1
                    continue
                slot = 0 if W0 >= s0 else 1
                assert (b, slot) not in ws_parts
                ws_parts[(b, slot)] = gsb
                assert ((b * 2 + slot) + 1) * part_floats <= ws_part_floats
                nseg_of[gsb] = nseg
                counters[gsb] += 1
                if counters[gsb] == nseg:
                    emitted[gsb] += 1
                    for c in range(wg_of(s0), wg_of(s1 - 1) + 1):
                        cs = 0 if first_unit(c * WAVES, U, NW) >= s0 else 1
                        assert ws_parts.get((c, cs)) == gsb, (c, cs, gsb)
        assert read == set(lds_parts), (b, set(lds_parts) - read)
    assert len(covered) == U and sorted(covered) == list(range(U))
    assert all(n == 2 for n in swaps.values())
    for gsb in range(total_sbs):
        assert emitted[gsb] == 1, gsb
        if gsb in nseg_of:
            assert counters[gsb] == nseg_of[gsb]
    # every column block is in exactly one super-block
    for pr in table:
        assert pr["NSB"] * nbw >= pr["NCB"] > (pr["NSB"] - 1) * nbw
    return dict(U=U, NW=NW, wgs=wgs, lds=lds, xlds=xlds, nbw=nbw, swapped=len(swaps),
                counted=len(nseg_of))


LAYER = [(7168, 5120), (5120, 6144), (34816, 5120), (5120, 17408)]


@pytest.mark.parametrize("M", [1, 2, 16])
def test_layer_set_grouped(M):
    info = simulate(LAYER, M, 128)
    assert info["NW"] == (4096 if info["nbw"] == 1 else 2048)
    if M == 1:
        assert info["xlds"] and info["lds"] <= LDS_BUDGET and info["nbw"] == 1
    if M == 16:
        assert not info["xlds"] and info["nbw"] == wide(128)


@pytest.mark.parametrize("nbw", [1, 3, 6])
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


def test_both_cross_workgroup_forms_occur():
    """The layer set takes the two-workgroup swap; a narrow, deep problem (one
    column block, many groups) has super-blocks spread over three or more
    workgroups and takes the counted form."""
    info = simulate(LAYER, 1, 128)
    assert info["swapped"] > 0 and info["counted"] == 0
    info = simulate([(16, 8192)], 1, 32)
    assert info["counted"] > 0
