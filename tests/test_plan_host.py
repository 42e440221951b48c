"""Host-only tests of planned calls (w4a16_plan_build, w4a16_gemm_planned): the
plan's byte image against an independent model of its fields (problem table
offsets, the first problem of every workgroup, workspace layout, checksum), and
every error path, which returns before any launch. No call here reaches a
kernel: the problem pointers are aligned dummy addresses."""
import numpy as np
import pytest

import w4a16_weight_only_gemm_amd as w4

HDR = np.dtype([("magic", "<u4"), ("version", "<u4"), ("kind", "<i4"), ("count", "<i4"),
                ("M", "<i4"), ("group", "<i4"), ("grid", "<i4"), ("nwaves", "<i4"),
                ("nbw", "<i4"), ("rows", "<i4"), ("xlds", "<i4"), ("lds_bytes", "<i4"),
                ("lds_part_off", "<i4"), ("table_off", "<i4"), ("wgfirst_off", "<i4"),
                ("tiles", "<i4"), ("units", "<i8"), ("total_columns", "<i8"),
                ("counters_off", "<i8"), ("slots_off", "<i8"), ("part_off", "<i8"),
                ("workspace_bytes", "<i8"), ("checksum", "<u8"), ("pad1", "<u8", 5)])
SK = np.dtype([("x", "<u8"), ("qw", "<u8"), ("sp", "<u8"), ("y", "<u8"), ("N", "<i4"),
               ("K", "<i4"), ("G", "<i4"), ("NCB", "<i4"), ("NSB", "<i4"), ("pad", "<i4"),
               ("u_begin", "<i8"), ("sb_begin", "<i4"), ("pad2", "<i4")])
LG = np.dtype([("x", "<u8"), ("qw", "<u8"), ("sp", "<u8"), ("y", "<u8"), ("N", "<i4"),
               ("K", "<i4"), ("G", "<i4"), ("NCB", "<i4"), ("MT", "<i4"), ("NT", "<i4"),
               ("KT", "<i4"), ("pad", "<i4"), ("u_begin", "<i8"), ("t_begin", "<i4"),
               ("pad2", "<i4")])
MAGIC = 0x4C503457
CUS = 256  # the library's compute-unit count when no device is visible
WIDE = {32: 6, 64: 6, 128: 6, 256: 3}


def fnv1a64(data: bytes) -> int:
    h = 0xcbf29ce484222325
    for b in data:
        h ^= b
        h = (h * 0x100000001b3) & 0xFFFFFFFFFFFFFFFF
    return h


def _problems(shapes, base=1 << 20):
    """(x, qweight, scales, y, N, K) tuples with distinct 256-byte aligned dummy addresses."""
    out = []
    for i, (N, K) in enumerate(shapes):
        a = base + i * (1 << 16)
        out.append((a, a + 0x1000, a + 0x2000, a + 0x3000, N, K))
    return out


def _parse(plan):
    h = np.frombuffer(plan[:HDR.itemsize].tobytes(), HDR)[0]
    dt = SK if h["kind"] == 1 else LG
    tab = np.frombuffer(plan[h["table_off"]:h["table_off"] + dt.itemsize * h["count"]].tobytes(), dt)
    wgf = np.frombuffer(plan[h["wgfirst_off"]:h["wgfirst_off"] + 4 * h["grid"]].tobytes(), "<i4")
    return h, tab, wgf


def _checksum(plan):
    """FNV-1a over the whole plan with its checksum field (bytes 112..119) read as zero."""
    b = bytearray(plan.tobytes())
    b[112:120] = bytes(8)
    return fnv1a64(bytes(b))


def _owner(u_begin, u):
    return int(np.searchsorted(u_begin, u, side="right") - 1)


SHAPES = [(7168, 5120), (5120, 6144), (34816, 5120), (5120, 17408)] * 3 + [(200, 384), (33, 256)]


@pytest.mark.parametrize("M", [1, 2, 5, 16])
@pytest.mark.parametrize("group", [32, 64, 128, 256])
def test_streamk_plan_fields(M, group):
    shapes = [(N, K) for N, K in SHAPES if K % group == 0]
    probs = _problems(shapes)
    plan = w4.w4a16_plan_build(probs, M, group)
    assert len(plan) == w4.w4a16_plan_bytes(len(probs))
    h, tab, wgf = _parse(plan)
    assert (h["magic"], h["kind"], h["count"], h["M"], h["group"]) == (MAGIC, 1, len(probs), M, group)
    nbw = int(h["nbw"])
    assert nbw == (1 if h["xlds"] else WIDE[group])
    if h["xlds"]:
        assert h["lds_bytes"] <= 78 * 1024
    # problem table: pointers, shapes, and prefix sums of units and super-blocks
    u = sb = 0
    for e, (x, qw, sp, y, N, K) in zip(tab, probs):
        assert (e["x"], e["qw"], e["sp"], e["y"], e["N"], e["K"]) == (x, qw, sp, y, N, K)
        G, NCB = int(K) // group, -(-int(N) // 16)
        NSB = -(-NCB // nbw)
        assert (e["G"], e["NCB"], e["NSB"], e["u_begin"], e["sb_begin"]) == (G, NCB, NSB, u, sb)
        u += NSB * G  # Python integers: the products exceed 32 bits
        sb += NSB
    assert h["units"] == u
    assert h["total_columns"] == sum(N for N, _ in shapes)
    # the grid: every counted wave owns at least one unit, eight waves per workgroup
    cap = CUS * (2 if nbw == 1 else 1) * 8
    cap = min(cap, 8192 if nbw == 1 else 4096)
    assert h["nwaves"] == min(cap, u)
    assert h["grid"] == -(-h["nwaves"] // 8)
    # the first problem of every workgroup holds its first unit
    for b in range(h["grid"]):
        first = u * (8 * b) // int(h["nwaves"])
        assert wgf[b] == _owner(tab["u_begin"], first)
    # workspace: counters per super-block, swap slots per output of every super-block, parts
    Mr = min(M, 16)
    cb = -(-sb * 4 // 256) * 256
    sl = -(-sb * nbw * Mr * 16 * 4 // 256) * 256
    assert (h["counters_off"], h["slots_off"], h["part_off"]) == (0, cb, cb + sl)
    assert h["workspace_bytes"] > h["part_off"]
    assert w4.w4a16_plan_workspace_bytes(plan) == h["workspace_bytes"]
    assert h["checksum"] == _checksum(plan)


@pytest.mark.parametrize("M", [17, 64, 65, 1024])
@pytest.mark.parametrize("group", [32, 64, 128])
def test_large_plan_fields(M, group):
    shapes = [(N, K) for N, K in SHAPES if K % group == 0]
    probs = _problems(shapes)
    plan = w4.w4a16_plan_build(probs, M, group)
    h, tab, wgf = _parse(plan)
    assert (h["magic"], h["kind"], h["count"], h["M"], h["group"]) == (MAGIC, 2, len(probs), M, group)
    rows = 32 if M <= 32 else (64 if M <= 64 else 128)
    assert h["rows"] == rows
    u = t = 0
    for e, (x, qw, sp, y, N, K) in zip(tab, probs):
        G, NCB = K // group, -(-N // 16)
        MT, NT, KT = -(-M // rows), -(-NCB // 16), -(-G // (128 // group))
        assert (e["G"], e["NCB"], e["MT"], e["NT"], e["KT"]) == (G, NCB, MT, NT, KT)
        assert (e["u_begin"], e["t_begin"]) == (u, t)
        u += MT * NT * KT
        t += MT * NT
    assert h["grid"] == min(CUS, 320, u)
    if t >= 16 * h["grid"]:
        # whole tiles dealt round robin: no stream-K split, no workspace
        assert h["tiles"] == 1 and h["units"] == t and h["workspace_bytes"] == 0
    else:
        assert h["tiles"] == 0 and h["units"] == u
        for w in range(h["grid"]):
            assert wgf[w] == _owner(tab["u_begin"], u * w // h["grid"])
        assert h["part_off"] == -(-t * 4 // 256) * 256
        regs = rows // 16 * 2 * 4
        assert h["workspace_bytes"] == h["part_off"] + 320 * 2 * 8 * regs * 64 * 4
    assert h["checksum"] == _checksum(plan)


def test_large_plan_of_many_tiles_deals_whole_tiles():
    # 64 layer sets at M = 1024: 104,448 tiles of 128 x 256, whole tiles per workgroup
    shapes = [(7168, 5120), (5120, 6144), (34816, 5120), (5120, 17408)] * 64
    plan = w4.w4a16_plan_build(_problems(shapes, base=1 << 24), 1024, 128)
    h, tab, _ = _parse(plan)
    assert h["tiles"] == 1 and h["units"] == 64 * 8 * (28 + 20 + 136 + 20)
    assert h["workspace_bytes"] == 0 and w4.w4a16_plan_workspace_bytes(plan) == 0
    assert list(tab["t_begin"][:5]) == [0, 224, 384, 1472, 1632]


def test_plan_errors_return_before_any_launch():
    probs = _problems([(512, 256), (64, 192)])
    assert w4.w4a16_plan_bytes(0) == 0 and w4.w4a16_plan_bytes(4097) == 0
    assert w4.w4a16_plan_bytes(4096) > w4.w4a16_plan_bytes(1) > 256
    ok, _ = w4.plan_build_status(probs, 1, 64)
    assert ok == w4.W4A16_OK
    assert w4.plan_build_status(probs, 0, 64)[0] == w4.W4A16_ERR_INVALID_ARG       # M = 0
    assert w4.plan_build_status(probs, 1, 48)[0] == w4.W4A16_ERR_UNSUPPORTED       # group
    assert w4.plan_build_status(probs, 1, 128)[0] == w4.W4A16_ERR_UNSUPPORTED      # K % group
    assert w4.plan_build_status(probs, 64, 256)[0] == w4.W4A16_ERR_UNSUPPORTED     # M > 16, g 256
    bad = [list(p) for p in probs]
    bad[1][3] += 8
    assert w4.plan_build_status([tuple(b) for b in bad], 1, 64)[0] == w4.W4A16_ERR_MISALIGNED
    bad = [list(p) for p in probs]
    bad[0][0] = 0
    assert w4.plan_build_status([tuple(b) for b in bad], 1, 64)[0] == w4.W4A16_ERR_INVALID_ARG
    bad = [list(p) for p in probs]
    bad[0][4] = -1
    assert w4.plan_build_status([tuple(b) for b in bad], 1, 64)[0] == w4.W4A16_ERR_INVALID_ARG
    # w4a16_gemm_planned refuses what is not a plan, and too small or misaligned workspaces
    plan = w4.w4a16_plan_build(probs, 1, 64)
    need = w4.w4a16_plan_workspace_bytes(plan)
    dev = 1 << 30  # a dummy device address: never used, every call below fails first
    junk = np.zeros_like(plan)
    assert w4.w4a16_plan_workspace_bytes(junk) == 0
    assert w4.planned_status(junk, dev, dev, need) == w4.W4A16_ERR_INVALID_ARG
    assert w4.planned_status(plan, dev, dev, need - 1) == w4.W4A16_ERR_INVALID_ARG
    assert w4.planned_status(plan, dev, 0, need) == w4.W4A16_ERR_INVALID_ARG
    assert w4.planned_status(plan, 0, dev, need) == w4.W4A16_ERR_INVALID_ARG
    assert w4.planned_status(plan, dev + 8, dev, need) == w4.W4A16_ERR_MISALIGNED
    assert w4.planned_status(plan, dev, dev + 16, need) == w4.W4A16_ERR_MISALIGNED
