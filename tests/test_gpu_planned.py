"""GPU parity of planned calls (w4a16_plan_build + w4a16_gemm_planned): many
independent GEMMs in one launch, descriptors read from a device copy of the
plan. Each output against the oracle within |y - y_ref| <= 1e-2 (1 + |y_ref|);
repeated calls on one workspace bit-identical; a plan of at most eight problems
bit-identical to w4a16_gemm_grouped on the same problems (same split of the
work); a device plan that is not the host's does nothing."""
import sys

import numpy as np
import pytest

import oracle
import synth
from gpu_util import bf16_bits_to_f64, dev_u16, dev_u32, tolerance_ratio

pytestmark = pytest.mark.gpu


def log(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible to torch")
    import w4a16_weight_only_gemm_amd  # noqa: F401  (fails loudly if the library is missing)
    yield


class Batch:
    """Packed weights, activations and outputs of several GEMMs sharing M and the group."""

    def __init__(self, case, M, shapes, g):
        import torch

        import w4a16_weight_only_gemm_amd as w4
        self.M, self.g, self.shapes = M, g, shapes
        self.host, self.dev = [], []
        for i, (N, K) in enumerate(shapes):
            q = synth.gen_q(synth.tensor_id(synth.KIND_Q, 800 + case, i), N, K)
            s = synth.gen_scales(synth.tensor_id(synth.KIND_SCALES, 800 + case, i), N, K // g)
            x = synth.gen_x(synth.tensor_id(synth.KIND_X, 800 + case, i, M), M, K)
            qw, sp = w4.w4a16_pack(q, s, g)
            self.host.append((x, q, s))
            self.dev.append((dev_u16(x).view(torch.bfloat16), dev_u32(qw), dev_u16(sp),
                             torch.empty((M, N), dtype=torch.bfloat16, device="cuda")))

    def entries(self):
        return [(x, qw, sp, y, N, K) for (x, qw, sp, y), (N, K) in zip(self.dev, self.shapes)]

    def outputs(self):
        import torch
        torch.cuda.synchronize()
        return [y.view(torch.int16).cpu().numpy().view(np.uint16) for (_, _, _, y) in self.dev]


def _planned(batch, ws=None, plan=None):
    """(plan, plan_dev, workspace) after one planned call."""
    import torch

    import w4a16_weight_only_gemm_amd as w4
    if plan is None:
        plan = w4.w4a16_plan_build(batch.entries(), batch.M, batch.g)
    plan_dev = torch.from_numpy(plan).to("cuda")
    if ws is None:
        nb = w4.w4a16_plan_workspace_bytes(plan)
        ws = torch.zeros((nb + 3) // 4, dtype=torch.int32, device="cuda")
    w4.w4a16_gemm_planned(plan, plan_dev, ws)
    return plan, plan_dev, ws


# Twelve to twenty problems of ragged shapes: more than the grouped call's eight.
MIXED = [(520, 1024), (7168, 512), (33, 768), (1000, 256), (64, 2048), (200, 384), (4096, 1024),
         (16, 512), (130, 1536), (2048, 768), (80, 5120), (300, 1024)]

CASES = [(1, 128), (1, 64), (2, 128), (5, 32), (16, 128), (16, 256), (17, 128), (40, 64),
         (64, 128), (100, 32), (300, 128), (1024, 64)]


@pytest.mark.parametrize("case", list(enumerate(CASES)), ids=lambda c: "M%d_g%d" % c[1])
def test_planned_mixed_shapes_against_oracle(case):
    cid, (M, g) = case
    shapes = [(N, K) for N, K in MIXED if K % g == 0]
    if M <= 16:
        shapes = shapes + shapes[:6]  # 18 problems
    log(f"planned M={M} g={g}: {len(shapes)} problems")
    b = Batch(cid, M, shapes, g)
    _, _, ws = _planned(b)
    ys = b.outputs()
    for i, ((x, q, s), y) in enumerate(zip(b.host, ys)):
        rows = slice(0, min(M, 96))  # the oracle over at most 96 rows, all columns
        ref = oracle.gemm(x[rows], q, s, g, threads=synth.default_threads())
        r = tolerance_ratio(y[rows], ref)
        assert r <= 1.0, f"problem {i} {shapes[i]}: ratio {r}"
    # a second call on the same workspace: the counters were left at zero, same bits
    _planned(b, ws=ws)
    for y0, y1 in zip(ys, b.outputs()):
        assert np.array_equal(y0, y1)


@pytest.mark.parametrize("M,g", [(1024, 128), (200, 64), (40, 32)])
def test_planned_whole_tiles_against_oracle(M, g):
    """Enough problems that the plan deals whole tiles round robin (no
    workspace): every row tile and ragged column tile against the oracle."""
    import w4a16_weight_only_gemm_amd as w4
    reps = {1024: 8, 200: 32, 40: 64}[M]
    shapes = [(N, K) for N, K in MIXED if K % g == 0 and K <= 2048] * reps
    b = Batch(30 + M, M, shapes, g)
    plan = w4.w4a16_plan_build(b.entries(), M, g)
    assert w4.w4a16_plan_workspace_bytes(plan) == 0, "expected the whole-tile form"
    log(f"planned whole tiles M={M} g={g}: {len(shapes)} problems")
    _planned(b, plan=plan)
    ys = b.outputs()
    rng = np.random.default_rng(M)
    rows = np.unique(np.concatenate([[0, M - 1], np.arange(127, M, 128), np.arange(128, M, 128),
                                     rng.choice(M, 8, replace=False)]))
    rows = rows[rows < M]
    for i, ((x, q, s), y) in enumerate(zip(b.host, ys)):
        if i % 3 and i >= len(MIXED):  # every problem of the first set, a third of the rest
            continue
        ref = oracle.gemm(x[rows], q, s, g, threads=synth.default_threads())
        r = tolerance_ratio(y[rows], ref)
        assert r <= 1.0, f"problem {i} {shapes[i]}: ratio {r}"
    # and again, same bits
    _planned(b, plan=plan)
    for y0, y1 in zip(ys, b.outputs()):
        assert np.array_equal(y0, y1)


@pytest.mark.parametrize("M", [1, 16, 64, 1024])
def test_planned_layer_is_bit_identical_to_grouped(M):
    """The four projections of a (scaled-down) layer: the plan splits the work as
    w4a16_gemm_grouped does, so the results are the same bits."""
    import torch

    import w4a16_weight_only_gemm_amd as w4
    shapes = [(1792, 1280), (1280, 1536), (8704, 1280), (1280, 4352)]
    b = Batch(50 + M, M, shapes, 128)
    _planned(b)
    yp = b.outputs()
    cols = sum(N for N, _ in shapes)
    nb = w4.w4a16_workspace_bytes(M, cols)
    ws = torch.zeros((nb + 3) // 4, dtype=torch.int32, device="cuda")
    w4.w4a16_gemm_grouped(b.entries(), M, 128, ws)
    for y0, y1 in zip(yp, b.outputs()):
        assert np.array_equal(y0, y1)


def test_planned_with_another_device_plan_does_nothing():
    import torch

    import w4a16_weight_only_gemm_amd as w4
    b = Batch(90, 4, [(512, 1024), (256, 512)], 128)
    other = w4.w4a16_plan_build(b.entries(), 3, 128)   # a different plan (M = 3)
    plan = w4.w4a16_plan_build(b.entries(), 4, 128)
    assert int(other[112:120].view(np.uint64)[0]) != int(plan[112:120].view(np.uint64)[0])
    for (_, _, _, y) in b.dev:
        y.view(torch.int16).fill_(0x7FC1)  # a sentinel NaN pattern
    nb = max(w4.w4a16_plan_workspace_bytes(plan), w4.w4a16_plan_workspace_bytes(other))
    ws = torch.zeros((nb + 3) // 4, dtype=torch.int32, device="cuda")
    w4.w4a16_gemm_planned(plan, torch.from_numpy(other).to("cuda"), ws)
    for y in b.outputs():
        assert np.all(y == 0x7FC1)
    # and with its own device copy it computes
    _planned(b, ws=ws, plan=plan)
    for (x, q, s), y in zip(b.host, b.outputs()):
        assert tolerance_ratio(y, oracle.gemm(x, q, s, 128)) <= 1.0
