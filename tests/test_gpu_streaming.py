"""GPU parity of the streaming entry points (w4a16_gemm_ws, w4a16_gemm_grouped)
against the CPU oracle: the persistent stream-K kernel, its workspace protocol
and the one-launch layer set."""
import sys

import numpy as np
import pytest

import oracle
import pins
import synth
from gpu_util import Problem, bf16_bits_to_f64, run_ws, tolerance_ratio, workspace

pytestmark = pytest.mark.gpu


def log(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible to torch")
    import w4a16_weight_only_gemm_amd  # noqa: F401
    yield


def _inputs(cid, M, N, K, g):
    q = synth.gen_q(synth.tensor_id(synth.KIND_Q, 600 + cid, 1), N, K)
    s = synth.gen_scales(synth.tensor_id(synth.KIND_SCALES, 600 + cid, 1), N, K // g)
    x = synth.gen_x(synth.tensor_id(synth.KIND_X, 600 + cid, 1, M), M, K)
    return x, q, s


def test_tiny_gemv_ws():
    x, q, s = synth.tiny_inputs()
    g = synth.TINY["group"]
    y = run_ws(Problem(x, q, s, g))
    assert tolerance_ratio(y, oracle.gemm(x, q, s, g)) <= 1.0


@pytest.mark.parametrize("shape", [(1, 512, 256, 64), (5, 48, 256, 64), (16, 64, 1024, 128),
                                   (9, 80, 5120, 128), (16, 96, 2048, 256), (3, 40, 512, 32)],
                         ids=lambda s: "x".join(map(str, s)))
def test_unit_scale_bit_exact_ws(shape):
    M, N, K, g = shape
    x, q, s, expect = pins.unit_scale_case(M, N, K, g)
    y = run_ws(Problem(x, q, s, g))
    assert np.array_equal(bf16_bits_to_f64(y), expect)


@pytest.mark.parametrize("kg", [(256, 64), (512, 128), (128, 32), (512, 256)], ids=str)
def test_one_hot_rows_recover_codes_ws(kg):
    """Sixteen one-hot activation rows per call, s = 1: y[m][n] = q[n][j_m] exactly;
    K/16 calls cover every k, so every code passes through every lane slot."""
    K, g = kg
    N = 40
    q = synth.gen_q(synth.tensor_id(synth.KIND_Q, 700, K), N, K)
    s = np.full((N, K // g), pins.FP16_ONE, np.uint16)
    got = np.zeros((K, N))
    for c in range(K // 16):
        js = np.arange(16) * (K // 16) + c
        x = np.zeros((16, K))
        x[np.arange(16), js] = 1.0
        y = run_ws(Problem(pins.bf16_bits(x), q, s, g))
        got[js] = bf16_bits_to_f64(y)
    assert np.array_equal(got, q.T.astype(np.float64))


RAGGED = [(1, 16, 128, 32), (1, 200, 384, 64), (2, 520, 1024, 128), (7, 33, 512, 128),
          (15, 64, 768, 256), (16, 1000, 640, 128), (1, 7, 4096, 128), (4, 3000, 2560, 64),
          (16, 5120, 17408, 128), (1, 34816, 5120, 128)]


@pytest.mark.parametrize("case", list(enumerate(RAGGED)), ids=lambda c: "x".join(map(str, c[1])))
def test_ragged_ws(case):
    cid, (M, N, K, g) = case
    log(f"ws ragged {(M, N, K, g)}")
    x, q, s = _inputs(cid, M, N, K, g)
    y = run_ws(Problem(x, q, s, g))
    cols = np.arange(N) if N <= 4096 else np.sort(np.random.default_rng(cid).choice(N, 512, False))
    ref = oracle.gemm(x, q[cols], s[cols], g, threads=synth.default_threads())
    assert tolerance_ratio(y[:, cols], ref) <= 1.0


def _layer_problems(M, layer=0):
    probs, data = [], []
    for pi, p in enumerate(synth.LAYER_PROJECTIONS):
        x, q, s = synth.layer_inputs(layer, pi, M)
        probs.append(Problem(x, q, s, synth.GROUP))
        data.append((x, q, s))
    return probs, data


@pytest.mark.parametrize("layer", [0, 63])
@pytest.mark.parametrize("M", [1, 2, 3, 4, 16])
def test_layer_set_grouped_full(M, layer):
    """The four projections of a layer in one launch, every output checked
    (layers 0 and 63: the first and last of the 64-layer stack). The launch
    forms: rows staged in LDS (M = 1, 2), six-column-block units with each
    wave reading its activation fragments (M = 3, 4, 16)."""
    import torch
    import w4a16_weight_only_gemm_amd as w4
    probs, data = _layer_problems(M, layer)
    ys = [torch.empty((M, p.N), dtype=torch.bfloat16, device="cuda") for p in probs]
    ws = workspace(M, sum(p.N for p in probs))
    entries = [(p.x, p.qw, p.sp, y, p.N, p.K) for p, y in zip(probs, ys)]
    for rep in range(2):  # the second call reuses the workspace the first left clean
        w4.w4a16_gemm_grouped(entries, M, synth.GROUP, ws)
        torch.cuda.synchronize()
        for (x, q, s), y, p in zip(data, ys, synth.LAYER_PROJECTIONS):
            yb = y.view(torch.int16).cpu().numpy().view(np.uint16)
            r = tolerance_ratio(yb, oracle.gemm(x, q, s, synth.GROUP, threads=synth.default_threads()))
            log(f"grouped M={M} {p.name} rep {rep}: ratio {r:.4f}")
            assert r <= 1.0
    assert _handoff_state_clean(ws, M, sum(p.N for p in probs))


def _handoff_state_clean(ws, M, total_columns):
    """True when the workspace's counters and swap slots (the regions that
    must be zero between calls) are zero. Region sizes as the library lays
    them out: counters, then one slot per output value of every super-block
    (column blocks plus 8 problems x 5 blocks of slack) for min(M, 16) rows."""
    import w4a16_weight_only_gemm_amd as w4
    ncount = w4.w4a16_workspace_bytes(0, total_columns)
    nslot = (((total_columns + 15) // 16 + 40) * 16 * min(M, 16) * 4 + 255) // 256 * 256
    return int(ws[:(ncount + nslot) // 4].abs().sum().item()) == 0


# Narrow, deep problems: super-blocks spread over three or more workgroups
# (the counted hand-off), several problems in one launch; the last case also
# has super-blocks shared by exactly two workgroups (the swap) at M = 1.
DEEP = [[(16, 8192, 32)], [(48, 16384, 64)], [(64, 8192, 32), (200, 4096, 32)],
        [(16, 2048, 32), (40, 8192, 32), (24, 1024, 32)], [(16, 16384, 32), (6144, 2048, 32)]]


@pytest.mark.parametrize("M", [1, 5, 16])
@pytest.mark.parametrize("case", list(enumerate(DEEP)), ids=lambda c: str(c[0]))
def test_deep_problems_handoff(case, M):
    import torch
    import w4a16_weight_only_gemm_amd as w4
    cid, shapes = case
    g = shapes[0][2]
    data = [_inputs(60 + 4 * cid + i, M, N, K, g) for i, (N, K, _) in enumerate(shapes)]
    probs = [Problem(x, q, s, g) for (x, q, s) in data]
    ys = [torch.empty((M, p.N), dtype=torch.bfloat16, device="cuda") for p in probs]
    total = sum(p.N for p in probs)
    ws = workspace(M, total)
    entries = [(p.x, p.qw, p.sp, y, p.N, p.K) for p, y in zip(probs, ys)]
    log(f"deep problems {shapes} M={M}")
    first = None
    for rep in range(3):
        w4.w4a16_gemm_grouped(entries, M, g, ws)
        torch.cuda.synchronize()
        outs = [y.view(torch.int16).cpu().numpy().view(np.uint16).copy() for y in ys]
        assert _handoff_state_clean(ws, M, total)
        if first is None:
            first = outs
            for (x, q, s), yb in zip(data, outs):
                assert tolerance_ratio(yb, oracle.gemm(x, q, s, g, threads=synth.default_threads())) <= 1.0
        else:
            assert all(np.array_equal(a, b) for a, b in zip(first, outs))


@pytest.mark.parametrize("M", [1, 4, 16])
def test_streaming_deterministic(M):
    x, q, s = _inputs(40 + M, M, 5120, 6144, 128)
    prob = Problem(x, q, s, 128)
    ws = workspace(M, 5120)
    a, b = run_ws(prob, ws), run_ws(prob, ws)
    assert np.array_equal(a, b)
    assert _handoff_state_clean(ws, M, 5120)
    assert tolerance_ratio(a, oracle.gemm(x, q, s, 128, threads=synth.default_threads())) <= 1.0


def test_workspace_errors():
    import torch
    import w4a16_weight_only_gemm_amd as w4
    M, N, K, g = 4, 64, 256, 64
    x, q, s = _inputs(90, M, N, K, g)
    prob = Problem(x, q, s, g)
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    ws = workspace(M, N)
    e = [(prob.x, prob.qw, prob.sp, y, N, K)]
    nb = ws.numel() * 4
    assert w4.grouped_status(e, M, g, ws, nb - 4) == w4.W4A16_ERR_INVALID_ARG
    assert w4.grouped_status(e, M, g, None, nb) == w4.W4A16_ERR_INVALID_ARG
    big = workspace(M, N + 8192)  # room for a 16-byte offset
    assert w4.grouped_status(e, M, g, big.data_ptr() + 16, nb) == w4.W4A16_ERR_MISALIGNED
    assert w4.grouped_status(e, M, g, ws, nb) == w4.W4A16_OK
    torch.cuda.synchronize()
    yb = y.view(torch.int16).cpu().numpy().view(np.uint16)
    assert tolerance_ratio(yb, oracle.gemm(x, q, s, g)) <= 1.0
