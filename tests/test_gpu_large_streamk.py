"""GPU parity of the stream-K large-M path (w4a16_gemm_grouped at M > 16, and
w4a16_gemm_ws where it runs it) against the CPU oracle: tiles of 32, 64 and 128
rows, tiles cut between workgroups and summed through the workspace, several
problems per launch, and repeated calls on one workspace (the counters must
come back to zero, and the parts are summed in a fixed order). A single
problem above 16 rows may run w4a16_gemm's kernels instead (when the time
models put them ahead), so the single-shape cases launch the problem twice in
one grouped call (run_streamk), which always takes the stream-K schedule."""
import sys

import numpy as np
import pytest

import oracle
import pins
import synth
from gpu_util import Problem, bf16_bits_to_f64, run_streamk, run_ws, tolerance_ratio, workspace

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


def _inputs(cid, M, N, K, g):
    q = synth.gen_q(synth.tensor_id(synth.KIND_Q, 800 + cid, 2), N, K)
    s = synth.gen_scales(synth.tensor_id(synth.KIND_SCALES, 800 + cid, 2), N, K // g)
    x = synth.gen_x(synth.tensor_id(synth.KIND_X, 800 + cid, 2, M), M, K)
    return x, q, s


# (M, N, K, g): each tile height (M <= 32, <= 64, larger), ragged rows,
# columns and k-tiles, one tile or many, K long enough that tiles are cut.
SHAPES = [(17, 272, 384, 128), (32, 512, 2048, 128), (33, 300, 640, 64), (64, 1040, 1536, 128),
          (65, 40, 96, 32), (100, 4112, 192, 64), (129, 520, 5120, 128), (200, 256, 17408, 128),
          (300, 72, 512, 32), (24, 16, 128, 128), (48, 2000, 3072, 64), (1000, 600, 1024, 128)]


@pytest.mark.parametrize("case", list(enumerate(SHAPES)), ids=lambda c: "x".join(map(str, c[1])))
def test_streamk_large_random_parity(case):
    cid, (M, N, K, g) = case
    log(f"stream-K large M={M} N={N} K={K} g={g}")
    x, q, s = _inputs(cid, M, N, K, g)
    prob = Problem(x, q, s, g)
    ws = workspace(M, 2 * N)
    a = run_streamk(prob, ws)
    ref = oracle.gemm(x, q, s, g, threads=synth.default_threads())
    r = max(tolerance_ratio(y, ref) for y in a)
    log(f"  tolerance ratio {r:.4f}")
    assert r <= 1.0
    b = run_streamk(prob, ws)
    assert all(np.array_equal(u, v) for u, v in zip(a, b))  # counters reset, fixed summation order


@pytest.mark.parametrize("shape", [(40, 272, 1024, 128), (130, 300, 384, 32), (70, 48, 4096, 64)],
                         ids=lambda s: "x".join(map(str, s)))
def test_streamk_large_unit_scale_exact(shape):
    M, N, K, g = shape
    x, q, s, expect = pins.unit_scale_case(M, N, K, g)
    for y in run_streamk(Problem(x, q, s, g)):
        assert np.array_equal(bf16_bits_to_f64(y), expect)


@pytest.mark.parametrize("kg", [(256, 64), (1024, 128), (128, 32)], ids=str)
def test_streamk_large_identity_exact(kg):
    """x = I (M = K rows), s = 1: y[m][n] = q[n][m] exactly through the cut tiles."""
    K, g = kg
    N = 48
    q = synth.gen_q(synth.tensor_id(synth.KIND_Q, 850, K), N, K)
    ys = run_streamk(Problem(pins.bf16_bits(np.eye(K)), q,
                             np.full((N, K // g), pins.FP16_ONE, np.uint16), g))
    for y in ys:
        assert np.array_equal(bf16_bits_to_f64(y), q.T.astype(np.float64))


@pytest.mark.parametrize("M", [20, 64, 128])
def test_streamk_large_grouped_problems(M):
    """Three problems of different shapes in one launch, twice on one workspace."""
    import torch
    import w4a16_weight_only_gemm_amd as w4
    shapes = [(520, 1024, 128), (48, 2048, 128), (1000, 384, 128)]
    data = [_inputs(30 + i, M, N, K, g) for i, (N, K, g) in enumerate(shapes)]
    probs = [Problem(x, q, s, 128) for (x, q, s) in data]
    ys = [torch.empty((M, p.N), dtype=torch.bfloat16, device="cuda") for p in probs]
    ws = workspace(M, sum(p.N for p in probs))
    entries = [(p.x, p.qw, p.sp, y, p.N, p.K) for p, y in zip(probs, ys)]
    first = None
    for rep in range(2):
        w4.w4a16_gemm_grouped(entries, M, 128, ws)
        torch.cuda.synchronize()
        outs = [y.view(torch.int16).cpu().numpy().view(np.uint16).copy() for y in ys]
        for (x, q, s), yb in zip(data, outs):
            assert tolerance_ratio(yb, oracle.gemm(x, q, s, 128, threads=synth.default_threads())) <= 1.0
        if first is None:
            first = outs
        else:
            assert all(np.array_equal(a, b) for a, b in zip(first, outs))


@pytest.mark.parametrize("layer", [0, 63])
@pytest.mark.parametrize("M", [64, 1024])
def test_streamk_large_layer_set_sampled(M, layer):
    """The four projections of a layer in one launch at full size: all rows of
    256 sampled columns of each (layers 0 and 63 of the 64-layer stack)."""
    import torch
    import w4a16_weight_only_gemm_amd as w4
    data = [synth.layer_inputs(layer, i, M) for i in range(4)]
    probs = [Problem(x, q, s, synth.GROUP) for (x, q, s) in data]
    ys = [torch.empty((M, p.N), dtype=torch.bfloat16, device="cuda") for p in probs]
    ws = workspace(M, sum(p.N for p in probs))
    w4.w4a16_gemm_grouped([(p.x, p.qw, p.sp, y, p.N, p.K) for p, y in zip(probs, ys)], M,
                          synth.GROUP, ws)
    torch.cuda.synchronize()
    for i, ((x, q, s), y, pj) in enumerate(zip(data, ys, synth.LAYER_PROJECTIONS)):
        cols = np.sort(np.random.default_rng(i * 5 + M + layer).choice(pj.N, 256, replace=False))
        cols[0], cols[-1] = 0, pj.N - 1
        yb = y.view(torch.int16).cpu().numpy().view(np.uint16)[:, cols]
        r = tolerance_ratio(yb, oracle.gemm(x, q[cols], s[cols], synth.GROUP,
                                            threads=synth.default_threads()))
        log(f"grouped M={M} {pj.name}: ratio {r:.4f}")
        assert r <= 1.0


def test_streamk_large_workspace_errors():
    import torch
    import w4a16_weight_only_gemm_amd as w4
    M, N, K, g = 40, 64, 256, 64
    x, q, s = _inputs(90, M, N, K, g)
    prob = Problem(x, q, s, g)
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    y2 = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    ws = workspace(M, 2 * N)
    # two problems: the stream-K schedule runs, so the workspace is checked
    e = [(prob.x, prob.qw, prob.sp, y, N, K), (prob.x, prob.qw, prob.sp, y2, N, K)]
    nb = w4.w4a16_workspace_bytes(M, 2 * N)
    assert w4.grouped_status(e, M, g, ws, nb - 4) == w4.W4A16_ERR_INVALID_ARG
    assert w4.grouped_status(e, M, g, None, nb) == w4.W4A16_ERR_INVALID_ARG
    big = workspace(M, 2 * N + 8192)
    assert w4.grouped_status(e, M, g, big.data_ptr() + 16, nb) == w4.W4A16_ERR_MISALIGNED
    assert w4.grouped_status(e, M, g, ws, nb) == w4.W4A16_OK
    torch.cuda.synchronize()
    yb = y.view(torch.int16).cpu().numpy().view(np.uint16)
    assert tolerance_ratio(yb, oracle.gemm(x, q, s, g)) <= 1.0


@pytest.mark.parametrize("M", [1, 16, 64])
def test_output_head_sampled(M):
    """The output-head shape (N = 248,320 rows of K = 5120) through the
    workspace entry point: all rows of 512 sampled columns, first and last
    included."""
    N, K, g = 248320, 5120, 128
    x, q, s = _inputs(70 + M, M, N, K, g)
    prob = Problem(x, q, s, g)
    y = run_ws(prob, workspace(M, N))
    cols = np.sort(np.random.default_rng(M).choice(N, 512, replace=False))
    cols[0], cols[-1] = 0, N - 1
    r = tolerance_ratio(y[:, cols], oracle.gemm(x, q[cols], s[cols], g, threads=synth.default_threads()))
    log(f"head M={M}: ratio {r:.4f}")
    assert r <= 1.0


def test_workspace_shared_by_every_kind_of_call():
    """One workspace, zero-filled once, serves a sequence of calls that use it
    in different layouts (MFMA stream-K at 64 and 1024 rows, the streaming
    kernel at 1 and 16 rows; each call holds its problem twice, so every one
    runs a stream-K schedule): each call leaves every byte at zero, so each
    result equals that of a call on a fresh workspace, bit for bit."""
    import torch

    import w4a16_weight_only_gemm_amd as w4
    from gpu_util import Problem
    N, K, g = 5120, 2048, 128
    need = max(w4.w4a16_workspace_bytes(M, 2 * N) for M in (1, 16, 64, 1024))
    ws = torch.zeros((need + 3) // 4, dtype=torch.int32, device="cuda")
    for i, M in enumerate((64, 1, 1024, 16, 1, 64)):
        q = synth.gen_q(synth.tensor_id(synth.KIND_Q, 990, i), N, K)
        s = synth.gen_scales(synth.tensor_id(synth.KIND_SCALES, 990, i), N, K // g)
        x = synth.gen_x(synth.tensor_id(synth.KIND_X, 990, i, M), M, K)
        prob = Problem(x, q, s, g)
        ys = run_streamk(prob, ws=ws)
        fresh = run_streamk(prob)
        assert all(np.array_equal(a, b) for a, b in zip(ys, fresh)), \
            f"call {i} (M={M}) differs on the shared workspace"
        torch.cuda.synchronize()
        assert int(torch.count_nonzero(ws)) == 0, f"call {i} (M={M}) left workspace bytes set"
