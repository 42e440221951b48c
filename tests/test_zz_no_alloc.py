"""w4a16_gemm_noalloc (the entry point for callers that cannot allocate) against
w4a16_gemm_ws, its workspace twin, through the C ABI: two calls in a row on the
shared static scratch, the second with a smaller input, each bit-identical to
the workspace call (same kernels, deterministic sums) and within the GEMM's
acceptance bound of the oracle on sampled columns; and the size limit."""
import sys

import numpy as np
import pytest

import oracle
import synth
from gpu_util import Problem, run_ws, tolerance_ratio

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


def _problem(case, M, N, K, g):
    q = synth.gen_q(synth.tensor_id(synth.KIND_Q, 700 + case, 0), N, K)
    s = synth.gen_scales(synth.tensor_id(synth.KIND_SCALES, 700 + case, 0), N, K // g)
    x = synth.gen_x(synth.tensor_id(synth.KIND_X, 700 + case, 0, M), M, K)
    return x, q, s, Problem(x, q, s, g)


def _noalloc(prob):
    import torch

    import w4a16_weight_only_gemm_amd as w4
    y = torch.empty((prob.M, prob.N), dtype=torch.bfloat16, device="cuda")
    w4.w4a16_gemm_noalloc(prob.x, prob.qw, prob.sp, y, prob.M, prob.N, prob.K, prob.group)
    torch.cuda.synchronize()
    return y.view(torch.int16).cpu().numpy().view(np.uint16)


def _check(case, M, N, K, g):
    log(f"noalloc case {case}: M={M} N={N} K={K} g={g}")
    x, q, s, prob = _problem(case, M, N, K, g)
    y = _noalloc(prob)
    y_ws = run_ws(prob)
    assert np.array_equal(y, y_ws), "differs from w4a16_gemm_ws"
    cols = np.sort(np.random.default_rng(case).choice(N, min(N, 48), replace=False))
    ref = oracle.gemm(x, q[cols], s[cols], g, threads=synth.default_threads())
    assert tolerance_ratio(y[:, cols], ref) <= 1.0


# (first call, second smaller call): both stream-K forms of the workspace path,
# and the single problems above 16 rows that run w4a16_gemm's kernels instead
PAIRS = [
    ((16, 7168, 5120, 128), (3, 1000, 1024, 128)),     # M <= 16 streaming kernel
    ((1, 34816, 5120, 128), (1, 520, 512, 64)),        # M = 1, activations staged in LDS
    ((1024, 48, 32768, 128), (64, 40, 65536, 128)),    # M > 16 MFMA stream-K (deep, narrow), twice
    ((64, 5120, 6144, 128), (20, 520, 512, 64)),       # M > 16, w4a16_gemm's kernels: no scratch used
    ((300, 72, 512, 256), (17, 40, 256, 256)),         # group 256 above 16 rows: no scratch used
]


@pytest.mark.parametrize("pair", PAIRS, ids=lambda p: "M%d_then_M%d" % (p[0][0], p[1][0]))
def test_noalloc_matches_workspace_call_twice(pair):
    first, second = pair
    case = 10 * PAIRS.index(pair)
    _check(case, *first)
    _check(case + 1, *second)


def test_noalloc_rejects_shapes_beyond_the_scratch():
    import w4a16_weight_only_gemm_amd as w4
    # M = 16 with two million columns needs about 128 MB of swap slots; the raw
    # addresses are never used, the call returns before any launch
    N = 2_000_000
    assert w4.w4a16_workspace_bytes(16, N) > w4.W4A16_NOALLOC_SCRATCH_BYTES
    assert w4.noalloc_status(256, 256, 256, 256, 16, N, 256, 64) == w4.W4A16_ERR_TOO_LARGE
    assert w4.noalloc_status(256, 256, 256, 256, 1, 64, 256, 48) == w4.W4A16_ERR_UNSUPPORTED
    assert w4.noalloc_status(256, 256, 256, 250, 1, 64, 256, 64) == w4.W4A16_ERR_MISALIGNED
    assert w4.noalloc_status(0, 256, 256, 256, 1, 64, 256, 64) == w4.W4A16_ERR_INVALID_ARG
    assert w4.noalloc_status(0, 0, 0, 0, 0, 64, 256, 64) == w4.W4A16_OK
