"""GPU parity of every kernel form w4a16_gemm can run, through the C ABI.

w4a16_gemm picks a form per shape from time models of its kernels (the
library's own choice; w4a16_select_form reports it): up to 16 rows the small-M
forms of the plain kernel (16 to 64 columns per workgroup of 4, 8 or 16 waves,
rows in LDS at one or two rows; from 9 rows at group 128 the forms below); from 17
rows either a plain-kernel form (16, 32 or 64 rows by 32 to 80 columns per
workgroup; at group 128 the activation fragments pass through a wave-private
LDS area) or the whole-K tile engine
(32, 64 or 128 rows by 256 columns; at 32 and 64 rows loads run three
k-tiles ahead). Each case below is a shape for which the automatic choice is
one given form (asserted first, on the host), ragged in M and N, with several
workgroups along N; the result is checked against the oracle,
|y - y_ref| <= 1e-2 (1 + |y_ref|): every output, or, above 24 rows where the
oracle would take long, 24 sampled rows (the first, the last, 22 at random). Forced paths cover
the tile engine at 1 and 16 rows and the plain kernel at several hundred."""
import sys

import numpy as np
import pytest

import oracle
import synth
from gpu_util import Problem, tolerance_ratio

pytestmark = pytest.mark.gpu

AUTO, SKINNY, LARGE = 0, 1, 2

# ((M, N, K, group), expected (path, rows, cols, waves))
FORM_CASES = [
    ((1, 3000, 4096, 128), (1, 16, 16, 16)),    # one row in LDS, one column block per workgroup
    ((5, 900, 2048, 128), (1, 16, 16, 16)),     # few column blocks: one per 16-wave workgroup
    ((3, 1000, 1024, 32), (1, 16, 16, 16)),
    ((1, 3000, 2048, 64), (1, 16, 16, 16)),
    ((2, 500, 2048, 256), (1, 16, 16, 16)),
    ((3, 17000, 512, 128), (1, 16, 48, 4)),     # wide N: 4-wave workgroups, fragments through LDS
    ((7, 17000, 512, 128), (1, 16, 80, 4)),
    ((5, 5000, 768, 128), (1, 16, 32, 8)),      # short K
    ((2, 17000, 512, 64), (1, 16, 32, 4)),      # wide N at group 64: rows in LDS, then operand order
    ((7, 17000, 512, 64), (1, 16, 64, 4)),
    ((7, 3000, 2048, 128), (1, 16, 32, 8)),     # two groups in flight at 7-12 rows
    ((9, 2000, 4096, 128), (1, 16, 32, 8)),
    ((11, 2000, 4096, 128), (1, 16, 32, 8)),
    ((13, 17000, 1024, 128), (1, 16, 80, 4)),
    ((16, 9000, 8192, 128), (1, 16, 64, 8)),
    ((11, 300, 128, 128), (1, 32, 32, 16)),     # 32-row forms below 17 rows: a padding row block
    ((15, 9000, 1152, 128), (1, 32, 48, 16)),
    ((17, 100, 4096, 128), (1, 16, 32, 8)),
    ((17, 5000, 8192, 128), (1, 16, 64, 8)),
    ((17, 9000, 8192, 128), (1, 16, 80, 8)),
    ((17, 100, 256, 128), (1, 32, 32, 16)),
    ((17, 9000, 256, 128), (1, 32, 48, 16)),
    ((37, 7001, 256, 128), (1, 32, 64, 16)),
    ((17, 17000, 1024, 128), (1, 32, 80, 4)),
    ((33, 9000, 2048, 128), (1, 32, 80, 8)),
    ((37, 9000, 256, 128), (1, 64, 64, 16)),
    ((17, 17000, 256, 128), (2, 32, 256, 8)),
    ((37, 35001, 256, 128), (2, 64, 256, 8)),
    ((517, 12001, 256, 128), (2, 128, 256, 8)),
    ((17, 100, 512, 64), (1, 32, 32, 4)),
    ((17, 17000, 2048, 64), (1, 32, 64, 4)),
    ((37, 100, 512, 64), (1, 64, 32, 4)),
    ((17, 520, 256, 64), (2, 32, 256, 8)),
    ((37, 35001, 256, 64), (2, 64, 256, 8)),
    ((517, 12001, 256, 64), (2, 128, 256, 8)),
    ((17, 100, 512, 32), (1, 32, 32, 4)),
    ((37, 100, 512, 32), (1, 64, 32, 4)),
    ((17, 520, 256, 32), (2, 32, 256, 8)),
    ((37, 35001, 256, 32), (2, 64, 256, 8)),
    ((17, 17000, 256, 256), (1, 32, 64, 4)),
    ((37, 100, 256, 256), (1, 64, 32, 4)),
    ((37, 17000, 256, 256), (1, 64, 64, 4)),
]

# ((M, N, K, group), forced path, expected form)
FORCED_CASES = [
    ((1, 1000, 1024, 128), LARGE, (2, 32, 256, 8)),
    ((16, 700, 512, 64), LARGE, (2, 32, 256, 8)),
    ((700, 300, 512, 128), SKINNY, None),
    ((517, 300, 512, 32), SKINNY, None),
]

SAMPLE_ABOVE = 2e8  # multiply-adds above which the oracle computes sampled rows only


def log(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible to torch")
    import w4a16_weight_only_gemm_amd  # noqa: F401  (fails loudly if the library is missing)
    yield


def _check(cid, M, N, K, g, path):
    q = synth.gen_q(synth.tensor_id(synth.KIND_Q, 700 + cid, 0), N, K)
    s = synth.gen_scales(synth.tensor_id(synth.KIND_SCALES, 700 + cid, 0), N, K // g)
    x = synth.gen_x(synth.tensor_id(synth.KIND_X, 700 + cid, 0, M), M, K)
    y = Problem(x, q, s, g).run(path)
    if M * N * K > SAMPLE_ABOVE and M > 24:
        rng = np.random.default_rng(cid)
        rows = np.unique(np.concatenate([[0, M - 1], rng.choice(M, 22, replace=False)]))
    else:
        rows = np.arange(M)
    ref = oracle.gemm(x[rows], q, s, g, threads=synth.default_threads())
    r = tolerance_ratio(y[rows], ref)
    log(f"  {len(rows)} rows checked, tolerance ratio {r:.4f}")
    assert r <= 1.0


@pytest.mark.parametrize("case", list(enumerate(FORM_CASES)),
                         ids=lambda c: "x".join(map(str, c[1][0])))
def test_auto_form_parity(case):
    import w4a16_weight_only_gemm_amd as w4
    cid, ((M, N, K, g), form) = case
    got = w4.w4a16_select_form(M, N, K, g)
    log(f"form case M={M} N={N} K={K} g={g}: form {got}")
    assert got == form
    _check(cid, M, N, K, g, AUTO)


@pytest.mark.parametrize("case", list(enumerate(FORCED_CASES)),
                         ids=lambda c: f"{'x'.join(map(str, c[1][0]))}-path{c[1][1]}")
def test_forced_form_parity(case):
    import w4a16_weight_only_gemm_amd as w4
    cid, ((M, N, K, g), path, form) = case
    got = w4.w4a16_select_form(M, N, K, g, path)
    log(f"forced case M={M} N={N} K={K} g={g} path={path}: form {got}")
    assert got[0] == path
    if form is not None:
        assert got == form
    _check(100 + cid, M, N, K, g, path)


# single problems on the workspace entry point: (M, N, K, group), whether the
# time models route them to w4a16_gemm's kernels
WS_SINGLE = [((64, 5120, 6144, 128), True), ((17, 272, 384, 128), True),
             ((64, 40, 65536, 128), False), ((500, 40, 16384, 128), False)]


@pytest.mark.parametrize("case", list(enumerate(WS_SINGLE)),
                         ids=lambda c: "x".join(map(str, c[1][0])))
def test_workspace_call_of_one_problem(case):
    """w4a16_gemm_ws with one problem above 16 rows: where the models put
    w4a16_gemm's kernels ahead it returns w4a16_gemm's result bit for bit and
    leaves the workspace untouched; either way the result is within the
    tolerance of the oracle (48 sampled columns)."""
    import torch

    from gpu_util import run_ws, workspace
    cid, ((M, N, K, g), whole) = case
    log(f"workspace call of one problem M={M} N={N} K={K} g={g}")
    q = synth.gen_q(synth.tensor_id(synth.KIND_Q, 760 + cid, 0), N, K)
    s = synth.gen_scales(synth.tensor_id(synth.KIND_SCALES, 760 + cid, 0), N, K // g)
    x = synth.gen_x(synth.tensor_id(synth.KIND_X, 760 + cid, 0, M), M, K)
    prob = Problem(x, q, s, g)
    ws = workspace(M, N)
    y = run_ws(prob, ws)
    assert int(torch.count_nonzero(ws)) == 0
    if whole:
        assert np.array_equal(y, prob.run(AUTO))
    cols = np.sort(np.random.default_rng(cid).choice(N, min(N, 48), replace=False))
    ref = oracle.gemm(x, q[cols], s[cols], g, threads=synth.default_threads())
    assert tolerance_ratio(y[:, cols], ref) <= 1.0
