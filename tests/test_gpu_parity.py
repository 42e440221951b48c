"""GPU parity of the HIP path against the CPU oracle, through the C ABI.

Acceptance: |y - y_ref| <= 1e-2 * (1 + |y_ref|) element by element (y decoded
from bf16, y_ref the oracle's fp64), on the seeded inputs; bit-exact results
where the exact answer is a small integer (unit scales, group-index sums,
identity activation), which pins the operand layouts of each kernel path.
"""
import sys

import numpy as np
import pytest

import oracle
import pins
import synth
from gpu_util import Problem, bf16_bits_to_f64, dev_u16, dev_u32, tolerance_ratio

pytestmark = pytest.mark.gpu

PATHS = [0, 1, 2]  # auto, skinny, large
PATH_IDS = ["auto", "skinny", "large"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible to torch")
    import w4a16_weight_only_gemm_amd  # noqa: F401  (fails loudly if the library is missing)
    yield


def _random_inputs(case_id, M, N, K, g):
    q = synth.gen_q(synth.tensor_id(synth.KIND_Q, 200 + case_id, 0), N, K)
    s = synth.gen_scales(synth.tensor_id(synth.KIND_SCALES, 200 + case_id, 0), N, K // g)
    x = synth.gen_x(synth.tensor_id(synth.KIND_X, 200 + case_id, 0, M), M, K)
    return x, q, s


@pytest.mark.parametrize("path", PATHS, ids=PATH_IDS)
def test_tiny_gemv(path):
    x, q, s = synth.tiny_inputs()
    t = synth.TINY
    log(f"tiny M={t['M']} K={t['K']} N={t['N']} g={t['group']} path={path}")
    y = Problem(x, q, s, t["group"]).run(path)
    ref = oracle.gemm(x, q, s, t["group"], threads=synth.default_threads())
    assert tolerance_ratio(y, ref) <= 1.0


UNIT_SHAPES = [(1, 512, 256, 64), (5, 48, 256, 64), (16, 64, 1024, 128), (37, 80, 5120, 128),
               (64, 32, 512, 32), (130, 96, 2048, 256)]


@pytest.mark.parametrize("path", PATHS, ids=PATH_IDS)
@pytest.mark.parametrize("shape", UNIT_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_unit_scale_bit_exact(path, shape):
    M, N, K, g = shape
    log(f"unit-scale {shape} path={path}")
    x, q, s, expect = pins.unit_scale_case(M, N, K, g)
    y = Problem(x, q, s, g).run(path)
    assert np.array_equal(bf16_bits_to_f64(y), expect)


@pytest.mark.parametrize("path", PATHS, ids=PATH_IDS)
@pytest.mark.parametrize("shape", [(1, 512, 256, 64), (3, 40, 1024, 128), (20, 16, 512, 32),
                                   (70, 24, 2048, 256)], ids=lambda s: "x".join(map(str, s)))
def test_group_index_bit_exact(path, shape):
    M, N, K, g = shape
    G = K // g
    log(f"group-index {shape} path={path}")
    s = pins.fp16_bits(np.tile(1.0 + np.arange(G), (N, 1)))
    x = np.full((M, K), pins.BF16_ONE, np.uint16)
    y = Problem(x, np.ones((N, K), np.int8), s, g).run(path)
    assert np.all(bf16_bits_to_f64(y) == g * G * (G + 1) / 2.0)


@pytest.mark.parametrize("path", PATHS, ids=PATH_IDS)
@pytest.mark.parametrize("kg", [(256, 64), (512, 128), (128, 32), (256, 256)], ids=str)
def test_identity_activation_recovers_codes(path, kg):
    """x = I (M = K), s = 1: y[m][n] = q[n][m] exactly -- every code through every lane."""
    K, g = kg
    N = 48
    q = synth.gen_q(synth.tensor_id(synth.KIND_Q, 300, K), N, K)
    log(f"identity K={K} g={g} path={path}")
    y = Problem(pins.bf16_bits(np.eye(K)), q, np.full((N, K // g), pins.FP16_ONE, np.uint16),
                g).run(path)
    assert np.array_equal(bf16_bits_to_f64(y), q.T.astype(np.float64))


RAGGED = [(1, 16, 128, 32), (1, 200, 384, 64), (2, 520, 1024, 128), (7, 33, 512, 128),
          (15, 64, 768, 256), (16, 1000, 640, 128), (17, 112, 1024, 64), (31, 48, 2048, 128),
          (33, 80, 1536, 128), (63, 64, 384, 128), (64, 256, 1024, 128), (65, 130, 768, 64),
          (100, 300, 1280, 128), (256, 160, 2048, 128), (300, 72, 512, 256)]


@pytest.mark.parametrize("path", PATHS, ids=PATH_IDS)
@pytest.mark.parametrize("case", list(enumerate(RAGGED)), ids=lambda c: "x".join(map(str, c[1])))
def test_ragged_shapes(path, case):
    cid, (M, N, K, g) = case
    log(f"ragged {(M, N, K, g)} path={path}")
    x, q, s = _random_inputs(cid, M, N, K, g)
    y = Problem(x, q, s, g).run(path)
    ref = oracle.gemm(x, q, s, g, threads=synth.default_threads())
    assert tolerance_ratio(y, ref) <= 1.0


@pytest.mark.parametrize("M", [1, 16])
@pytest.mark.parametrize("proj", range(4), ids=[p.name for p in synth.LAYER_PROJECTIONS])
def test_layer_set_full(M, proj):
    """The decode and verify layer sets at full size, every output checked."""
    p = synth.LAYER_PROJECTIONS[proj]
    log(f"layer-set full M={M} {p.name} K={p.K} N={p.N}")
    x, q, s = synth.layer_inputs(0, proj, M)
    y = Problem(x, q, s, synth.GROUP).run(0)
    ref = oracle.gemm(x, q, s, synth.GROUP, threads=synth.default_threads())
    r = tolerance_ratio(y, ref)
    log(f"  tolerance ratio {r:.4f}")
    assert r <= 1.0


@pytest.mark.parametrize("M", [64, 1024])
@pytest.mark.parametrize("proj", range(4), ids=[p.name for p in synth.LAYER_PROJECTIONS])
def test_layer_set_sampled(M, proj):
    """The batched layer sets at full size: all rows of 384 sampled columns."""
    p = synth.LAYER_PROJECTIONS[proj]
    log(f"layer-set sampled M={M} {p.name} K={p.K} N={p.N}")
    x, q, s = synth.layer_inputs(0, proj, M)
    y = Problem(x, q, s, synth.GROUP).run(0)
    cols = np.sort(np.random.default_rng(proj * 7 + M).choice(p.N, 384, replace=False))
    cols[0], cols[-1] = 0, p.N - 1
    ref = oracle.gemm(x, q[cols], s[cols], synth.GROUP, threads=synth.default_threads())
    r = tolerance_ratio(y[:, cols], ref)
    log(f"  tolerance ratio {r:.4f}")
    assert r <= 1.0


@pytest.mark.parametrize("path", PATHS, ids=PATH_IDS)
def test_deterministic(path):
    x, q, s = _random_inputs(50, 24, 512, 2048, 128)
    prob = Problem(x, q, s, 128)
    a = prob.run(path)
    b = prob.run(path)
    assert np.array_equal(a, b)


@pytest.mark.parametrize("path", PATHS, ids=PATH_IDS)
def test_output_guard_bands_untouched(path):
    import torch
    M, N, K, g = 19, 200, 1024, 128
    x, q, s = _random_inputs(51, M, N, K, g)
    prob = Problem(x, q, s, g)
    pad = 4096
    buf = torch.full((pad + M * N + pad,), 0x7E5A, dtype=torch.int16, device="cuda")
    y = buf[pad:pad + M * N].view(torch.bfloat16)
    yb = prob.run(path, y=y)
    host = buf.cpu().numpy().view(np.uint16)
    assert (host[:pad] == 0x7E5A).all() and (host[pad + M * N:] == 0x7E5A).all()
    ref = oracle.gemm(x, q, s, g)
    assert tolerance_ratio(yb.reshape(-1)[:M * N].reshape(M, N), ref) <= 1.0


def test_m_zero_is_a_noop():
    import torch
    import w4a16_weight_only_gemm_amd as w4
    y = torch.full((4, 64), 3.0, dtype=torch.bfloat16, device="cuda")
    x = torch.zeros((4, 256), dtype=torch.bfloat16, device="cuda")
    qw = torch.zeros((64, 32), dtype=torch.int32, device="cuda")
    sp = torch.zeros((4, 64), dtype=torch.int16, device="cuda")
    w4.w4a16_gemm(x, qw, sp, y, 0, 64, 256, 64)
    torch.cuda.synchronize()
    assert (y == 3.0).all()


def test_error_leaves_no_state_and_nondefault_stream():
    import torch
    import w4a16_weight_only_gemm_amd as w4
    M, N, K, g = 9, 96, 512, 128
    x, q, s = _random_inputs(52, M, N, K, g)
    prob = Problem(x, q, s, g)
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    # misaligned y, unsupported group: rejected on the host
    assert w4.gemm_status(prob.x, prob.qw, prob.sp, y.data_ptr() + 2, M, N, K, g) == \
        w4.W4A16_ERR_MISALIGNED
    assert w4.gemm_status(prob.x, prob.qw, prob.sp, y, M, N, K, 96) == w4.W4A16_ERR_UNSUPPORTED
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        w4.w4a16_gemm(prob.x, prob.qw, prob.sp, y, M, N, K, g, stream=stream)
    stream.synchronize()
    yb = y.view(torch.int16).cpu().numpy().view(np.uint16)
    assert tolerance_ratio(yb, oracle.gemm(x, q, s, g)) <= 1.0


def test_empty_n_tail_and_single_column():
    M, N, K, g = 3, 1, 256, 64
    x, q, s = _random_inputs(53, M, N, K, g)
    for path in PATHS:
        y = Problem(x, q, s, g).run(path)
        assert tolerance_ratio(y, oracle.gemm(x, q, s, g)) <= 1.0


# Every kernel instantiation: group sizes 32..256 against row-block counts
# 1 (M = 3 and 12, the two one-row-block split-K shapes), 2 and 4 (M = 24, 50)
# and two row tiles (M = 90), at K = 8 and 20 groups.
MATRIX = [(M, g, kg) for g in (32, 64, 128, 256) for M in (3, 12, 24, 50, 90) for kg in (8, 20)]


@pytest.mark.parametrize("path", PATHS, ids=PATH_IDS)
@pytest.mark.parametrize("case", list(enumerate(MATRIX)), ids=lambda c: "M%d-g%d-G%d" % c[1])
def test_instantiation_matrix(path, case):
    cid, (M, g, kg) = case
    N, K = 80, kg * g
    log(f"matrix M={M} N={N} K={K} g={g} path={path}")
    x, q, s = _random_inputs(100 + cid, M, N, K, g)
    y = Problem(x, q, s, g).run(path)
    assert tolerance_ratio(y, oracle.gemm(x, q, s, g)) <= 1.0


# Activations of standard deviation 1000 against codes that are zero over whole
# groups: the exact sums of those groups are 0, while the kernels' biased
# dequantization adds and removes 24 * (row sum) in fp32 around them, an error
# that grows with |x|, not |y|. Columns 0..15 are zero over all of K (y = 0
# exactly, where the bound is tightest), columns 16..31 zero in every other
# group, the rest random. The two cases of 16,400 columns run w4a16_gemm's
# 4-wave forms for wide N.
WIDE = [(1, 64, 17408, 128), (3, 48, 5120, 128), (16, 64, 6144, 64), (20, 48, 2048, 32),
        (70, 80, 17408, 128), (200, 64, 4096, 128), (4, 16400, 1024, 128), (20, 16400, 1024, 128)]


def _wide_inputs(case, M, N, K, g):
    q = synth.gen_q(synth.tensor_id(synth.KIND_Q, 900 + case, 0), N, K)
    q[:16] = 0
    for t in range(0, K // g, 2):
        q[16:32, t * g:(t + 1) * g] = 0
    s = synth.gen_scales(synth.tensor_id(synth.KIND_SCALES, 900 + case, 0), N, K // g)
    x = synth.gen_x(synth.tensor_id(synth.KIND_X, 900 + case, 0, M), M, K, sigma=1000.0)
    return x, q, s


@pytest.mark.parametrize("path", PATHS + ["ws", "noalloc"], ids=PATH_IDS + ["ws", "noalloc"])
@pytest.mark.parametrize("case", list(enumerate(WIDE)), ids=lambda c: "x".join(map(str, c[1])))
def test_wide_range_activations(path, case):
    from gpu_util import run_ws
    cid, (M, N, K, g) = case
    log(f"wide-range x (sigma 1000) {(M, N, K, g)} path={path}")
    x, q, s = _wide_inputs(cid, M, N, K, g)
    prob = Problem(x, q, s, g)
    if path == "ws":
        y = run_ws(prob)
    elif path == "noalloc":
        import torch

        import w4a16_weight_only_gemm_amd as w4
        yt = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        w4.w4a16_gemm_noalloc(prob.x, prob.qw, prob.sp, yt, M, N, K, g)
        torch.cuda.synchronize()
        y = yt.view(torch.int16).cpu().numpy().view(np.uint16)
    else:
        y = prob.run(path)
    ref = oracle.gemm(x, q, s, g, threads=synth.default_threads())
    assert np.all(ref[:, :16] == 0.0)
    r_zero = tolerance_ratio(y[:, :16], ref[:, :16])
    r = tolerance_ratio(y, ref)
    log(f"  ratio {r:.3f} (all-zero columns {r_zero:.3f})")
    assert r <= 1.0
