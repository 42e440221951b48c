"""GPU parity of the large-M kernel (forced path, and the automatic choice at
large M) against the CPU oracle, through the C ABI: shapes spanning several
128-row and 256-column tiles with ragged edges in M, N and K, every group
size, and closed-form cases that must come out exact."""
import sys

import numpy as np
import pytest

import oracle
import pins
import synth
from gpu_util import Problem, bf16_bits_to_f64, tolerance_ratio

pytestmark = pytest.mark.gpu

LARGE = 2


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
    q = synth.gen_q(synth.tensor_id(synth.KIND_Q, 400 + cid, 0), N, K)
    s = synth.gen_scales(synth.tensor_id(synth.KIND_SCALES, 400 + cid, 0), N, K // g)
    x = synth.gen_x(synth.tensor_id(synth.KIND_X, 400 + cid, 0, M), M, K)
    return x, q, s


# (M, N, K, g): several row and column tiles, ragged in every dimension; K not
# a multiple of the 128-wide k-tile for groups 32 and 64.
SHAPES = [(129, 272, 384, 128), (256, 512, 1152, 128), (130, 257, 160, 32), (200, 40, 96, 32),
          (300, 4112, 192, 64), (1024, 1040, 2048, 128), (513, 300, 640, 64), (128, 256, 128, 128),
          (65, 16, 32, 32), (384, 768, 4096, 128), (97, 1000, 1344, 64), (260, 600, 1024, 256)]


@pytest.mark.parametrize("case", list(enumerate(SHAPES)), ids=lambda c: "x".join(map(str, c[1])))
def test_large_random_parity(case):
    cid, (M, N, K, g) = case
    log(f"large random M={M} N={N} K={K} g={g}")
    x, q, s = _inputs(cid, M, N, K, g)
    y = Problem(x, q, s, g).run(LARGE)
    r = tolerance_ratio(y, oracle.gemm(x, q, s, g, threads=synth.default_threads()))
    log(f"  tolerance ratio {r:.4f}")
    assert r <= 1.0


@pytest.mark.parametrize("shape", [(130, 272, 512, 128), (256, 300, 384, 32), (200, 48, 1024, 64)],
                         ids=lambda s: "x".join(map(str, s)))
def test_large_unit_scale_exact(shape):
    M, N, K, g = shape
    log(f"large unit-scale {shape}")
    x, q, s, expect = pins.unit_scale_case(M, N, K, g)
    assert np.array_equal(bf16_bits_to_f64(Problem(x, q, s, g).run(LARGE)), expect)


@pytest.mark.parametrize("g", [32, 64, 128])
def test_large_group_index_exact(g):
    """s[n][j] = j + 1, q = 1, x = 1: y = g * G (G + 1) / 2 -- every group's
    scale applied to its own k range, including the groups of a ragged last
    k-tile."""
    M, N, K = 140, 272, 11 * g
    G = K // g
    s = pins.fp16_bits(np.tile(1.0 + np.arange(G), (N, 1)))
    x = np.full((M, K), pins.BF16_ONE, np.uint16)
    y = Problem(x, np.ones((N, K), np.int8), s, g).run(LARGE)
    assert np.all(bf16_bits_to_f64(y) == g * G * (G + 1) / 2.0)


def test_large_row_sums_are_per_row_and_group():
    """One-hot rows: row m of x is 1 at k = m only, so its group's bias sum is 1
    and every other group's is 0; y[m][n] = q[n][m] exactly (s = 1)."""
    M, N, K, g = 256, 64, 256, 32
    q = synth.gen_q(synth.tensor_id(synth.KIND_Q, 450, 0), N, K)
    x = pins.bf16_bits(np.eye(M, K))
    y = Problem(x, q, np.full((N, K // g), pins.FP16_ONE, np.uint16), g).run(LARGE)
    assert np.array_equal(bf16_bits_to_f64(y), q.T[:M].astype(np.float64))


def test_large_deterministic_and_auto_choice():
    import w4a16_weight_only_gemm_amd as w4
    M, N, K, g = 512, 4096, 1024, 128   # 16 column tiles: the tile engine's shape
    assert w4.w4a16_select_path(M, N, K, g) == LARGE
    x, q, s = _inputs(90, M, N, K, g)
    prob = Problem(x, q, s, g)
    a, b, c = prob.run(LARGE), prob.run(LARGE), prob.run(0)
    assert np.array_equal(a, b) and np.array_equal(a, c)
