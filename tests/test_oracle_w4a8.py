"""The W4A8 half of the CPU oracle (int8 activations with one scale per row,
int4 weights) pinned to things other than itself: quantization closed forms
(exact grid values, ties to even, zero rows, power-of-two scaling), the
quantization error bound, brute force in Python integers, exact agreement
with the W4A16 oracle when the activations already sit on the int8 grid, the
W4A16-to-W4A8 difference within the propagated quantization bound, and the
device arrangement of the quantized activations. Planted mistakes (wrappers
around the oracle, on the CPU) fail the pins."""
from fractions import Fraction

import numpy as np
import pytest

import oracle
import pins


# ------------------------------------------------------------ quantization

def pin_quantize_grid_and_ties(quantize):
    """Row maximum 127 (exact in bf16): inv = 1, so each code is the value
    rounded to the nearest integer with ties to even, and sx = 1."""
    vals = [127.0, -127.0, 0.5, 1.5, 2.5, -0.5, -1.5, 3.0, 0.0, 126.5, -2.5, 64.0]
    xq, sx = quantize(pins.bf16_bits([vals]))
    assert np.array_equal(xq[0], [127, -127, 0, 2, 2, 0, -2, 3, 0, 126, -2, 64])
    assert sx[0] == np.float32(1.0)


def pin_quantize_zero_and_scaling(quantize):
    """A zero row gives zero codes and scale 0; multiplying a row by a power
    of two leaves its codes unchanged and multiplies its scale by it."""
    rng = np.random.default_rng(11)
    xf = rng.standard_normal((3, 96)).astype(np.float32)
    xb = (xf.view(np.uint32) >> 16).astype(np.uint16)
    xb[1] = 0
    xq, sx = quantize(xb)
    assert not xq[1].any() and sx[1] == 0
    for p in (2.0, 0.25, 1024.0):
        x2 = pins.bf16_bits(pins.bf16_to_f64(xb) * p)
        xq2, sx2 = quantize(x2)
        assert np.array_equal(xq2, xq)
        assert np.array_equal(sx2.astype(np.float64), sx.astype(np.float64) * p)


def pin_quantize_bounds(quantize):
    """Codes lie in [-127, 127], the row maximum maps to +-127, and every
    value is within 0.5 * sx of its code times sx, plus three binary32
    roundings (of inv, of x * inv and of sx) relative to |x| <= 127 sx."""
    rng = np.random.default_rng(12)
    xf = (rng.standard_normal((8, 512)) * rng.uniform(0.01, 100, size=(8, 1))).astype(np.float32)
    xb = (xf.view(np.uint32) >> 16).astype(np.uint16)
    xq, sx = quantize(xb)
    xv = pins.bf16_to_f64(xb)
    assert np.abs(xq.astype(int)).max() <= 127
    for m in range(8):
        i = np.argmax(np.abs(xv[m]))
        assert abs(int(xq[m, i])) == 127 and np.sign(xq[m, i]) == np.sign(xv[m, i])
        err = np.abs(xv[m] - xq[m].astype(np.float64) * float(sx[m]))
        assert err.max() <= float(sx[m]) * (0.5 + 127 * 3 * 2.0**-24), m


QUANT_PINS = [pin_quantize_grid_and_ties, pin_quantize_zero_and_scaling, pin_quantize_bounds]


@pytest.mark.parametrize("pin", QUANT_PINS, ids=lambda f: f.__name__)
def test_oracle_quantize_pins(pin):
    pin(oracle.quantize_rows)


def _quantize_truncating(x):
    """Planted mistake: truncation instead of rounding to nearest."""
    xq, sx = oracle.quantize_rows(x)
    xv = pins.bf16_to_f64(x)
    out = np.where(sx[:, None] > 0, np.trunc(xv / np.where(sx > 0, sx, 1)[:, None]), 0)
    return np.clip(out, -127, 127).astype(np.int8), sx


def _quantize_half_up(x):
    """Planted mistake: ties rounded away from zero."""
    xq, sx = oracle.quantize_rows(x)
    xv = pins.bf16_to_f64(x).astype(np.float32)
    a = np.abs(xv).max(axis=1)
    inv = np.where(a > 0, np.float32(127) / np.where(a > 0, a, 1), 0).astype(np.float32)
    t = (xv * inv[:, None]).astype(np.float32)
    return np.clip(np.sign(t) * np.floor(np.abs(t) + 0.5), -127, 127).astype(np.int8), sx


def _quantize_scale_255(x):
    """Planted mistake: scale from 255 levels instead of 127."""
    xq, sx = oracle.quantize_rows(x)
    return xq, (sx * np.float32(127.0 / 255.0)).astype(np.float32)


@pytest.mark.parametrize("bad", [_quantize_truncating, _quantize_half_up, _quantize_scale_255],
                         ids=lambda f: f.__name__)
def test_quantize_pins_catch_planted_mistakes(bad):
    failed = 0
    for pin in QUANT_PINS:
        try:
            pin(bad)
        except AssertionError:
            failed += 1
    assert failed >= 1


# -------------------------------------------------------------------- GEMM

def _exact_w4a8(xq, sx, q, s_bits, g):
    """Exact rational y (Python integers and Fractions), from the definition."""
    M, K = xq.shape
    N = q.shape[0]
    sv = pins.fp16_to_f64(s_bits)
    out = [[Fraction(0)] * N for _ in range(M)]
    for m in range(M):
        for n in range(N):
            tot = Fraction(0)
            for t in range(K // g):
                acc = sum(int(xq[m, k]) * int(q[n, k]) for k in range(t * g, (t + 1) * g))
                tot += Fraction(float(sv[n, t])) * acc
            out[m][n] = Fraction(float(sx[m])) * tot
    return out


def pin_w4a8_bruteforce(gemm8):
    rng = np.random.default_rng(13)
    for (M, N, K, g) in [(1, 3, 64, 64), (2, 5, 128, 64), (3, 4, 256, 128), (2, 7, 128, 32)]:
        xq = rng.integers(-127, 128, size=(M, K)).astype(np.int8)
        sx = rng.uniform(0.001, 0.1, size=M).astype(np.float32)
        q = rng.integers(-8, 8, size=(N, K)).astype(np.int8)
        s = rng.uniform(0.005, 0.02, size=(N, K // g)).astype(np.float16).view(np.uint16)
        y = gemm8(xq, sx, q, s, g)
        ex = _exact_w4a8(xq, sx, q, s, g)
        for m in range(M):
            for n in range(N):
                mag = abs(float(ex[m][n])) + float(sx[m]) * 127 * 8 * 0.02 * K
                assert abs(Fraction(float(y[m, n])) - ex[m][n]) <= Fraction(mag * 2.0**-50), (m, n)


def pin_w4a8_grid_equals_w4a16(gemm8):
    """Activations already on the int8 grid of their row (row maximum
    127 * 2^-e, every value a multiple of 2^-e): quantization is exact, and
    the W4A8 product equals the W4A16 oracle's bit for bit."""
    rng = np.random.default_rng(14)
    M, N, K, g = 4, 24, 512, 128
    codes = rng.integers(-127, 128, size=(M, K))
    codes[:, 0] = 127
    e = np.array([0, 3, 6, 9])
    x = pins.bf16_bits(codes * 2.0 ** (-e[:, None]))
    q = rng.integers(-8, 8, size=(N, K)).astype(np.int8)
    s = rng.uniform(0.005, 0.02, size=(N, K // g)).astype(np.float16).view(np.uint16)
    xq, sx = oracle.quantize_rows(x)
    assert np.array_equal(xq.astype(int), codes)
    assert np.array_equal(gemm8(xq, sx, q, s, g), oracle.gemm(x, q, s, g))


def pin_w4a8_quantization_bound(gemm8):
    """Against the W4A16 product of the unquantized activations: the
    difference is at most sum_k |w[n][k]| * |x[m][k] - xq[m][k] * sx[m]|
    (plus double rounding)."""
    rng = np.random.default_rng(15)
    for (M, N, K, g) in [(3, 16, 256, 64), (2, 40, 1024, 128)]:
        x, q, s = pins.random_case(rng, M, N, K, g)
        xq, sx = oracle.quantize_rows(x)
        y8 = gemm8(xq, sx, q, s, g)
        y16 = oracle.gemm(x, q, s, g)
        w = np.abs(q.astype(np.float64) * np.repeat(pins.fp16_to_f64(s), g, axis=1))   # [N, K]
        dx = np.abs(pins.bf16_to_f64(x) - xq.astype(np.float64) * sx.astype(np.float64)[:, None])
        bound = dx @ w.T
        assert np.all(np.abs(y8 - y16) <= bound * (1 + 1e-9) + 1e-12)
        # and the quantization matters: the two products do differ
        assert np.abs(y8 - y16).max() > 0


GEMM8_PINS = [pin_w4a8_bruteforce, pin_w4a8_grid_equals_w4a16, pin_w4a8_quantization_bound]


@pytest.mark.parametrize("pin", GEMM8_PINS, ids=lambda f: f.__name__)
def test_oracle_w4a8_pins(pin):
    pin(oracle.gemm_w4a8)


def _w4a8_no_row_scale(xq, sx, q, s, g):
    """Planted mistake: the row scale left out."""
    return oracle.gemm_w4a8(xq, np.ones_like(sx), q, s, g)


def _w4a8_group_shift(xq, sx, q, s, g):
    """Planted mistake: group t scaled by the scale of group t + 1."""
    return oracle.gemm_w4a8(xq, sx, q, np.roll(s, -1, axis=1), g)


def _w4a8_sign(xq, sx, q, s, g):
    """Planted mistake: a sign flip of the codes' top value (-8 read as +8)."""
    y = oracle.gemm_w4a8(xq, sx, q, s, g)
    extra = oracle.gemm_w4a8(xq, sx, (q == -8).astype(np.int8) * 16, s, g)
    return y + extra


def _w4a8_dropped_term(xq, sx, q, s, g):
    """Planted mistake: the last k of every group left out."""
    q2 = q.copy()
    q2[:, g - 1::g] = 0
    return oracle.gemm_w4a8(xq, sx, q2, s, g)


@pytest.mark.parametrize("bad", [_w4a8_no_row_scale, _w4a8_group_shift, _w4a8_sign, _w4a8_dropped_term],
                         ids=lambda f: f.__name__)
def test_w4a8_pins_catch_planted_mistakes(bad):
    failed = 0
    for pin in GEMM8_PINS:
        try:
            pin(bad)
        except AssertionError:
            failed += 1
    assert failed >= 1


# ---------------------------------------------------- device arrangement

def test_arrange_xq_positions():
    """Codes equal to their own k (mod 128, as int8): each aligned block of 16
    lands in the order 0,4,1,5,2,6,3,7, 8,12,9,13,10,14,11,15, and the group
    sums are the plain sums."""
    K, g = 64, 32
    xq = (np.arange(K) - 32).astype(np.int8)[None, :]
    out, xs = oracle.arrange_xq(xq, g)
    order = [0, 4, 1, 5, 2, 6, 3, 7, 8, 12, 9, 13, 10, 14, 11, 15]
    expect = np.array([16 * b + order[j] for b in range(K // 16) for j in range(16)]) - 32
    assert np.array_equal(out[0].astype(int), expect)
    assert np.array_equal(xs[0], [sum(range(-32, 0)), sum(range(0, 32))])
