"""Pins for the W4A16 GEMM and its packed format.

Each pin checks a ``gemm(x_bits, q, s_bits, group) -> float64 [M, N]`` or a
``pack(q, s_bits, group) -> (qweight, scales)`` against something fixed by the
format's definition or by mathematics, never by re-running the function under
test: hand-derived packed words, closed-form sums, exact rational brute force,
invariants (identity activation, one-hot activation, linearity) and a library
matmul over weights dequantized by separate code. The same checks run against
planted mistakes (``test_oracle_pins.py``) to show that each one bites.

Conventions (packed format, a reading of pages that leave it open):
  q int8 [N, K] in -8..7; x bf16 bits [M, K]; s fp16 bits [N, K/group];
  qweight uint32 [N, K/8], code of q[n][8j+i] in bits 4i..4i+3 (two's complement);
  packed scales fp16 bits [K/group, N] (group-major).
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np

BF16_ONE = 0x3F80
FP16_ONE = 0x3C00


def bf16_bits(values) -> np.ndarray:
    """bf16 bit patterns of values that bf16 holds exactly (small integers, powers of two)."""
    f = np.asarray(values, dtype=np.float32)
    b = f.view(np.uint32)
    if np.any(b & 0xFFFF):
        raise ValueError("value not exact in bf16")
    return (b >> 16).astype(np.uint16)


def fp16_bits(values) -> np.ndarray:
    h = np.asarray(values, dtype=np.float16)
    if not np.array_equal(h.astype(np.float64), np.asarray(values, dtype=np.float64)):
        raise ValueError("value not exact in fp16")
    return h.view(np.uint16)


def bf16_to_f64(bits) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint32) << 16).view(np.float32).astype(np.float64)


def fp16_to_f64(bits) -> np.ndarray:
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


# ---------------------------------------------------------------- packing

# (codes q[0..7] of one word, expected uint32), derived by hand: the code of
# q[i] is q[i] & 0xF, placed at bits 4i..4i+3.
GOLDEN_WORDS = [
    ([0, 1, 2, 3, 4, 5, 6, 7], 0x76543210),
    ([-1] * 8, 0xFFFFFFFF),
    ([-8] * 8, 0x88888888),
    ([7, -8, 0, 0, 0, 0, 0, 0], 0x00000087),
    ([0, 0, 0, 0, 0, 0, 0, -1], 0xF0000000),
    ([-8, -7, -6, -5, -4, -3, -2, -1], 0xFEDCBA98),
    ([1, 0, 0, 0, 0, 0, 0, 0], 0x00000001),
    ([0, 0, 0, 0, 0, 0, 0, 7], 0x70000000),
]


def pin_golden_words(pack):
    q = np.array([c for c, _ in GOLDEN_WORDS], dtype=np.int8)           # N = 8 columns, K = 8
    s = fp16_bits(np.ones((len(GOLDEN_WORDS), 1)))
    qw, _ = pack(q, s, 8)
    expect = np.array([[w] for _, w in GOLDEN_WORDS], dtype=np.uint32)
    assert np.array_equal(qw, expect), [hex(v) for v in qw.ravel()]
    # two words in one column: word j holds k = 8j..8j+7
    q2 = np.array([[0, 1, 2, 3, 4, 5, 6, 7, -1, -1, -1, -1, -1, -1, -1, -1]], dtype=np.int8)
    qw2, _ = pack(q2, fp16_bits([[1.0]]), 16)
    assert qw2.tolist() == [[0x76543210, 0xFFFFFFFF]], [hex(v) for v in qw2.ravel()]


def pin_scale_layout(pack):
    N, K, g = 3, 32, 8
    s = fp16_bits(np.arange(N * (K // g), dtype=np.float64).reshape(N, K // g) + 1.0)
    _, sp = pack(np.zeros((N, K), dtype=np.int8), s, g)
    # group-major: sp[j][n] == s[n][j]
    assert sp.shape == (K // g, N)
    for n in range(N):
        for j in range(K // g):
            assert sp[j, n] == s[n, j]


def pin_pack_roundtrip(pack, unpack):
    rng = np.random.default_rng(7)
    # every combination of the four low codes of a word, high codes random, and vice versa
    combos = np.array(np.meshgrid(*[np.arange(-8, 8)] * 4, indexing="ij")).reshape(4, -1).T
    hi = rng.integers(-8, 8, size=(combos.shape[0], 4))
    for q in (np.concatenate([combos, hi], axis=1), np.concatenate([hi, combos], axis=1)):
        q = q.astype(np.int8)
        qw, _ = pack(q, fp16_bits(np.ones((q.shape[0], 1))), 8)
        assert np.array_equal(unpack(qw, 8), q)
    # random matrices at the workload's group sizes
    for (N, K, g) in [(5, 256, 64), (3, 1024, 128), (17, 128, 128)]:
        q = rng.integers(-8, 8, size=(N, K)).astype(np.int8)
        qw, _ = pack(q, fp16_bits(np.ones((N, K // g))), g)
        assert np.array_equal(unpack(qw, K), q)
    # pack(unpack(w)) == w for arbitrary words (every 32-bit word is a valid packing)
    words = rng.integers(0, 1 << 32, size=(64, 32), dtype=np.uint64).astype(np.uint32)
    words[0, :8] = [0, 0xFFFFFFFF, 0x88888888, 0x77777777, 0x12345678, 0x87654321, 0xF0F0F0F0, 1]
    q = unpack(words, 256)
    qw, _ = pack(q, fp16_bits(np.ones((64, 2))), 128)
    assert np.array_equal(qw, words)


def pin_pack_rejects(pack):
    bad = np.zeros((2, 16), dtype=np.int8)
    bad[1, 3] = 8
    for q, g in [(bad, 8), (np.full((1, 8), -9, dtype=np.int8), 8)]:
        try:
            pack(q, fp16_bits(np.ones((q.shape[0], q.shape[1] // g))), g)
        except ValueError:
            pass
        else:
            raise AssertionError("out-of-range code accepted")


# ---------------------------------------------------------------- the GEMM

def unit_scale_case(M, N, K, g):
    """s = 1, x = 1, q[n][k] = ((k + n) mod 16) - 8: every 16 consecutive k sum to -8."""
    k = np.arange(K)[None, :]
    n = np.arange(N)[:, None]
    q = (((k + n) % 16) - 8).astype(np.int8)
    x = np.full((M, K), BF16_ONE, dtype=np.uint16)
    s = np.full((N, K // g), FP16_ONE, dtype=np.uint16)
    return x, q, s, np.full((M, N), -K / 2.0)


def pin_unit_scale_closed_form(gemm):
    for (M, N, K, g) in [(1, 16, 16, 8), (3, 7, 64, 16), (2, 32, 256, 64), (1, 512, 256, 64),
                         (4, 24, 1024, 128)]:
        x, q, s, expect = unit_scale_case(M, N, K, g)
        y = gemm(x, q, s, g)
        assert np.array_equal(y, expect), (M, N, K, g)


def pin_hand_cases(gemm):
    # K = 8, one group of 8, s = 1: x = 1..8 against q = 0..7 gives sum_{k=1..8} k(k-1) = 168
    x = bf16_bits([[1, 2, 3, 4, 5, 6, 7, 8]])
    s = fp16_bits([[1.0]])
    assert gemm(x, np.array([[0, 1, 2, 3, 4, 5, 6, 7]], dtype=np.int8), s, 8)[0, 0] == 168.0
    # x = 1 against q = -8..-1 gives -36
    x1 = np.full((1, 8), BF16_ONE, dtype=np.uint16)
    assert gemm(x1, np.arange(-8, 0, dtype=np.int8)[None, :], s, 8)[0, 0] == -36.0
    # a non-unit scale: 0.5 * (x = 1..8 against q = 7..0) = 0.5 * 84
    q = np.arange(7, -1, -1, dtype=np.int8)[None, :]
    assert gemm(x, q, fp16_bits([[0.5]]), 8)[0, 0] == 42.0


def pin_group_index(gemm):
    # s[n][j] = 1 + j, q = 1, x = 1 -> y = g * G (G + 1) / 2
    for (M, N, K, g) in [(1, 4, 64, 8), (2, 8, 256, 64), (1, 512, 256, 64), (1, 3, 1024, 128)]:
        G = K // g
        s = fp16_bits(np.tile(1.0 + np.arange(G), (N, 1)))
        y = gemm(np.full((M, K), BF16_ONE, dtype=np.uint16), np.ones((N, K), dtype=np.int8), s, g)
        assert np.all(y == g * G * (G + 1) / 2.0), (M, N, K, g)
    # one-hot x = e_j picks q[n][j] * s[n][floor(j/g)] for every j
    rng = np.random.default_rng(3)
    N, K, g = 5, 64, 16
    q = rng.integers(-8, 8, size=(N, K)).astype(np.int8)
    s = fp16_bits(rng.integers(1, 64, size=(N, K // g)) / 16.0)
    x = bf16_bits(np.eye(K))
    y = gemm(x, q, s, g)
    expect = q.T.astype(np.float64) * np.repeat(fp16_to_f64(s), g, axis=1).T
    assert np.array_equal(y, expect)


def pin_identity_activation(gemm):
    # M = K, x = I, s = 1 -> y[m][n] = q[n][m]: the whole weight matrix comes back
    rng = np.random.default_rng(4)
    for (N, K, g) in [(48, 32, 8), (16, 256, 64), (512, 256, 64)]:
        q = rng.integers(-8, 8, size=(N, K)).astype(np.int8)
        y = gemm(bf16_bits(np.eye(K)), q, np.full((N, K // g), FP16_ONE, dtype=np.uint16), g)
        assert np.array_equal(y, q.T.astype(np.float64)), (N, K, g)


def pin_linearity(gemm):
    rng = np.random.default_rng(5)
    M, N, K, g = 4, 24, 256, 64
    q = rng.integers(-8, 8, size=(N, K)).astype(np.int8)
    s = fp16_bits(rng.integers(80, 320, size=(N, K // g)) / 16384.0)
    xa = rng.integers(-64, 64, size=(M, K)) / 32.0
    y = gemm(bf16_bits(xa), q, s, g)
    # doubling x or s doubles y exactly (scaling by 2 commutes with every rounding)
    assert np.array_equal(gemm(bf16_bits(2 * xa), q, s, g), 2 * y)
    assert np.array_equal(gemm(bf16_bits(xa), q, fp16_bits(2 * fp16_to_f64(s)), g), 2 * y)
    # additivity over disjoint supports of x
    mask = rng.random((M, K)) < 0.5
    ya = gemm(bf16_bits(np.where(mask, xa, 0.0)), q, s, g)
    yb = gemm(bf16_bits(np.where(mask, 0.0, xa)), q, s, g)
    assert np.allclose(ya + yb, y, rtol=0, atol=1e-12 * (1 + np.abs(y).max()))


def random_case(rng, M, N, K, g):
    """Random bf16 activations (standard normal, truncated to bf16), codes and fp16 scales."""
    xf = rng.standard_normal((M, K)).astype(np.float32)
    x = (xf.view(np.uint32) >> 16).astype(np.uint16)
    q = rng.integers(-8, 8, size=(N, K)).astype(np.int8)
    s = rng.uniform(0.005, 0.02, size=(N, K // g)).astype(np.float16).view(np.uint16)
    return x, q, s


def exact_gemm(x_bits, q, s_bits, g):
    """Exact rational y[m][n] (Fractions), written from the definition."""
    xv = bf16_to_f64(x_bits)
    sv = fp16_to_f64(s_bits)
    M, K = xv.shape
    N = q.shape[0]
    out = [[Fraction(0)] * N for _ in range(M)]
    for m in range(M):
        for n in range(N):
            acc = Fraction(0)
            for k in range(K):
                acc += Fraction(float(xv[m, k])) * int(q[n, k]) * Fraction(float(sv[n, k // g]))
            out[m][n] = acc
    return out


def pin_bruteforce_exact(gemm):
    rng = np.random.default_rng(6)
    for (M, N, K, g) in [(1, 3, 8, 8), (2, 5, 32, 16), (3, 8, 64, 32), (3, 4, 64, 64), (2, 6, 48, 8)]:
        x, q, s = random_case(rng, M, N, K, g)
        y = gemm(x, q, s, g)
        ex = exact_gemm(x, q, s, g)
        xv, sv = bf16_to_f64(x), fp16_to_f64(s)
        for m in range(M):
            for n in range(N):
                terms = np.abs(xv[m] * q[n] * np.repeat(sv[n], g))
                bound = K * 2.0**-53 * terms.sum()
                assert abs(Fraction(float(y[m, n])) - ex[m][n]) <= Fraction(bound), (M, N, K, g, m, n)


def pin_library_matmul(gemm):
    """The oracle against a textbook float64 matmul over weights dequantized here."""
    rng = np.random.default_rng(8)
    for (M, N, K, g) in [(3, 40, 256, 64), (16, 64, 1024, 128), (1, 33, 640, 128)]:
        x, q, s = random_case(rng, M, N, K, g)
        w = q.astype(np.float64) * np.repeat(fp16_to_f64(s), g, axis=1)      # [N, K]
        ref = bf16_to_f64(x) @ w.T
        y = gemm(x, q, s, g)
        assert np.allclose(y, ref, rtol=1e-12, atol=1e-12), (M, N, K, g)
