"""Pins for the W4A16 GEMM and its packed format.

Each pin checks a ``gemm(x_bits, q, s_bits, group) -> float64 [M, N]`` or a
``pack(q, s_bits, group) -> (qweight, scales)`` against something fixed by the
format's definition or by mathematics, never by re-running the function under
test: hand-derived packed words, closed-form sums, exact rational brute force,
invariants (identity activation, one-hot activation, linearity) and a library
matmul over weights dequantized by separate code. The same checks run against
planted mistakes (``test_oracle_pins.py``) to show that each one bites.

Conventions: q int8 [N, K] in -8..7; x bf16 bits [M, K]; s fp16 bits
[N, K/group]; the packed arrangement is described above pin_golden_words.
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
#
# Device arrangement (oracle.c states it in full): word j of column n holds
# the codes of k = 8j..8j+7 (two's complement), the code of k = 8j+i in nibble
# (i // 2) + 4 (i % 2): even k in nibbles 0..3, odd k in nibbles 4..7; tiles of
# 16 columns x one group are stored lane-major, lane l holding g/32 consecutive
# words of column 16b + l%16 starting at word t*g/8 + (l//16)*g/32; scales are
# [block][group][16].

# (codes q[0..7] of one word, expected uint32), derived by hand: with
# c_i = q[i] & 0xF, the hex digits from the most significant down are
# c7 c5 c3 c1 c6 c4 c2 c0.
GOLDEN_WORDS = [
    ([0, 1, 2, 3, 4, 5, 6, 7], 0x75316420),
    ([-1] * 8, 0xFFFFFFFF),
    ([-8] * 8, 0x88888888),
    ([7, -8, 0, 0, 0, 0, 0, 0], 0x00080007),
    ([0, 0, 0, 0, 0, 0, 0, -1], 0xF0000000),
    ([-8, -7, -6, -5, -4, -3, -2, -1], 0xFDB9ECA8),
    ([1, 0, 0, 0, 0, 0, 0, 0], 0x00000001),
    ([0, 1, 0, 0, 0, 0, 0, 0], 0x00010000),
    ([0, 0, 0, 0, 0, 0, 0, 7], 0x70000000),
]


def pin_golden_words(pack):
    # N = 9 columns (one block, padded to 16), K = 32, group 32 (one word per
    # lane, one group): lane l holds word l // 16 of column l % 16. The golden
    # codes fill k = 0..7 of each column, so lanes 0..8 hold the golden words
    # and every other lane (padding columns, or words 1..3) is zero.
    n = len(GOLDEN_WORDS)
    q = np.zeros((n, 32), dtype=np.int8)
    q[:, :8] = np.array([c for c, _ in GOLDEN_WORDS], dtype=np.int8)
    qw, _ = pack(q, fp16_bits(np.ones((n, 1))), 32)
    expect = np.zeros(64, dtype=np.uint32)
    expect[:n] = [w for _, w in GOLDEN_WORDS]
    assert np.array_equal(np.asarray(qw).ravel(), expect), [hex(v) for v in np.asarray(qw).ravel()]
    # one column, codes 0..7 then eight -1: words 0x75316420, 0xFFFFFFFF, 0, 0
    # land in lanes 0, 16, 32, 48
    q2 = np.zeros((1, 32), dtype=np.int8)
    q2[0, :16] = [0, 1, 2, 3, 4, 5, 6, 7] + [-1] * 8
    qw2 = np.asarray(pack(q2, fp16_bits([[1.0]]), 32)[0]).ravel()
    expect2 = np.zeros(64, dtype=np.uint32)
    expect2[0], expect2[16] = 0x75316420, 0xFFFFFFFF
    assert np.array_equal(qw2, expect2), [hex(v) for v in qw2]


def pin_tile_positions(pack):
    """Three codes placed by hand in N = 20 (two blocks), K = 128, group 64
    (two words per lane, eight words per column per group, two groups)."""
    q = np.zeros((20, 128), dtype=np.int8)
    q[17, 100] = -3   # block 1, column 1; word 12 = group 1, word 4 of it -> lane 2*16+1 = 33,
    #                   word 0 of the lane; index ((1*2+1)*64+33)*2 = 450; k = 8*12 + 4, so
    #                   i = 4 -> nibble 2: 0xD << 8
    q[2, 7] = 5       # block 0, column 2; word 0, i = 7 -> nibble 7 -> lane 2, index 4; 5 << 28
    q[19, 127] = -8   # block 1, column 3; word 15 = group 1, word 7 -> lane 3*16+3 = 51,
    #                   word 1 of the lane; index ((1*2+1)*64+51)*2+1 = 487; i = 7: 0x8 << 28
    qw = np.asarray(pack(q, fp16_bits(np.ones((20, 2))), 64)[0]).ravel()
    assert qw.size == 2 * 16 * 128 // 8
    expect = np.zeros(512, dtype=np.uint32)
    expect[450], expect[4], expect[487] = 0x00000D00, 0x50000000, 0x80000000
    assert np.array_equal(qw, expect), [(i, hex(v)) for i, v in enumerate(qw) if v]


def pin_scale_layout(pack):
    # N = 20 (two blocks), K = 64, group 32: s[n][t] = 2n + t + 1 (exact in fp16),
    # stored as [block][group][16] with zero scales for the padding columns.
    N, K, g = 20, 64, 32
    s = fp16_bits(2.0 * np.arange(N)[:, None] + np.arange(K // g)[None, :] + 1.0)
    sp = np.asarray(pack(np.zeros((N, K), dtype=np.int8), s, g)[1]).ravel()
    v = fp16_to_f64(sp)
    assert v.size == 2 * 2 * 16
    assert v[0] == 1.0 and v[1] == 3.0 and v[15] == 31.0      # block 0, group 0: n = 0, 1, 15
    assert v[16] == 2.0 and v[31] == 32.0                     # block 0, group 1: n = 0, 15
    assert v[32] == 33.0 and v[35] == 39.0 and v[36] == 0.0   # block 1, group 0: n = 16, 19, pad
    assert v[48] == 34.0 and v[51] == 40.0 and v[52:].sum() == 0.0  # block 1, group 1
    assert np.count_nonzero(v) == N * (K // g)


def pin_pack_roundtrip(pack, unpack):
    rng = np.random.default_rng(7)
    # every combination of four codes of a word (others random), both halves
    combos = np.array(np.meshgrid(*[np.arange(-8, 8)] * 4, indexing="ij")).reshape(4, -1).T
    for half in range(2):
        N = combos.shape[0] // 64                   # 1024 columns, 64 combinations each
        q = rng.integers(-8, 8, size=(N, 512)).astype(np.int8)
        blk = combos.reshape(N, 64, 4)
        for c in range(64):
            q[:, 8 * c + 4 * half: 8 * c + 4 * half + 4] = blk[:, c, :]
        qw, _ = pack(q, fp16_bits(np.ones((N, 4))), 128)
        assert np.array_equal(unpack(qw, N, 512, 128), q)
    # random matrices, ragged and whole column blocks, every group size
    for (N, K, g) in [(5, 256, 64), (3, 1024, 128), (17, 128, 128), (40, 512, 256), (33, 96, 32)]:
        q = rng.integers(-8, 8, size=(N, K)).astype(np.int8)
        qw, _ = pack(q, fp16_bits(np.ones((N, K // g))), g)
        assert np.array_equal(unpack(qw, N, K, g), q)
    # pack(unpack(w)) == w for arbitrary words when N fills whole blocks
    words = rng.integers(0, 1 << 32, size=64 * 32, dtype=np.uint64).astype(np.uint32)
    words[:8] = [0, 0xFFFFFFFF, 0x88888888, 0x77777777, 0x12345678, 0x87654321, 0xF0F0F0F0, 1]
    q = unpack(words, 32, 512, 128)
    qw, _ = pack(q, fp16_bits(np.ones((32, 4))), 128)
    assert np.array_equal(np.asarray(qw).ravel(), words)


def pin_pack_rejects(pack):
    bad = np.zeros((2, 64), dtype=np.int8)
    bad[1, 3] = 8
    cases = [(bad, 32), (np.full((1, 32), -9, dtype=np.int8), 32),
             (np.zeros((1, 48), dtype=np.int8), 16),       # group not a multiple of 32
             (np.zeros((1, 96), dtype=np.int8), 64)]       # K not a multiple of the group
    for q, g in cases:
        try:
            pack(q, fp16_bits(np.ones((q.shape[0], max(q.shape[1] // g, 1)))), g)
        except ValueError:
            pass
        else:
            raise AssertionError(f"accepted bad input (K={q.shape[1]}, group={g})")


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
