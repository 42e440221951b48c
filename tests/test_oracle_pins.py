"""The CPU oracle pinned to things other than itself, and planted mistakes
(wrong sign, dropped term, wrong group or column index, transposed operand,
wrong nibble order or sign code, reduced precision) shown to fail the pins.

The planted mistakes are wrappers around the oracle on the CPU; the oracle
itself is never modified."""
import numpy as np
import pytest

import oracle
import pins


def gemm(x, q, s, g):
    return oracle.gemm(x, q, s, g, threads=2)


GEMM_PINS = [pins.pin_unit_scale_closed_form, pins.pin_hand_cases, pins.pin_group_index,
             pins.pin_identity_activation, pins.pin_linearity, pins.pin_bruteforce_exact,
             pins.pin_library_matmul]


@pytest.mark.parametrize("pin", GEMM_PINS, ids=lambda f: f.__name__)
def test_oracle_gemm_pins(pin):
    pin(gemm)


def test_oracle_golden_words():
    pins.pin_golden_words(oracle.pack)


def test_oracle_scale_layout():
    pins.pin_scale_layout(oracle.pack)


def test_oracle_tile_positions():
    pins.pin_tile_positions(oracle.pack)


def test_oracle_pack_roundtrip():
    pins.pin_pack_roundtrip(oracle.pack, oracle.unpack)


def test_oracle_pack_rejects_out_of_range():
    pins.pin_pack_rejects(oracle.pack)


def test_oracle_rejects_bad_shapes():
    x = np.zeros((1, 24), np.uint16)
    q = np.zeros((2, 24), np.int8)
    with pytest.raises(ValueError):
        oracle.gemm(x, q, np.zeros((2, 1), np.uint16), 16)  # K % group != 0
    with pytest.raises(ValueError):
        oracle.pack(np.zeros((2, 48), np.int8), np.zeros((2, 1), np.uint16), 48)  # group % 32


def test_oracle_thread_count_invariant():
    rng = np.random.default_rng(11)
    x, q, s = pins.random_case(rng, 5, 77, 512, 128)
    a = oracle.gemm(x, q, s, 128, threads=1)
    b = oracle.gemm(x, q, s, 128, threads=8)
    assert np.array_equal(a, b)


def test_oracle_empty_shapes():
    assert oracle.gemm(np.zeros((0, 64), np.uint16), np.zeros((8, 64), np.int8),
                       np.zeros((8, 1), np.uint16), 64).shape == (0, 8)
    assert oracle.gemm(np.zeros((2, 64), np.uint16), np.zeros((0, 64), np.int8),
                       np.zeros((0, 1), np.uint16), 64).shape == (2, 0)


def test_oracle_number_decoding():
    # bf16 and fp16 decoding against values fixed by the IEEE formats
    assert oracle.bf16_to_f64(0x3F80) == 1.0 and oracle.bf16_to_f64(0xC100) == -8.0
    assert oracle.bf16_to_f64(0x0001) == 2.0**-133
    assert oracle.fp16_to_f64(0x3C00) == 1.0 and oracle.fp16_to_f64(0x7BFF) == 65504.0
    assert oracle.fp16_to_f64(0x0001) == 2.0**-24 and oracle.fp16_to_f64(0x0400) == 2.0**-14
    assert oracle.fp16_to_f64(0xC000) == -2.0 and oracle.fp16_to_f64(0x3555) == 1365 / 4096
    assert np.isinf(oracle.fp16_to_f64(0x7C00)) and np.isnan(oracle.fp16_to_f64(0x7E00))


# ------------------------------------------------------------ planted mistakes

def _mut_sign(x, q, s, g):
    return oracle.gemm(x, (-q.astype(np.int16)).clip(-128, 127).astype(np.int8), s, g)


def _mut_drop_last_term(x, q, s, g):
    x = x.copy()
    x[:, -1] = 0
    return oracle.gemm(x, q, s, g)


def _mut_group_index(x, q, s, g):
    # uses s[n][floor(k/g) + 1] (clamped): an off-by-one group index
    s2 = np.concatenate([s[:, 1:], s[:, -1:]], axis=1)
    return oracle.gemm(x, q, s2, g)


def _mut_scale_column(x, q, s, g):
    return oracle.gemm(x, q, np.roll(s, 1, axis=0), g)


def _mut_transposed_q(x, q, s, g):
    # reads q as if it were stored k-major ([K][N]): element (n, k) taken from flat index k*N + n
    N, K = q.shape
    return oracle.gemm(x, q.reshape(-1).reshape(K, N).T.copy(), s, g)


def _mut_fp32_accumulate(x, q, s, g):
    w = (q.astype(np.float32) * np.repeat(pins.fp16_to_f64(s).astype(np.float32), g, axis=1))
    xv = pins.bf16_to_f64(x).astype(np.float32)
    y = np.zeros((x.shape[0], q.shape[0]), dtype=np.float32)
    for k in range(x.shape[1]):
        y += np.outer(xv[:, k], w[:, k])
    return y.astype(np.float64)


def _mut_bf16_weights(x, q, s, g):
    w = q.astype(np.float64) * np.repeat(pins.fp16_to_f64(s), g, axis=1)
    wb = (w.astype(np.float32).view(np.uint32) + 0x8000) & 0xFFFF0000  # round w to bf16
    return pins.bf16_to_f64(x) @ wb.view(np.float32).astype(np.float64).T


GEMM_MUTANTS = [_mut_sign, _mut_drop_last_term, _mut_group_index, _mut_scale_column,
                _mut_transposed_q, _mut_fp32_accumulate, _mut_bf16_weights]


def _fails_some_pin(pin_fns):
    caught = []
    for pin in pin_fns:
        try:
            pin()
        except (AssertionError, ValueError):
            caught.append(pin)
    return caught


@pytest.mark.parametrize("mutant", GEMM_MUTANTS, ids=lambda f: f.__name__)
def test_planted_gemm_mistake_is_caught(mutant):
    caught = _fails_some_pin([lambda p=p: p(mutant) for p in GEMM_PINS])
    assert caught, f"{mutant.__name__} passed every pin"


def _pack_nibbles_reversed(q, s, g):
    return oracle.pack(q.reshape(q.shape[0], -1, 8)[:, :, ::-1].reshape(q.shape).copy(), s, g)


def _pack_sequential_nibbles(q, s, g):
    # code of k = 8j+i in nibble i (not interleaved): feed the oracle codes
    # reordered so that its nibble (i // 2) + 4 (i % 2) receives q[8j + that nibble]
    sigma = [i // 2 + 4 * (i % 2) for i in range(8)]
    return oracle.pack(q.reshape(q.shape[0], -1, 8)[:, :, sigma].reshape(q.shape).copy(), s, g)


def _pack_offset_binary(q, s, g):
    qw, sp = oracle.pack(q, s, g)
    return qw ^ np.uint32(0x88888888), sp


def _pack_scales_row_major(q, s, g):
    qw, sp = oracle.pack(q, s, g)
    flat = np.zeros_like(sp)
    flat[:s.size] = s.ravel()
    return qw, flat


def _pack_untiled(q, s, g):
    # words in plain [N][K/8] order (columns padded to 16), no lane tiling
    qw, sp = oracle.pack(q, s, g)
    N, K = q.shape
    Np = oracle.blocks(N) * 16
    qp = np.zeros((Np, K), np.int8)
    qp[:N] = q
    words = np.zeros((Np, K // 8), np.uint32)
    codes = (qp.astype(np.int64) & 0xF).astype(np.uint32).reshape(Np, K // 8, 8)
    for i in range(8):
        words |= codes[:, :, i] << np.uint32(4 * i)
    return words.ravel(), sp


def _unpack_offset_binary(qw, N, K, g):
    return oracle.unpack(qw ^ np.uint32(0x88888888), N, K, g)


@pytest.mark.parametrize("mutant", [_pack_nibbles_reversed, _pack_sequential_nibbles,
                                    _pack_offset_binary, _pack_scales_row_major, _pack_untiled],
                         ids=lambda f: f.__name__)
def test_planted_pack_mistake_is_caught(mutant):
    caught = _fails_some_pin([lambda: pins.pin_golden_words(mutant),
                              lambda: pins.pin_tile_positions(mutant),
                              lambda: pins.pin_scale_layout(mutant)])
    assert caught, f"{mutant.__name__} passed every pin"


def test_planted_unpack_mistake_is_caught():
    caught = _fails_some_pin([lambda: pins.pin_pack_roundtrip(oracle.pack, _unpack_offset_binary)])
    assert caught
