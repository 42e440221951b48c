"""The seeded input generator: SplitMix64 known answers, the rounding of its
fp16/bf16 conversions, the value distributions, and slice regeneration."""
import numpy as np
import pytest

import synth

MASK = (1 << 64) - 1


def _py_splitmix64_stream(state, n):
    """Reference SplitMix64 written from its published definition, in Python ints."""
    out = []
    for _ in range(n):
        state = (state + 0x9E3779B97F4A7C15) & MASK
        z = state
        z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & MASK
        z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & MASK
        out.append(z ^ (z >> 31))
    return out


def test_splitmix64_seed0_known_outputs():
    # The first outputs of SplitMix64 seeded with 0, as listed with its public reference code.
    expect = [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]
    assert [synth.splitmix64(0, i) for i in range(3)] == expect
    assert _py_splitmix64_stream(0, 3) == expect


@pytest.mark.parametrize("key", [0, 1, 0xDEADBEEF, MASK, 0x0123456789ABCDEF])
def test_splitmix64_counter_matches_stream(key):
    ref = _py_splitmix64_stream(key, 40)
    assert [synth.splitmix64(key, i) for i in range(40)] == ref


def test_fp16_rounding_matches_numpy():
    rng = np.random.default_rng(1)
    vals = np.concatenate([
        rng.uniform(0.005, 0.02, 20000),
        rng.uniform(-70000, 70000, 2000),
        rng.uniform(-1e-4, 1e-4, 2000),     # subnormal range
        np.array([0.0, -0.0, 1.0, 65504.0, 65519.99, 65520.0, 2.0**-24, 2.0**-25, 3 * 2.0**-26]),
    ])
    ours = np.array([synth.f64_to_fp16_bits(v) for v in vals], dtype=np.uint16)
    with np.errstate(over="ignore"):
        ref = vals.astype(np.float16).view(np.uint16)  # numpy rounds double -> half to nearest even
    np.testing.assert_array_equal(ours, ref)


def _bf16_value(bits):
    return float(np.array([int(bits) << 16], dtype=np.uint32).view(np.float32)[0])


def test_bf16_rounding_is_nearest_even():
    rng = np.random.default_rng(2)
    vals = np.concatenate([rng.standard_normal(5000), rng.uniform(-1e30, 1e30, 500),
                           np.array([1.0 + 2.0**-8, 1.0 + 3 * 2.0**-8, -(1.0 + 2.0**-8)])])
    for v in vals:
        b = synth.f64_to_bf16_bits(v)
        err = abs(_bf16_value(b) - v)
        # the neighbouring patterns b-1 and b+1 are the next bf16 values of the same sign
        for nb in (b - 1, b + 1):
            if (nb & 0x7FFF) == 0 or (nb & 0x7FFF) >= 0x7F80:
                continue
            d = abs(_bf16_value(nb) - v)
            assert err <= d, (v, hex(b), hex(nb))
            if err == d:
                assert (b & 1) == 0, (v, hex(b))  # a tie goes to the even pattern
    # exact ties: 1 + 2^-8 lies halfway between 1 and 1 + 2^-7 -> even (1.0)
    assert synth.f64_to_bf16_bits(1.0 + 2.0**-8) == 0x3F80
    assert synth.f64_to_bf16_bits(1.0 + 3 * 2.0**-8) == 0x3F82


def test_q_distribution_and_range():
    q = synth.gen_q(synth.tensor_id(synth.KIND_Q, 0, 0), 256, 1024)
    assert q.min() == -8 and q.max() == 7
    counts = np.bincount(q.ravel().astype(np.int64) + 8, minlength=16)
    assert counts.min() > 0.9 * q.size / 16 and counts.max() < 1.1 * q.size / 16
    assert abs(q.mean() + 0.5) < 0.02
    assert abs((q.astype(np.float64) ** 2).mean() - 21.5) < 0.2


def test_scales_distribution_and_range():
    s = synth.gen_scales(synth.tensor_id(synth.KIND_SCALES, 0, 0), 512, 64)
    v = s.view(np.float16).astype(np.float64)
    assert v.min() >= 0.005 - 1e-6 and v.max() <= 0.02 + 1e-5
    assert abs(v.mean() - 0.0125) < 2e-4


def test_x_distribution():
    x = synth.gen_x(synth.tensor_id(synth.KIND_X, 0, 0, 64), 64, 4096)
    v = (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    assert abs(v.mean()) < 0.01 and abs(v.std() - 1.0) < 0.01
    assert np.isfinite(v).all()


def test_slices_regenerate_exactly():
    tid = synth.tensor_id(synth.KIND_Q, 3, 1)
    full = synth.gen_q(tid, 100, 64)
    np.testing.assert_array_equal(synth.gen_q(tid, 100, 64, rows=(37, 58)), full[37:58])
    tid = synth.tensor_id(synth.KIND_X, 3, 1, 16)
    full = synth.gen_x(tid, 16, 256)
    np.testing.assert_array_equal(synth.gen_x(tid, 16, 256, rows=(5, 9)), full[5:9])
    tid = synth.tensor_id(synth.KIND_SCALES, 3, 1)
    full = synth.gen_scales(tid, 40, 8)
    np.testing.assert_array_equal(synth.gen_scales(tid, 40, 8, rows=(0, 1)), full[:1])


def test_threads_do_not_change_values():
    tid = synth.tensor_id(synth.KIND_X, 1, 2, 8)
    a = synth.gen_x(tid, 8, 1000, threads=1)
    b = synth.gen_x(tid, 8, 1000, threads=7)
    np.testing.assert_array_equal(a, b)


def test_tensors_are_distinct():
    a = synth.gen_q(synth.tensor_id(synth.KIND_Q, 0, 0), 4, 64)
    b = synth.gen_q(synth.tensor_id(synth.KIND_Q, 1, 0), 4, 64)
    c = synth.gen_q(synth.tensor_id(synth.KIND_Q, 0, 1), 4, 64)
    assert (a != b).any() and (a != c).any()


def test_scaled_activations():
    """sigma = 1 is gen_x bit for bit; sigma = 1000 is 1000 times the same normal,
    each side rounded to bf16 once (relative difference at most 2 * 2^-8)."""
    tid = synth.tensor_id(synth.KIND_X, 3, 1, 4)
    a = synth.gen_x(tid, 4, 512)
    assert np.array_equal(a, synth.gen_x(tid, 4, 512, sigma=1.0))
    b = synth.gen_x(tid, 4, 512, sigma=1000.0)
    fa = (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    fb = (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    nz = fa != 0
    assert np.all(np.abs(fb[nz] / (1000.0 * fa[nz]) - 1.0) <= 2.0 ** -7)
    assert 900.0 < np.std(fb) < 1100.0
