"""GPU parity of the W4A8 entry points against the CPU oracle, through the C ABI.

w4a8_quantize decides integers (the codes) in fp32 on both sides, so its
codes, their arrangement and the row scales must match the oracle bit for bit.
w4a8_gemm: |y - y_ref| <= 1e-2 * (1 + |y_ref|) element by element against the
oracle's W4A8 product (exact integer sums, fp64 scaling), and bit-exact where
the exact answer is a small integer (one-hot activations, group-index sums),
which pins the operand layouts and the group-to-scale mapping.
"""
import sys

import numpy as np
import pytest

import oracle
import pins
import synth
from gpu_util import bf16_bits_to_f64, dev_u16, dev_u32, tolerance_ratio

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


def _torch():
    import torch
    return torch


def gpu_quantize(x_bits):
    """(arranged codes [M][K] int8, row scales [M] fp32) from the GPU."""
    import w4a16_weight_only_gemm_amd as w4
    torch = _torch()
    M, K = x_bits.shape
    x = dev_u16(x_bits).view(torch.bfloat16)
    xq = torch.full((M, K), 99, dtype=torch.int8, device="cuda")
    sx = torch.full((max(M, 1),), -1.0, dtype=torch.float32, device="cuda")
    w4.w4a8_quantize(x, xq, sx, M, K)
    torch.cuda.synchronize()
    return xq.cpu().numpy(), sx.cpu().numpy()[:M]


class Q8Problem:
    """Packed weights plus arranged int8 codes and row scales on the device."""

    def __init__(self, xq_arranged, sx, q, s_bits, group):
        import w4a16_weight_only_gemm_amd as w4
        torch = _torch()
        self.M, self.K = xq_arranged.shape
        self.N = q.shape[0]
        self.group = group
        qw, sp = w4.w4a16_pack(q, s_bits, group)
        self.qw = dev_u32(qw)
        self.sp = dev_u16(sp)
        self.xq = torch.from_numpy(np.ascontiguousarray(xq_arranged)).to("cuda")
        self.sx = torch.from_numpy(np.ascontiguousarray(sx, dtype=np.float32)).to("cuda")

    def run(self) -> np.ndarray:
        import w4a16_weight_only_gemm_amd as w4
        torch = _torch()
        y = torch.full((self.M, self.N), float("nan"), dtype=torch.bfloat16, device="cuda")
        w4.w4a8_gemm(self.xq, self.sx, self.qw, self.sp, y, self.M, self.N, self.K, self.group)
        torch.cuda.synchronize()
        return y.view(torch.int16).cpu().numpy().view(np.uint16)


def arranged(xq):
    return oracle.arrange_xq(xq, 16)[0]


def _random_inputs(case_id, M, N, K, g):
    q = synth.gen_q(synth.tensor_id(synth.KIND_Q, 300 + case_id, 0), N, K)
    s = synth.gen_scales(synth.tensor_id(synth.KIND_SCALES, 300 + case_id, 0), N, K // g)
    x = synth.gen_x(synth.tensor_id(synth.KIND_X, 300 + case_id, 0, M), M, K)
    return x, q, s


# ------------------------------------------------------------ quantization

QUANT_SHAPES = [(1, 16), (1, 256), (2, 4096), (3, 5120), (37, 272), (300, 1024), (5, 17408)]


@pytest.mark.parametrize("shape", QUANT_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_quantize_bit_exact(shape):
    M, K = shape
    log(f"w4a8 quantize {shape}")
    x = synth.gen_x(synth.tensor_id(synth.KIND_X, 310, 0, M), M, K)
    if M >= 3:
        x[1] = 0                                                       # zero row
        x[2] = pins.bf16_bits([(np.arange(K) % 255 - 127) * 0.5])[0]   # ties at n + 0.5 ...
        x[2, 0] = pins.bf16_bits([[127.0]])[0, 0]                       # ... once inv = 1
    xq, sx = gpu_quantize(x)
    eq, es = oracle.quantize_rows(x)
    assert np.array_equal(sx.view(np.uint32), es.view(np.uint32))
    assert np.array_equal(xq, arranged(eq))


def test_quantize_scaled_rows_and_extremes():
    """Rows spanning many binades (tiny, huge, one nonzero value, negative
    maximum) against the oracle, bit for bit."""
    K = 512
    rng = np.random.default_rng(21)
    rows = [rng.standard_normal(K) * 1e-30, rng.standard_normal(K) * 1e30,
            np.where(np.arange(K) == 17, -3.0, 0.0), -np.abs(rng.standard_normal(K)),
            np.full(K, 1.0), rng.standard_normal(K) * 3.0]
    x = (np.array(rows, np.float32).view(np.uint32) >> 16).astype(np.uint16)  # truncated to bf16
    log("w4a8 quantize extremes")
    xq, sx = gpu_quantize(x)
    eq, es = oracle.quantize_rows(x)
    assert np.array_equal(sx.view(np.uint32), es.view(np.uint32))
    assert np.array_equal(xq, arranged(eq))


# -------------------------------------------------------------------- GEMM

def test_gemm_one_hot_bit_exact():
    """Row m holds the code 1 at k = (37 m) mod K and zeros elsewhere, unit
    scales: y[m][n] = q[n][(37 m) mod K] exactly. Every k position of every
    lane group and k-tile is hit, so a wrong byte order or piece index fails."""
    for (M, N, K, g) in [(256, 48, 1024, 128), (200, 40, 640, 64), (700, 264, 512, 128)]:
        log(f"w4a8 one-hot {(M, N, K, g)}")
        rng = np.random.default_rng(22)
        q = rng.integers(-8, 8, size=(N, K)).astype(np.int8)
        s = pins.fp16_bits(np.ones((N, K // g)))
        ks = (37 * np.arange(M)) % K
        xq = np.zeros((M, K), np.int8)
        xq[np.arange(M), ks] = 1
        y = Q8Problem(arranged(xq), np.ones(M, np.float32), q, s, g).run()
        assert np.array_equal(bf16_bits_to_f64(y), q[:, ks].T.astype(np.float64))


def test_gemm_group_index_bit_exact():
    """Codes 1 everywhere, unit weights, scale t + 1 on group t, row scale 2^-e:
    y = 2^-e * g * G (G + 1) / 2, exact."""
    for (M, N, K, g) in [(130, 32, 1024, 128), (70, 24, 1472, 64), (600, 272, 1472, 64)]:
        G = K // g
        log(f"w4a8 group-index {(M, N, K, g)}")
        s = pins.fp16_bits(np.tile(1.0 + np.arange(G), (N, 1)))
        sx = (2.0 ** -(np.arange(M) % 5)).astype(np.float32)
        y = Q8Problem(np.ones((M, K), np.int8), sx, np.ones((N, K), np.int8), s, g).run()
        expect = sx.astype(np.float64)[:, None] * (g * G * (G + 1) / 2.0) * np.ones((1, N))
        assert np.array_equal(bf16_bits_to_f64(y), expect)


def test_gemm_extreme_codes_bit_exact():
    """Codes -127 against weights -8 over a whole group, one group: the
    largest magnitude an int32 group sum reaches here, 1016 g; the result
    127 * 8 * g * scale must come out exactly (scale a power of two)."""
    M, N, K, g = 64, 32, 256, 128
    log("w4a8 extreme codes")
    xq = np.full((M, K), -127, np.int8)
    q = np.full((N, K), -8, np.int8)
    s = pins.fp16_bits(np.full((N, K // g), 2.0 ** -10))
    y = Q8Problem(arranged(xq), np.ones(M, np.float32), q, s, g).run()
    assert np.all(bf16_bits_to_f64(y) == 127 * 8 * K * 2.0 ** -10)


# M <= 256 runs 4-wave workgroups (128 x 128 tiles), larger M 8-wave ones (128 x 256)
GEMM_SHAPES = [(1, 16, 64, 64), (5, 40, 320, 64), (128, 256, 1024, 128), (130, 300, 640, 64),
               (257, 520, 2048, 128), (300, 1000, 1088, 64), (64, 7168, 512, 128),
               (512, 136, 384, 128), (513, 300, 640, 64), (700, 520, 1152, 128)]


@pytest.mark.parametrize("shape", GEMM_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_gemm_parity(shape):
    M, N, K, g = shape
    log(f"w4a8 gemm {shape}")
    x, q, s = _random_inputs(GEMM_SHAPES.index(shape), M, N, K, g)
    xq, sx = oracle.quantize_rows(x)
    y = Q8Problem(arranged(xq), sx, q, s, g).run()
    ref = oracle.gemm_w4a8(xq, sx, q, s, g)
    assert tolerance_ratio(y, ref) <= 1.0


@pytest.mark.parametrize("shape", [(256, 520, 2048, 128), (333, 96, 5120, 64)],
                         ids=lambda s: "x".join(map(str, s)))
def test_quantize_then_gemm(shape):
    """The device chain (quantize, then GEMM) against the oracle's chain."""
    import w4a16_weight_only_gemm_amd as w4
    torch = _torch()
    M, N, K, g = shape
    log(f"w4a8 chain {shape}")
    x, q, s = _random_inputs(20 + K // 64, M, N, K, g)
    xd = dev_u16(x).view(torch.bfloat16)
    xq = torch.empty((M, K), dtype=torch.int8, device="cuda")
    sx = torch.empty((M,), dtype=torch.float32, device="cuda")
    qw, sp = w4.w4a16_pack(q, s, g)
    qwd, spd = dev_u32(qw), dev_u16(sp)
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    w4.w4a8_quantize(xd, xq, sx, M, K)
    w4.w4a8_gemm(xq, sx, qwd, spd, y, M, N, K, g)
    torch.cuda.synchronize()
    eq, es = oracle.quantize_rows(x)
    ref = oracle.gemm_w4a8(eq, es, q, s, g)
    assert tolerance_ratio(y.view(torch.int16).cpu().numpy().view(np.uint16), ref) <= 1.0


def test_mlp_projections_m1024_sampled():
    """The MLP projections of the layer at M = 1024 (gate+up fused 5120 x
    34816, down 17408 x 5120), group 128, in the launch configuration of the
    benchmark: quantize and GEMM on the device over the full shape; the
    oracle recomputes sampled rows and columns."""
    import w4a16_weight_only_gemm_amd as w4
    torch = _torch()
    M, g = 1024, 128
    rng = np.random.default_rng(23)
    for proj in (2, 3):
        p = synth.LAYER_PROJECTIONS[proj]
        log(f"w4a8 sampled proj={proj} M={M} N={p.N} K={p.K}")
        x, q, s = synth.layer_inputs(0, proj, M, group=g)
        xd = dev_u16(x).view(torch.bfloat16)
        xq = torch.empty((M, p.K), dtype=torch.int8, device="cuda")
        sx = torch.empty((M,), dtype=torch.float32, device="cuda")
        qw, sp = w4.w4a16_pack(q, s, g)
        y = torch.empty((M, p.N), dtype=torch.bfloat16, device="cuda")
        w4.w4a8_quantize(xd, xq, sx, M, p.K)
        w4.w4a8_gemm(xq, sx, dev_u32(qw), dev_u16(sp), y, M, p.N, p.K, g)
        torch.cuda.synchronize()
        rows = np.unique(np.concatenate([[0, M - 1], rng.integers(0, M, 14)]))
        cols = np.unique(np.concatenate([[0, p.N - 1], rng.integers(0, p.N, 30)]))
        eq, es = oracle.quantize_rows(x[rows])
        assert np.array_equal(sx.cpu().numpy()[rows].view(np.uint32), es.view(np.uint32))
        assert np.array_equal(xq.cpu().numpy()[rows], arranged(eq))
        ref = oracle.gemm_w4a8(eq, es, q[cols], s[cols], g)
        yb = y.view(torch.int16).cpu().numpy().view(np.uint16)[np.ix_(rows, cols)]
        assert tolerance_ratio(yb, ref) <= 1.0


def test_gemm_deterministic_and_stream():
    """Same inputs, same bits, on a non-default stream too."""
    import w4a16_weight_only_gemm_amd as w4
    torch = _torch()
    M, N, K, g = 200, 600, 2048, 128
    log("w4a8 determinism")
    x, q, s = _random_inputs(40, M, N, K, g)
    xq, sx = oracle.quantize_rows(x)
    pr = Q8Problem(arranged(xq), sx, q, s, g)
    a = pr.run()
    st = torch.cuda.Stream()
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    with torch.cuda.stream(st):
        w4.w4a8_gemm(pr.xq, pr.sx, pr.qw, pr.sp, y, M, N, K, g, stream=st)
    st.synchronize()
    b = y.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(a, b)


# ----------------------------------------------------------------- grouped

def test_grouped_quantize_matches_oracle():
    """One launch over three inputs of different K, bit-exact against the oracle."""
    import w4a16_weight_only_gemm_amd as w4
    torch = _torch()
    M = 37
    entries, xs, outs = [], [], []
    for i, K in enumerate((5120, 272, 1024)):
        x = synth.gen_x(synth.tensor_id(synth.KIND_X, 320 + i, 0, M), M, K)
        xd = dev_u16(x).view(torch.bfloat16)
        xq = torch.full((M, K), 99, dtype=torch.int8, device="cuda")
        sx = torch.full((M,), -1.0, dtype=torch.float32, device="cuda")
        entries.append((xd, xq, sx, K))
        xs.append(x)
        outs.append((xq, sx))
    log("w4a8 grouped quantize")
    w4.w4a8_quantize_grouped(entries, M)
    torch.cuda.synchronize()
    for x, (xq, sx) in zip(xs, outs):
        eq, es = oracle.quantize_rows(x)
        assert np.array_equal(sx.cpu().numpy().view(np.uint32), es.view(np.uint32))
        assert np.array_equal(xq.cpu().numpy(), arranged(eq))


@pytest.mark.parametrize("g", [64, 128])
def test_grouped_gemm_parity_and_identity(g):
    """One launch over problems of different N and K (the deepest K is
    dispatched first, whatever its position in the list): each result within
    tolerance of the oracle and bit-identical to its single-problem call."""
    import w4a16_weight_only_gemm_amd as w4
    torch = _torch()
    M = 130
    shapes = [(300, 640), (1000, 1152), (48, 2048), (520, 256)]
    probs, refs = [], []
    for i, (N, K) in enumerate(shapes):
        x, q, s = _random_inputs(50 + i, M, N, K, g)
        xq, sx = oracle.quantize_rows(x)
        probs.append(Q8Problem(arranged(xq), sx, q, s, g))
        refs.append(oracle.gemm_w4a8(xq, sx, q, s, g))
    ys = [torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda") for N, _ in shapes]
    log(f"w4a8 grouped gemm g={g}")
    w4.w4a8_gemm_grouped([(p.xq, p.sx, p.qw, p.sp, y, p.N, p.K) for p, y in zip(probs, ys)], M, g)
    torch.cuda.synchronize()
    for p, y, ref in zip(probs, ys, refs):
        yb = y.view(torch.int16).cpu().numpy().view(np.uint16)
        assert tolerance_ratio(yb, ref) <= 1.0
        assert np.array_equal(yb, p.run())


def test_grouped_layer_set_m256_sampled():
    """The four projections of a layer at M = 256 (group 128) through the
    grouped quantize and grouped GEMM, as the benchmark runs them; the oracle
    recomputes sampled rows and columns of every projection."""
    import w4a16_weight_only_gemm_amd as w4
    torch = _torch()
    M, g = 256, 128
    rng = np.random.default_rng(24)
    qents, gents, keep = [], [], []
    for proj, p in enumerate(synth.LAYER_PROJECTIONS):
        x, q, s = synth.layer_inputs(1, proj, M, group=g)
        qw, sp = w4.w4a16_pack(q, s, g)
        xd = dev_u16(x).view(torch.bfloat16)
        xq = torch.empty((M, p.K), dtype=torch.int8, device="cuda")
        sx = torch.empty((M,), dtype=torch.float32, device="cuda")
        y = torch.empty((M, p.N), dtype=torch.bfloat16, device="cuda")
        qwd, spd = dev_u32(qw), dev_u16(sp)
        qents.append((xd, xq, sx, p.K))
        gents.append((xq, sx, qwd, spd, y, p.N, p.K))
        keep.append((x, q, s, y, p, xd, qwd, spd))
    log("w4a8 grouped layer set M=256")
    w4.w4a8_quantize_grouped(qents, M)
    w4.w4a8_gemm_grouped(gents, M, g)
    torch.cuda.synchronize()
    for x, q, s, y, p, *_ in keep:
        rows = np.unique(np.concatenate([[0, M - 1], rng.integers(0, M, 10)]))
        cols = np.unique(np.concatenate([[0, p.N - 1], rng.integers(0, p.N, 24)]))
        eq, es = oracle.quantize_rows(x[rows])
        ref = oracle.gemm_w4a8(eq, es, q[cols], s[cols], g)
        yb = y.view(torch.int16).cpu().numpy().view(np.uint16)[np.ix_(rows, cols)]
        assert tolerance_ratio(yb, ref) <= 1.0
