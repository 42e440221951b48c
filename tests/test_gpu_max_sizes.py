"""GPU tests at the size limits of 32-bit buffer offsets: activations larger
than 4 GB, which the kernels address in row chunks of one launch each. The
activations are drawn on the device (seeded); the oracle recomputes the rows
on both sides of every chunk boundary and the first and last rows.

Acceptance as everywhere: |y - y_ref| <= 1e-2 * (1 + |y_ref|) per element.
"""
import sys

import numpy as np
import pytest

import oracle
import synth
from gpu_util import dev_u16, dev_u32, tolerance_ratio

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
    torch.cuda.empty_cache()


def _weights(case, N, K, g):
    q = synth.gen_q(synth.tensor_id(synth.KIND_Q, 400 + case, 0), N, K)
    s = synth.gen_scales(synth.tensor_id(synth.KIND_SCALES, 400 + case, 0), N, K // g)
    return q, s


def _device_x(M, K, seed):
    import torch
    gen = torch.Generator(device="cuda")
    gen.manual_seed(seed)
    return torch.randn((M, K), generator=gen, device="cuda", dtype=torch.float32).to(torch.bfloat16)


def _rows_bits(x, rows):
    import torch
    return x[rows].view(torch.int16).cpu().numpy().view(np.uint16)


def test_w4a16_large_path_activations_over_4gb():
    """w4a16_gemm_ex on the one-workgroup-per-tile path with 4.3 GB of
    activations (K = 32768): two row chunks, the first of 65,408 rows; then
    w4a16_gemm and w4a16_gemm_ws (plain_kernel) on the same input."""
    import torch

    import w4a16_weight_only_gemm_amd as w4
    M, N, K, g = 65600, 48, 32768, 128
    assert 2 * M * K > 2**32
    q, s = _weights(0, N, K, g)
    qw, sp = w4.w4a16_pack(q, s, g)
    x = _device_x(M, K, 401)
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    log(f"w4a16 large path M={M} K={K} N={N} ({2 * M * K / 2**30:.2f} GiB of x)")
    w4.w4a16_gemm_ex(x, dev_u32(qw), dev_u16(sp), y, M, N, K, g, w4.W4A16_PATH_LARGE)
    torch.cuda.synchronize()
    rows = [0, 65407, 65408, 65409, M - 1]
    ref = oracle.gemm(_rows_bits(x, rows), q, s, g)
    yb = y[rows].view(torch.int16).cpu().numpy().view(np.uint16)
    assert tolerance_ratio(yb, ref) <= 1.0
    # w4a16_gemm runs plain_kernel here (three column blocks: the tile engine
    # would leave most compute units idle), and the workspace entry point
    # routes this one problem to w4a16_gemm's kernels
    assert w4.w4a16_select_form(M, N, K, g)[0] == w4.W4A16_PATH_SKINNY
    y2 = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    w4.w4a16_gemm(x, dev_u32(qw), dev_u16(sp), y2, M, N, K, g)
    torch.cuda.synchronize()
    yb2 = y2[rows].view(torch.int16).cpu().numpy().view(np.uint16)
    assert tolerance_ratio(yb2, ref) <= 1.0
    nb = w4.w4a16_workspace_bytes(M, N)
    ws = torch.zeros((nb + 3) // 4, dtype=torch.int32, device="cuda")
    y3 = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    w4.w4a16_gemm_ws(x, dev_u32(qw), dev_u16(sp), y3, M, N, K, g, ws)
    torch.cuda.synchronize()
    assert torch.equal(y2.view(torch.int16), y3.view(torch.int16))
    del x, y, y2, y3, ws


def test_w4a8_activations_over_4gb():
    """w4a8_quantize and w4a8_gemm with 4.3 GB of int8 codes (K = 32768): the
    GEMM runs in two row chunks, the first of 130,944 rows; codes and row
    scales of the sampled rows are checked bit for bit."""
    import torch

    import w4a16_weight_only_gemm_amd as w4
    M, N, K, g = 131100, 48, 32768, 128
    assert M * K > 2**32
    q, s = _weights(1, N, K, g)
    qw, sp = w4.w4a16_pack(q, s, g)
    x = _device_x(M, K, 402)
    xq = torch.empty((M, K), dtype=torch.int8, device="cuda")
    sx = torch.empty((M,), dtype=torch.float32, device="cuda")
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    log(f"w4a8 M={M} K={K} N={N} ({M * K / 2**30:.2f} GiB of codes)")
    w4.w4a8_quantize(x, xq, sx, M, K)
    w4.w4a8_gemm(xq, sx, dev_u32(qw), dev_u16(sp), y, M, N, K, g)
    torch.cuda.synchronize()
    rows = [0, 130943, 130944, 130945, M - 1]
    eq, es = oracle.quantize_rows(_rows_bits(x, rows))
    assert np.array_equal(sx[rows].cpu().numpy().view(np.uint32), es.view(np.uint32))
    assert np.array_equal(xq[rows].cpu().numpy(), oracle.arrange_xq(eq, 16)[0])
    ref = oracle.gemm_w4a8(eq, es, q, s, g)
    yb = y[rows].view(torch.int16).cpu().numpy().view(np.uint16)
    assert tolerance_ratio(yb, ref) <= 1.0
    del x, xq, sx, y
