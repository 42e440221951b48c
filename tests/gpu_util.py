"""Helpers of the GPU tests: device buffers from the generator's arrays, one call
through the C ABI, and the acceptance check against the oracle."""
from __future__ import annotations

import numpy as np

TOL = 1e-2  # |y - y_ref| <= TOL * (1 + |y_ref|), the GEMM's acceptance bound


def torch_mod():
    import torch
    return torch


def dev_u16(a: np.ndarray):
    torch = torch_mod()
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to("cuda")


def dev_u32(a: np.ndarray):
    torch = torch_mod()
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int32)).to("cuda")


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


class Problem:
    """Packed weights and activations of one GEMM, resident on the device."""

    def __init__(self, x_bits, q, s_bits, group):
        import w4a16_weight_only_gemm_amd as w4
        torch = torch_mod()
        self.M, self.K = x_bits.shape
        self.N = q.shape[0]
        self.group = group
        qw, sp = w4.w4a16_pack(q, s_bits, group)
        self.qw = dev_u32(qw)
        self.sp = dev_u16(sp)
        self.x = dev_u16(x_bits).view(torch.bfloat16)

    def run(self, path=0, y=None, stream=None) -> np.ndarray:
        import w4a16_weight_only_gemm_amd as w4
        torch = torch_mod()
        if y is None:
            y = torch.empty((self.M, self.N), dtype=torch.bfloat16, device="cuda")
        w4.w4a16_gemm_ex(self.x, self.qw, self.sp, y, self.M, self.N, self.K, self.group, path,
                         stream=stream)
        torch.cuda.synchronize()
        return y.view(torch.int16).cpu().numpy().view(np.uint16)


def tolerance_ratio(y_bits: np.ndarray, y_ref: np.ndarray) -> float:
    """max over elements of |y - y_ref| / (TOL * (1 + |y_ref|)); <= 1 passes."""
    y = bf16_bits_to_f64(y_bits)
    if y.size == 0:
        return 0.0
    if not np.isfinite(y).all():
        return float("inf")
    return float(np.max(np.abs(y - y_ref) / (TOL * (1.0 + np.abs(y_ref)))))


def workspace(M: int, total_columns: int):
    """A zero-filled device workspace for the streaming entry points."""
    import w4a16_weight_only_gemm_amd as w4
    torch = torch_mod()
    nbytes = w4.w4a16_workspace_bytes(M, total_columns)
    return torch.zeros((nbytes + 3) // 4, dtype=torch.int32, device="cuda")


def run_streamk(prob: "Problem", ws=None) -> np.ndarray:
    """One w4a16_gemm_grouped launch holding the problem twice, with two outputs:
    the stream-K schedule runs whatever the shape (w4a16_gemm_ws may run
    w4a16_gemm's kernels for a single problem above 16 rows). Both outputs are
    returned; the copies are cut differently, so their bits may differ."""
    import w4a16_weight_only_gemm_amd as w4
    torch = torch_mod()
    if ws is None:
        ws = workspace(prob.M, 2 * prob.N)
    ys = [torch.empty((prob.M, prob.N), dtype=torch.bfloat16, device="cuda") for _ in range(2)]
    w4.w4a16_gemm_grouped([(prob.x, prob.qw, prob.sp, y, prob.N, prob.K) for y in ys], prob.M,
                          prob.group, ws)
    torch.cuda.synchronize()
    return [y.view(torch.int16).cpu().numpy().view(np.uint16) for y in ys]


def run_ws(prob: "Problem", ws=None) -> np.ndarray:
    """One call of w4a16_gemm_ws (streaming kernel for M <= 16)."""
    import w4a16_weight_only_gemm_amd as w4
    torch = torch_mod()
    if ws is None:
        ws = workspace(prob.M, prob.N)
    y = torch.empty((prob.M, prob.N), dtype=torch.bfloat16, device="cuda")
    w4.w4a16_gemm_ws(prob.x, prob.qw, prob.sp, y, prob.M, prob.N, prob.K, prob.group, ws)
    torch.cuda.synchronize()
    return y.view(torch.int16).cpu().numpy().view(np.uint16)
