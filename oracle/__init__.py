"""CPU oracle of the W4A16 weight-only GEMM (fp64), loaded with ctypes.

TEST INFRASTRUCTURE ONLY: the tests, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` are the only callers. The product path (the
``w4a16_weight_only_gemm_amd`` package and its HIP library) never imports this
package, and this package never imports that one.

``oracle.c`` states what is computed and the packed format. Every function
here is a thin ctypes wrapper around it.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
# W4A16_ORACLE_LIB names another build of oracle.c (the sanitizer test runs the
# pins against an address/undefined-behaviour sanitizer build through it).
_LIB_PATH = os.environ.get("W4A16_ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so next to it (gcc -O2; strict IEEE double)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(
            ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-Wall", "-Wextra",
             "-ffp-contract=off", "-fno-fast-math", _SRC, "-o", tmp, "-lm", "-lpthread"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=False)
        lib = ctypes.CDLL(_LIB_PATH)
        vp, c_int = ctypes.c_void_p, ctypes.c_int
        lib.oracle_bf16_to_f64.restype = ctypes.c_double
        lib.oracle_bf16_to_f64.argtypes = [ctypes.c_uint16]
        lib.oracle_fp16_to_f64.restype = ctypes.c_double
        lib.oracle_fp16_to_f64.argtypes = [ctypes.c_uint16]
        lib.oracle_gemm_f64.restype = c_int
        lib.oracle_gemm_f64.argtypes = [vp, vp, vp, vp, c_int, c_int, c_int, c_int, c_int]
        lib.oracle_pack.restype = c_int
        lib.oracle_pack.argtypes = [vp, vp, vp, vp, c_int, c_int, c_int]
        lib.oracle_unpack.restype = c_int
        lib.oracle_unpack.argtypes = [vp, vp, c_int, c_int, c_int]
        lib.oracle_quantize_rows.restype = c_int
        lib.oracle_quantize_rows.argtypes = [vp, vp, vp, c_int, c_int]
        lib.oracle_gemm_w4a8.restype = c_int
        lib.oracle_gemm_w4a8.argtypes = [vp, vp, vp, vp, vp, c_int, c_int, c_int, c_int]
        lib.oracle_arrange_xq.restype = c_int
        lib.oracle_arrange_xq.argtypes = [vp, vp, vp, c_int, c_int, c_int]
        _lib = lib
    return _lib


def _c(a: np.ndarray, dtype) -> np.ndarray:
    a = np.ascontiguousarray(a)
    if a.dtype != dtype:
        raise TypeError(f"expected {np.dtype(dtype)}, got {a.dtype}")
    return a


def bf16_to_f64(bits: int) -> float:
    return float(_load().oracle_bf16_to_f64(int(bits)))


def fp16_to_f64(bits: int) -> float:
    return float(_load().oracle_fp16_to_f64(int(bits)))


def gemm(x_bf16: np.ndarray, q: np.ndarray, s_fp16: np.ndarray, group: int,
         threads: int = 1) -> np.ndarray:
    """y[M][N] (float64) for x bf16 bits [M][K], q int8 [N][K], s fp16 bits [N][K/group]."""
    x = _c(x_bf16, np.uint16)
    q = _c(q, np.int8)
    s = _c(s_fp16, np.uint16)
    M, K = x.shape
    N, Kq = q.shape
    if Kq != K or s.shape != (N, K // group if group else 0):
        raise ValueError("shape mismatch")
    y = np.empty((M, N), dtype=np.float64)
    rc = _load().oracle_gemm_f64(x.ctypes.data, q.ctypes.data, s.ctypes.data, y.ctypes.data,
                                 M, N, K, group, threads)
    if rc != 0:
        raise ValueError(f"oracle_gemm_f64 failed with code {rc}")
    return y


def blocks(N: int) -> int:
    return (N + 15) // 16


def pack(q: np.ndarray, s_fp16: np.ndarray, group: int):
    """(qweight uint32 [blocks*16*K/8], scales fp16 bits [blocks*(K/group)*16]) in the
    device arrangement described in oracle.c."""
    q = _c(q, np.int8)
    s = _c(s_fp16, np.uint16)
    N, K = q.shape
    if group <= 0 or group % 32 or K % group or s.shape != (N, K // group):
        raise ValueError("oracle_pack: bad shape")
    B = blocks(N)
    qw = np.empty(B * 16 * K // 8, dtype=np.uint32)
    sp = np.empty(B * (K // group) * 16, dtype=np.uint16)
    rc = _load().oracle_pack(q.ctypes.data, s.ctypes.data, qw.ctypes.data, sp.ctypes.data,
                             N, K, group)
    if rc != 0:
        raise ValueError("oracle_pack rejected the input")
    return qw, sp


def unpack(qweight: np.ndarray, N: int, K: int, group: int) -> np.ndarray:
    qw = _c(qweight, np.uint32)
    if qw.size != blocks(N) * 16 * K // 8:
        raise ValueError("oracle_unpack: bad size")
    q = np.empty((N, K), dtype=np.int8)
    rc = _load().oracle_unpack(qw.ctypes.data, q.ctypes.data, N, K, group)
    if rc != 0:
        raise ValueError("oracle_unpack rejected the input")
    return q


def quantize_rows(x_bf16: np.ndarray):
    """W4A8 activation quantization (oracle.c): (xq int8 [M][K], sx float32 [M])."""
    x = _c(x_bf16, np.uint16)
    M, K = x.shape
    xq = np.empty((M, K), dtype=np.int8)
    sx = np.empty(M, dtype=np.float32)
    rc = _load().oracle_quantize_rows(x.ctypes.data, xq.ctypes.data, sx.ctypes.data, M, K)
    if rc != 0:
        raise ValueError("oracle_quantize_rows rejected the input")
    return xq, sx


def gemm_w4a8(xq: np.ndarray, sx: np.ndarray, q: np.ndarray, s_fp16: np.ndarray,
              group: int) -> np.ndarray:
    """y[M][N] (float64) of the W4A8 product (oracle.c): exact integer sums per
    group, scaled in double."""
    xq = _c(xq, np.int8)
    sx = _c(sx, np.float32)
    q = _c(q, np.int8)
    s = _c(s_fp16, np.uint16)
    M, K = xq.shape
    N = q.shape[0]
    if q.shape != (N, K) or sx.shape != (M,) or s.shape != (N, K // group):
        raise ValueError("shape mismatch")
    y = np.empty((M, N), dtype=np.float64)
    rc = _load().oracle_gemm_w4a8(xq.ctypes.data, sx.ctypes.data, q.ctypes.data, s.ctypes.data,
                                  y.ctypes.data, M, N, K, group)
    if rc != 0:
        raise ValueError("oracle_gemm_w4a8 rejected the input")
    return y


def arrange_xq(xq: np.ndarray, group: int):
    """Device arrangement of quantized activations and their group sums
    (oracle.c): (int8 [M][K], int32 [M][K/group])."""
    xq = _c(xq, np.int8)
    M, K = xq.shape
    out = np.empty((M, K), dtype=np.int8)
    xs = np.empty((M, K // group), dtype=np.int32)
    rc = _load().oracle_arrange_xq(xq.ctypes.data, out.ctypes.data, xs.ctypes.data, M, K, group)
    if rc != 0:
        raise ValueError("oracle_arrange_xq rejected the input")
    return out, xs
