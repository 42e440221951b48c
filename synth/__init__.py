"""Seeded synthetic inputs for the W4A16 weight-only GEMM, shared by the CPU
oracle and the GPU library.

This package only draws numbers and names workloads; it holds none of the
GEMM's arithmetic. The generator is SplitMix64 over a 64-bit counter (Steele,
Lea and Flood, OOPSLA 2014), implemented in ``synth.c`` and loaded with ctypes.
Every tensor has its own id, so any slice can be regenerated independently.

Workload shapes are those of a 27B-class dense decoder layer, the model whose
decode throughput the source pages discuss ("One weight read, shared by every
stream" and "Where the line bends" on the Qwen3.8-27B throughput page): four
projections per layer, MLP width 17,408, 64 layers. M is the number of
activation rows sharing one weight read: streams times verified positions.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "synth.c")
_LIB_PATH = os.path.join(_HERE, "libsynth.so")
_lib = None

SEED = 0

KIND_Q, KIND_SCALES, KIND_X = 1, 2, 3


def build(force: bool = True) -> str:
    """Compile synth.c into libsynth.so next to it (gcc, -O2)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(
            ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-Wall", "-Wextra",
             _SRC, "-o", tmp, "-lm", "-lpthread"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=False)
        lib = ctypes.CDLL(_LIB_PATH)
        u64, i64, c_int = ctypes.c_uint64, ctypes.c_int64, ctypes.c_int
        lib.synth_splitmix64.restype = u64
        lib.synth_splitmix64.argtypes = [u64, u64]
        lib.synth_stream_key.restype = u64
        lib.synth_stream_key.argtypes = [u64, u64]
        lib.synth_f64_to_fp16_rne.restype = ctypes.c_uint16
        lib.synth_f64_to_fp16_rne.argtypes = [ctypes.c_double]
        lib.synth_f64_to_bf16_rne.restype = ctypes.c_uint16
        lib.synth_f64_to_bf16_rne.argtypes = [ctypes.c_double]
        for name in ("synth_q", "synth_scales", "synth_x"):
            fn = getattr(lib, name)
            fn.restype = c_int
            fn.argtypes = [u64, u64, ctypes.c_void_p, i64, i64, i64, c_int]
        lib.synth_x_sigma.restype = c_int
        lib.synth_x_sigma.argtypes = [u64, u64, ctypes.c_void_p, i64, i64, i64, ctypes.c_double,
                                      c_int]
        _lib = lib
    return _lib


def default_threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def tensor_id(kind: int, layer: int, proj: int, m: int = 0) -> int:
    """Id of one synthetic tensor: kind (q / scales / x), layer, projection and,
    for activations, the row count M (so each M gets its own activations)."""
    return (kind << 56) | (m << 32) | (layer << 12) | proj


def splitmix64(key: int, i: int) -> int:
    return int(_load().synth_splitmix64(key, i))


def stream_key(seed: int, tid: int) -> int:
    return int(_load().synth_stream_key(seed, tid))


def f64_to_fp16_bits(v: float) -> int:
    return int(_load().synth_f64_to_fp16_rne(float(v)))


def f64_to_bf16_bits(v: float) -> int:
    return int(_load().synth_f64_to_bf16_rne(float(v)))


def gen_q(tid: int, N: int, K: int, rows=None, seed: int = SEED, threads: int | None = None):
    """int8 [n1-n0, K] codes in [-8, 7] for rows [n0, n1) of q[N][K]."""
    n0, n1 = (0, N) if rows is None else rows
    out = np.empty((n1 - n0, K), dtype=np.int8)
    rc = _load().synth_q(seed, tid, out.ctypes.data, K, n0, n1, threads or default_threads())
    assert rc == 0
    return out


def gen_scales(tid: int, N: int, G: int, rows=None, seed: int = SEED, threads: int | None = None):
    """uint16 fp16 bit patterns [n1-n0, G] for rows [n0, n1) of s[N][G]."""
    n0, n1 = (0, N) if rows is None else rows
    out = np.empty((n1 - n0, G), dtype=np.uint16)
    rc = _load().synth_scales(seed, tid, out.ctypes.data, G, n0, n1, threads or default_threads())
    assert rc == 0
    return out


def gen_x(tid: int, M: int, K: int, rows=None, seed: int = SEED, threads: int | None = None,
          sigma: float = 1.0):
    """uint16 bf16 bit patterns [m1-m0, K] for rows [m0, m1) of x[M][K]: the
    standard normal times sigma, rounded to bf16 (sigma = 1: the workloads)."""
    m0, m1 = (0, M) if rows is None else rows
    out = np.empty((m1 - m0, K), dtype=np.uint16)
    if sigma == 1.0:
        rc = _load().synth_x(seed, tid, out.ctypes.data, K, m0, m1, threads or default_threads())
    else:
        rc = _load().synth_x_sigma(seed, tid, out.ctypes.data, K, m0, m1, float(sigma),
                                   threads or default_threads())
    assert rc == 0
    return out


# ---------------------------------------------------------------- workloads

@dataclass(frozen=True)
class Projection:
    name: str
    K: int
    N: int


# One layer of the 27B-class dense stand-in: (K, N) of y[M,N] = x[M,K] . W[K,N].
LAYER_PROJECTIONS = (
    Projection("qkv", 5120, 7168),
    Projection("o", 6144, 5120),
    Projection("gate_up", 5120, 34816),
    Projection("down", 17408, 5120),
)
GROUP = 128
N_LAYERS = 64

# One GPU's share of the same layer under 8-way tensor parallelism: qkv and
# gate_up split by columns (N / 8), o and down by rows of K (K / 8; each GPU
# then holds a partial y that an all-reduce sums). Their tensors take
# projection slots SHARD_PROJ_BASE + index, apart from the full layer's.
TP8_SHARD_PROJECTIONS = (
    Projection("qkv", 5120, 896),
    Projection("o", 768, 5120),
    Projection("gate_up", 5120, 4352),
    Projection("down", 2176, 5120),
)
SHARD_PROJ_BASE = 8

# The small GEMV case the oracle finishes instantly.
TINY = dict(M=1, K=256, N=512, group=64)
TINY_PROJ = 15  # projection slot reserved for the tiny case's tensor ids

# Row counts: single-stream decode, a 15-draft + 1 verify block, 64 streams,
# 64 streams x 16 verified positions; and the full-step sweep.
M_DECODE, M_VERIFY, M_STREAMS, M_BATCH = 1, 16, 64, 1024
M_SWEEP = (1, 2, 4, 8, 16, 32, 64, 128, 256, 512, 1024)


def layer_inputs(layer: int, proj_index: int, M: int, rows_n=None, rows_m=None,
                 group: int = GROUP, seed: int = SEED):
    """(x bf16 bits [M,K], q int8 [N,K], s fp16 bits [N,K/group]) of one projection."""
    p = LAYER_PROJECTIONS[proj_index]
    q = gen_q(tensor_id(KIND_Q, layer, proj_index), p.N, p.K, rows_n, seed)
    s = gen_scales(tensor_id(KIND_SCALES, layer, proj_index), p.N, p.K // group, rows_n, seed)
    x = gen_x(tensor_id(KIND_X, layer, proj_index, M), M, p.K, rows_m, seed)
    return x, q, s


def tiny_inputs(seed: int = SEED):
    t = TINY
    q = gen_q(tensor_id(KIND_Q, 0, TINY_PROJ), t["N"], t["K"], seed=seed)
    s = gen_scales(tensor_id(KIND_SCALES, 0, TINY_PROJ), t["N"], t["K"] // t["group"], seed=seed)
    x = gen_x(tensor_id(KIND_X, 0, TINY_PROJ, t["M"]), t["M"], t["K"], seed=seed)
    return x, q, s
