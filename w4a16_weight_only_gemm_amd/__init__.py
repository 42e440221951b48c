"""Python binding of the MI355X W4A16 weight-only GEMM library (``libw4a16.so``).

Argument marshalling only: every step of the GEMM runs in the library's HIP
kernels, and packing runs in its host code. The names match the C ABI in
``include/w4a16.h``. PyTorch, when used, only provides device memory and the
current HIP stream. There is no fallback: if the library has not been built
(``python w4a16_weight_only_gemm_amd/_build.py`` or ``__graft_entry__.build()``),
importing this package raises.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

try:  # load torch's HIP runtime first so the library binds to the same one
    import torch as _torch
except ImportError:  # pragma: no cover - torch is optional for host-only use
    _torch = None

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libw4a16.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build it with `python w4a16_weight_only_gemm_amd/_build.py`")

_lib = ctypes.CDLL(LIB_PATH)

W4A16_OK = 0
W4A16_ERR_INVALID_ARG = 1
W4A16_ERR_UNSUPPORTED = 2
W4A16_ERR_MISALIGNED = 3
W4A16_ERR_LAUNCH = 4
W4A16_ERR_TOO_LARGE = 5
W4A16_NOALLOC_SCRATCH_BYTES = 96 << 20

W4A16_PATH_AUTO = 0
W4A16_PATH_SKINNY = 1
W4A16_PATH_LARGE = 2

W4A16_MAX_PROBLEMS = 8
W4A16_PLAN_MAX_PROBLEMS = 4096


class w4a16_problem(ctypes.Structure):
    _fields_ = [("x", ctypes.c_void_p), ("qweight", ctypes.c_void_p), ("scales", ctypes.c_void_p),
                ("y", ctypes.c_void_p), ("N", ctypes.c_int), ("K", ctypes.c_int)]

class w4a8_quantize_problem(ctypes.Structure):
    _fields_ = [("x", ctypes.c_void_p), ("xq", ctypes.c_void_p), ("sx", ctypes.c_void_p),
                ("K", ctypes.c_int)]


class w4a8_problem(ctypes.Structure):
    _fields_ = [("xq", ctypes.c_void_p), ("sx", ctypes.c_void_p), ("qweight", ctypes.c_void_p),
                ("scales", ctypes.c_void_p), ("y", ctypes.c_void_p), ("N", ctypes.c_int),
                ("K", ctypes.c_int)]

# Every symbol include/w4a16.h declares, with its ctypes signature.
_vp, _int, _sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
SIGNATURES = {
    "w4a16_qweight_bytes": (_sz, [_int, _int]),
    "w4a16_scales_bytes": (_sz, [_int, _int, _int]),
    "w4a16_pack": (_int, [_vp, _vp, _vp, _vp, _int, _int, _int]),
    "w4a16_gemm": (_int, [_vp, _vp, _vp, _vp, _int, _int, _int, _int, _vp]),
    "w4a16_gemm_ex": (_int, [_vp, _vp, _vp, _vp, _int, _int, _int, _int, _int, _vp]),
    "w4a16_workspace_bytes": (_sz, [_int, ctypes.c_longlong]),
    "w4a16_gemm_ws": (_int, [_vp, _vp, _vp, _vp, _int, _int, _int, _int, _vp, _sz, _vp]),
    "w4a16_gemm_grouped": (_int, [_vp, _int, _int, _int, _vp, _sz, _vp]),
    "w4a16_gemm_noalloc": (_int, [_vp, _vp, _vp, _vp, _int, _int, _int, _int, _vp]),
    "w4a16_plan_bytes": (_sz, [_int]),
    "w4a16_plan_build": (_int, [_vp, _int, _int, _int, _vp, _sz]),
    "w4a16_plan_workspace_bytes": (_sz, [_vp]),
    "w4a16_gemm_planned": (_int, [_vp, _vp, _vp, _sz, _vp]),
    "w4a16_select_path": (_int, [_int, _int, _int, _int]),
    "w4a16_select_form": (_int, [_int, _int, _int, _int, _int, _vp, _vp, _vp]),
    "w4a8_quantize": (_int, [_vp, _vp, _vp, _int, _int, _vp]),
    "w4a8_gemm": (_int, [_vp, _vp, _vp, _vp, _vp, _int, _int, _int, _int, _vp]),
    "w4a8_quantize_grouped": (_int, [_vp, _int, _int, _vp]),
    "w4a8_gemm_grouped": (_int, [_vp, _int, _int, _int, _vp]),
    "w4a16_status_string": (ctypes.c_char_p, [_int]),
    "w4a16_version": (_int, []),
    "w4a16_read_probe": (_int, [_vp, _sz, _vp, _sz, _vp]),
}
for _name, (_res, _args) in SIGNATURES.items():
    _fn = getattr(_lib, _name)
    _fn.restype = _res
    _fn.argtypes = _args


class W4A16Error(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {w4a16_status_string(status)}")


def w4a16_status_string(status: int) -> str:
    return _lib.w4a16_status_string(int(status)).decode()


def w4a16_version() -> int:
    return int(_lib.w4a16_version())


def w4a16_qweight_bytes(N: int, K: int) -> int:
    return int(_lib.w4a16_qweight_bytes(N, K))


def w4a16_scales_bytes(N: int, K: int, group: int) -> int:
    return int(_lib.w4a16_scales_bytes(N, K, group))


def w4a16_select_path(M: int, N: int, K: int, group: int) -> int:
    return int(_lib.w4a16_select_path(M, N, K, group))


def w4a16_select_form(M: int, N: int, K: int, group: int, path: int = 0):
    """(path, rows, cols, waves) of the kernel form w4a16_gemm_ex runs for the
    shape, or None for an unsupported shape."""
    r, c, w = ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
    p = int(_lib.w4a16_select_form(M, N, K, group, path, ctypes.byref(r), ctypes.byref(c),
                                   ctypes.byref(w)))
    return None if p < 0 else (p, r.value, c.value, w.value)


def w4a16_pack(q: np.ndarray, scales: np.ndarray, group: int):
    """Host packing: q int8 [N, K] in -8..7 and fp16 scales [N, K/group] (float16 or
    uint16 bit patterns) -> (qweight uint32, scales uint16) as flat arrays in the
    device arrangement (w4a16_qweight_bytes / w4a16_scales_bytes long)."""
    q = np.ascontiguousarray(q)
    if q.dtype != np.int8 or q.ndim != 2:
        raise TypeError("q must be a 2-D int8 array")
    s = np.ascontiguousarray(scales)
    if s.dtype == np.float16:
        s = s.view(np.uint16)
    if s.dtype != np.uint16 or s.ndim != 2:
        raise TypeError("scales must be a 2-D float16 or uint16 array")
    N, K = q.shape
    if group <= 0 or group % 32 != 0 or K % group != 0 or s.shape != (N, K // group):
        raise W4A16Error(W4A16_ERR_INVALID_ARG, "w4a16_pack")
    qw = np.empty(w4a16_qweight_bytes(N, K) // 4, dtype=np.uint32)
    sp = np.empty(w4a16_scales_bytes(N, K, group) // 2, dtype=np.uint16)
    rc = _lib.w4a16_pack(q.ctypes.data, s.ctypes.data, qw.ctypes.data, sp.ctypes.data, N, K, group)
    if rc != W4A16_OK:
        raise W4A16Error(rc, "w4a16_pack")
    return qw, sp


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if _torch is not None and isinstance(t, _torch.Tensor):
        if not t.is_cuda:
            raise ValueError("device tensor expected")
        if not t.is_contiguous():
            raise ValueError("contiguous tensor expected")
        return t.data_ptr()
    raise TypeError(f"unsupported buffer type {type(t)}")


def _stream(stream):
    if stream is None:
        if _torch is not None and _torch.cuda.is_available():
            return _torch.cuda.current_stream().cuda_stream
        return None
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream  # torch.cuda.Stream


def _packed_bytes(N: int, K: int, group: int):
    """Bytes the kernels read of the packed weights and scales: the device
    arrangement pads N up to whole 16-column blocks (w4a16_qweight_bytes and
    w4a16_scales_bytes), so a buffer of N * K / 2 bytes is too short when
    N % 16 != 0."""
    return int(_lib.w4a16_qweight_bytes(N, K)), int(_lib.w4a16_scales_bytes(N, K, group))


def _check_tensors(x, qweight, scales, y, M, N, K, group):
    """Size and dtype checks for torch tensors (raw addresses are the caller's business).
    Raises before anything reaches the library."""
    if _torch is None:
        return
    qbytes, sbytes = _packed_bytes(N, K, group)
    need = {"x": (x, 2 * M * K, True), "y": (y, 2 * M * N, True),
            "qweight": (qweight, qbytes, False), "scales": (scales, sbytes, False)}
    for name, (t, nbytes, bf16) in need.items():
        if isinstance(t, _torch.Tensor):
            if bf16 and t.dtype != _torch.bfloat16:
                raise TypeError(f"{name} must be torch.bfloat16")
            have = t.numel() * t.element_size()
            if have < nbytes:
                raise ValueError(f"{name} holds {have} bytes, needs {nbytes}")


def w4a16_gemm_ex(x, qweight, scales, y, M: int, N: int, K: int, group: int, path: int,
                  stream=None) -> None:
    """y[M, N] = x[M, K] . dequant(qweight, scales) on the GPU, asynchronously on `stream`
    (default: torch's current stream). Buffers are torch device tensors or raw device
    addresses. Raises W4A16Error on a non-OK status."""
    if group > 0 and K % group == 0:
        _check_tensors(x, qweight, scales, y, M, N, K, group)
    rc = _lib.w4a16_gemm_ex(_ptr(x), _ptr(qweight), _ptr(scales), _ptr(y), M, N, K, group, path,
                            _stream(stream))
    if rc != W4A16_OK:
        raise W4A16Error(rc, "w4a16_gemm_ex")


def w4a16_gemm(x, qweight, scales, y, M: int, N: int, K: int, group: int, stream=None) -> None:
    if group > 0 and K % group == 0:
        _check_tensors(x, qweight, scales, y, M, N, K, group)
    rc = _lib.w4a16_gemm(_ptr(x), _ptr(qweight), _ptr(scales), _ptr(y), M, N, K, group,
                         _stream(stream))
    if rc != W4A16_OK:
        raise W4A16Error(rc, "w4a16_gemm")


def gemm_status(x, qweight, scales, y, M, N, K, group, path=W4A16_PATH_AUTO, stream=None) -> int:
    """Raw status of w4a16_gemm_ex, without raising (for tests of the error paths)."""
    return int(_lib.w4a16_gemm_ex(_ptr(x), _ptr(qweight), _ptr(scales), _ptr(y), M, N, K, group,
                                  path, _stream(stream)))


def pack_status(q_ptr, s_ptr, qw_ptr, sp_ptr, N, K, group) -> int:
    """Raw status of w4a16_pack on raw host addresses (for tests of the error paths)."""
    return int(_lib.w4a16_pack(q_ptr, s_ptr, qw_ptr, sp_ptr, N, K, group))


def w4a16_workspace_bytes(M: int, total_columns: int) -> int:
    return int(_lib.w4a16_workspace_bytes(M, total_columns))


def w4a16_gemm_ws(x, qweight, scales, y, M: int, N: int, K: int, group: int, workspace,
                  workspace_bytes: int | None = None, stream=None) -> None:
    """As w4a16_gemm, with a zero-initialised device workspace (torch tensor or address);
    M <= 16 runs the streaming kernel."""
    if group > 0 and K % group == 0:
        _check_tensors(x, qweight, scales, y, M, N, K, group)
    if workspace_bytes is None:
        workspace_bytes = workspace.numel() * workspace.element_size()
    rc = _lib.w4a16_gemm_ws(_ptr(x), _ptr(qweight), _ptr(scales), _ptr(y), M, N, K, group,
                            _ptr(workspace), workspace_bytes, _stream(stream))
    if rc != W4A16_OK:
        raise W4A16Error(rc, "w4a16_gemm_ws")


def w4a16_gemm_noalloc(x, qweight, scales, y, M: int, N: int, K: int, group: int,
                       stream=None) -> None:
    """As w4a16_gemm_ws, with the library's static device scratch in place of a
    workspace (allocates nothing). Calls that can overlap on one GPU race."""
    if group > 0 and K % group == 0:
        _check_tensors(x, qweight, scales, y, M, N, K, group)
    rc = _lib.w4a16_gemm_noalloc(_ptr(x), _ptr(qweight), _ptr(scales), _ptr(y), M, N, K, group,
                                 _stream(stream))
    if rc != W4A16_OK:
        raise W4A16Error(rc, "w4a16_gemm_noalloc")


def noalloc_status(x, qweight, scales, y, M, N, K, group, stream=None) -> int:
    """Raw status of w4a16_gemm_noalloc, without raising (for tests of the error paths)."""
    return int(_lib.w4a16_gemm_noalloc(_ptr(x), _ptr(qweight), _ptr(scales), _ptr(y), M, N, K,
                                       group, _stream(stream)))


def make_problems(entries):
    """ctypes array of w4a16_problem from (x, qweight, scales, y, N, K) tuples."""
    arr = (w4a16_problem * len(entries))()
    for i, (x, qw, sp, y, N, K) in enumerate(entries):
        arr[i] = w4a16_problem(_ptr(x), _ptr(qw), _ptr(sp), _ptr(y), N, K)
    return arr


def w4a16_gemm_grouped(problems, M: int, group: int, workspace, workspace_bytes: int | None = None,
                       stream=None) -> None:
    """Several GEMMs sharing M and the group size; `problems` is a list of
    (x, qweight, scales, y, N, K) tuples or a make_problems() array."""
    if not isinstance(problems, ctypes.Array):
        for (x, qw, sp, y, N, K) in problems:
            if group > 0 and K % group == 0:
                _check_tensors(x, qw, sp, y, M, N, K, group)
    arr = problems if isinstance(problems, ctypes.Array) else make_problems(problems)
    if workspace_bytes is None:
        workspace_bytes = workspace.numel() * workspace.element_size()
    rc = _lib.w4a16_gemm_grouped(ctypes.cast(arr, ctypes.c_void_p), len(arr), M, group,
                                 _ptr(workspace), workspace_bytes, _stream(stream))
    if rc != W4A16_OK:
        raise W4A16Error(rc, "w4a16_gemm_grouped")


def w4a16_plan_bytes(count: int) -> int:
    return int(_lib.w4a16_plan_bytes(count))


def plan_build_status(problems, M: int, group: int):
    """(status, plan) of w4a16_plan_build: `plan` is a host uint8 array."""
    arr = problems if isinstance(problems, ctypes.Array) else make_problems(problems)
    nbytes = w4a16_plan_bytes(len(arr))
    plan = np.zeros(max(1, nbytes), dtype=np.uint8)
    rc = int(_lib.w4a16_plan_build(ctypes.cast(arr, ctypes.c_void_p), len(arr), M, group,
                                   plan.ctypes.data, nbytes))
    return rc, plan


def w4a16_plan_build(problems, M: int, group: int) -> np.ndarray:
    """Host plan (uint8 array) of GEMMs sharing M and the group size, from
    (x, qweight, scales, y, N, K) tuples or a make_problems() array; copy it to
    device memory and pass both copies to w4a16_gemm_planned."""
    if not isinstance(problems, ctypes.Array):
        for (x, qw, sp, y, N, K) in problems:
            if group > 0 and K % group == 0:
                _check_tensors(x, qw, sp, y, M, N, K, group)
    rc, plan = plan_build_status(problems, M, group)
    if rc != W4A16_OK:
        raise W4A16Error(rc, "w4a16_plan_build")
    return plan


def w4a16_plan_workspace_bytes(plan: np.ndarray) -> int:
    return int(_lib.w4a16_plan_workspace_bytes(plan.ctypes.data))


def planned_status(plan: np.ndarray, plan_dev, workspace, workspace_bytes: int,
                   stream=None) -> int:
    return int(_lib.w4a16_gemm_planned(plan.ctypes.data, _ptr(plan_dev), _ptr(workspace),
                                       workspace_bytes, _stream(stream)))


def w4a16_gemm_planned(plan: np.ndarray, plan_dev, workspace, workspace_bytes: int | None = None,
                       stream=None) -> None:
    """Every GEMM of a plan in one launch; plan_dev is a device copy of `plan`. A
    plan whose w4a16_plan_workspace_bytes is 0 takes workspace=None."""
    if workspace_bytes is None:
        workspace_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    rc = planned_status(plan, plan_dev, workspace, workspace_bytes, stream)
    if rc != W4A16_OK:
        raise W4A16Error(rc, "w4a16_gemm_planned")


def grouped_status(problems, M, group, workspace, workspace_bytes, stream=None) -> int:
    arr = problems if isinstance(problems, ctypes.Array) else make_problems(problems)
    return int(_lib.w4a16_gemm_grouped(ctypes.cast(arr, ctypes.c_void_p), len(arr), M, group,
                                       _ptr(workspace), workspace_bytes, _stream(stream)))


def _check_sizes(**need):
    """name=(tensor or address, bytes needed): size checks for torch tensors."""
    if _torch is None:
        return
    for name, (t, nbytes) in need.items():
        if isinstance(t, _torch.Tensor):
            have = t.numel() * t.element_size()
            if have < nbytes:
                raise ValueError(f"{name} holds {have} bytes, needs {nbytes}")


def w4a8_quantize(x, xq, sx, M: int, K: int, stream=None) -> None:
    """Row-wise int8 quantization of bf16 x[M][K] on the GPU: codes xq[M][K]
    (int8, arranged for the int8 MFMA) and row scales sx[M] (fp32)."""
    if _torch is not None and isinstance(x, _torch.Tensor) and x.dtype != _torch.bfloat16:
        raise TypeError("x must be torch.bfloat16")
    _check_sizes(x=(x, 2 * M * K), xq=(xq, M * K), sx=(sx, 4 * M))
    rc = _lib.w4a8_quantize(_ptr(x), _ptr(xq), _ptr(sx), M, K, _stream(stream))
    if rc != W4A16_OK:
        raise W4A16Error(rc, "w4a8_quantize")


def w4a8_gemm(xq, sx, qweight, scales, y, M: int, N: int, K: int, group: int,
              stream=None) -> None:
    """y[M][N] (bf16) = W4A8 product of the codes and row scales written by
    w4a8_quantize and the packed weights written by w4a16_pack."""
    if group > 0 and K % group == 0:
        qbytes, sbytes = _packed_bytes(N, K, group)
        _check_sizes(xq=(xq, M * K), sx=(sx, 4 * M), y=(y, 2 * M * N),
                     qweight=(qweight, qbytes), scales=(scales, sbytes))
    rc = _lib.w4a8_gemm(_ptr(xq), _ptr(sx), _ptr(qweight), _ptr(scales), _ptr(y), M, N, K, group,
                        _stream(stream))
    if rc != W4A16_OK:
        raise W4A16Error(rc, "w4a8_gemm")


def w4a8_quantize_status(x, xq, sx, M, K, stream=None) -> int:
    """Raw status of w4a8_quantize, without raising (for tests of the error paths)."""
    return int(_lib.w4a8_quantize(_ptr(x), _ptr(xq), _ptr(sx), M, K, _stream(stream)))


def w4a8_gemm_status(xq, sx, qweight, scales, y, M, N, K, group, stream=None) -> int:
    """Raw status of w4a8_gemm, without raising (for tests of the error paths)."""
    return int(_lib.w4a8_gemm(_ptr(xq), _ptr(sx), _ptr(qweight), _ptr(scales), _ptr(y), M, N, K,
                              group, _stream(stream)))


def make_w4a8_quantize_problems(entries):
    """ctypes array of w4a8_quantize_problem from (x, xq, sx, K) tuples."""
    arr = (w4a8_quantize_problem * len(entries))()
    for i, (x, xq, sx, K) in enumerate(entries):
        arr[i] = w4a8_quantize_problem(_ptr(x), _ptr(xq), _ptr(sx), K)
    return arr


def make_w4a8_problems(entries):
    """ctypes array of w4a8_problem from (xq, sx, qweight, scales, y, N, K) tuples."""
    arr = (w4a8_problem * len(entries))()
    for i, (xq, sx, qw, sp, y, N, K) in enumerate(entries):
        arr[i] = w4a8_problem(_ptr(xq), _ptr(sx), _ptr(qw), _ptr(sp), _ptr(y), N, K)
    return arr


def w4a8_quantize_grouped_status(problems, M, stream=None) -> int:
    arr = problems if isinstance(problems, ctypes.Array) else make_w4a8_quantize_problems(problems)
    return int(_lib.w4a8_quantize_grouped(ctypes.cast(arr, ctypes.c_void_p), len(arr), M,
                                          _stream(stream)))


def w4a8_quantize_grouped(problems, M: int, stream=None) -> None:
    """Several row-wise quantizations sharing M in one launch; `problems` is a
    list of (x, xq, sx, K) tuples or a make_w4a8_quantize_problems() array."""
    if not isinstance(problems, ctypes.Array):
        for (x, xq, sx, K) in problems:
            _check_sizes(x=(x, 2 * M * K), xq=(xq, M * K), sx=(sx, 4 * M))
    rc = w4a8_quantize_grouped_status(problems, M, stream)
    if rc != W4A16_OK:
        raise W4A16Error(rc, "w4a8_quantize_grouped")


def w4a8_gemm_grouped_status(problems, M, group, stream=None) -> int:
    arr = problems if isinstance(problems, ctypes.Array) else make_w4a8_problems(problems)
    return int(_lib.w4a8_gemm_grouped(ctypes.cast(arr, ctypes.c_void_p), len(arr), M, group,
                                      _stream(stream)))


def w4a8_gemm_grouped(problems, M: int, group: int, stream=None) -> None:
    """Several W4A8 GEMMs sharing M and the group size in one launch; `problems`
    is a list of (xq, sx, qweight, scales, y, N, K) tuples or a
    make_w4a8_problems() array."""
    if not isinstance(problems, ctypes.Array):
        for (xq, sx, qw, sp, y, N, K) in problems:
            if group > 0 and K % group == 0:
                qbytes, sbytes = _packed_bytes(N, K, group)
                _check_sizes(xq=(xq, M * K), sx=(sx, 4 * M), y=(y, 2 * M * N),
                             qweight=(qw, qbytes), scales=(sp, sbytes))
    rc = w4a8_gemm_grouped_status(problems, M, group, stream)
    if rc != W4A16_OK:
        raise W4A16Error(rc, "w4a8_gemm_grouped")


READ_PROBE_SINK_BYTES = 8192


def read_probe_status(buf, nbytes: int, sink, sink_bytes: int = READ_PROBE_SINK_BYTES,
                      stream=None) -> int:
    return int(_lib.w4a16_read_probe(_ptr(buf), nbytes, _ptr(sink), sink_bytes, _stream(stream)))


def w4a16_read_probe(buf, nbytes: int, sink, sink_bytes: int = READ_PROBE_SINK_BYTES,
                     stream=None) -> None:
    """Read `nbytes` of device memory at `buf` once in the weight-stream access
    pattern (a measurement aid: the practical read-bandwidth ceiling); one
    32-bit wrapping sum per workgroup goes into the zero-filled `sink`."""
    rc = read_probe_status(buf, nbytes, sink, sink_bytes, stream)
    if rc != W4A16_OK:
        raise W4A16Error(rc, "w4a16_read_probe")
