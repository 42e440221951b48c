"""Host-only tests of the C-ABI library: it loads without a GPU, exports every
function include/w4a16.h declares, packs bit for bit like the oracle, and
rejects bad arguments before any launch (no call here reaches a kernel)."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle
import pins
import synth
import w4a16_weight_only_gemm_amd as w4

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    text = open(os.path.join(ROOT, "include", "w4a16.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(w4a(?:16|8)_\w+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    names = _declared_functions()
    assert len(names) >= 8, names
    for name in ("w4a8_quantize", "w4a8_gemm", "w4a8_quantize_grouped", "w4a8_gemm_grouped"):
        assert name in names, name
    lib = ctypes.CDLL(w4.LIB_PATH)
    for name in names:
        assert hasattr(lib, name), f"{name} not exported"
        assert name in w4.SIGNATURES, f"{name} has no binding"


def test_version_and_status_strings():
    assert w4.w4a16_version() >= 100
    for st in range(6):
        assert w4.w4a16_status_string(st).startswith("W4A16_")
    assert "unknown" in w4.w4a16_status_string(99)


def test_sizes():
    assert w4.w4a16_qweight_bytes(7168, 5120) == 7168 * 5120 // 2
    assert w4.w4a16_scales_bytes(7168, 5120, 128) == 7168 * 40 * 2
    assert w4.w4a16_qweight_bytes(20, 64) == 32 * 64 // 2   # padded to 2 blocks of 16
    assert w4.w4a16_scales_bytes(20, 64, 32) == 32 * 2 * 2
    assert w4.w4a16_qweight_bytes(4, 48) == 0          # K % 32
    assert w4.w4a16_scales_bytes(4, 96, 64) == 0       # K % group
    assert w4.w4a16_qweight_bytes(-1, 8) == 0


def _lib_pack(q, s, g):
    try:
        return w4.w4a16_pack(q, s, g)
    except w4.W4A16Error as e:  # the pins expect ValueError for rejected input
        raise ValueError(str(e)) from e


def test_library_pack_golden_words():
    pins.pin_golden_words(_lib_pack)
    pins.pin_scale_layout(_lib_pack)
    pins.pin_pack_rejects(_lib_pack)


@pytest.mark.parametrize("shape", [(512, 256, 64), (96, 1024, 128), (40, 768, 256), (24, 64, 32)])
def test_library_pack_matches_oracle(shape):
    N, K, g = shape
    q = synth.gen_q(synth.tensor_id(synth.KIND_Q, 9, 0), N, K)
    s = synth.gen_scales(synth.tensor_id(synth.KIND_SCALES, 9, 0), N, K // g)
    qw_lib, sp_lib = w4.w4a16_pack(q, s, g)
    qw_ref, sp_ref = oracle.pack(q, s, g)
    assert np.array_equal(qw_lib, qw_ref)
    assert np.array_equal(sp_lib, sp_ref)


def test_library_pack_matches_oracle_full_projection():
    # the largest projection of the layer set (gate+up, 5120 x 34816), bit for bit
    p = synth.LAYER_PROJECTIONS[2]
    q = synth.gen_q(synth.tensor_id(synth.KIND_Q, 0, 2), p.N, p.K)
    s = synth.gen_scales(synth.tensor_id(synth.KIND_SCALES, 0, 2), p.N, p.K // synth.GROUP)
    qw_lib, sp_lib = w4.w4a16_pack(q, s, synth.GROUP)
    qw_ref, sp_ref = oracle.pack(q, s, synth.GROUP)
    assert np.array_equal(qw_lib, qw_ref) and np.array_equal(sp_lib, sp_ref)


def test_pack_rejects_and_writes_nothing():
    N, K, g = 4, 64, 32
    q = np.zeros((N, K), np.int8)
    q[3, 63] = -9
    s = np.ones((N, K // g), np.uint16)
    qw = np.full(w4.w4a16_qweight_bytes(N, K) // 4, 0xDEADBEEF, np.uint32)
    sp = np.full(w4.w4a16_scales_bytes(N, K, g) // 2, 0xABCD, np.uint16)
    rc = w4.pack_status(q.ctypes.data, s.ctypes.data, qw.ctypes.data, sp.ctypes.data, N, K, g)
    assert rc == w4.W4A16_ERR_INVALID_ARG
    assert (qw == 0xDEADBEEF).all() and (sp == 0xABCD).all()
    # bad shapes
    for (K2, g2) in [(60, 30), (64, 12), (64, 48), (12, 4), (96, 64)]:
        assert w4.pack_status(q.ctypes.data, s.ctypes.data, qw.ctypes.data, sp.ctypes.data,
                              N, K2, g2) == w4.W4A16_ERR_INVALID_ARG
    # null pointers with a non-empty shape, and the empty shape
    assert w4.pack_status(None, s.ctypes.data, qw.ctypes.data, sp.ctypes.data, N, K, g) == 1
    assert w4.pack_status(None, None, None, None, 0, K, g) == w4.W4A16_OK
    # a valid call right after the failures succeeds
    q[3, 63] = 7
    assert w4.pack_status(q.ctypes.data, s.ctypes.data, qw.ctypes.data, sp.ctypes.data, N, K, g) == 0
    # column 3, k = 63: logical word 7 = group 1 (4 words per column per group of 32),
    # its word 3 -> lane 3*16 + 3 = 51 of tile 1 -> word 64 + 51 = 115; code 7 at nibble 7
    assert qw[115] == 0x70000000 and np.count_nonzero(qw) == 1


# Fake, never-dereferenced addresses: every call below fails its host checks
# before any HIP call, so no device is needed.
A = 0x10000  # 16-byte aligned


def test_gemm_argument_checks_without_launch():
    st = w4.gemm_status
    assert st(A, A, A, A, 0, 512, 256, 64) == w4.W4A16_OK                     # M == 0: no-op
    assert st(None, None, None, None, 0, 512, 256, 64) == w4.W4A16_OK
    assert st(None, A, A, A, 1, 512, 256, 64) == w4.W4A16_ERR_INVALID_ARG     # null x
    assert st(A, A, A, None, 1, 512, 256, 64) == w4.W4A16_ERR_INVALID_ARG     # null y
    assert st(A, A, A, A, -1, 512, 256, 64) == w4.W4A16_ERR_INVALID_ARG
    assert st(A, A, A, A, 1, -5, 256, 64) == w4.W4A16_ERR_INVALID_ARG
    assert st(A, A, A, A, 1, 512, 256, 48) == w4.W4A16_ERR_UNSUPPORTED       # group
    assert st(A, A, A, A, 1, 512, 250, 64) == w4.W4A16_ERR_UNSUPPORTED       # K % group
    assert st(A, A, A, A, 1, 0, 256, 64) == w4.W4A16_ERR_UNSUPPORTED
    assert st(A, A, A, A, 1, 512, 0, 64) == w4.W4A16_ERR_UNSUPPORTED
    # past plain_kernel's 65535 row tiles only the tile engine runs: not at group 256
    big = 65535 * 16 + 1
    assert st(A, A, A, A, big, 512, 256, 256) == w4.W4A16_ERR_UNSUPPORTED
    assert st(A, A, A, A, big, 512, 256, 256, path=w4.W4A16_PATH_SKINNY) == w4.W4A16_ERR_UNSUPPORTED
    assert st(A + 2, A, A, A, 1, 512, 256, 64) == w4.W4A16_ERR_MISALIGNED
    assert st(A, A + 8, A, A, 1, 512, 256, 64) == w4.W4A16_ERR_MISALIGNED
    assert st(A, A, A + 4, A, 1, 512, 256, 64) == w4.W4A16_ERR_MISALIGNED
    assert st(A, A, A, A + 2, 1, 512, 256, 64) == w4.W4A16_ERR_MISALIGNED
    assert st(A, A, A, A, 1, 512, 256, 64, path=7) == w4.W4A16_ERR_INVALID_ARG


def test_select_path():
    S, L = w4.W4A16_PATH_SKINNY, w4.W4A16_PATH_LARGE
    assert w4.w4a16_select_path(1, 7168, 5120, 128) == S
    assert w4.w4a16_select_path(16, 5120, 17408, 128) == S
    assert w4.w4a16_select_path(16, 34816, 5120, 128) == S          # up to 16 rows: always
    assert w4.w4a16_select_path(17, 34816, 5120, 128) == S          # 4-wave 32-row XS form
    assert w4.w4a16_select_path(33, 34816, 5120, 128) == L          # 136 column tiles fill the CUs
    assert w4.w4a16_select_path(64, 34816, 5120, 128) == L
    assert w4.w4a16_select_path(64, 5120, 17408, 128) == S          # 20 column tiles do not
    assert w4.w4a16_select_path(192, 5120, 6144, 128) == S
    assert w4.w4a16_select_path(320, 5120, 6144, 128) == L
    assert w4.w4a16_select_path(1024, 5120, 6144, 128) == L
    assert w4.w4a16_select_path(1024, 16, 256, 128) == S            # one column block
    assert w4.w4a16_select_path(512, 896, 5120, 128) == S           # narrow: 4 column tiles
    assert w4.w4a16_select_path(65535 * 16 + 1, 896, 5120, 128) == L  # past plain_kernel's grid
    assert w4.w4a16_select_path(65535 * 16 + 1, 896, 5120, 256) == -1  # and no tile engine
    assert w4.w4a16_select_path(65535 * 16, 896, 5120, 256) == S
    assert w4.w4a16_select_path(64, 34816, 5120, 256) == S          # no tile engine at group 256
    assert w4.w4a16_select_path(1, 512, 256, 48) == -1
    assert w4.w4a16_select_path(-1, 512, 256, 64) == -1


# (M, N, K, group) -> (path, rows, cols, waves) that w4a16_gemm runs: the
# decode layer set (qkv 5120x7168, o 6144x5120, gate_up 5120x34816, down
# 17408x5120) at the row counts of its sweep, the time models' choices.
FORMS = {
    (1, 7168, 5120, 128): (1, 16, 16, 16), (1, 34816, 5120, 128): (1, 16, 48, 4),
    (1, 5120, 17408, 128): (1, 16, 32, 16), (16, 34816, 5120, 128): (1, 16, 80, 4),
    (8, 34816, 5120, 128): (1, 16, 80, 4), (1, 5120, 768, 128): (1, 16, 32, 8), (12, 5120, 17408, 128): (1, 16, 32, 8),
    (2, 7168, 5120, 128): (1, 16, 32, 8), (4, 896, 5120, 128): (1, 16, 16, 16),
    (8, 34816, 5120, 64): (1, 16, 64, 4), (1, 896, 17408, 128): (1, 16, 32, 16),
    (32, 7168, 5120, 128): (1, 32, 32, 16), (32, 34816, 5120, 128): (1, 32, 80, 4),
    (32, 5120, 17408, 128): (1, 16, 64, 8), (64, 7168, 5120, 128): (1, 32, 64, 16),
    (64, 5120, 6144, 128): (1, 32, 48, 16), (64, 34816, 5120, 128): (2, 64, 256, 8),
    (64, 5120, 17408, 128): (1, 16, 80, 8), (128, 7168, 5120, 128): (1, 64, 64, 16),
    (128, 5120, 17408, 128): (1, 32, 80, 8), (256, 7168, 5120, 128): (2, 32, 256, 8),
    (1024, 34816, 5120, 128): (2, 128, 256, 8), (1024, 5120, 17408, 128): (2, 32, 256, 8),
    (64, 5120, 17408, 64): (1, 64, 32, 4), (64, 34816, 5120, 64): (2, 64, 256, 8),
}


def test_select_form():
    for (M, N, K, g), want in FORMS.items():
        got = w4.w4a16_select_form(M, N, K, g)
        assert got == want, ((M, N, K, g), got, want)
        assert got[0] == w4.w4a16_select_path(M, N, K, g)
    # forced paths: the tile engine at any M (32-row tiles at 1 row), the small-M
    # kernel at any M; group 256 has no tile engine (w4a16_gemm_ex falls back)
    assert w4.w4a16_select_form(1, 7168, 5120, 128, w4.W4A16_PATH_LARGE) == (2, 32, 256, 8)
    assert w4.w4a16_select_form(1024, 5120, 6144, 128, w4.W4A16_PATH_SKINNY)[0] == 1
    assert w4.w4a16_select_form(1024, 5120, 6144, 256, w4.W4A16_PATH_LARGE)[0] == 1
    # past plain_kernel's grid: the tile engine on every path, or no kernel at group 256
    big = 65535 * 16 + 1
    assert w4.w4a16_select_form(big, 896, 5120, 128, w4.W4A16_PATH_SKINNY)[0] == 2
    assert w4.w4a16_select_form(big, 896, 5120, 256) is None
    assert w4.w4a16_select_form(big - 1, 896, 5120, 256)[0] == 1
    assert w4.w4a16_select_form(1, 512, 256, 48) is None
    assert w4.w4a16_select_form(1, 512, 256, 64, path=7) is None
    assert w4.w4a16_select_form(-1, 512, 256, 64) is None
    r = ctypes.c_int(-5)
    assert w4._lib.w4a16_select_form(1, 512, 256, 64, 0, None, ctypes.byref(r), ctypes.byref(r)) == -1
    assert r.value == -5


def test_select_form_bounds():
    """Every chosen form exists and tiles the output: rows 16..128, columns
    16..256 in 16-column blocks, 4..16 waves, over a grid of shapes."""
    for M in (1, 2, 3, 5, 9, 16, 17, 31, 33, 64, 65, 100, 200, 320, 321, 700, 5000):
        for N in (1, 16, 100, 1000, 5000, 34816, 248320):
            for K, g in ((128, 32), (256, 64), (5120, 128), (17408, 128), (4096, 256)):
                p, r, c, w = w4.w4a16_select_form(M, N, K, g)
                assert p in (1, 2) and r in (16, 32, 64, 128) and c % 16 == 0
                assert 16 <= c <= 256 and w in (4, 8, 16)


def test_workspace_sizes():
    assert w4.w4a16_workspace_bytes(-1, 10) == 0
    a = w4.w4a16_workspace_bytes(1, 52224)
    b = w4.w4a16_workspace_bytes(16, 52224)
    assert 0 < a < b
    # M > 16: per-tile counters and register-major parts of the MFMA tiles,
    # growing with the tile height (32, 64, 128 rows)
    c, d, e = (w4.w4a16_workspace_bytes(m, 52224) for m in (17, 64, 1024))
    assert 0 < c < d < e
    assert w4.w4a16_workspace_bytes(65, 52224) == w4.w4a16_workspace_bytes(128, 52224)
    assert w4.w4a16_workspace_bytes(0, 160) % 256 == 0


def test_grouped_argument_checks_without_launch():
    st = w4.grouped_status
    ok = (A, A, A, A, 512, 256)
    nb = w4.w4a16_workspace_bytes(4, 512)
    assert st([ok], 0, 64, A * 16, nb) == w4.W4A16_OK                        # M == 0
    assert st([ok] * 9, 4, 64, A * 16, nb) == w4.W4A16_ERR_INVALID_ARG        # too many
    assert st([ok], -1, 64, A * 16, nb) == w4.W4A16_ERR_INVALID_ARG
    assert st([ok], 4, 48, A * 16, nb) == w4.W4A16_ERR_UNSUPPORTED
    assert st([(A, A, A, A, 512, 200)], 4, 64, A * 16, nb) == w4.W4A16_ERR_UNSUPPORTED
    assert st([(A, None, A, A, 512, 256)], 4, 64, A * 16, nb) == w4.W4A16_ERR_INVALID_ARG
    assert st([(A + 4, A, A, A, 512, 256)], 4, 64, A * 16, nb) == w4.W4A16_ERR_MISALIGNED
    assert st([ok], 4, 64, None, nb) == w4.W4A16_ERR_INVALID_ARG              # no workspace
    assert st([ok], 4, 64, A * 16, nb - 1) == w4.W4A16_ERR_INVALID_ARG        # too small
    assert st([ok], 4, 64, A * 16 + 16, nb) == w4.W4A16_ERR_MISALIGNED        # not 256-aligned


def test_w4a8_argument_checks_without_launch():
    q = w4.w4a8_quantize_status
    assert q(A, A, A, 0, 256) == w4.W4A16_OK                                  # M == 0: no-op
    assert q(None, None, None, 0, 256) == w4.W4A16_OK
    assert q(A, A, A, -1, 256) == w4.W4A16_ERR_INVALID_ARG
    assert q(A, A, A, 1, -16) == w4.W4A16_ERR_INVALID_ARG
    assert q(None, A, A, 1, 256) == w4.W4A16_ERR_INVALID_ARG
    assert q(A, A, None, 1, 256) == w4.W4A16_ERR_INVALID_ARG
    assert q(A, A, A, 1, 200) == w4.W4A16_ERR_UNSUPPORTED                     # K % 16
    assert q(A, A, A, 1, 0) == w4.W4A16_ERR_UNSUPPORTED
    assert q(A + 2, A, A, 1, 256) == w4.W4A16_ERR_MISALIGNED
    assert q(A, A + 8, A, 1, 256) == w4.W4A16_ERR_MISALIGNED
    assert q(A, A, A + 4, 1, 256) == w4.W4A16_ERR_MISALIGNED
    g = w4.w4a8_gemm_status
    assert g(A, A, A, A, A, 0, 512, 256, 64) == w4.W4A16_OK                   # M == 0
    assert g(A, A, A, A, A, -1, 512, 256, 64) == w4.W4A16_ERR_INVALID_ARG
    assert g(A, None, A, A, A, 1, 512, 256, 64) == w4.W4A16_ERR_INVALID_ARG   # null sx
    assert g(A, A, A, A, None, 1, 512, 256, 64) == w4.W4A16_ERR_INVALID_ARG   # null y
    for group in (32, 256, 48):
        assert g(A, A, A, A, A, 1, 512, 1024, group) == w4.W4A16_ERR_UNSUPPORTED
    assert g(A, A, A, A, A, 1, 512, 320, 128) == w4.W4A16_ERR_UNSUPPORTED     # K % group
    assert g(A, A, A, A, A, 1, 0, 256, 64) == w4.W4A16_ERR_UNSUPPORTED
    assert g(A, A, A, A, A, 1, 1 << 20, 1 << 14, 128) == w4.W4A16_ERR_UNSUPPORTED  # 8 GB of weights
    for i in range(5):
        args = [A] * 5
        args[i] = A + 4
        assert g(*args, 1, 512, 256, 64) == w4.W4A16_ERR_MISALIGNED, i


def test_w4a8_grouped_argument_checks_without_launch():
    q = w4.w4a8_quantize_grouped_status
    ok = (A, A, A, 256)
    assert q([ok], 0) == w4.W4A16_OK                                          # M == 0
    assert q([ok] * 9, 4) == w4.W4A16_ERR_INVALID_ARG                         # too many
    assert q([ok], -1) == w4.W4A16_ERR_INVALID_ARG
    assert q([ok, (A, A, A, -16)], 4) == w4.W4A16_ERR_INVALID_ARG
    assert q([ok, (A, None, A, 256)], 4) == w4.W4A16_ERR_INVALID_ARG
    assert q([ok, (A, A, A, 40)], 4) == w4.W4A16_ERR_UNSUPPORTED
    assert q([ok, (A, A, A + 4, 256)], 4) == w4.W4A16_ERR_MISALIGNED
    g = w4.w4a8_gemm_grouped_status
    ok = (A, A, A, A, A, 512, 256)
    assert g([ok], 0, 64) == w4.W4A16_OK
    assert g([ok] * 9, 4, 64) == w4.W4A16_ERR_INVALID_ARG
    assert g([ok], -1, 64) == w4.W4A16_ERR_INVALID_ARG
    assert g([ok, (A, A, A, A, A, -1, 256)], 4, 64) == w4.W4A16_ERR_INVALID_ARG
    assert g([ok, (A, A, None, A, A, 512, 256)], 4, 64) == w4.W4A16_ERR_INVALID_ARG
    assert g([ok], 4, 32) == w4.W4A16_ERR_UNSUPPORTED
    assert g([ok, (A, A, A, A, A, 512, 352)], 4, 64) == w4.W4A16_ERR_UNSUPPORTED
    assert g([ok, (A, A, A, A, A + 2, 512, 256)], 4, 64) == w4.W4A16_ERR_MISALIGNED


def test_read_probe_rejects_bad_arguments_before_launch():
    """The read-bandwidth probe checks its arguments on the host; none of these
    calls reaches a kernel (bytes == 0 returns before any launch)."""
    ok, bad, mis = w4.W4A16_OK, w4.W4A16_ERR_INVALID_ARG, w4.W4A16_ERR_MISALIGNED
    buf, sink = 0x10000, 0x20000  # never dereferenced on these paths
    assert w4.read_probe_status(buf, 24, sink) == bad            # not a multiple of 16
    assert w4.read_probe_status(buf, 0, None) == bad             # no sink
    assert w4.read_probe_status(buf, 0, sink, 8188) == bad       # sink below 2,048 words
    assert w4.read_probe_status(buf, 0, sink + 2) == mis         # sink not 4-byte aligned
    assert w4.read_probe_status(0, 0, sink) == ok                # empty read: nothing launched
    assert w4.read_probe_status(None, 32, sink) == bad           # null buffer
    assert w4.read_probe_status(buf + 8, 32, sink) == mis        # buffer not 16-byte aligned


def test_binding_requires_padded_packed_sizes():
    """With N % 16 != 0 the kernels read whole 16-column blocks of the packed
    weights and scales: tensors sized to the unpadded N*K/2 and N*(K/group)*2
    must be rejected by the binding before anything reaches the library."""
    torch = pytest.importorskip("torch")
    M, N, K, g = 3, 20, 256, 64
    x = torch.zeros((M, K), dtype=torch.bfloat16)
    y = torch.zeros((M, N), dtype=torch.bfloat16)
    qw_short = torch.zeros(N * K // 8, dtype=torch.int32)            # N*K/2 bytes
    sp_short = torch.zeros(N * (K // g), dtype=torch.int16)          # N*(K/g)*2 bytes
    qw_full = torch.zeros(w4.w4a16_qweight_bytes(N, K) // 4, dtype=torch.int32)
    sp_full = torch.zeros(w4.w4a16_scales_bytes(N, K, g) // 2, dtype=torch.int16)
    assert qw_full.numel() * 4 > qw_short.numel() * 4
    for qw, sp, what in ((qw_short, sp_full, "qweight"), (qw_full, sp_short, "scales")):
        with pytest.raises(ValueError, match=what):
            w4.w4a16_gemm(x, qw, sp, y, M, N, K, g)
        with pytest.raises(ValueError, match=what):
            w4.w4a16_gemm_ex(x, qw, sp, y, M, N, K, g, w4.W4A16_PATH_SKINNY)
        with pytest.raises(ValueError, match=what):
            w4.w4a16_gemm_ws(x, qw, sp, y, M, N, K, g, torch.zeros(64, dtype=torch.int32))
        with pytest.raises(ValueError, match=what):
            w4.w4a16_gemm_grouped([(x, qw, sp, y, N, K)], M, g, torch.zeros(64, dtype=torch.int32))
        xq = torch.zeros((M, K), dtype=torch.int8)
        sx = torch.zeros((M,), dtype=torch.float32)
        with pytest.raises(ValueError, match=what):
            w4.w4a8_gemm(xq, sx, qw, sp, y, M, N, K, g)
        with pytest.raises(ValueError, match=what):
            w4.w4a8_gemm_grouped([(xq, sx, qw, sp, y, N, K)], M, g)
    # padded sizes pass the size check and only then meet the device check
    with pytest.raises(ValueError, match="device tensor"):
        w4.w4a16_gemm(x, qw_full, sp_full, y, M, N, K, g)
