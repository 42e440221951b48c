"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

The library's host half (packing, every argument check, sizes, the plan
builder) is rebuilt with the sanitizers on its host code only (device code as
usual: `-Xarch_host -fsanitize=...` on the hipcc line) and driven in a child
process that preloads the sanitizer runtime: every call that returns before a
launch, across valid and invalid shapes, with packed words and plans compared
byte for byte against the ordinary build. The oracle (plain C) is rebuilt with
gcc's sanitizers and its pins are run against that build. Any sanitizer report
aborts the child, which fails the test. No GPU is used.
"""
import os
import subprocess
import sys
import textwrap

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "w4a16_weight_only_gemm_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SOURCES = ["w4a16_host.cpp", "w4a16_plain.hip", "w4a16_skinny.hip", "w4a16_large.hip", "w4a8.hip",
           "w4a16_probe.hip", "w4a16_noalloc.hip"]
SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1:abort_on_error=1",
           "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}


def _tool_out(cmd):
    return subprocess.run(cmd, capture_output=True, text=True).stdout.strip()


@pytest.fixture(scope="module")
def sanitized_lib(tmp_path_factory):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    out = str(tmp_path_factory.mktemp("asan") / "libw4a16_san.so")
    cmd = [HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-shared",
           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-I", os.path.join(ROOT, "include"), *[os.path.join(CSRC, s) for s in SOURCES],
           "-Wl,-rpath,/opt/rocm/lib", "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    runtime = _tool_out([HIPCC, "-print-file-name=libclang_rt.asan-x86_64.so"])
    assert os.path.exists(runtime), runtime
    return out, runtime


DRIVER = textwrap.dedent(r'''
    import ctypes, sys
    import numpy as np
    sys.path.insert(0, ROOT)
    import w4a16_weight_only_gemm_amd as w4   # the ordinary build, for comparison
    san = ctypes.CDLL(LIB)
    for name, (res, args) in w4.SIGNATURES.items():
        fn = getattr(san, name)
        fn.restype, fn.argtypes = res, args
    ref = w4._lib
    rng = np.random.default_rng(0)
    # packing: every group size, ragged N, bytes identical to the ordinary build
    for (N, K, g) in [(1, 32, 32), (20, 256, 64), (33, 512, 128), (16, 256, 256), (70, 1024, 32),
                      (5, 96, 32), (48, 384, 128)]:
        if K % g:
            continue
        q = rng.integers(-8, 8, (N, K)).astype(np.int8)
        s = rng.integers(0, 1 << 16, (N, K // g)).astype(np.uint16)
        outs = []
        for lib in (san, ref):
            qw = np.zeros(lib.w4a16_qweight_bytes(N, K) // 4, np.uint32)
            sp = np.zeros(lib.w4a16_scales_bytes(N, K, g) // 2, np.uint16)
            assert lib.w4a16_pack(q.ctypes.data, s.ctypes.data, qw.ctypes.data, sp.ctypes.data,
                                  N, K, g) == 0
            outs.append((qw, sp))
        assert np.array_equal(outs[0][0], outs[1][0]) and np.array_equal(outs[0][1], outs[1][1])
        bad = q.copy(); bad[N - 1, K - 1] = 8
        qw = np.zeros(san.w4a16_qweight_bytes(N, K) // 4, np.uint32)
        sp = np.zeros(san.w4a16_scales_bytes(N, K, g) // 2, np.uint16)
        assert san.w4a16_pack(bad.ctypes.data, s.ctypes.data, qw.ctypes.data, sp.ctypes.data,
                              N, K, g) == 1
        assert not qw.any()
    for args in [(-1, 64, 32), (4, 48, 32), (4, 96, 64), (4, 64, 0), (4, 64, 48)]:
        assert san.w4a16_pack(None, None, None, None, *args) == 1
    assert san.w4a16_pack(None, None, None, None, 0, 64, 32) == 0
    # sizes and the dispatch
    for M in (0, 1, 16, 17, 64, 192, 193, 1024, 100000):
        for cols in (0, 1, 52224, 248320):
            assert san.w4a16_workspace_bytes(M, cols) == ref.w4a16_workspace_bytes(M, cols)
        assert san.w4a16_select_path(M, 512, 256, 64) == ref.w4a16_select_path(M, 512, 256, 64)
    # the form models (host arithmetic over the shape): same choice in both builds
    outs = [(ctypes.c_int * 3)() for _ in range(2)]
    for M in (1, 2, 9, 16, 17, 64, 129, 320, 321, 4096):
        for (N, K, g) in ((1, 128, 32), (100, 2048, 64), (5120, 17408, 128), (34816, 5120, 128),
                          (248320, 5120, 128), (7000, 4096, 256)):
            for path in (0, 1, 2):
                rs = [lib.w4a16_select_form(M, N, K, g, path, ctypes.byref(o, 0), ctypes.byref(o, 4),
                                            ctypes.byref(o, 8)) for lib, o in zip((san, ref), outs)]
                assert rs[0] == rs[1] and list(outs[0]) == list(outs[1]), (M, N, K, g, path)
    for st in range(-1, 8):
        assert san.w4a16_status_string(st) == ref.w4a16_status_string(st)
    # argument checks of every GEMM entry point: each returns before any launch
    A, B = 1 << 20, (1 << 20) + 8    # aligned and misaligned dummy device addresses
    for fn in (san.w4a16_gemm,):
        assert fn(A, A, A, A, -1, 64, 256, 64, None) == 1
        assert fn(A, A, A, A, 0, 64, 256, 64, None) == 0
        assert fn(None, A, A, A, 1, 64, 256, 64, None) == 1
        assert fn(A, A, A, A, 1, 64, 256, 48, None) == 2
        assert fn(A, A, A, A, 1, 64, 200, 64, None) == 2
        assert fn(B, A, A, A, 1, 64, 256, 64, None) == 3
    assert san.w4a16_gemm_ex(A, A, A, A, 1, 64, 256, 64, 7, None) == 1
    assert san.w4a16_gemm_ws(A, A, A, A, 1, 64, 256, 64, None, 0, None) == 1
    assert san.w4a16_gemm_ws(A, A, A, A, 1, 64, 256, 64, B, 1 << 30, None) == 3
    assert san.w4a16_gemm_noalloc(A, A, A, A, 16, 2000000, 256, 64, None) == 5
    assert san.w4a16_gemm_noalloc(B, A, A, A, 1, 64, 256, 64, None) == 3
    probs = (w4.w4a16_problem * 9)()
    for i in range(9):
        probs[i] = w4.w4a16_problem(A, A, A, A, 64, 256)
    pp = ctypes.cast(probs, ctypes.c_void_p)
    assert san.w4a16_gemm_grouped(pp, 9, 1, 64, A, 1 << 30, None) == 1
    assert san.w4a16_gemm_grouped(pp, 2, 1, 64, None, 0, None) == 1
    assert san.w4a8_quantize(A, A, A, 1, 24, None) == 2
    assert san.w4a8_gemm(A, A, A, A, A, 1, 64, 256, 32, None) == 2
    assert san.w4a16_read_probe(A, 24, A, 8192, None) == 1
    # plans: many shapes and counts, bytes identical to the ordinary build
    shapes = [(7168, 5120), (5120, 6144), (34816, 5120), (5120, 17408), (200, 384), (33, 256)]
    for count in (1, 4, 8, 9, 256, 4096):
        arr = (w4.w4a16_problem * count)()
        for i in range(count):
            N, K = shapes[i % len(shapes)]
            base = (1 << 24) + i * (1 << 16)
            arr[i] = w4.w4a16_problem(base, base + 4096, base + 8192, base + 12288, N, K)
        ap = ctypes.cast(arr, ctypes.c_void_p)
        nb = san.w4a16_plan_bytes(count)
        for M in (1, 2, 16, 17, 64, 1024):
            plans = []
            for lib in (san, ref):
                plan = np.zeros(nb, np.uint8)
                assert lib.w4a16_plan_build(ap, count, M, 128, plan.ctypes.data, nb) == 0
                plans.append(plan)
            assert np.array_equal(plans[0], plans[1])
            ws = san.w4a16_plan_workspace_bytes(plans[0].ctypes.data)
            if ws:  # a workspace one byte short: refused before any launch
                assert san.w4a16_gemm_planned(plans[0].ctypes.data, A, A, ws - 1, None) == 1
        small = np.zeros(nb - 1, np.uint8)
        assert san.w4a16_plan_build(ap, count, 1, 128, small.ctypes.data, nb - 1) == 1
    assert san.w4a16_plan_bytes(0) == 0 and san.w4a16_plan_bytes(4097) == 0
    junk = np.zeros(4096, np.uint8)
    assert san.w4a16_plan_workspace_bytes(junk.ctypes.data) == 0
    assert san.w4a16_gemm_planned(junk.ctypes.data, A, A, 0, None) == 1
    print("SANITIZED_HOST_OK")
''')


def _run_child(code, env_extra, preload):
    env = dict(os.environ, **SAN_ENV, **env_extra)
    env["LD_PRELOAD"] = preload
    return subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, env=env,
                          timeout=600)


def test_host_library_under_sanitizers(sanitized_lib):
    lib, runtime = sanitized_lib
    code = f"ROOT = {ROOT!r}\nLIB = {lib!r}\n" + DRIVER
    r = _run_child(code, {}, runtime)
    assert r.returncode == 0 and "SANITIZED_HOST_OK" in r.stdout, (r.stdout[-2000:] + r.stderr[-4000:])
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr


def test_oracle_pins_under_sanitizers(tmp_path):
    out = str(tmp_path / "liboracle_san.so")
    r = subprocess.run(["gcc", "-O1", "-g", "-std=c11", "-fPIC", "-shared", "-Wall", "-Wextra",
                        "-ffp-contract=off", "-fno-fast-math", "-fsanitize=address,undefined",
                        "-fno-sanitize-recover=undefined", os.path.join(ROOT, "oracle", "oracle.c"),
                        "-o", out, "-lm", "-lpthread"], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    runtime = _tool_out(["gcc", "-print-file-name=libasan.so"])
    code = ("import sys, pytest\n"
            f"sys.exit(pytest.main(['-q', '-p', 'no:cacheprovider', "
            f"{os.path.join(ROOT, 'tests', 'test_oracle_pins.py')!r}, "
            f"{os.path.join(ROOT, 'tests', 'test_oracle_w4a8.py')!r}]))\n")
    r = _run_child(code, {"W4A16_ORACLE_LIB": out}, runtime)
    assert r.returncode == 0, (r.stdout[-3000:] + r.stderr[-3000:])
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr
