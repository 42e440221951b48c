"""In-tree build of the HIP library libw4a16.so for gfx950 (hipcc, no JIT)."""
from __future__ import annotations

import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libw4a16.so")
SOURCES = ["w4a16_host.cpp", "w4a16_plain.hip", "w4a16_skinny.hip", "w4a16_large.hip", "w4a8.hip",
           "w4a16_probe.hip", "w4a16_noalloc.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def command(out: str) -> list[str]:
    return [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
            "-Wall", "-Werror=return-type",
            # no packed-fp32 VALU forms anywhere in the device code
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", os.path.join(ROOT, "include"),
            *[os.path.join(CSRC, s) for s in SOURCES],
            "-Wl,-rpath,/opt/rocm/lib", "-o", out]


def build() -> str:
    tmp = LIB + ".tmp"
    proc = subprocess.run(command(tmp), capture_output=True, text=True)
    if proc.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + proc.stdout + proc.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
