"""Build libmgemm for gfx950 in-tree (async_global_shared_amd/_build/).

Produces the shared library and, beside it, the device assembly of the same
translation unit (used by the tests that inspect the generated ISA).
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(HERE, "csrc", "mgemm.hip")
OUT = os.path.join(HERE, "_build")
LIB = os.path.join(OUT, "libmgemm.so")
ISA = os.path.join(OUT, "mgemm-gfx950.s")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-ffp-contract=off",
    # packed fp32 (v_pk_*_f32) stays off: plain v_fma_f32 and MFMA only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I" + os.path.join(ROOT, "include"), "-Wall",
]


def _run(cmd):
    p = subprocess.run(cmd, capture_output=True, text=True)
    noise = "'-packed-fp32-ops' is not a recognized feature"
    err = "\n".join(l for l in p.stderr.splitlines() if noise not in l and "unused during compilation" not in l)
    if p.returncode != 0:
        raise RuntimeError(f"build failed: {' '.join(cmd)}\n{err}")
    if err.strip():
        sys.stderr.write(err + "\n")


def build() -> str:
    """Compile (always) and return the library path."""
    os.makedirs(OUT, exist_ok=True)
    tmp = LIB + ".tmp%d" % os.getpid()
    lib_cmd = [HIPCC, *FLAGS, "-fPIC", "-shared", SRC, "-o", tmp]
    isa_cmd = [HIPCC, *FLAGS, "--cuda-device-only", "-S", SRC, "-o", ISA + ".tmp"]
    procs = [subprocess.Popen(c, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True) for c in (lib_cmd, isa_cmd)]
    for cmd, p in zip((lib_cmd, isa_cmd), procs):
        _, err = p.communicate()
        if p.returncode != 0:
            raise RuntimeError(f"build failed: {' '.join(cmd)}\n{err}")
    os.replace(tmp, LIB)
    os.replace(ISA + ".tmp", ISA)
    return LIB


if __name__ == "__main__":
    print(build())
