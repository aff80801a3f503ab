"""The C ABI from C: include/mgemm.h compiles as C99 (and as C++17), and a C
program linked against libmgemm calls the host-only entry points (version,
status strings, validation before any HIP call, launch plans, the ring
schedule) with plain pointers and sizes. No GPU needed."""
import os
import shutil
import subprocess

import pytest

import async_global_shared_amd as m

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
INC = os.path.join(ROOT, "include")

PROGRAM = r"""
#include <stdio.h>
#include <string.h>
#include "mgemm.h"

#define CHECK(c) do { if (!(c)) { printf("failed: %s\n", #c); return 1; } } while (0)

int main(void) {
    mgemm_plan_t p;
    int ev[4096];
    const float *A = (const float *)(uintptr_t)0x100000000ull;
    const float *B = (const float *)(uintptr_t)0x1000000000ull;
    float *C = (float *)(uintptr_t)0x10000000000ull;
    CHECK(mgemm_version() == MGEMM_VERSION);
    CHECK(mgemm_status_string(MGEMM_ERR_ARG) != NULL && strlen(mgemm_status_string(MGEMM_ERR_ARG)) > 0);
    /* validation precedes any HIP call */
    CHECK(mgemm_sgemm(-1, 8, 8, A, 8, B, 8, C, 8, 2, MGEMM_FILL_PIPED, NULL) == MGEMM_ERR_ARG);
    CHECK(mgemm_sgemm(8, 8, 8, A, 8, B, 8, C, 8, 0, MGEMM_FILL_PIPED, NULL) == MGEMM_ERR_ARG);
    CHECK(mgemm_sgemm(8, 8, 8, A, 8, B, 8, (float *)A, 8, 2, MGEMM_FILL_PIPED, NULL) == MGEMM_ERR_ALIAS);
    CHECK(mgemm_tile_copy(10, 10, A, 9, C, 10, 2, NULL) == MGEMM_ERR_ARG);
    /* the timed configuration's plan: 128x128 MFMA tile, 2-stage asynchronous ring */
    CHECK(mgemm_plan_sgemm(8192, 8192, 8192, A, 8192, B, 8192, C, 8192, 2, MGEMM_FILL_PIPED,
                           MGEMM_COMPUTE_MFMA, MGEMM_TILE_128x128, MGEMM_LOADER_AUTO, &p) == MGEMM_OK);
    CHECK(p.bm == 128 && p.bn == 128 && p.blocks == 4096 && p.slices == 512 && p.load_bytes == 16);
    CHECK(p.lds_bytes == 2 * (128 * 16 + 16 * 128) * 4 && p.threads == 256);
    /* the ring schedule of 2 stages over 5 slices is enumerable on the host */
    CHECK(mgemm_ring_trace(0, 2, MGEMM_FILL_PIPED, 5, ev, 4096) > 0);
    printf("ok %d %d %d\n", p.bm, p.blocks, p.slices);
    return 0;
}
"""


@pytest.fixture(scope="module")
def built():
    if not os.path.exists(m.LIB_PATH):
        pytest.skip("libmgemm is not built")
    return os.path.dirname(m.LIB_PATH)


def test_header_compiles_as_c99_and_cxx17(tmp_path):
    src = tmp_path / "h.c"
    src.write_text('#include "mgemm.h"\nint main(void) { return mgemm_version() == MGEMM_VERSION ? 0 : 1; }\n')
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror", "-fsyntax-only", "-I", INC,
                    str(src)], check=True)
    subprocess.run(["g++", "-std=c++17", "-Wall", "-Wextra", "-pedantic", "-Werror", "-fsyntax-only", "-x", "c++",
                    "-I", INC, str(src)], check=True)


def test_c_program_calls_the_abi(tmp_path, built):
    if shutil.which("gcc") is None:
        pytest.skip("no gcc")
    src = tmp_path / "abi.c"
    src.write_text(PROGRAM)
    exe = tmp_path / "abi"
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-I", INC, str(src), "-o", str(exe), "-L", built,
                    "-lmgemm", "-Wl,-rpath," + built, "-Wl,-rpath-link,/opt/rocm/lib"], check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.startswith("ok 128 4096 512"), r.stdout
