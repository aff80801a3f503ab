"""The oracle against facts fixed by mathematics and the pages (CPU only)."""
import os
import subprocess
import tempfile

import numpy as np
import pytest

import oracle
from tests import oracle16_pins, oracle_attn_pins, oracle_pins


@pytest.fixture(scope="module")
def lib():
    oracle.build()
    return oracle.load()


ALL = list(oracle_pins.ALL_PINS) + list(oracle16_pins.ALL_PINS16) + list(oracle_attn_pins.ALL_ATTN_PINS)


@pytest.mark.parametrize("pin", ALL, ids=lambda f: f.__name__)
def test_pin(lib, pin):
    pin(lib)


def test_thread_count_does_not_change_results(lib):
    """Each output row is one thread's sequential sum, so the oracle's thread
    count (set for timing) changes no bit of its result."""
    import datagen
    A = datagen.matrix("uniform", 41, 37, 53)
    B = datagen.matrix("uniform", 42, 53, 29)
    threads = oracle.num_threads(lib)
    try:
        oracle.set_threads(1, lib)
        assert oracle.num_threads(lib) == 1
        one = oracle.gemm_f64(A, B)
    finally:
        oracle.set_threads(threads, lib)
    assert oracle.num_threads(lib) == threads
    assert oracle.gemm_f64(A, B).tobytes() == one.tobytes()


def test_bound_formula():
    # slack 4, K terms, unit roundoff 2^-24 of fp32 round-to-nearest
    Abs = np.array([[1.0, 2.0]])
    assert np.array_equal(oracle.bound(1024, Abs), 4 * 1024 * 2.0 ** -24 * Abs)


# Deliberate mistakes planted in copies of the oracle's source. Each must be
# caught by at least one pin, which shows the pins can see that class of bug.
MUTANTS = {
    "drop_last_term": ("for (p = 0; p < K; ++p) {\n            const double a = (double)A",
                       "for (p = 0; p < K - 1; ++p) {\n            const double a = (double)A"),
    "transpose_A": ("(double)A[i * lda + p]", "(double)A[p * lda + i]"),
    "ignore_lda": ("(double)A[i * lda + p]", "(double)A[i * K + p]"),
    "wrong_sign": ("c[j] += a * (double)b[j];", "c[j] -= a * (double)b[j];"),
    "column_shift": ("c[j] += a * (double)b[j];", "c[j] += a * (double)b[(j + 1) % N];"),
    "abs_drops_sign_of_B": ("a * fabs((double)b[j])", "a * (double)b[j]"),
    "copy_short_row": ("(size_t)cols * sizeof(float)", "(size_t)(cols - 1) * sizeof(float)"),
    "f16_bias_off_by_one": ("x = ldexp((double)(f | 0x400), e - 25);", "x = ldexp((double)(f | 0x400), e - 24);"),
    "f16_no_subnormals": ("x = ldexp((double)f, -24);", "x = 0.0;"),
    "f16_drops_sign": ("return sign ? -x : x;", "return x;"),
    "bf16_wrong_shift": ("v.u = (uint32_t)h << 16;", "v.u = (uint32_t)h << 15;"),
    "gemm16_abs_keeps_b_sign": ("c[j] += a * (absolute ? fabs(bv) : bv);", "c[j] += a * bv;"),
    "gemm16_drops_first_term": ("for (p = 0; p < K; ++p) {\n            double a = oracle_decode16", "for (p = 1; p < K; ++p) {\n            double a = oracle_decode16"),
    "attn_drops_scale": ("s[j] = scale * acc;", "s[j] = acc;"),
    "attn_transposed_K": ("oracle_decode16(K[j * ldk + d], fmt)", "oracle_decode16(K[d * ldk + j], fmt)"),
    "attn_no_max": ("s[j] = exp(s[j] - mx);", "s[j] = exp(s[j]);"),
    "attn_max_of_first_key": ("if (s[j] > mx)", "if (j == 0)"),
    "attn_unnormalised": ("const double w = s[j] / sum;", "const double w = s[j];"),
    "attn_drops_last_key": ("for (j = 0; j < Sk; ++j) {\n            const double w", "for (j = 0; j < Sk - 1; ++j) {\n            const double w"),
    "attn_abs_keeps_sign": ("Wabs[i * ldo + c] += w * fabs(v);", "Wabs[i * ldo + c] += w * v;"),
    "attn_ignores_ldv": ("V[j * ldv + c]", "V[j * Dv + c]"),
    "attn_ignores_ldq": ("Q[i * ldq + d]", "Q[i * D + d]"),
    "attn_g_drops_abs_of_k": ("mag += fabs(q[d]) * fabs(k);", "mag += fabs(q[d]) * k;"),
    "attn_g_of_first_key": ("if (mag > gmax)", "if (j == 0)"),
    "attn_vmax_keeps_sign": ("const double v = fabs(oracle_decode16(V[j * ldv + c], fmt));", "const double v = oracle_decode16(V[j * ldv + c], fmt);"),
    "attn_query_shift": ("q[d] = oracle_decode16(Q[i * ldq + d], fmt);", "q[d] = oracle_decode16(Q[((i + 1) % Sq) * ldq + d], fmt);"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    old, new = MUTANTS[name]
    src = open(oracle.SRC).read()
    assert src.count(old) >= 1, name
    mutated = src.replace(old, new, 1)
    with tempfile.TemporaryDirectory() as d:
        path = os.path.join(d, "mut.c")
        with open(path, "w") as f:
            f.write(mutated)
        so = os.path.join(d, "libmut.so")
        subprocess.run(["gcc", *oracle.CFLAGS, path, "-o", so, "-lm"], check=True)
        lib = oracle.load(so)
        failed = []
        for pin in ALL:
            try:
                pin(lib)
            except (AssertionError, ValueError, OverflowError):
                # a NaN or inf read from padding surfaces as ValueError
                failed.append(pin.__name__)
        assert failed, f"mutant {name} passed every pin"
