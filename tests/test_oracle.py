"""The oracle against facts fixed by mathematics and the pages (CPU only)."""
import os
import subprocess
import tempfile

import numpy as np
import pytest

import oracle
from tests import oracle_pins


@pytest.fixture(scope="module")
def lib():
    oracle.build()
    return oracle.load()


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(lib, pin):
    pin(lib)


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
        for pin in oracle_pins.ALL_PINS:
            try:
                pin(lib)
            except (AssertionError, ValueError, OverflowError):
                # a NaN or inf read from padding surfaces as ValueError
                failed.append(pin.__name__)
        assert failed, f"mutant {name} passed every pin"
