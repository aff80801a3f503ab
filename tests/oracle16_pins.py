"""Pins of the oracle's 16-bit (bfloat16 / binary16) decoders and GEMM, each a
function of a loaded oracle library that raises AssertionError on mismatch."""
from fractions import Fraction

import numpy as np

import datagen
import oracle


def _decoded_by_library(bits: np.ndarray, fmt: str) -> np.ndarray:
    """Values of 16-bit patterns via library conversions (numpy binary16,
    torch bfloat16), not the oracle."""
    if fmt == "f16":
        return bits.astype(np.uint16).view(np.float16).astype(np.float64)
    import torch
    t = torch.from_numpy(bits.astype(np.uint16).view(np.int16).copy()).view(torch.bfloat16)
    return t.to(torch.float64).numpy()


def pin_decoders_all_patterns(lib):
    allbits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    for fmt in ("f16", "bf16"):
        want = _decoded_by_library(allbits, fmt)
        got = np.array([lib.oracle_decode16(int(b), oracle.FMT[fmt]) for b in allbits])
        nan = np.isnan(want)
        assert np.array_equal(np.isnan(got), nan), fmt
        assert np.array_equal(got[~nan], want[~nan]), fmt
        assert np.array_equal(np.signbit(got[~nan]), np.signbit(want[~nan])), fmt


def pin_gemm16_bruteforce(lib, cases=30):
    rng = np.random.default_rng(5)
    for c in range(cases):
        fmt = ("bf16", "f16")[c % 2]
        M, N, K = (int(x) for x in rng.integers(1, 9, size=3))
        A = datagen.matrix16(300 + c, M, K, fmt, ld=K + int(rng.integers(0, 3)))[:, :K]
        B = datagen.matrix16(400 + c, K, N, fmt, ld=N + int(rng.integers(0, 3)))[:, :N]
        C = oracle.gemm16_f64(A, B, fmt, lib=lib)
        S = oracle.gemm16_f64(A, B, fmt, absolute=True, lib=lib)
        a = _decoded_by_library(np.ascontiguousarray(A), fmt)
        b = _decoded_by_library(np.ascontiguousarray(B), fmt)
        for i in range(M):
            for j in range(N):
                e = sum((Fraction(a[i, k]) * Fraction(b[k, j]) for k in range(K)), Fraction(0))
                ea = sum((abs(Fraction(a[i, k])) * abs(Fraction(b[k, j])) for k in range(K)), Fraction(0))
                assert Fraction(C[i, j]) == e and Fraction(S[i, j]) == ea, (fmt, M, N, K, i, j)


def pin_gemm16_closed_forms(lib):
    for fmt in ("bf16", "f16"):
        M, N, K = 33, 21, 70
        ones_a = datagen.matrix16(0, M, K, fmt, kind="ones")
        ones_b = datagen.matrix16(0, K, N, fmt, kind="ones")
        assert np.all(oracle.gemm16_f64(ones_a, ones_b, fmt, lib=lib) == K)
        B = datagen.matrix16(9, K, N, fmt)
        I = datagen.to_bits16(np.eye(K, dtype=np.float32), fmt)
        assert np.array_equal(oracle.gemm16_f64(I, B, fmt, lib=lib), _decoded_by_library(B, fmt))
        # integer-exact grid: 16 x values are small integers, numpy's int64 matmul is exact
        A = datagen.matrix16(11, M, K, fmt, kind="coarse")
        Bc = datagen.matrix16(12, K, N, fmt, kind="coarse")
        Ai = (_decoded_by_library(A, fmt) * 16).astype(np.int64)
        Bi = (_decoded_by_library(Bc, fmt) * 16).astype(np.int64)
        assert np.array_equal(oracle.gemm16_f64(A, Bc, fmt, lib=lib), (Ai @ Bi) / 256.0)
        assert np.array_equal(oracle.gemm16_f64(A, Bc, fmt, absolute=True, lib=lib),
                              (np.abs(Ai) @ np.abs(Bi)) / 256.0)


ALL_PINS16 = (pin_decoders_all_patterns, pin_gemm16_bruteforce, pin_gemm16_closed_forms)
