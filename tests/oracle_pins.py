"""Checks that tie the oracle to facts other than itself.

Each ``pin_*`` function takes a loaded oracle library (ctypes handle) and
raises AssertionError when the oracle disagrees with the fact it checks. The
test module runs them on the real oracle (they must pass) and on deliberately
broken copies of its source (at least one must fail each copy).
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np

import datagen
import oracle


def _padded(a: np.ndarray, extra: int, fill=np.nan) -> np.ndarray:
    """Return a view of a copy of ``a`` whose rows are ``extra`` floats longer."""
    out = np.full((a.shape[0], a.shape[1] + extra), fill, dtype=np.float32)
    out[:, :a.shape[1]] = a
    return out[:, :a.shape[1]]


def _exact(A, B):
    M, K = A.shape
    N = B.shape[1]
    C = [[Fraction(0)] * N for _ in range(M)]
    S = [[Fraction(0)] * N for _ in range(M)]
    for i in range(M):
        for j in range(N):
            s = Fraction(0)
            t = Fraction(0)
            for k in range(K):
                a = Fraction(float(A[i, k]))
                b = Fraction(float(B[k, j]))
                s += a * b
                t += abs(a) * abs(b)
            C[i][j] = s
            S[i][j] = t
    return C, S


def pin_bruteforce_exact(lib, cases: int = 40, seed: int = 11) -> None:
    """Tiny shapes 1..9 with padded leading dimensions vs exact rational sums.
    U[-1,1) values on the 2^-23 grid: each product lies on the 2^-46 grid
    and |sum| <= 9 < 2^4, so 50 bits hold every partial sum and the fp64
    result must equal the exact rational value."""
    rng = np.random.default_rng(seed)
    for c in range(cases):
        M, N, K = (int(x) for x in rng.integers(1, 10, size=3))
        A = datagen.uniform_pm1(100 + c, M * K).reshape(M, K)
        B = datagen.uniform_pm1(200 + c, K * N).reshape(K, N)
        Ap = _padded(A, int(rng.integers(0, 5)))
        Bp = _padded(B, int(rng.integers(0, 5)))
        C = oracle.gemm_f64(Ap, Bp, lib=lib)
        S = oracle.abs_gemm_f64(Ap, Bp, lib=lib)
        Ce, Se = _exact(A, B)
        for i in range(M):
            for j in range(N):
                assert Fraction(C[i, j]) == Ce[i][j], (M, N, K, i, j)
                assert Fraction(S[i, j]) == Se[i][j], (M, N, K, i, j)


def pin_closed_forms(lib) -> None:
    """Products whose value is fixed by algebra, exact in any order."""
    M, N, K = 37, 29, 53
    ones_a = np.ones((M, K), np.float32)
    ones_b = np.ones((K, N), np.float32)
    C = oracle.gemm_f64(_padded(ones_a, 3), _padded(ones_b, 5), lib=lib)
    assert np.all(C == K)
    A = datagen.uniform_pm1(7, M * K).reshape(M, K)
    # A . I = A
    I = np.eye(K, dtype=np.float32)
    assert np.array_equal(oracle.gemm_f64(_padded(A, 2), _padded(I, 1), lib=lib), A.astype(np.float64))
    # I . A = A
    Im = np.eye(M, dtype=np.float32)
    assert np.array_equal(oracle.gemm_f64(Im, A, lib=lib), A.astype(np.float64))
    # P . A = A with permuted rows: (P A)[i] = A[perm[i]]
    perm = np.random.default_rng(3).permutation(M)
    P = np.zeros((M, M), np.float32)
    P[np.arange(M), perm] = 1.0
    assert np.array_equal(oracle.gemm_f64(P, _padded(A, 4), lib=lib), A[perm].astype(np.float64))
    # one nonzero a at (i0, k0): C = a * B[k0, :] on row i0, zero elsewhere
    B = datagen.uniform_pm1(8, K * N).reshape(K, N)
    E = np.zeros((M, K), np.float32)
    i0, k0 = 5, 41
    E[i0, k0] = 0.75
    C = oracle.gemm_f64(_padded(E, 2), _padded(B, 3), lib=lib)
    want = np.zeros((M, N))
    want[i0] = 0.75 * B[k0].astype(np.float64)
    assert np.array_equal(C, want)
    # K = 1: outer product
    a = datagen.uniform_pm1(9, M).reshape(M, 1)
    b = datagen.uniform_pm1(10, N).reshape(1, N)
    assert np.array_equal(oracle.gemm_f64(a, b, lib=lib), a.astype(np.float64) * b.astype(np.float64))
    # K = 0: empty sum
    assert np.all(oracle.gemm_f64(np.zeros((M, 0), np.float32), np.zeros((0, N), np.float32), lib=lib) == 0.0)


def pin_coarse_grid_integer(lib) -> None:
    """Values on the 2^-4 grid: 16A and 16B are small integers, so 256*C is an
    exact int64 matrix product (numpy's integer matmul, no rounding)."""
    for (M, N, K) in ((64, 64, 256), (33, 70, 129)):
        A = datagen.matrix("coarse", 21, M, K)
        B = datagen.matrix("coarse", 22, K, N)
        Ai = (A * 16).astype(np.int64)
        Bi = (B * 16).astype(np.int64)
        want = (Ai @ Bi).astype(np.float64) / 256.0
        assert np.array_equal(oracle.gemm_f64(_padded(A, 3), B, lib=lib), want)
        wabs = (np.abs(Ai) @ np.abs(Bi)).astype(np.float64) / 256.0
        assert np.array_equal(oracle.abs_gemm_f64(A, _padded(B, 1), lib=lib), wabs)


def pin_slice_sentinel(lib) -> None:
    """A = 1 and B[k, j] = floor(k / 16) (and the mirror) give
    C_ij = 16 T (T-1) / 2 + r T with T = K // 16, r = K % 16."""
    for K in (1, 15, 16, 17, 200, 1537):
        T, r = K // 16, K % 16
        want = 16 * T * (T - 1) // 2 + r * T
        M, N = 9, 11
        C = oracle.gemm_f64(np.ones((M, K), np.float32), datagen.slice_sentinel(K, N, axis=0), lib=lib)
        assert np.all(C == want), K
        C = oracle.gemm_f64(datagen.slice_sentinel(M, K, axis=1), np.ones((K, N), np.float32), lib=lib)
        assert np.all(C == want), K


def pin_numpy_f64(lib) -> None:
    """Agreement with numpy's fp64 matmul (a different summation order)
    within the fp64 bound 2 K 2^-53 (|A||B|)."""
    M, N, K = 150, 170, 700
    A = datagen.matrix("uniform", 31, M, K)
    B = datagen.matrix("uniform", 32, K, N)
    C = oracle.gemm_f64(_padded(A, 7), _padded(B, 9), lib=lib)
    S = oracle.abs_gemm_f64(A, B, lib=lib)
    ref = A.astype(np.float64) @ B.astype(np.float64)
    sref = np.abs(A.astype(np.float64)) @ np.abs(B.astype(np.float64))
    assert np.all(np.abs(C - ref) <= 2 * K * 2.0 ** -53 * sref)
    assert np.allclose(S, sref, rtol=K * 2.0 ** -52, atol=0)


def pin_copy(lib) -> None:
    src = datagen.matrix("normal", 3, 45, 70, ld=77)
    dst = oracle.copy_f32(src[:, :70], lib=lib)
    assert dst.tobytes() == np.ascontiguousarray(src[:, :70]).tobytes()


ALL_PINS = (pin_bruteforce_exact, pin_closed_forms, pin_coarse_grid_integer,
            pin_slice_sentinel, pin_numpy_f64, pin_copy)
