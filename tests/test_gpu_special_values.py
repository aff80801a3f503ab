"""IEEE special values through the C ABI. An infinity or a NaN in A decides
its row of C exactly in any summation order: with B finite and non-zero,
A[i][k0] = +inf gives C[i][j] = sign(B[k0][j]) * inf, and A[i][k0] = NaN gives
NaN across row i. The same holds for infinities and NaNs in one column of B.
Every fill and depth must reproduce the oracle's class (and the sign of each
infinity) on those rows and columns, and stay within the bound elsewhere."""
import numpy as np
import pytest
import torch

import async_global_shared_amd as m
import datagen
import oracle
from tests.gpu_util import TILES, full_rows, out_device, padded_device
from tests.test_gpu_gemm16 import dev16

pytestmark = pytest.mark.gpu

M, N, K = 200, 150, 70


def _nonzero_uniform(seed, rows, cols):
    x = datagen.matrix("uniform", seed, rows, cols)
    x[x == 0] = 0.5
    return x


def _plant(A, B):
    A, B = A.copy(), B.copy()
    A[3, 10] = np.inf
    A[7, 0] = -np.inf
    A[11, K - 1] = np.nan
    B[20, 5] = np.inf
    B[K - 1, 9] = np.nan
    return A, B


def _check_classes(C, ref, what):
    """Rows 3, 7, 11 and columns 5, 9: same NaN / infinity pattern and signs
    as the fp64 oracle; elsewhere both are finite."""
    for sel in (np.s_[[3, 7, 11], :], np.s_[:, [5, 9]]):
        c, r = C[sel].astype(np.float64), ref[sel]
        assert np.array_equal(np.isnan(c), np.isnan(r)), what
        assert np.array_equal(np.isposinf(c), np.isposinf(r)), what
        assert np.array_equal(np.isneginf(c), np.isneginf(r)), what
    mask = np.ones((M, N), bool)
    mask[[3, 7, 11], :] = False
    mask[:, [5, 9]] = False
    assert np.all(np.isfinite(C[mask])) and np.all(np.isfinite(ref[mask])), what
    return mask


def _check_finite_part(C, ref, bnd, mask, what):
    err = np.abs(C[mask].astype(np.float64) - ref[mask])
    assert np.all(err <= bnd[mask]), what


def test_fp32_special_values():
    A, B = _plant(_nonzero_uniform(1, M, K), _nonzero_uniform(2, K, N))
    ref = oracle.gemm_f64(A, B)
    with np.errstate(invalid="ignore"):
        bnd = oracle.bound(K, oracle.abs_gemm_f64(A, B))
    Ad, Bd = padded_device(A, poison=0.0), padded_device(B, poison=0.0)
    for compute, tile in TILES:
        for fill in ("sync", "piped"):
            for S in (1, 2, 3):
                Cd = out_device(M, N)
                m.sgemm(Ad, Bd, Cd, stages=S, fill=fill, compute=compute, tile=tile)
                torch.cuda.synchronize()
                C = full_rows(Cd)[:, :N]
                what = (compute, tile, fill, S)
                _check_finite_part(C, ref, bnd, _check_classes(C, ref, what), what)


@pytest.mark.parametrize("fmt", ["bf16", "f16"])
def test_gemm16_special_values(fmt):
    K16 = 72
    A = datagen.matrix16(3, M, K16, fmt)
    B = datagen.matrix16(4, K16, N, fmt)
    inf, ninf = {"bf16": (0x7F80, 0xFF80), "f16": (0x7C00, 0xFC00)}[fmt]
    nan = {"bf16": 0x7FC0, "f16": 0x7E00}[fmt]
    zero = (A == 0) | (A == 0x8000)
    A[zero] = {"bf16": 0x3F00, "f16": 0x3800}[fmt]  # 0.5: no zero meets an infinity
    zero = (B == 0) | (B == 0x8000)
    B[zero] = {"bf16": 0x3F00, "f16": 0x3800}[fmt]
    A[3, 10], A[7, 0], A[11, K16 - 1] = inf, ninf, nan
    B[20, 5], B[K16 - 1, 9] = inf, nan
    ref = oracle.gemm16_f64(A, B, fmt)
    Ad, Bd = dev16(A, fmt), dev16(B, fmt)
    for tile in ("128x128", "256x128", "256x256"):
        for fill, S in (("sync", 1), ("sync", 2), ("piped", 1), ("piped", 2)):
            Cd = out_device(M, N)
            m.gemm16(Ad, Bd, Cd, stages=S, fill=fill, tile=tile)
            torch.cuda.synchronize()
            _check_classes(full_rows(Cd)[:, :N], ref, (fmt, tile, fill, S))
