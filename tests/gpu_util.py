"""Shared helpers of the GPU parity tests (device buffers with padding and
poison, variant lists, checks against the oracle)."""
from __future__ import annotations

import numpy as np
import torch

import async_global_shared_amd as m
import oracle

DEV = torch.device("cuda:0")
SENTINEL = -12345.0

# (compute, tile) pairs, each with its own shared compute tile
TILES = [("valu", "64x64"), ("valu", "128x128"), ("mfma", "64x64"), ("mfma", "128x128"), ("mfma", "256x128")]
FILLS = ["sync", "piped"]
STAGES = [1, 2, 3]


def padded_device(a: np.ndarray, ld: int | None = None, extra_rows: int = 2, poison=np.nan,
                  offset: int = 0) -> torch.Tensor:
    """Device copy of ``a`` as a view with leading dimension ``ld``; the padding
    columns, ``extra_rows`` rows past the end and ``offset`` leading elements
    hold ``poison``, so a read outside the matrix turns into NaN in C."""
    rows, cols = a.shape
    ld = cols if ld is None else ld
    buf = torch.full((offset + (rows + extra_rows) * ld,), poison, dtype=torch.float32)
    view = buf[offset:offset + rows * ld].view(rows, ld)
    view[:, :cols] = torch.from_numpy(np.ascontiguousarray(a))
    dbuf = buf.to(DEV)
    return dbuf[offset:offset + rows * ld].view(rows, ld)[:, :cols]


def out_device(M: int, N: int, ldc: int | None = None, offset: int = 0) -> torch.Tensor:
    """Output view of M x N with leading dimension ldc; every cell (including
    the padding, which must stay untouched) starts as SENTINEL."""
    ldc = N if ldc is None else ldc
    buf = torch.full((offset + (M + 1) * ldc,), SENTINEL, dtype=torch.float32, device=DEV)
    return buf[offset:offset + M * ldc].view(M, ldc)[:, :N]


def ring_fits(M, N, K, **kw) -> bool:
    """Whether the library plans this launch; the only refusal expected of a
    valid call is a ring deeper than the CU's LDS (MGEMM_ERR_UNSUPPORTED)."""
    try:
        m.plan(M, N, K, **kw)
        return True
    except m.MgemmError as e:
        assert e.status == m.ERR_UNSUPPORTED, (M, N, K, kw, e.status)
        return False


def run(Ad, Bd, Cd, *, compute, tile, fill, stages, loader="auto"):
    m.sgemm(Ad, Bd, Cd, stages=stages, fill=fill, compute=compute, tile=tile, loader=loader)
    torch.cuda.synchronize()
    return Cd


def full_rows(Cd: torch.Tensor) -> np.ndarray:
    """Host copy of the whole padded storage rows of a C view."""
    M, N = Cd.shape
    ldc = Cd.stride(0)
    base = Cd.as_strided((M, ldc), (ldc, 1))
    return base.cpu().numpy()


def check_bound(C: np.ndarray, A: np.ndarray, B: np.ndarray, rows=None, what=""):
    """|C - C_ref| <= 4 K 2^-24 (|A||B|) elementwise, on all rows or on ``rows``."""
    K = A.shape[1]
    if rows is not None:
        A = np.ascontiguousarray(A[rows])
        C = C[rows]
    ref = oracle.gemm_f64(A, B)
    bnd = oracle.bound(K, oracle.abs_gemm_f64(A, B))
    err = np.abs(C.astype(np.float64) - ref)
    bad = ~(err <= bnd)
    if bad.any():
        i, j = np.argwhere(bad)[0]
        raise AssertionError(f"{what}: {bad.sum()} elements outside the bound, first ({i},{j}): "
                             f"got {C[i, j]!r} want {ref[i, j]!r} bound {bnd[i, j]!r}")
    return float(np.max(err / np.maximum(bnd, 1e-300))) if err.size else 0.0


def same_bits(x: np.ndarray, y: np.ndarray) -> bool:
    return x.shape == y.shape and x.tobytes() == y.tobytes()
