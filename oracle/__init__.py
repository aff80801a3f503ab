"""TEST INFRASTRUCTURE: the CPU oracle for the pipelined GEMMs (fp32 and 16-bit
inputs), the tile copy and scaled dot-product attention.

Only the tests, the smoke check and the CPU-baseline leg of the benchmark may
import this package. The product library never loads it, and it shares no code
with the HIP sources (see ref_gemm.c for the definitions and their sources).

The numeric work happens in ``ref_gemm.c`` (plain C, fp64, OpenMP over rows);
this module only compiles it with gcc and marshals numpy arrays through ctypes.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import time
from typing import NamedTuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(_HERE, "ref_gemm.c")
LIB = os.path.join(_HERE, "_build", "liboracle.so")
CFLAGS = ["-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
          "-shared", "-fPIC", "-std=c99", "-Wall"]

_lib = None


def build(src: str = SRC, out: str = LIB) -> str:
    """Compile the oracle with gcc (always recompiles)."""
    os.makedirs(os.path.dirname(out), exist_ok=True)
    tmp = out + ".tmp%d" % os.getpid()
    subprocess.run(["gcc", *CFLAGS, src, "-o", tmp, "-lm"], check=True)
    os.replace(tmp, out)
    return out


def load(path: str | None = None):
    """Load (building first if absent) the oracle library."""
    global _lib
    if path is not None:
        return _bind(ctypes.CDLL(path))
    if _lib is None:
        if not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
            build()
        _lib = _bind(ctypes.CDLL(LIB))
    return _lib


def _bind(lib):
    i64, fp, dp = ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p
    for name in ("oracle_gemm_f64", "oracle_abs_gemm_f64"):
        f = getattr(lib, name)
        f.argtypes = [i64, i64, i64, fp, i64, fp, i64, dp, i64]
        f.restype = None
    lib.oracle_copy_f32.argtypes = [i64, i64, fp, i64, fp, i64]
    lib.oracle_copy_f32.restype = None
    lib.oracle_num_threads.restype = ctypes.c_int
    lib.oracle_set_threads.argtypes = [ctypes.c_int]
    lib.oracle_set_threads.restype = None
    lib.oracle_decode16.argtypes = [ctypes.c_uint16, ctypes.c_int]
    lib.oracle_decode16.restype = ctypes.c_double
    lib.oracle_gemm16_f64.argtypes = [i64, i64, i64, fp, i64, fp, i64, dp, i64, ctypes.c_int, ctypes.c_int]
    lib.oracle_gemm16_f64.restype = None
    lib.oracle_attention_f64.argtypes = [i64, i64, i64, i64, fp, i64, fp, i64, fp, i64, ctypes.c_double,
                                         ctypes.c_int, dp, dp, i64, dp, dp]
    lib.oracle_attention_f64.restype = ctypes.c_int
    return lib


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def _check_operands(M, N, K, A, B):
    for name, x in (("A", A), ("B", B)):
        if x.dtype != np.float32 or x.ndim != 2 or (x.size and x.strides[1] != 4):
            raise TypeError(f"{name} must be a 2-D fp32 array with unit column stride")
    if A.shape[0] < M or A.shape[1] < K or B.shape[0] < K or B.shape[1] < N:
        raise ValueError("operand smaller than M x K / K x N")


def gemm_f64(A: np.ndarray, B: np.ndarray, M=None, N=None, K=None, lib=None) -> np.ndarray:
    """C_ref = A[:M,:K] @ B[:K,:N] in fp64 (k ascending). A and B may be
    views with a row stride larger than their width (their leading dimension)."""
    M = A.shape[0] if M is None else M
    K = A.shape[1] if K is None else K
    N = B.shape[1] if N is None else N
    _check_operands(M, N, K, A, B)
    C = np.empty((M, N), dtype=np.float64)
    (lib or load()).oracle_gemm_f64(M, N, K, _ptr(A), A.strides[0] // 4,
                                    _ptr(B), B.strides[0] // 4, _ptr(C), N)
    return C


def abs_gemm_f64(A: np.ndarray, B: np.ndarray, M=None, N=None, K=None, lib=None) -> np.ndarray:
    """Abs = |A[:M,:K]| @ |B[:K,:N]| in fp64."""
    M = A.shape[0] if M is None else M
    K = A.shape[1] if K is None else K
    N = B.shape[1] if N is None else N
    _check_operands(M, N, K, A, B)
    C = np.empty((M, N), dtype=np.float64)
    (lib or load()).oracle_abs_gemm_f64(M, N, K, _ptr(A), A.strides[0] // 4,
                                        _ptr(B), B.strides[0] // 4, _ptr(C), N)
    return C


FMT = {"bf16": 1, "f16": 2}


def decode16(bits: int, fmt: str, lib=None) -> float:
    """Value of one 16-bit pattern in format ``fmt`` ("bf16" or "f16")."""
    return float((lib or load()).oracle_decode16(int(bits) & 0xFFFF, FMT[fmt]))


def gemm16_f64(A: np.ndarray, B: np.ndarray, fmt: str, absolute: bool = False, lib=None) -> np.ndarray:
    """C_ref = dec(A) @ dec(B) in fp64 for uint16 bit-pattern arrays A (M x K)
    and B (K x N), which may be views with a larger row stride."""
    for name, x in (("A", A), ("B", B)):
        if x.dtype != np.uint16 or x.ndim != 2 or (x.size and x.strides[1] != 2):
            raise TypeError(f"{name} must be a 2-D uint16 array with unit column stride")
    M, K = A.shape
    K2, N = B.shape
    if K2 != K:
        raise ValueError("inner dimensions differ")
    C = np.empty((M, N), dtype=np.float64)
    (lib or load()).oracle_gemm16_f64(M, N, K, A.ctypes.data, A.strides[0] // 2, B.ctypes.data,
                                      B.strides[0] // 2, C.ctypes.data, N, FMT[fmt], int(absolute))
    return C


def copy_f32(src: np.ndarray, rows=None, cols=None, lib=None) -> np.ndarray:
    rows = src.shape[0] if rows is None else rows
    cols = src.shape[1] if cols is None else cols
    dst = np.full((rows, cols), np.nan, dtype=np.float32)  # unwritten cells stay NaN
    (lib or load()).oracle_copy_f32(rows, cols, _ptr(src), src.strides[0] // 4, _ptr(dst), cols)
    return dst


def bound(K: int, Abs: np.ndarray, slack: float = 4.0) -> np.ndarray:
    """Elementwise acceptance bound slack * K * 2^-24 * (|A||B|)_ij for an fp32
    GEMM against this fp64 reference."""
    return slack * K * 2.0 ** -24 * Abs


def num_threads(lib=None) -> int:
    return int((lib or load()).oracle_num_threads())


def set_threads(n: int, lib=None) -> None:
    """Thread count of the oracle's parallel loops (timing only)."""
    (lib or load()).oracle_set_threads(int(n))


def timed_gemm_rows(A: np.ndarray, B: np.ndarray, rows: int, lib=None):
    """Run oracle_gemm_f64 on the first ``rows`` rows of A (full N and K) and
    return (seconds, flop). Used only for the CPU baseline."""
    M, K = rows, A.shape[1]
    N = B.shape[1]
    C = np.empty((M, N), dtype=np.float64)
    lib = lib or load()
    t0 = time.perf_counter()
    lib.oracle_gemm_f64(M, N, K, _ptr(A), A.strides[0] // 4, _ptr(B), B.strides[0] // 4, _ptr(C), N)
    dt = time.perf_counter() - t0
    return dt, 2.0 * M * N * K


def timed_copy(src: np.ndarray, lib=None):
    """Run oracle_copy_f32 on the whole of ``src`` into a fresh array and
    return (seconds, copy). Used only for the CPU baseline of the tile copy."""
    lib = lib or load()
    rows, cols = src.shape
    dst = np.empty((rows, cols), dtype=np.float32)
    dst.fill(0.0)  # touch every page before the clock starts
    t0 = time.perf_counter()
    lib.oracle_copy_f32(rows, cols, _ptr(src), src.strides[0] // 4, _ptr(dst), cols)
    return time.perf_counter() - t0, dst


class AttnRef(NamedTuple):
    """The attention oracle's result and the magnitudes its bound needs."""
    O: np.ndarray     # (..., Sq, Dv) softmax(scale Q K^T) V
    Wabs: np.ndarray  # (..., Sq, Dv) sum_j w_j |v_jc|
    G: np.ndarray     # (..., Sq) max_j sum_d |q_d||k_jd|
    Vmax: np.ndarray  # (..., Dv) max_j |v_jc|
    D: int
    Sk: int


def attention_f64(Q: np.ndarray, K: np.ndarray, V: np.ndarray, fmt: str, scale: float, with_abs: bool = False,
                  lib=None):
    """softmax(scale * Q K^T) V in fp64 for 16-bit patterns Q (..., Sq, D),
    K (..., Sk, D), V (..., Sk, Dv) with any leading (batch, head) axes and
    unit stride along the last axis; returns O (..., Sq, Dv), or with
    ``with_abs`` an AttnRef that also carries the magnitudes of the bound."""
    lib = lib or load()
    for name, x in (("Q", Q), ("K", K), ("V", V)):
        if x.dtype != np.uint16 or x.ndim < 2 or (x.size and x.strides[-1] != 2):
            raise TypeError(f"{name} must hold uint16 patterns with unit stride along its last axis")
    lead = Q.shape[:-2]
    if K.shape[:-2] != lead or V.shape[:-2] != lead:
        raise ValueError("Q, K and V need the same leading axes")
    Sq, D = Q.shape[-2:]
    Sk, Dv = V.shape[-2:]
    if K.shape[-2:] != (Sk, D):
        raise ValueError("K must be Sk x D")
    if Sk < 1:
        raise ValueError("softmax over an empty key set is undefined")
    O = np.zeros(lead + (Sq, Dv))
    W = np.zeros(lead + (Sq, Dv))
    G = np.zeros(lead + (Sq,))
    Vm = np.zeros(lead + (Dv,))
    for idx in np.ndindex(*lead):
        q, k, v = Q[idx], K[idx], V[idx]
        o, w, g, vm = O[idx], W[idx], G[idx], Vm[idx]
        st = lib.oracle_attention_f64(Sq, Sk, D, Dv, _ptr(q), q.strides[0] // 2, _ptr(k), k.strides[0] // 2,
                                      _ptr(v), v.strides[0] // 2, float(scale), FMT[fmt], _ptr(o),
                                      _ptr(w) if with_abs else None, Dv, _ptr(g) if with_abs else None,
                                      _ptr(vm) if with_abs else None)
        if st != 0:
            raise MemoryError("oracle_attention_f64: out of memory")
    return AttnRef(O, W, G, Vm, int(D), int(Sk)) if with_abs else O


def attention_bound(ref: AttnRef, fmt: str, scale: float) -> np.ndarray:
    """Acceptance bound of the attention kernels, elementwise:
    (e_p + 4 delta_i) sum_j w_j |v_jc| + Sk tau max_j |v_jc|.
    e_p = 2^-6 (bfloat16) or 2^-8 (binary16): the probabilities are rounded
    to the 16-bit format before the P V product (unit roundoff 2^-8 or
    2^-11), which moves each weight by at most about twice that, with fp32
    accumulation and rescaling adding far less for key counts below 2^14.
    delta_i = |scale| (D + 8) 2^-24 G_i bounds the error of every score of
    query row i (fp32 sums of D exact products, then the fp32 scaling into
    the exponent and the shift by the row maximum); perturbing every score by
    at most delta moves each softmax weight by a factor within
    exp(+-2 delta), so O by at most 2 delta sum_j w_j |v_jc|, taken twice.
    The last term covers probabilities too small for a relative error: the
    kernels' probabilities are taken against a running reference at most 8
    (log2 units) below the row maximum, so they lie in [0, 2^8] with a row
    sum of at least 1 (the row maximum contributes 2^0 or more), and each
    key's rounded probability is off
    by at most tau in absolute terms below the format's normal range. For
    bfloat16 (fp32's exponent range) that is fp32 underflow, tau = 2^-125;
    binary16 stops at subnormals spaced 2^-24 (nothing below 2^-25 survives
    the rounding), so tau = 2^-25."""
    e_p = 2.0 ** -6 if fmt == "bf16" else 2.0 ** -8
    tau = 2.0 ** -125 if fmt == "bf16" else 2.0 ** -25
    delta = abs(scale) * (ref.D + 8) * 2.0 ** -24 * ref.G
    return (e_p + 4.0 * delta[..., None]) * ref.Wabs + ref.Sk * tau * ref.Vmax[..., None, :]
