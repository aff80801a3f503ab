"""Python binding of libmgemm: the MI355X (gfx950) pipelined FP32 GEMM and tile copy.

The functions named ``mgemm_*`` are the C entry points of ``include/mgemm.h``
with the same arguments (device pointers as integers, ``stream`` as the
integer value of a hipStream_t). ``sgemm`` and ``tile_copy`` are conveniences
that read pointers, leading dimensions and the current stream off torch
tensors. Every step of the computation runs in the HIP kernels of
``csrc/``; this module only marshals arguments. If the compiled library is
missing, importing the functions raises instead of computing anything.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "_build", "libmgemm.so")
ISA_PATH = os.path.join(_HERE, "_build", "mgemm-gfx950.s")

# constants of include/mgemm.h
MGEMM_VERSION = 100
FILL_SYNC, FILL_PIPED, FILL_PIPED_WS = 0, 1, 2
COMPUTE_VALU, COMPUTE_MFMA = 0, 1
TILE_AUTO, TILE_64x64, TILE_128x128, TILE_256x128, TILE_256x256 = 0, 1, 2, 3, 4
LOADER_AUTO, LOADER_B128, LOADER_B32 = 0, 1, 2
OK, ERR_ARG, ERR_ALIAS, ERR_ARCH, ERR_LAUNCH, ERR_UNSUPPORTED = 0, -1, -2, -3, -4, -5
DTYPE_BF16, DTYPE_F16 = 1, 2

_FILL = {"sync": FILL_SYNC, "piped": FILL_PIPED, "piped_ws": FILL_PIPED_WS}
_COMPUTE = {"valu": COMPUTE_VALU, "mfma": COMPUTE_MFMA}
_TILE = {"auto": TILE_AUTO, "64x64": TILE_64x64, "128x128": TILE_128x128, "256x128": TILE_256x128, "256x256": TILE_256x256}
_LOADER = {"auto": LOADER_AUTO, "b128": LOADER_B128, "b32": LOADER_B32}


class MgemmError(RuntimeError):
    def __init__(self, status: int, what: str = ""):
        self.status = status
        super().__init__(f"{what}: {mgemm_status_string(status)} (status {status})")


class Plan(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int) for n in (
        "compute", "tile", "bm", "bn", "bk", "threads", "blocks", "load_bytes", "slices",
        "stages", "fill_mode", "lds_bytes", "loads_per_slice", "max_vmcnt")]

    def as_dict(self):
        return {n: getattr(self, n) for n, _ in self._fields_}


_lib = None


def lib():
    """The loaded libmgemm (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"libmgemm is not built ({LIB_PATH} missing); run __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        i64, vp, ci = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
        L.mgemm_sgemm.argtypes = [i64, i64, i64, vp, i64, vp, i64, vp, i64, ci, ci, vp]
        L.mgemm_sgemm_ex.argtypes = [i64, i64, i64, vp, i64, vp, i64, vp, i64, ci, ci, ci, ci, ci, vp]
        L.mgemm_tile_copy.argtypes = [i64, i64, vp, i64, vp, i64, ci, vp]
        L.mgemm_plain_copy.argtypes = [i64, i64, vp, i64, vp, i64, vp]
        L.mgemm_plan_sgemm.argtypes = [i64, i64, i64, vp, i64, vp, i64, vp, i64, ci, ci, ci, ci, ci,
                                       ctypes.POINTER(Plan)]
        L.mgemm_ring_trace.argtypes = [ci, ci, ci, ci, ctypes.POINTER(ctypes.c_int), ci]
        L.mgemm_fill_trace.argtypes = [ci, ci, ci, ctypes.POINTER(ctypes.c_int), ci]
        L.mgemm_gemm16.argtypes = [i64, i64, i64, vp, i64, vp, i64, vp, i64, ci, ci, ci, ci, vp]
        L.mgemm_plan_gemm16.argtypes = [i64, i64, i64, vp, i64, vp, i64, vp, i64, ci, ci, ci, ci,
                                        ctypes.POINTER(Plan)]
        L.mgemm_attention.argtypes = [i64, i64, i64, i64, i64, vp, i64, i64, i64, vp, i64, i64, i64, vp, i64, i64,
                                      i64, vp, i64, i64, i64, ctypes.c_float, ci, ci, ci, vp]
        L.mgemm_plan_attention.argtypes = [i64, i64, i64, i64, i64, vp, i64, i64, i64, vp, i64, i64, i64, vp, i64,
                                           i64, i64, vp, i64, i64, i64, ci, ci, ci, ctypes.POINTER(Plan)]
        L.mgemm_blocks_per_cu.argtypes = [i64, i64, i64, vp, i64, vp, i64, vp, i64, ci, ci, ci, ci, ci,
                                          ctypes.POINTER(ctypes.c_int)]
        L.mgemm_status_string.argtypes = [ci]
        L.mgemm_status_string.restype = ctypes.c_char_p
        for f in (L.mgemm_sgemm, L.mgemm_sgemm_ex, L.mgemm_tile_copy, L.mgemm_plain_copy, L.mgemm_plan_sgemm,
                  L.mgemm_ring_trace, L.mgemm_fill_trace, L.mgemm_version, L.mgemm_blocks_per_cu, L.mgemm_gemm16,
                  L.mgemm_plan_gemm16, L.mgemm_attention, L.mgemm_plan_attention):
            f.restype = ci
        _lib = L
    return _lib


# ---- the C entry points, same names and arguments ---------------------------

def mgemm_sgemm(M, N, K, A, lda, B, ldb, C, ldc, stages, fill_mode, stream) -> int:
    return lib().mgemm_sgemm(M, N, K, A, lda, B, ldb, C, ldc, stages, fill_mode, stream)


def mgemm_sgemm_ex(M, N, K, A, lda, B, ldb, C, ldc, stages, fill_mode, compute, tile, loader, stream) -> int:
    return lib().mgemm_sgemm_ex(M, N, K, A, lda, B, ldb, C, ldc, stages, fill_mode, compute, tile, loader, stream)


def mgemm_gemm16(M, N, K, A, lda, B, ldb, C, ldc, dtype, stages, fill_mode, tile, stream) -> int:
    return lib().mgemm_gemm16(M, N, K, A, lda, B, ldb, C, ldc, dtype, stages, fill_mode, tile, stream)


def mgemm_plan_gemm16(M, N, K, A, lda, B, ldb, C, ldc, dtype, stages, fill_mode, tile):
    p = Plan()
    st = lib().mgemm_plan_gemm16(M, N, K, A, lda, B, ldb, C, ldc, dtype, stages, fill_mode, tile, ctypes.byref(p))
    return st, p


def mgemm_attention(batch, heads, seq_q, seq_k, head_dim, Q, q_sb, q_sh, q_ld, K, k_sb, k_sh, k_ld, V, v_sb, v_sh,
                    v_ld, O, o_sb, o_sh, o_ld, scale, dtype, stages, fill_mode, stream) -> int:
    return lib().mgemm_attention(batch, heads, seq_q, seq_k, head_dim, Q, q_sb, q_sh, q_ld, K, k_sb, k_sh, k_ld, V,
                                 v_sb, v_sh, v_ld, O, o_sb, o_sh, o_ld, scale, dtype, stages, fill_mode, stream)


def mgemm_plan_attention(batch, heads, seq_q, seq_k, head_dim, Q, q_sb, q_sh, q_ld, K, k_sb, k_sh, k_ld, V, v_sb,
                         v_sh, v_ld, O, o_sb, o_sh, o_ld, dtype, stages, fill_mode):
    p = Plan()
    st = lib().mgemm_plan_attention(batch, heads, seq_q, seq_k, head_dim, Q, q_sb, q_sh, q_ld, K, k_sb, k_sh, k_ld,
                                    V, v_sb, v_sh, v_ld, O, o_sb, o_sh, o_ld, dtype, stages, fill_mode,
                                    ctypes.byref(p))
    return st, p


def mgemm_tile_copy(rows, cols, src, lds, dst, ldd, stages, stream) -> int:
    return lib().mgemm_tile_copy(rows, cols, src, lds, dst, ldd, stages, stream)


def mgemm_plain_copy(rows, cols, src, lds, dst, ldd, stream) -> int:
    return lib().mgemm_plain_copy(rows, cols, src, lds, dst, ldd, stream)


def mgemm_status_string(status: int) -> str:
    return lib().mgemm_status_string(status).decode()


def mgemm_version() -> int:
    return lib().mgemm_version()


def mgemm_plan_sgemm(M, N, K, A, lda, B, ldb, C, ldc, stages, fill_mode, compute, tile, loader):
    """(status, Plan) for these arguments; no device access."""
    p = Plan()
    st = lib().mgemm_plan_sgemm(M, N, K, A, lda, B, ldb, C, ldc, stages, fill_mode, compute, tile, loader,
                                ctypes.byref(p))
    return st, p


def mgemm_blocks_per_cu(M, N, K, A, lda, B, ldb, C, ldc, stages, fill_mode, compute, tile, loader):
    """(status, resident blocks per CU) of the kernel that would be launched."""
    out = ctypes.c_int(0)
    st = lib().mgemm_blocks_per_cu(M, N, K, A, lda, B, ldb, C, ldc, stages, fill_mode, compute, tile, loader,
                                   ctypes.byref(out))
    return st, out.value


def mgemm_fill_trace(kind: int, load_bytes: int, fill_mode: int):
    """One slice's loader map as (header, events): header = (slot bytes, rows0,
    cols0, rows1, cols1); events = (operand, wave, lds byte, row, col, layout
    byte) per lane and unit (see include/mgemm.h)."""
    n = lib().mgemm_fill_trace(kind, load_bytes, fill_mode, None, 0)
    if n < 0:
        raise MgemmError(n, "mgemm_fill_trace")
    buf = (ctypes.c_int * (6 * max(n, 1)))()
    lib().mgemm_fill_trace(kind, load_bytes, fill_mode, buf, n)
    ev = [tuple(buf[6 * i:6 * i + 6]) for i in range(n)]
    assert ev[0][0] == -1
    return ev[0][1:], ev[1:]


def mgemm_ring_trace(kind: int, stages: int, fill_mode: int, slices: int):
    """The ring schedule as a list of (op, a, b) events (see include/mgemm.h)."""
    n = lib().mgemm_ring_trace(kind, stages, fill_mode, slices, None, 0)
    if n < 0:
        raise MgemmError(n, "mgemm_ring_trace")
    buf = (ctypes.c_int * (3 * max(n, 1)))()
    lib().mgemm_ring_trace(kind, stages, fill_mode, slices, buf, n)
    return [(buf[3 * i], buf[3 * i + 1], buf[3 * i + 2]) for i in range(n)]


# ---- torch conveniences (pointers, leading dimensions and stream only) ------

def _mat(t, name):
    import torch
    if not isinstance(t, torch.Tensor) or t.dtype != torch.float32 or t.dim() != 2:
        raise TypeError(f"{name} must be a 2-D float32 torch tensor")
    if not t.is_cuda:
        raise TypeError(f"{name} must be on a GPU")
    if t.numel() and t.stride(1) != 1:
        raise TypeError(f"{name} must have unit column stride")
    return t.data_ptr(), _ld(t)


def _ld(t):
    """The row stride passed as the leading dimension. A single row has no
    meaningful stride (the width stands in); with two rows or more the
    stride goes through as it is, so an overlapping view (an expanded row,
    stride 0, or any stride below the width) reaches the C ABI's ld < cols
    check and is refused before any launch."""
    return max(t.stride(0), t.shape[1]) if t.shape[0] <= 1 else t.stride(0)


def _stream(stream):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream if hasattr(s, "cuda_stream") else int(s)


def sgemm(A, B, C=None, *, stages: int = 2, fill: str = "piped", compute: str = "valu",
          tile: str = "auto", loader: str = "auto", stream=None):
    """C = A @ B through mgemm_sgemm_ex on the current (or given) stream."""
    import torch
    M, K = A.shape
    K2, N = B.shape
    if K2 != K:
        raise ValueError("inner dimensions differ")
    if C is None:
        C = torch.empty((M, N), dtype=torch.float32, device=A.device)
    if tuple(C.shape) != (M, N):
        raise ValueError("C has the wrong shape")
    pa, lda = _mat(A, "A")
    pb, ldb = _mat(B, "B")
    pc, ldc = _mat(C, "C")
    st = mgemm_sgemm_ex(M, N, K, pa, lda, pb, ldb, pc, ldc, stages, _FILL[fill], _COMPUTE[compute],
                        _TILE[tile], _LOADER[loader], _stream(stream))
    if st != OK:
        raise MgemmError(st, "mgemm_sgemm_ex")
    return C


def _mat16(t, name):
    import torch
    if not isinstance(t, torch.Tensor) or t.dtype not in (torch.bfloat16, torch.float16) or t.dim() != 2:
        raise TypeError(f"{name} must be a 2-D bfloat16 or float16 torch tensor")
    if not t.is_cuda:
        raise TypeError(f"{name} must be on a GPU")
    if t.numel() and t.stride(1) != 1:
        raise TypeError(f"{name} must have unit column stride")
    return t.data_ptr(), _ld(t)


def gemm16(A, B, C=None, *, stages: int = 2, fill: str = "piped", tile: str = "auto", stream=None):
    """C (fp32) = A @ B for bfloat16 or float16 A and B, through mgemm_gemm16."""
    import torch
    if A.dtype != B.dtype:
        raise TypeError("A and B must have the same 16-bit format")
    M, K = A.shape
    K2, N = B.shape
    if K2 != K:
        raise ValueError("inner dimensions differ")
    if C is None:
        C = torch.empty((M, N), dtype=torch.float32, device=A.device)
    pa, lda = _mat16(A, "A")
    pb, ldb = _mat16(B, "B")
    pc, ldc = _mat(C, "C")
    dtype = DTYPE_BF16 if A.dtype == torch.bfloat16 else DTYPE_F16
    st = mgemm_gemm16(M, N, K, pa, lda, pb, ldb, pc, ldc, dtype, stages, _FILL[fill], _TILE[tile], _stream(stream))
    if st != OK:
        raise MgemmError(st, "mgemm_gemm16")
    return C


def plan16(M, N, K, *, dtype="bf16", stages=2, fill="piped", tile="auto", lda=None, ldb=None, ldc=None,
           a_ptr=0x10000, b_ptr=0x40000000, c_ptr=0x80000000):
    st, p = mgemm_plan_gemm16(M, N, K, a_ptr, K if lda is None else lda, b_ptr, N if ldb is None else ldb, c_ptr,
                              N if ldc is None else ldc, DTYPE_BF16 if dtype == "bf16" else DTYPE_F16, stages,
                              _FILL[fill], _TILE[tile])
    if st != OK:
        raise MgemmError(st, "mgemm_plan_gemm16")
    return p.as_dict()


def _attn_view(t, name, fp32=False):
    import torch
    want = (torch.float32,) if fp32 else (torch.bfloat16, torch.float16)
    if not isinstance(t, torch.Tensor) or t.dim() != 4 or t.dtype not in want:
        raise TypeError(f"{name} must be a 4-D (batch, heads, seq, dim) torch tensor of "
                        f"{'float32' if fp32 else 'bfloat16 or float16'}")
    if not t.is_cuda:
        raise TypeError(f"{name} must be on a GPU")
    if t.numel() and t.stride(3) != 1:
        raise TypeError(f"{name} must have unit stride along its last axis")
    sb, sh, ld, _ = t.stride()
    return t.data_ptr(), sb, sh, ld


def attention(Q, K, V, O=None, *, scale=None, stages: int = 2, fill: str = "piped", stream=None):
    """O (fp32) = softmax(scale Q K^T) V per (batch, head) through
    mgemm_attention; Q (B, H, Sq, D), K and V (B, H, Sk, D) of one 16-bit
    format; scale defaults to 1/sqrt(D)."""
    import torch
    if not (Q.dtype == K.dtype == V.dtype):
        raise TypeError("Q, K and V must have the same 16-bit format")
    B, H, Sq, D = Q.shape
    Sk = K.shape[2]
    if K.shape != (B, H, Sk, D) or V.shape != (B, H, Sk, D):
        raise ValueError("K and V must be (batch, heads, seq_k, head_dim) matching Q")
    if O is None:
        O = torch.empty((B, H, Sq, D), dtype=torch.float32, device=Q.device)
    scale = D ** -0.5 if scale is None else float(scale)
    q, k, v = _attn_view(Q, "Q"), _attn_view(K, "K"), _attn_view(V, "V")
    o = _attn_view(O, "O", fp32=True)
    dtype = DTYPE_BF16 if Q.dtype == torch.bfloat16 else DTYPE_F16
    st = mgemm_attention(B, H, Sq, Sk, D, *q, *k, *v, *o, scale, dtype, stages, _FILL[fill], _stream(stream))
    if st != OK:
        raise MgemmError(st, "mgemm_attention")
    return O


def plan_attention(batch, heads, seq_q, seq_k, head_dim, *, dtype="bf16", stages=2, fill="piped", align=16):
    """Launch plan of attention on contiguous (batch, heads, seq, dim)
    tensors at fake addresses aligned to `align` bytes (no device access)."""
    D = head_dim
    qa, ka, va, oa = (1 << 32) + align % 16, 1 << 36, 1 << 37, 1 << 40
    st, p = mgemm_plan_attention(batch, heads, seq_q, seq_k, D, qa, heads * seq_q * D, seq_q * D, D,
                                 ka, heads * seq_k * D, seq_k * D, D, va, heads * seq_k * D, seq_k * D, D,
                                 oa, heads * seq_q * D, seq_q * D, D, DTYPE_BF16 if dtype == "bf16" else DTYPE_F16,
                                 stages, _FILL[fill])
    if st != OK:
        raise MgemmError(st, "mgemm_plan_attention")
    return p.as_dict()


def tile_copy(src, dst=None, *, stages: int = 3, stream=None):
    """dst = src through mgemm_tile_copy."""
    import torch
    if dst is None:
        dst = torch.empty(src.shape, dtype=torch.float32, device=src.device)
    if tuple(dst.shape) != tuple(src.shape):
        raise ValueError("dst has the wrong shape")
    ps, lds = _mat(src, "src")
    pd, ldd = _mat(dst, "dst")
    st = mgemm_tile_copy(src.shape[0], src.shape[1], ps, lds, pd, ldd, stages, _stream(stream))
    if st != OK:
        raise MgemmError(st, "mgemm_tile_copy")
    return dst


def plain_copy(src, dst=None, *, stream=None):
    """dst = src through mgemm_plain_copy (no LDS ring: the copy ceiling)."""
    import torch
    if dst is None:
        dst = torch.empty(src.shape, dtype=torch.float32, device=src.device)
    if tuple(dst.shape) != tuple(src.shape):
        raise ValueError("dst has the wrong shape")
    ps, lds = _mat(src, "src")
    pd, ldd = _mat(dst, "dst")
    st = mgemm_plain_copy(src.shape[0], src.shape[1], ps, lds, pd, ldd, _stream(stream))
    if st != OK:
        raise MgemmError(st, "mgemm_plain_copy")
    return dst


def blocks_per_cu(M, N, K, *, stages=2, fill="piped", compute="valu", tile="auto", loader="auto"):
    """Resident blocks per CU of the kernel for this problem (aligned layout)."""
    st, n = mgemm_blocks_per_cu(M, N, K, 0x10000, K, 0x40000000, N, 0x80000000, N, stages, _FILL[fill],
                                _COMPUTE[compute], _TILE[tile], _LOADER[loader])
    if st != OK:
        raise MgemmError(st, "mgemm_blocks_per_cu")
    return n


def plan(M, N, K, *, stages=2, fill="piped", compute="valu", tile="auto", loader="auto",
         a_ptr=0x10000, lda=None, b_ptr=0x40000000, ldb=None, c_ptr=0x80000000, ldc=None):
    """Launch plan for a problem (defaults: aligned, non-overlapping fake addresses)."""
    st, p = mgemm_plan_sgemm(M, N, K, a_ptr, K if lda is None else lda, b_ptr, N if ldb is None else ldb,
                             c_ptr, N if ldc is None else ldc, stages, _FILL[fill], _COMPUTE[compute],
                             _TILE[tile], _LOADER[loader])
    if st != OK:
        raise MgemmError(st, "mgemm_plan_sgemm")
    return p.as_dict()
