"""Seeded synthetic inputs shared by the oracle side and the HIP side.

This module only draws numbers; it contains none of the GEMM or copy
arithmetic. Every value is a pure function of (seed, index), so the CPU and
the GPU sides of a test receive identical bytes.

Generator: SplitMix64 (Steele, Lea and Flood, "Fast splittable pseudorandom
number generators", OOPSLA 2014) used counter-style. The 64-bit word for
stream ``seed`` at position ``i`` is ``mix64(GAMMA * (seed * 2**40 + i + 1))``
where ``mix64`` is SplitMix64's output finaliser. Distributions built on it:

* ``uniform_pm1``: U[-1, 1) on the 2**-23 grid, ``(top24 - 2**23) * 2**-23``,
  exact in fp32 and fp64 and never -0.0 (values in [-1, 1 - 2**-23]).
* ``normal01``: Box-Muller in fp64 from two 24-bit uniforms (the first mapped
  to (0, 1]), rounded to fp32.
* ``coarse_pm1``: the 2**-4 grid in [-1, 15/16]; with K <= 8192 every fp32
  partial sum of products of such values is exact.
* ``page_pattern_a/b``: the inputs of the day-74 program on the
  "pipelined_gemm.cu" page (main: a[i] = (i % 97) * 0.01f,
  b[i] = (i % 53) * 0.02f - 0.5f).
"""
from __future__ import annotations

import numpy as np

GAMMA = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)
_CHUNK = 1 << 22

SEED_A = 1
SEED_B = 2
SEED_COPY = 3


def mix64(z: np.ndarray) -> np.ndarray:
    """SplitMix64's output finaliser on a uint64 array (wrapping arithmetic)."""
    z = z.copy()
    z ^= z >> np.uint64(30)
    z *= _M1
    z ^= z >> np.uint64(27)
    z *= _M2
    z ^= z >> np.uint64(31)
    return z


def words(seed: int, start: int, count: int) -> np.ndarray:
    """64-bit words of stream ``seed`` at positions start .. start+count-1."""
    ctr = np.arange(start + 1, start + 1 + count, dtype=np.uint64)
    ctr += np.uint64((seed << 40) & 0xFFFFFFFFFFFFFFFF)
    with np.errstate(over="ignore"):
        return mix64(ctr * GAMMA)


def _fill(n: int, fn) -> np.ndarray:
    out = np.empty(n, dtype=np.float32)
    for s in range(0, n, _CHUNK):
        c = min(_CHUNK, n - s)
        out[s:s + c] = fn(s, c)
    return out


def uniform_pm1(seed: int, n: int) -> np.ndarray:
    """n values of U[-1, 1) on the 2**-23 grid (fp32, exact)."""
    def part(s, c):
        top = (words(seed, s, c) >> np.uint64(40)).astype(np.int64)
        return ((top - (1 << 23)).astype(np.float64) * 2.0 ** -23).astype(np.float32)
    return _fill(n, part)


def coarse_pm1(seed: int, n: int) -> np.ndarray:
    """n values on the 2**-4 grid in [-1, 15/16] (fp32, exact)."""
    def part(s, c):
        top = (words(seed, s, c) >> np.uint64(59)).astype(np.int64)
        return ((top - 16).astype(np.float64) / 16.0).astype(np.float32)
    return _fill(n, part)


def normal01(seed: int, n: int) -> np.ndarray:
    """n values ~ N(0, 1): Box-Muller in fp64, rounded to fp32."""
    def part(s, c):
        w = words(seed, 2 * s, 2 * c)
        u1 = ((w[0::2] >> np.uint64(40)).astype(np.float64) + 1.0) * 2.0 ** -24
        u2 = (w[1::2] >> np.uint64(40)).astype(np.float64) * 2.0 ** -24
        return (np.sqrt(-2.0 * np.log(u1)) * np.cos(2.0 * np.pi * u2)).astype(np.float32)
    return _fill(n, part)


def page_pattern_a(n: int) -> np.ndarray:
    i = np.arange(n, dtype=np.int64)
    return (i % 97).astype(np.float32) * np.float32(0.01)


def page_pattern_b(n: int) -> np.ndarray:
    i = np.arange(n, dtype=np.int64)
    return (i % 53).astype(np.float32) * np.float32(0.02) - np.float32(0.5)


def matrix(kind: str, seed: int, rows: int, cols: int, ld: int | None = None,
           pad: float = float("nan")) -> np.ndarray:
    """A rows x ld fp32 array whose [:, :cols] block holds the stream's first
    rows*cols values in row-major order; columns cols..ld-1 hold ``pad``."""
    ld = cols if ld is None else ld
    if ld < cols:
        raise ValueError("ld < cols")
    n = rows * cols
    gen = {"uniform": uniform_pm1, "coarse": coarse_pm1, "normal": normal01}
    if kind in gen:
        v = gen[kind](seed, n)
    elif kind == "ones":
        v = np.ones(n, dtype=np.float32)
    elif kind == "page_a":
        v = page_pattern_a(n)
    elif kind == "page_b":
        v = page_pattern_b(n)
    else:
        raise ValueError(kind)
    out = np.full((rows, ld), pad, dtype=np.float32)
    out[:, :cols] = v.reshape(rows, cols)
    return out


def slice_sentinel(rows: int, cols: int, axis: int, group: int = 16) -> np.ndarray:
    """Matrix whose entry is floor(index_along_axis / group); used as the B
    operand (axis=0, index k) or the A operand (axis=1, index k)."""
    idx = np.arange(rows if axis == 0 else cols, dtype=np.int64) // group
    if axis == 0:
        return np.repeat(idx[:, None], cols, axis=1).astype(np.float32)
    return np.repeat(idx[None, :], rows, axis=0).astype(np.float32)


# ---- torch twin (same numbers, generated on any torch device) -------------

def _torch_words(seed: int, start: int, count: int, device):
    import torch
    def u(x):  # uint64 constant as a wrapped int64
        return x - (1 << 64) if x >= (1 << 63) else x
    ctr = torch.arange(start + 1, start + 1 + count, dtype=torch.int64, device=device)
    ctr = ctr + u((seed << 40) & 0xFFFFFFFFFFFFFFFF)
    z = ctr * u(int(GAMMA))

    def lsr(x, s):  # logical shift right on int64 bit patterns
        return (x >> s) & ((1 << (64 - s)) - 1)
    z = z ^ lsr(z, 30)
    z = z * u(int(_M1))
    z = z ^ lsr(z, 27)
    z = z * u(int(_M2))
    z = z ^ lsr(z, 31)
    return z, lsr


def uniform_pm1_torch(seed: int, n: int, device="cpu"):
    """Same values as uniform_pm1, produced by torch on ``device``."""
    import torch
    out = torch.empty(n, dtype=torch.float32, device=device)
    step = 1 << 24
    for s in range(0, n, step):
        c = min(step, n - s)
        z, lsr = _torch_words(seed, s, c, device)
        top = lsr(z, 40)
        out[s:s + c] = ((top - (1 << 23)).to(torch.float64) * 2.0 ** -23).to(torch.float32)
    return out


def normal01_torch(seed: int, n: int, device="cpu"):
    """Same values as normal01, produced by torch on ``device``."""
    import torch
    out = torch.empty(n, dtype=torch.float32, device=device)
    step = 1 << 23
    for s in range(0, n, step):
        c = min(step, n - s)
        z, lsr = _torch_words(seed, 2 * s, 2 * c, device)
        u1 = (lsr(z[0::2], 40).to(torch.float64) + 1.0) * 2.0 ** -24
        u2 = lsr(z[1::2], 40).to(torch.float64) * 2.0 ** -24
        out[s:s + c] = (torch.sqrt(-2.0 * torch.log(u1)) * torch.cos(2.0 * np.pi * u2)).to(torch.float32)
    return out


# ---- 16-bit inputs (bfloat16 / binary16 bit patterns) ------------------------

def grid_pm1(seed: int, n: int, bits: int) -> np.ndarray:
    """n values (top `bits` bits of the stream word - 2^(bits-1)) * 2^-(bits-1):
    a 2^-(bits-1) grid in [-1, 1), exact in any format with >= `bits`
    significand bits (bits=8 for bfloat16, 11 for binary16)."""
    def part(s, c):
        top = (words(seed, s, c) >> np.uint64(64 - bits)).astype(np.int64)
        return ((top - (1 << (bits - 1))).astype(np.float64) * 2.0 ** -(bits - 1)).astype(np.float32)
    return _fill(n, part)


def grid16_torch(seed: int, rows: int, cols: int, fmt: str, device="cpu"):
    """rows x cols torch bfloat16 / float16 tensor holding the values of
    grid_pm1(seed, rows * cols, bits) (the "grid" kind of matrix16, no
    padding), produced by torch on ``device``."""
    import torch
    bits = 8 if fmt == "bf16" else 11
    n = rows * cols
    out = torch.empty(n, dtype=torch.bfloat16 if fmt == "bf16" else torch.float16, device=device)
    step = 1 << 24
    for s in range(0, n, step):
        c = min(step, n - s)
        z, lsr = _torch_words(seed, s, c, device)
        top = lsr(z, 64 - bits)
        out[s:s + c] = ((top - (1 << (bits - 1))).to(torch.float64) * 2.0 ** -(bits - 1)).to(out.dtype)
    return out.view(rows, cols)


def to_bits16(x: np.ndarray, fmt: str) -> np.ndarray:
    """uint16 bit patterns of fp32 values that the format represents exactly
    ("bf16": upper half of the binary32 pattern; "f16": IEEE binary16)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if fmt == "bf16":
        u = x.view(np.uint32)
        if np.any(u & np.uint32(0xFFFF)):
            raise ValueError("value not exact in bfloat16")
        return (u >> np.uint32(16)).astype(np.uint16)
    if fmt == "f16":
        h = x.astype(np.float16)
        if not np.array_equal(h.astype(np.float32), x, equal_nan=True):
            raise ValueError("value not exact in binary16")
        return h.view(np.uint16)
    raise ValueError(fmt)


def matrix16(seed: int, rows: int, cols: int, fmt: str, kind: str = "grid", ld: int | None = None) -> np.ndarray:
    """rows x ld uint16 bit patterns; [:, :cols] holds the stream's values on the
    format's grid ("grid"), the 2^-4 grid ("coarse") or ones; padding holds the
    format's NaN pattern."""
    ld = cols if ld is None else ld
    n = rows * cols
    if kind == "grid":
        v = grid_pm1(seed, n, 8 if fmt == "bf16" else 11)
    elif kind == "coarse":
        v = coarse_pm1(seed, n)
    elif kind == "ones":
        v = np.ones(n, np.float32)
    else:
        raise ValueError(kind)
    out = np.full((rows, ld), 0x7FC0 if fmt == "bf16" else 0x7E00, dtype=np.uint16)
    out[:, :cols] = to_bits16(v, fmt).reshape(rows, cols)
    return out


# ---- structured attention inputs (full-size slice checks) --------------------
#
# Patterns, not draws: every value is a small integer or +-1, exact in both
# 16-bit formats. They are built with torch on any device (the full-size
# tensors are large) and returned as float32; callers cast to bfloat16 or
# float16, which changes no value.

def attn_slice_sentinel_v(batch: int, heads: int, seq: int, dim: int, group: int = 64, device="cpu"):
    """V[b, h, j, c] = floor(j / group) + ((c + 7 h + 3 b) mod dim).

    Integers below 2^8 for seq <= 64 group and dim <= 128 (exact in
    bfloat16 and binary16); with uniform weights the mean over keys of a
    column is a closed form, and a skipped or repeated group of keys moves
    it."""
    import torch
    j = torch.arange(seq, device=device, dtype=torch.int64) // group
    c = torch.arange(dim, device=device, dtype=torch.int64)
    b = torch.arange(batch, device=device, dtype=torch.int64)[:, None]
    h = torch.arange(heads, device=device, dtype=torch.int64)[None, :]
    r = (c[None, None, :] + 7 * h[..., None] + 3 * b[..., None]) % dim  # (batch, heads, dim)
    return (j[None, None, :, None] + r[:, :, None, :]).to(torch.float32)


def attn_peaked_winner(batch: int, heads: int, seq_q: int, group: int = 64, groups: int = 64, device="cpu"):
    """Key index w[b, h, i] = group * a + t that query i of head (b, h) is
    built to single out: a = (i + 5 h + 11 b) mod groups (its group of keys),
    t = (floor(i / groups) + 3 h + b) mod group (its place in the group). For
    seq_q = groups * group every key of a head is some query's winner once."""
    import torch
    i = torch.arange(seq_q, device=device, dtype=torch.int64)[None, None, :]
    b = torch.arange(batch, device=device, dtype=torch.int64)[:, None, None]
    h = torch.arange(heads, device=device, dtype=torch.int64)[None, :, None]
    a = (i + 5 * h + 11 * b) % groups
    t = (i // groups + 3 * h + b) % group
    return group * a + t


def _pm1_code(x, half):
    """(position, sign) of the signed one-hot code of x in [0, 2 half):
    position x mod half, sign +1 below half and -1 from half on."""
    import torch
    return x % half, torch.where(x < half, 1.0, -1.0)


def attn_peaked_qk(batch: int, heads: int, seq_q: int, seq_k: int, dim: int, group: int = 64, groups: int = 64,
                   device="cpu"):
    """(Q, K) as float32 (batch, heads, seq, dim) tensors of 0 and +-1.

    Key j = group * s + t carries the signed one-hot code of t (in dims
    0 .. group/2 - 1) and of s (in dims group/2 .. group - 1); query i carries
    the codes of its winner attn_peaked_winner(...)[b, h, i]. The dot product
    is +2 for the winner and at most +1 for every other key (each code
    contributes +1 on a match, 0 or -1 otherwise). Needs dim >= group,
    seq_k <= group * groups and groups <= group."""
    import torch
    half = group // 2
    if dim < group or seq_k > group * groups or groups > group:
        raise ValueError("peaked pattern needs dim >= group, seq_k <= group * groups, groups <= group")
    j = torch.arange(seq_k, device=device, dtype=torch.int64)
    K = torch.zeros((seq_k, dim), device=device, dtype=torch.float32)
    pt, st = _pm1_code(j % group, half)
    ps, ss = _pm1_code(j // group, half)
    K[j, pt] = st
    K[j, half + ps] = ss
    w = attn_peaked_winner(batch, heads, seq_q, group, groups, device=device)  # (batch, heads, seq_q)
    Q = torch.zeros((batch, heads, seq_q, dim), device=device, dtype=torch.float32)
    qt, qst = _pm1_code(w % group, half)
    qs, qss = _pm1_code(w // group, half)
    Q.scatter_(3, qt[..., None], qst[..., None])
    Q.scatter_(3, (half + qs)[..., None], qss[..., None])
    return Q, K.expand(batch, heads, seq_k, dim)
