"""A numpy model of the rounding the attention kernels perform, used to check
the oracle's acceptance bound from the other side: a bound that a plausible
kernel's arithmetic can exceed is too tight, and one that a kernel which
skips or repeats a slice of keys still meets is too loose.

It follows the tile loop of the async copy article ("from cp.async to
memcpy_async", section 6.2, "FlashAttention's tile pipeline") in the form the
library computes it (64-key slices, scores in the log2 domain, a running
reference that moves only when a slice's maximum exceeds it by more than 8,
probabilities rounded to the 16-bit input format before the P.V product, fp32
everywhere else). Nothing here is shared with the oracle or the HIP sources;
it is a test model, not a reference: the oracle's definition stays the fp64
softmax.

Two summation models bracket the hardware's order inside a matrix
instruction: "chunk" rounds once per 16 products (an exact dot product per
instruction, then the fp32 accumulation), "serial" rounds after every product
(the most rounding any fp32 order performs).
"""
from __future__ import annotations

import numpy as np

LOG2E = 1.4426950408889634
SLICE = 64
LAZY = 8.0

f32 = np.float32


def round16(x: np.ndarray, fmt: str) -> np.ndarray:
    """fp32 values rounded to nearest-even in bfloat16 or binary16, returned as fp32."""
    x = np.ascontiguousarray(x, dtype=f32)
    if fmt == "f16":
        return x.astype(np.float16).astype(f32)
    u = x.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(f32)


def _dot_fp32(a: np.ndarray, b: np.ndarray, model: str) -> np.ndarray:
    """a (n x d) . b^T (m x d) accumulated in fp32 under a summation model;
    the inputs are exact 16-bit values, so each product is exact in fp32."""
    n, d = a.shape
    acc = np.zeros((n, b.shape[0]), f32)
    if model == "chunk":
        for d0 in range(0, d, 16):
            part = a[:, d0:d0 + 16].astype(np.float64) @ b[:, d0:d0 + 16].T.astype(np.float64)
            acc = (acc.astype(np.float64) + part).astype(f32)
    else:
        for e in range(d):
            prod = np.outer(a[:, e], b[:, e]).astype(f32)
            acc = (acc + prod).astype(f32)
    return acc


def kernel_model(q: np.ndarray, k: np.ndarray, v: np.ndarray, fmt: str, scale: float, model: str = "chunk",
                 drop=(), repeat=None, ftz: bool = False) -> np.ndarray:
    """O (Sq x Dv, fp32) for decoded 16-bit inputs q (Sq x D), k (Sk x D), v
    (Sk x Dv). `drop` lists slices the modelled kernel skips entirely;
    `repeat = (s, r)` makes it read slice r's keys and values in place of
    slice s's (a ring slot mix-up); `ftz` flushes probabilities and rescale
    factors below fp32's normal range (2^-126) to zero, as an exponential
    unit without denormal results would."""
    q = np.asarray(q, f32)
    k = np.asarray(k, f32)
    v = np.asarray(v, f32)
    Sq, Sk = q.shape[0], k.shape[0]
    c = f32(scale * LOG2E)
    if c < 0:  # a negative scale is folded into the sign of q
        q, c = -q, f32(-c)
    m = np.full(Sq, -np.inf, f32)
    l = np.zeros(Sq, f32)
    o = np.zeros((Sq, v.shape[1]), f32)
    T = (Sk + SLICE - 1) // SLICE
    for t in range(T):
        if t in drop:
            continue
        src = repeat[1] if repeat is not None and repeat[0] == t else t
        ks = k[src * SLICE:min(Sk, (src + 1) * SLICE)]
        vs = v[src * SLICE:min(Sk, (src + 1) * SLICE)]
        s = _dot_fp32(q, ks, model)  # Sq x keys
        ext = s.max(axis=1)
        mcand = np.maximum(m, (c * ext).astype(f32))
        mnew = np.where(mcand > (m + f32(LAZY)).astype(f32), mcand, m).astype(f32)
        with np.errstate(invalid="ignore"):
            alpha = np.exp2((m.astype(np.float64) - mnew)).astype(f32)
        alpha = np.where(np.isneginf(m), f32(0), alpha).astype(f32)
        if ftz:
            alpha = np.where(alpha < f32(2.0 ** -126), f32(0), alpha).astype(f32)
        # x = fma(s, c, -m): the product is exact in fp64, one rounding to fp32
        x = (s.astype(np.float64) * np.float64(c) - mnew[:, None]).astype(f32)
        p = np.exp2(x.astype(np.float64)).astype(f32)
        if ftz:
            p = np.where(p < f32(2.0 ** -126), f32(0), p).astype(f32)
        rs = np.zeros(Sq, f32)
        for j in range(p.shape[1]):
            rs = (rs + p[:, j]).astype(f32)
        l = ((l * alpha).astype(f32) + rs).astype(f32)
        m = mnew
        o = (o * alpha[:, None]).astype(f32)
        pr = round16(p, fmt)
        o = (o + _dot_fp32(pr, vs.T.copy(), model)).astype(f32)
    inv = (f32(1) / l).astype(f32)
    return (o * inv[:, None]).astype(f32)
