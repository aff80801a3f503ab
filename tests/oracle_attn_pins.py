"""Pins of the oracle's attention (softmax(scale Q K^T) V over 16-bit inputs),
each a function of a loaded oracle library that raises AssertionError on a
mismatch. None of them reuses the oracle's arithmetic: they compare with a
library softmax, closed forms and invariants of the definition."""
import math
from fractions import Fraction

import numpy as np
import scipy.special

import datagen
import oracle
from tests.oracle16_pins import _decoded_by_library


def _lib_attention(Q, K, V, fmt, scale):
    """softmax(scale q k^T) v through numpy / scipy on library-decoded values."""
    q, k, v = (_decoded_by_library(x, fmt) for x in (Q, K, V))
    s = scale * (q @ np.swapaxes(k, -1, -2))
    w = scipy.special.softmax(s, axis=-1)
    return w @ v, w @ np.abs(v), (np.abs(q) @ np.abs(np.swapaxes(k, -1, -2))).max(axis=-1)


def _m(seed, rows, cols, fmt, kind="grid", pad=0):
    return datagen.matrix16(seed, rows, cols, fmt, kind=kind, ld=cols + pad)[:, :cols]


def pin_attention_matches_library_softmax(lib, cases=24):
    rng = np.random.default_rng(11)
    for c in range(cases):
        fmt = ("bf16", "f16")[c % 2]
        Sq, Sk, D, Dv = (int(x) for x in rng.integers(1, 12, size=4))
        pads = [int(x) for x in rng.integers(0, 3, size=3)]
        Q = _m(500 + c, Sq, D, fmt, pad=pads[0])
        K = _m(600 + c, Sk, D, fmt, pad=pads[1])
        V = _m(700 + c, Sk, Dv, fmt, pad=pads[2])
        scale = float(rng.uniform(0.05, 3.0))
        O, W, G, Vm, Dd, Skk = oracle.attention_f64(Q, K, V, fmt, scale, with_abs=True, lib=lib)
        Or, Wr, Gr = _lib_attention(Q, K, V, fmt, scale)
        assert np.allclose(O, Or, rtol=1e-12, atol=1e-14), (c, np.abs(O - Or).max())
        assert np.allclose(W, Wr, rtol=1e-12, atol=1e-14), c
        assert np.allclose(G, Gr, rtol=1e-13, atol=0), c
        assert np.array_equal(Vm, np.abs(_decoded_by_library(V, fmt)).max(axis=0)) and (Dd, Skk) == (D, Sk), c


def pin_attention_single_key(lib):
    # one key: its weight is exp(0) / exp(0) = 1 exactly, so O is that V row
    for fmt in ("bf16", "f16"):
        Q, K, V = _m(1, 6, 8, fmt), _m(2, 1, 8, fmt), _m(3, 1, 5, fmt)
        O = oracle.attention_f64(Q, K, V, fmt, 0.7, lib=lib)
        want = _decoded_by_library(V, fmt)[0]
        assert np.array_equal(O, np.broadcast_to(want, O.shape)), fmt


def pin_attention_equal_keys_average_v(lib):
    # identical keys (or scale 0): uniform weights, O = mean of the V rows
    fmt = "bf16"
    Sk = 7
    Q = _m(4, 3, 16, fmt)
    K = np.repeat(_m(5, 1, 16, fmt), Sk, axis=0)
    V = _m(6, Sk, 4, fmt)
    vd = _decoded_by_library(V, fmt)
    mean = [float(sum(Fraction(x) for x in vd[:, c]) / Sk) for c in range(4)]
    for KK, scale in ((K, 1.3), (_m(7, Sk, 16, fmt), 0.0)):
        O = oracle.attention_f64(Q, KK, V, fmt, scale, lib=lib)
        assert np.allclose(O, np.broadcast_to(mean, O.shape), rtol=4e-16, atol=4e-16), scale


def pin_attention_two_keys_logistic(lib):
    # s0 - s1 = scale (k0 - k1) with q = 1: w0 is the logistic function of it
    fmt = "bf16"
    for k0, k1, scale, v0, v1 in ((0.5, -0.25, 2.0, 1.0, -3.0), (0.75, 0.5, 40.0, 0.125, 2.0),
                                  (-1.0, 1.0, 0.5, 4.0, -4.0)):
        Q = datagen.to_bits16(np.array([[1.0]], np.float32), fmt)
        K = datagen.to_bits16(np.array([[k0], [k1]], np.float32), fmt)
        V = datagen.to_bits16(np.array([[v0], [v1]], np.float32), fmt)
        O = oracle.attention_f64(Q, K, V, fmt, scale, lib=lib)
        w0 = 1.0 / (1.0 + math.exp(-scale * (k0 - k1)))
        assert abs(O[0, 0] - (w0 * v0 + (1 - w0) * v1)) <= 1e-14 * (abs(v0) + abs(v1)), (k0, k1, scale)


def pin_attention_weights_sum_to_one(lib):
    # V = 1: every output is the weight sum, 1; the magnitudes equal it
    for fmt in ("bf16", "f16"):
        Q, K = _m(8, 9, 12, fmt), _m(9, 13, 12, fmt)
        V = _m(0, 13, 3, fmt, kind="ones")
        O, W = oracle.attention_f64(Q, K, V, fmt, 1.7, with_abs=True, lib=lib)[:2]
        assert np.allclose(O, 1.0, rtol=0, atol=1e-14) and np.allclose(W, 1.0, rtol=0, atol=1e-14), fmt


def pin_attention_key_permutation(lib):
    fmt = "f16"
    Q, K, V = _m(10, 5, 8, fmt), _m(11, 9, 8, fmt), _m(12, 9, 6, fmt)
    perm = np.random.default_rng(3).permutation(9)
    O = oracle.attention_f64(Q, K, V, fmt, 0.9, lib=lib)
    Op = oracle.attention_f64(Q, np.ascontiguousarray(K[perm]), np.ascontiguousarray(V[perm]), fmt, 0.9, lib=lib)
    assert np.allclose(O, Op, rtol=1e-13, atol=1e-15)


def pin_attention_shift_invariance(lib):
    # K + u (the same u for every key) adds scale * q.u to each score of a
    # row; softmax ignores it. Coarse-grid values keep K + u exact.
    fmt = "bf16"
    Q, K, V = _m(13, 4, 8, fmt, "coarse"), _m(14, 6, 8, fmt, "coarse"), _m(15, 6, 5, fmt)
    u = datagen.coarse_pm1(16, 8).astype(np.float32)
    Kf = _decoded_by_library(K, fmt).astype(np.float32) + u
    K2 = datagen.to_bits16(Kf, fmt)
    O = oracle.attention_f64(Q, K, V, fmt, 1.1, lib=lib)
    O2 = oracle.attention_f64(Q, K2, V, fmt, 1.1, lib=lib)
    assert np.allclose(O, O2, rtol=1e-12, atol=1e-14)


def pin_attention_linear_in_v(lib):
    fmt = "bf16"
    Q, K = _m(17, 4, 8, fmt), _m(18, 7, 8, fmt)
    V1, V2 = _m(19, 7, 5, fmt, "coarse"), _m(20, 7, 5, fmt, "coarse")
    V12 = datagen.to_bits16(_decoded_by_library(V1, fmt).astype(np.float32) +
                            _decoded_by_library(V2, fmt).astype(np.float32), fmt)
    O1, O2, O12 = (oracle.attention_f64(Q, K, v, fmt, 0.6, lib=lib) for v in (V1, V2, V12))
    assert np.allclose(O1 + O2, O12, rtol=1e-13, atol=1e-14)


def pin_attention_huge_scores(lib):
    # scale 1e6: scores up to ~1e7 (exp overflows unless the row maximum is
    # taken out) and distinct scores at least 1e6 * 2^-14 = 61 apart, so each
    # row returns the V row of its unique best key to within exp(-61)
    fmt = "bf16"
    Q, K, V = _m(21, 6, 4, fmt), _m(22, 10, 4, fmt), _m(23, 10, 3, fmt)
    s = _decoded_by_library(Q, fmt) @ _decoded_by_library(K, fmt).T
    O = oracle.attention_f64(Q, K, V, fmt, 1e6, lib=lib)
    assert np.all(np.isfinite(O))
    vd = _decoded_by_library(V, fmt)
    checked = 0
    for i in range(6):
        top = np.sort(s[i])[::-1]
        if top[0] - top[1] >= 2.0 ** -14:
            assert np.allclose(O[i], vd[int(np.argmax(s[i]))], rtol=0, atol=1e-20), i
            checked += 1
    assert checked >= 3


def pin_attention_leading_axes(lib):
    # (batch, head) axes, including a non-contiguous head view, match per-head calls
    fmt = "f16"
    Q = datagen.matrix16(24, 2 * 3 * 5, 8, fmt).reshape(2, 3, 5, 8)
    K = datagen.matrix16(25, 2 * 4 * 6, 8, fmt).reshape(2, 4, 6, 8)[:, 1:]
    V = datagen.matrix16(26, 2 * 3 * 6, 4, fmt).reshape(2, 3, 6, 4)
    O = oracle.attention_f64(Q, K, V, fmt, 0.8, lib=lib)
    for b in range(2):
        for h in range(3):
            Or, _, _ = _lib_attention(Q[b, h], K[b, h], V[b, h], fmt, 0.8)
            assert np.allclose(O[b, h], Or, rtol=1e-12, atol=1e-14), (b, h)


ALL_ATTN_PINS = [pin_attention_matches_library_softmax, pin_attention_single_key, pin_attention_equal_keys_average_v,
                 pin_attention_two_keys_logistic, pin_attention_weights_sum_to_one, pin_attention_key_permutation,
                 pin_attention_shift_invariance, pin_attention_linear_in_v, pin_attention_huge_scores,
                 pin_attention_leading_axes]
