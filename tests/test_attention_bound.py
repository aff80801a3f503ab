"""The attention acceptance bound, pinned from outside its own formula.

The oracle's bound (oracle.attention_bound) is
(e_p + 4 delta_i) sum_j w_j |v_jc| + Sk tau max_j |v_jc|. Restating that
formula in a test would pin nothing, so this file checks it against two
things that do not contain it:

* a numpy model of the kernels' rounding (tests/attn_kernel_model.py: fp32
  scores under two summation orders, fp32 exponentials and sums, 16-bit
  probabilities): on seeded and adversarial inputs it must land inside the
  bound with a margin, while the same model with a slice of keys skipped or
  read from the wrong slot must land outside it. For each of the bound's
  terms there is a crafted input that the model only meets with that term
  present (for binary16 the floor tau is its subnormal spacing: the model
  found that probabilities of 2^-43 round to zero there, which the fp32
  underflow floor alone did not cover);
* the closed forms of the two full-size slice sentinels that the GPU tests
  compare with bit for bit (or within 2^-22 relative): the oracle reproduces
  them at 4096 keys, and the model of a kernel that drops or repeats any one
  of the 64 slices misses them in every column.

The tile loop is the async copy article's ("from cp.async to memcpy_async",
section 6.2, "FlashAttention's tile pipeline"); the readings of its precision
are the oracle's.
"""
import math

import numpy as np
import pytest
import torch

import datagen
import oracle
from tests.attn_kernel_model import LOG2E, SLICE, kernel_model
from tests.oracle16_pins import _decoded_by_library as dec


def _m16(seed, rows, cols, fmt):
    return datagen.matrix16(seed, rows, cols, fmt)


def _bits(x, fmt):
    return datagen.to_bits16(np.asarray(x, np.float32), fmt)


def _ratio(O, ref, fmt, scale, bound=None):
    b = oracle.attention_bound(ref, fmt, scale) if bound is None else bound
    return float(np.max(np.abs(O.astype(np.float64) - ref.O) / b))


SEEDED = [  # Sq, Sk, D, scale
    (16, 64, 64, 0.125), (16, 200, 64, 64 ** -0.5), (16, 513, 16, 2.0), (8, 300, 64, 40.0), (8, 130, 64, -1.5),
    (8, 256, 128, 0.0), (8, 1, 64, 1.0), (8, 100, 64, 200.0), (4, 65, 128, 128 ** -0.5),
]


@pytest.mark.parametrize("fmt", ["bf16", "f16"])
@pytest.mark.parametrize("case", SEEDED, ids=lambda c: "x".join(map(str, c)))
def test_kernel_rounding_lands_inside_with_margin(fmt, case):
    Sq, Sk, D, scale = case
    Q, K, V = _m16(1, Sq, D, fmt), _m16(2, Sk, D, fmt), _m16(3, Sk, D, fmt)
    ref = oracle.attention_f64(Q, K, V, fmt, scale, with_abs=True)
    for model in ("chunk", "serial"):
        O = kernel_model(dec(Q, fmt), dec(K, fmt), dec(V, fmt), fmt, scale, model)
        assert _ratio(O, ref, fmt, scale) <= 0.5, (fmt, case, model)


@pytest.mark.parametrize("fmt", ["bf16", "f16"])
@pytest.mark.parametrize("Sk", [200, 256])
def test_a_skipped_or_repeated_slice_lands_outside(fmt, Sk):
    """At a few slices the bound sees every single-slice mistake: each slice
    dropped, and each slice read from its predecessor's slot."""
    Sq, D, scale = 8, 64, 64 ** -0.5
    Q, K, V = _m16(4, Sq, D, fmt), _m16(5, Sk, D, fmt), _m16(6, Sk, D, fmt)
    ref = oracle.attention_f64(Q, K, V, fmt, scale, with_abs=True)
    q, k, v = dec(Q, fmt), dec(K, fmt), dec(V, fmt)
    T = (Sk + SLICE - 1) // SLICE
    for s in range(T):
        assert _ratio(kernel_model(q, k, v, fmt, scale, drop=(s,)), ref, fmt, scale) > 1.0, ("drop", s)
        if s > 0:
            assert _ratio(kernel_model(q, k, v, fmt, scale, repeat=(s, s - 1)), ref, fmt, scale) > 1.0, ("repeat", s)


def test_probability_rounding_term_is_needed():
    """q = 1, one key at 1 and 199 at 1/2, V = 1: every non-maximal weight
    is just below 1/2 + 2^-9, which bfloat16 rounds down to 1/2 (relative
    error near its unit roundoff 2^-8), all in one direction. The model sits
    at about a quarter of the bound; e_p cut to 2^-9 would refuse it."""
    fmt, Sk = "bf16", 200
    c = -math.log2(0.5 + 2.0 ** -9 - 2.0 ** -14) / 0.5
    scale = c / LOG2E
    Q, K, V = _bits([[1.0]], fmt), _bits([[1.0]] + [[0.5]] * (Sk - 1), fmt), _bits([[1.0]] * Sk, fmt)
    ref = oracle.attention_f64(Q, K, V, fmt, scale, with_abs=True)
    O = kernel_model(dec(Q, fmt), dec(K, fmt), dec(V, fmt), fmt, scale)
    r = _ratio(O, ref, fmt, scale)
    assert 0.15 < r <= 0.5, r
    b = oracle.attention_bound(ref, fmt, scale)
    e_p = 2.0 ** -6
    assert _ratio(O, ref, fmt, scale, bound=b - (e_p - 2.0 ** -9) * ref.Wabs) > 1.0


def test_score_rounding_term_is_needed():
    """q = (256, 2^-5), k0 = (256, 2^-4), k1 = (256, 0): the exact scores
    65536 + 2^-9 and 65536 differ, but an fp32 sum cannot hold the first, so
    the kernel's two weights come out equal where the true ones are 2 : 1.
    Only the delta term (fp32 score error, scaled by the score magnitude G)
    covers that."""
    fmt = "bf16"
    Q, K, V = _bits([[256.0, 2 ** -5]], fmt), _bits([[256.0, 2 ** -4], [256.0, 0.0]], fmt), _bits([[1.0], [-1.0]], fmt)
    scale = 2.0 ** 9 / LOG2E
    ref = oracle.attention_f64(Q, K, V, fmt, scale, with_abs=True)
    assert abs(ref.O[0, 0] - 1.0 / 3.0) < 1e-8  # fp64 scores near 2^24 carry about 1e-9
    O = kernel_model(dec(Q, fmt), dec(K, fmt), dec(V, fmt), fmt, scale)
    assert O[0, 0] == 0.0
    assert _ratio(O, ref, fmt, scale) <= 0.5
    b_no_delta = 2.0 ** -6 * ref.Wabs + ref.Sk * 2.0 ** -125 * ref.Vmax[None, :]
    assert _ratio(O, ref, fmt, scale, bound=b_no_delta) > 1.0


def test_underflow_term_is_needed():
    """One key scores 1 (its value 0), 199 keys score 0 (value 1), scale such
    that their probabilities are 2^-130: an exponential without denormal
    results returns 0 for them, so O = 0 where the exact value is about
    199 2^-130. Only the underflow term covers a weight that small."""
    fmt, Sk = "bf16", 200
    scale = 130.0 / LOG2E
    Q, K = _bits([[1.0]], fmt), _bits([[1.0]] + [[0.0]] * (Sk - 1), fmt)
    V = _bits([[0.0]] + [[1.0]] * (Sk - 1), fmt)
    ref = oracle.attention_f64(Q, K, V, fmt, scale, with_abs=True)
    O = kernel_model(dec(Q, fmt), dec(K, fmt), dec(V, fmt), fmt, scale, ftz=True)
    assert O[0, 0] == 0.0 and ref.O[0, 0] > 0.0
    assert _ratio(O, ref, fmt, scale) <= 0.5
    b_no_floor = (2.0 ** -6 + 4.0 * abs(scale) * (ref.D + 8) * 2.0 ** -24 * ref.G[..., None]) * ref.Wabs
    assert _ratio(O, ref, fmt, scale, bound=b_no_floor) > 1.0


def test_binary16_underflow_term_is_needed():
    """The peaked pattern at scale 30 in binary16: the runners-up weigh about
    2^-43, below binary16's smallest subnormal, so the kernel's P V product
    sees them as 0. Where the winner's value is 0 the exact output is a sum
    of those tiny weights and the kernel's is 0: only the floor of 2^-25 per
    key (half the subnormal spacing) covers it; fp32's 2^-125 does not."""
    fmt, D, scale = "f16", 128, 30.0
    Qf, Kf = datagen.attn_peaked_qk(1, 1, FULL_SK, FULL_SK, D)
    rows = np.array([0, 1, 63, 64, 2000, FULL_SK - 1])
    Q, K = _bits(Qf[0, 0].numpy()[rows], fmt), _bits(Kf[0, 0].numpy(), fmt)
    V = _m16(9, FULL_SK, D, fmt)
    ref = oracle.attention_f64(Q, K, V, fmt, scale, with_abs=True)
    O = kernel_model(dec(Q, fmt), dec(K, fmt), dec(V, fmt), fmt, scale)
    assert _ratio(O, ref, fmt, scale) <= 0.5
    b_fp32_floor = (oracle.attention_bound(ref, fmt, scale) - ref.Sk * (2.0 ** -25 - 2.0 ** -125) *
                    ref.Vmax[None, :])
    assert _ratio(O, ref, fmt, scale, bound=b_fp32_floor) > 1.0


# ---- the full-size slice sentinels (closed forms the GPU tests compare with) ----

FULL_SK, FULL_D = 4096, 128


def _first_queries(x, n):
    return np.ascontiguousarray(x[:n])


@pytest.mark.parametrize("fmt", ["bf16", "f16"])
def test_uniform_sentinel_closed_form_and_its_misses(fmt):
    """scale = 0 and V[j, c] = floor(j/64) + r_c: uniform weights, so
    O[i, c] = 31.5 + r_c, exactly representable and reached exactly by fp32
    sums of integers below 2^20. The oracle reproduces it at 4096 keys; the
    model of a kernel that drops or repeats any single slice misses it in
    every column."""
    Vt = datagen.attn_slice_sentinel_v(1, 2, FULL_SK, FULL_D)  # (1, 2, Sk, D) float32
    r = (np.arange(FULL_D)[None, :] + 7 * np.arange(2)[:, None]) % FULL_D  # r_c per head
    want = 31.5 + r.astype(np.float64)
    Qa = _m16(7, 3, FULL_D, fmt)
    Ka = _m16(8, FULL_SK, FULL_D, fmt)
    for h in range(2):
        V = _bits(Vt[0, h].numpy(), fmt)
        O = oracle.attention_f64(Qa, Ka, V, fmt, 0.0)
        assert np.array_equal(O, np.broadcast_to(want[h], O.shape)), h
    q, k, v = dec(Qa, fmt)[:2], dec(Ka, fmt), dec(_bits(Vt[0, 0].numpy(), fmt), fmt)
    assert np.array_equal(kernel_model(q, k, v, fmt, 0.0), np.broadcast_to(want[0], (2, FULL_D)).astype(np.float32))
    T = FULL_SK // SLICE
    for s in (0, 1, 6, T // 2, T - 1):
        for kw in ({"drop": (s,)}, {"repeat": (s, s - 1 if s else 1)}):
            O = kernel_model(q, k, v, fmt, 0.0, **kw)
            assert np.all(O != want[0].astype(np.float32)), (s, kw)


@pytest.mark.parametrize("fmt", ["bf16", "f16"])
@pytest.mark.parametrize("D", [64, 128])
def test_peaked_sentinel_closed_form_and_its_misses(fmt, D):
    """The peaked pattern at scale 30: each query's winner scores 2, every
    other key at most 1, so the runners-up weigh 2^-43 each and O is the
    winner's V row to within 2^-22 relative (+1e-9). The oracle agrees; the
    model of a kernel that drops the winner's slice, or reads it from the
    neighbouring slot, misses by far more than that."""
    Sq, scale = 6, 30.0
    Qf, Kf = datagen.attn_peaked_qk(1, 1, FULL_SK, FULL_SK, D)
    w = datagen.attn_peaked_winner(1, 1, FULL_SK)[0, 0].numpy()
    rows = np.array([0, 1, 63, 64, 2000, FULL_SK - 1])
    Q = _bits(Qf[0, 0].numpy()[rows], fmt)
    K = _bits(Kf[0, 0].numpy(), fmt)
    V = _m16(9, FULL_SK, D, fmt)
    vw = dec(V, fmt)[w[rows]]
    tol = 2.0 ** -22 * np.abs(vw) + 1e-9
    ref = oracle.attention_f64(Q, K, V, fmt, scale, with_abs=True)
    assert np.all(np.abs(ref.O - vw) <= tol)
    q, k, v = dec(Q, fmt), dec(K, fmt), dec(V, fmt)
    O = kernel_model(q, k, v, fmt, scale)
    assert np.all(np.abs(O - vw) <= tol)
    assert _ratio(O, ref, fmt, scale) <= 0.5
    for i in range(Sq):
        s = int(w[rows[i]]) // SLICE
        for kw in ({"drop": (s,)}, {"repeat": (s, s - 1 if s else 1)}):
            Oi = kernel_model(q[i:i + 1], k, v, fmt, scale, **kw)
            assert np.sum(np.abs(Oi[0] - vw[i]) > tol[i]) >= D // 2, (i, kw)


def test_peaked_pattern_structure():
    """Winners: every key of a head exactly once over 4096 queries, every
    slice 64 times; the winner's score is 2 and every other score at most 1."""
    Q, K = datagen.attn_peaked_qk(2, 3, FULL_SK, FULL_SK, 64)
    w = datagen.attn_peaked_winner(2, 3, FULL_SK)
    for b in range(2):
        for h in range(3):
            assert torch.equal(torch.sort(w[b, h]).values, torch.arange(FULL_SK))
    s = Q[0, 1, :256] @ K[0, 1].T
    top = s.topk(2, dim=1)
    assert torch.equal(top.indices[:, 0], w[0, 1, :256])
    assert bool(torch.all(top.values[:, 0] == 2)) and bool(torch.all(top.values[:, 1] <= 1))
