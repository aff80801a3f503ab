"""Parity of the attention kernels with the oracle, through the C ABI:
|O - O_ref| <= (e_p + 4 delta_i) sum_j w_j |v_jc| + Sk tau max_j |v_jc|
elementwise (e_p = 2^-6 for bfloat16, 2^-8 for binary16: the probabilities'
rounding; delta_i = |scale| (D + 8) 2^-24 max_j sum_d |q_id||k_jd|: the
scores' fp32 rounding; tau = 2^-125 for bfloat16 (fp32 underflow), 2^-25 for
binary16 (its smallest subnormal spacing, halved): weights too small for a
relative error),
bit-identical across fills and ring depths, O's padding untouched. Inputs: the 16-bit seeded grid generator (values on the format's
grid in [-1, 1))."""
import numpy as np
import pytest
import torch

import async_global_shared_amd as m
import datagen
import oracle

pytestmark = pytest.mark.gpu

TORCH16 = {"bf16": torch.bfloat16, "f16": torch.float16}
SENTINEL = -12345.0


def host16(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def dev_qkv(seed, B, H, S, D, fmt, layout="bhsd", offset=0):
    """(B, H, S, D) 16-bit device view of seeded grid values; layout "bshd"
    stores it as (B, S, H, D); `offset` elements of NaN sit before it."""
    n = B * H * S * D
    vals = datagen.grid16_torch(seed, 1, n, fmt, device="cuda").view(-1)
    buf = torch.full((n + offset + 64,), float("nan"), dtype=TORCH16[fmt], device="cuda")
    if layout == "bhsd":
        buf[offset:offset + n] = vals
        return buf[offset:offset + n].view(B, H, S, D)
    store = buf[offset:offset + n].view(B, S, H, D)
    store.copy_(vals.view(B, H, S, D).permute(0, 2, 1, 3))
    return store.permute(0, 2, 1, 3)


def out_view(B, H, S, D, pad=0):
    """fp32 (B, H, S, D) view with rows of D + pad floats; padding holds SENTINEL."""
    buf = torch.full((B, H, S, D + pad), SENTINEL, dtype=torch.float32, device="cuda")
    return buf[..., :D], buf


def fits(stages, fill, D=128):
    try:
        m.plan_attention(1, 1, 128, 128, D, stages=stages, fill=fill)
        return True
    except m.MgemmError:
        return False


VARIANTS = [(f, S) for f in ("sync", "piped") for S in (1, 2, 3, 4) if not (f == "sync" and S == 4)]


def check(O, Q, K, V, fmt, scale, what, heads=None, rows=None):
    """O (B, H, Sq, D) device result against the oracle on all or some heads / rows."""
    Qh, Kh, Vh = host16(Q), host16(K), host16(V)
    Oh = O.cpu().numpy()
    B, H = Qh.shape[:2]
    for b, h in (heads or [(b, h) for b in range(B) for h in range(H)]):
        q = Qh[b, h] if rows is None else np.ascontiguousarray(Qh[b, h][rows])
        ref = oracle.attention_f64(q, Kh[b, h], Vh[b, h], fmt, scale, with_abs=True)
        got = Oh[b, h] if rows is None else Oh[b, h][rows]
        err = np.abs(got.astype(np.float64) - ref.O)
        bnd = oracle.attention_bound(ref, fmt, scale)
        bad = ~(err <= bnd)
        if bad.any():
            i, c = np.argwhere(bad)[0]
            raise AssertionError(f"{what} head ({b},{h}): {bad.sum()} outside the bound, first ({i},{c}): got "
                                 f"{got[i, c]!r} want {ref.O[i, c]!r} bound {bnd[i, c]!r}")


SHAPES = [  # B, H, Sq, Sk, D
    (1, 2, 130, 77, 64),
    (2, 1, 256, 256, 128),
    (1, 3, 200, 300, 64),
    (1, 1, 33, 1, 128),
    (1, 1, 1, 513, 128),
    (1, 2, 70, 192, 128),  # 3 key slices: the two-set synchronous ring's masked last load
    (1, 1, 90, 256, 64),  # 4 key slices: no masked load
]


@pytest.mark.parametrize("fmt", ["bf16", "f16"])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_every_variant(fmt, shape):
    B, H, Sq, Sk, D = shape
    Q = dev_qkv(1, B, H, Sq, D, fmt)
    K = dev_qkv(2, B, H, Sk, D, fmt)
    V = dev_qkv(3, B, H, Sk, D, fmt)
    scale = D ** -0.5
    ref = None
    for fill, S in VARIANTS:
        if not fits(S, fill, D):
            continue
        O, buf = out_view(B, H, Sq, D, pad=3)
        m.attention(Q, K, V, O, scale=scale, stages=S, fill=fill)
        torch.cuda.synchronize()
        assert bool(torch.all(buf[..., D:] == SENTINEL)), (fill, S)
        if ref is None:
            check(O, Q, K, V, fmt, scale, f"{fmt} {shape} {fill} S{S}")
            ref = O.clone()
        else:
            assert torch.equal(O.view(torch.int32), ref.view(torch.int32)), (fmt, shape, fill, S)


@pytest.mark.parametrize("fmt", ["bf16", "f16"])
@pytest.mark.parametrize("D", [64, 128])
def test_long_key_sequence(fmt, D):
    """32805 keys (513 slices, the last one ragged) for 70 queries of two
    heads: the online softmax over a long ring, every fill and depth that
    fits, within the bound and bit-identical."""
    B, H, Sq, Sk = 1, 2, 70, 32805
    Q = dev_qkv(13, B, H, Sq, D, fmt)
    K = dev_qkv(14, B, H, Sk, D, fmt)
    V = dev_qkv(15, B, H, Sk, D, fmt)
    scale = D ** -0.5
    ref = None
    for fill, S in VARIANTS:
        if not fits(S, fill, D):
            continue
        O, buf = out_view(B, H, Sq, D, pad=2)
        m.attention(Q, K, V, O, scale=scale, stages=S, fill=fill)
        torch.cuda.synchronize()
        assert bool(torch.all(buf[..., D:] == SENTINEL)), (fill, S)
        if ref is None:
            check(O, Q, K, V, fmt, scale, f"{fmt} D{D} long keys {fill} S{S}")
            ref = O.clone()
        else:
            assert torch.equal(O.view(torch.int32), ref.view(torch.int32)), (fmt, D, fill, S)


@pytest.mark.parametrize("D", [64, 128])
def test_many_heads(D):
    """5 x 37 (batch, head) pairs of 300 queries: 370 blocks, not a multiple
    of the 8 XCDs, so the block -> (batch, head, query block) map runs with a
    remainder; (batch, seq, head, dim) storage. Six heads against the oracle,
    every head bit-identical across fills and depths."""
    fmt, B, H, Sq, Sk = "bf16", 5, 37, 300, 130
    Q = dev_qkv(16, B, H, Sq, D, fmt, layout="bshd")
    K = dev_qkv(17, B, H, Sk, D, fmt, layout="bshd")
    V = dev_qkv(18, B, H, Sk, D, fmt, layout="bshd")
    assert m.plan_attention(B, H, Sq, Sk, D)["blocks"] == B * H * 2
    scale = D ** -0.5
    ref = None
    for fill, S in (("sync", 1), ("piped", 2), ("piped", 3)):
        O, buf = out_view(B, H, Sq, D, pad=1)
        m.attention(Q, K, V, O, scale=scale, stages=S, fill=fill)
        torch.cuda.synchronize()
        assert bool(torch.all(buf[..., D:] == SENTINEL)), (fill, S)
        if ref is None:
            check(O, Q, K, V, fmt, scale, f"many heads D{D}", heads=[(0, 0), (0, 36), (2, 17), (3, 5), (4, 0), (4, 36)])
            ref = O.clone()
        else:
            assert torch.equal(O.view(torch.int32), ref.view(torch.int32)), (D, fill, S)


@pytest.mark.parametrize("fmt", ["bf16", "f16"])
def test_layouts(fmt):
    """(batch, seq, head, dim) storage, misaligned bases (4-byte loads) and a
    padded output give the same bits as contiguous inputs."""
    B, H, Sq, Sk, D = 2, 3, 150, 190, 128
    base = [dev_qkv(s, B, H, n, D, fmt) for s, n in ((4, Sq), (5, Sk), (6, Sk))]
    O0 = m.attention(*base)
    torch.cuda.synchronize()
    check(O0, *base, fmt, D ** -0.5, f"{fmt} contiguous", heads=[(0, 0), (1, 2)])
    assert m.plan_attention(B, H, Sq, Sk, D)["load_bytes"] == 16
    for layout, offset in (("bshd", 0), ("bhsd", 2), ("bshd", 6)):
        qkv = [dev_qkv(s, B, H, n, D, fmt, layout=layout, offset=offset) for s, n in ((4, Sq), (5, Sk), (6, Sk))]
        for t, ref in zip(qkv, base):
            assert torch.equal(t, ref)
        O, buf = out_view(B, H, Sq, D, pad=1)
        for fill, S in (("piped", 2), ("sync", 1)):
            m.attention(*qkv, O, stages=S, fill=fill)
            torch.cuda.synchronize()
            assert torch.equal(O.contiguous().view(torch.int32), O0.view(torch.int32)), (layout, offset, fill, S)
            assert bool(torch.all(buf[..., D:] == SENTINEL))


@pytest.mark.parametrize("scale", [0.0, 2.0, 40.0, -1.5])
def test_scales(scale):
    """scale 0 (uniform weights: the mean of V), peaked and nearly one-hot
    softmax rows, and a negative scale (the row maximum of scale * s is then
    scale * min(s))."""
    fmt, B, H, Sq, Sk, D = "bf16", 1, 2, 96, 200, 64
    Q, K, V = (dev_qkv(s, B, H, n, D, fmt) for s, n in ((7, Sq), (8, Sk), (9, Sk)))
    O = m.attention(Q, K, V, scale=scale)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(O).all())
    check(O, Q, K, V, fmt, scale, f"scale {scale}")


@pytest.mark.parametrize("scale", [1.0, 4.0, 6.0])
def test_scores_rising_across_slices(scale):
    """Scores that climb with the key index, by about 1.4, 5.8 and 8.7 (log2
    units) per 64-key slice: the running reference stays behind the true
    maximum for several slices (probabilities up to 2^8) or moves every
    slice, and the result still matches the oracle."""
    fmt, B, H, Sq, Sk, D = "bf16", 1, 1, 64, 1000, 64
    q = np.zeros((Sq, D), np.float32)
    q[:, 0] = 1.0
    q[:, 1] = np.linspace(-0.5, 0.5, Sq)
    k = np.zeros((Sk, D), np.float32)
    k[:, 0] = np.arange(Sk) / 64.0
    k[:, 1] = np.cos(np.arange(Sk))
    Q, K = (torch.from_numpy(x).to(torch.bfloat16).cuda().view(B, H, -1, D) for x in (q, k))  # rounded to bf16
    V = dev_qkv(31, B, H, Sk, D, fmt)
    O = m.attention(Q, K, V, scale=scale)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(O).all())
    check(O, Q, K, V, fmt, scale, f"rising scores, scale {scale}")


def test_one_key_returns_its_value_row():
    fmt, D = "bf16", 128
    Q, K, V = dev_qkv(10, 1, 1, 70, D, fmt), dev_qkv(11, 1, 1, 1, D, fmt), dev_qkv(12, 1, 1, 1, D, fmt)
    O = m.attention(Q, K, V)
    torch.cuda.synchronize()
    assert torch.equal(O[0, 0], V[0, 0].float().expand(70, D))


def test_refused_arguments():
    Q = torch.zeros((1, 1, 8, 64), dtype=torch.bfloat16, device="cuda")
    K0 = torch.zeros((1, 1, 0, 64), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(m.MgemmError) as e:
        m.attention(Q, K0, K0)
    assert e.value.status == m.ERR_ARG
    Q96 = torch.zeros((1, 1, 8, 96), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(m.MgemmError):
        m.attention(Q96, Q96, Q96)
    E = torch.zeros((1, 1, 0, 64), dtype=torch.bfloat16, device="cuda")
    m.attention(E, Q, Q)  # no queries: nothing to do


@pytest.mark.parametrize("fmt", ["bf16", "f16"])
def test_full_size(fmt):
    """B = H = 16, Sq = Sk = 4096, D = 128, in the benchmark's launch
    configuration: nine whole heads (every query row; a different head index
    in each of nine batches, the corners included) against the oracle, bit
    identity across fills and depths on the whole output."""
    B, H, S, D = 16, 16, 4096, 128
    Q, K, V = (dev_qkv(s, B, H, S, D, fmt) for s in (21, 22, 23))
    ref = m.attention(Q, K, V, stages=2, fill="piped")
    other = torch.empty_like(ref)
    for fill, St in (("sync", 1), ("piped", 3), ("piped", 1)):
        other.fill_(float("nan"))
        m.attention(Q, K, V, other, stages=St, fill=fill)
        torch.cuda.synchronize()
        assert torch.equal(other.view(torch.int32), ref.view(torch.int32)), (fmt, fill, St)
    heads = [(0, 0), (15, 15)] + [(b, (5 * b + 3) % H) for b in range(1, 15, 2)]
    print(f"{fmt} full size: oracle on {len(heads)} whole heads", flush=True)
    check(ref, Q, K, V, fmt, D ** -0.5, f"{fmt} full size", heads=heads)


# ---- full-size slice sentinels -------------------------------------------------------
# At B = H = 16, Sq = Sk = 4096 a skipped or repeated 64-key slice stays inside
# the bound on seeded random inputs (the bound scales with the output's own
# size), so two structured inputs check every slice at that size instead; the
# CPU tests in test_attention_bound.py show that the oracle reproduces both
# closed forms and that a kernel which drops or repeats one slice misses them.

FULL_B, FULL_H, FULL_S = 16, 16, 4096


@pytest.mark.parametrize("fmt", ["bf16", "f16"])
@pytest.mark.parametrize("D", [128, 64])
def test_full_size_uniform_slice_sentinel(fmt, D):
    """scale 0 (every weight 1/4096) and V[b, h, j, c] = floor(j/64) + r with
    r = (c + 7h + 3b) mod D: every output is exactly 31.5 + r, on the whole
    output, for every fill and depth."""
    B, H, S = FULL_B, FULL_H, FULL_S
    Q, K = dev_qkv(41, B, H, S, D, fmt), dev_qkv(42, B, H, S, D, fmt)
    V = datagen.attn_slice_sentinel_v(B, H, S, D, device="cuda").to(TORCH16[fmt])
    c = torch.arange(D, device="cuda")
    r = (c[None, None, :] + 7 * torch.arange(H, device="cuda")[None, :, None] +
         3 * torch.arange(B, device="cuda")[:, None, None]) % D
    want = (31.5 + r.to(torch.float32))[:, :, None, :].expand(B, H, S, D)
    O = torch.empty((B, H, S, D), device="cuda")
    for fill, St in VARIANTS:
        if not fits(St, fill, D):
            continue
        print(f"uniform slice sentinel {fmt} D={D} {fill} S={St}", flush=True)
        O.fill_(float("nan"))
        m.attention(Q, K, V, O, scale=0.0, stages=St, fill=fill)
        torch.cuda.synchronize()
        assert torch.equal(O, want), (fmt, D, fill, St)


@pytest.mark.parametrize("fmt", ["bf16", "f16"])
@pytest.mark.parametrize("D", [128, 64])
def test_full_size_peaked_winner(fmt, D):
    """Each query's winning key scores 2 and every other key at most 1
    (datagen.attn_peaked_qk); at scale 30 the output is the winner's V row
    to within 2^-22 relative (+1e-9). Over a head's 4096 queries every key
    wins once, so a slice read from the wrong slot or skipped changes whole
    output rows. Whole output, every fill and depth; bit identity across
    them; sampled heads and rows against the oracle's bound."""
    B, H, S = FULL_B, FULL_H, FULL_S
    scale = 30.0
    Qf, Kf = datagen.attn_peaked_qk(B, H, S, S, D, device="cuda")
    Q, K = Qf.to(TORCH16[fmt]), Kf.to(TORCH16[fmt]).contiguous()
    del Qf, Kf
    V = dev_qkv(43, B, H, S, D, fmt)
    w = datagen.attn_peaked_winner(B, H, S, device="cuda")
    Vw = torch.gather(V.float(), 2, w[..., None].expand(B, H, S, D))
    tol = 2.0 ** -22 * Vw.abs() + 1e-9
    O = torch.empty((B, H, S, D), device="cuda")
    ref = None
    for fill, St in VARIANTS:
        if not fits(St, fill, D):
            continue
        print(f"peaked winner {fmt} D={D} {fill} S={St}", flush=True)
        O.fill_(float("nan"))
        m.attention(Q, K, V, O, scale=scale, stages=St, fill=fill)
        torch.cuda.synchronize()
        bad = ~((O - Vw).abs() <= tol)
        assert not bool(bad.any()), (fmt, D, fill, St, int(bad.sum()))
        if ref is None:
            ref = O.clone()
        else:
            assert torch.equal(O.view(torch.int32), ref.view(torch.int32)), (fmt, D, fill, St)
    rows = np.array([0, 1, 63, 64, 2047, S - 1])
    check(ref, Q, K, V, fmt, scale, f"{fmt} D={D} peaked", heads=[(0, 0), (9, 5)], rows=rows)
