"""Seeded random shapes, leading dimensions and base offsets, through the C
ABI: the fp32 GEMM on every (compute, tile, fill, depth), the 16-bit GEMM on
every (tile, fill, depth), attention on every (fill, depth) and the tile copy
on every depth. Each result is checked against the oracle (its bound; the copy
bitwise), bits are compared across fills and depths, and nothing outside the
output may change. Sizes stay small enough for the oracle to finish in
seconds, but cross tile, slice and ragged-edge boundaries."""
import os

import numpy as np
import pytest
import torch

import async_global_shared_amd as m
import datagen
import oracle
from tests.gpu_util import SENTINEL, TILES, check_bound, full_rows, out_device, padded_device, same_bits
from tests.test_gpu_attention import check as check_attention
from tests.test_gpu_attention import dev_qkv
from tests.test_gpu_gemm16 import check16, dev16, fits

pytestmark = pytest.mark.gpu

SEED = 20261202
# cases per operation; MGEMM_RANDOM_CASES widens the sweep (e.g. 1096)
CASES = range(int(os.environ.get("MGEMM_RANDOM_CASES", "16")))
PLAIN_CASES = CASES if "MGEMM_RANDOM_CASES" in os.environ else range(8)


def _rng(case):
    return np.random.default_rng([SEED, case])


@pytest.mark.parametrize("case", CASES)
def test_fp32_gemm_random(case):
    rng = _rng(case)
    M, N, K = (int(x) for x in rng.integers(1, 600, size=3))
    pa, pb, pc = (int(x) for x in rng.integers(0, 9, size=3))
    oa, ob, oc = (int(x) for x in rng.integers(0, 4, size=3))  # element offsets: most bases not 16-byte aligned
    A = datagen.matrix("uniform", 100 + case, M, K)
    B = datagen.matrix("uniform", 200 + case, K, N)
    Ad, Bd = padded_device(A, K + pa, offset=oa), padded_device(B, N + pb, offset=ob)
    what = f"case {case}: {M}x{N}x{K} ld+({pa},{pb},{pc}) offsets ({oa},{ob},{oc})"
    for compute, tile in TILES:
        ref = None
        for fill in ("sync", "piped"):
            for S in (1, 2, 3):
                Cd = out_device(M, N, N + pc, offset=oc)
                m.sgemm(Ad, Bd, Cd, stages=S, fill=fill, compute=compute, tile=tile)
                torch.cuda.synchronize()
                full = full_rows(Cd)
                assert np.all(full[:, N:] == SENTINEL), (what, compute, tile, fill, S)
                C = np.ascontiguousarray(full[:, :N])
                if ref is None:
                    check_bound(C, A, B, what=f"{what} {compute} {tile}")
                    ref = C
                else:
                    assert same_bits(C, ref), (what, compute, tile, fill, S)


@pytest.mark.parametrize("case", CASES)
def test_gemm16_random(case):
    rng = _rng(100 + case)
    fmt = ("bf16", "f16")[case % 2]
    M = int(rng.integers(1, 520))
    N, K = (2 * int(x) for x in rng.integers(1, 260, size=2))
    pa, pb, pc = (int(x) for x in rng.integers(0, 5, size=3))
    oa, ob = (2 * int(x) for x in rng.integers(0, 5, size=2))  # even: 4-byte aligned bases
    A = datagen.matrix16(300 + case, M, K, fmt)
    B = datagen.matrix16(400 + case, K, N, fmt)
    Ad, Bd = dev16(A, fmt, K + 2 * pa, oa), dev16(B, fmt, N + 2 * pb, ob)
    what = f"case {case} {fmt}: {M}x{N}x{K} ld+({2 * pa},{2 * pb},{pc}) offsets ({oa},{ob})"
    for tile in ("128x128", "256x128", "256x256"):
        ref = None
        for fill in ("sync", "piped"):
            for S in (1, 2, 3, 4):
                if not fits(tile, S) or (fill == "sync" and S == 4):
                    continue
                Cd = out_device(M, N, N + pc)
                m.gemm16(Ad, Bd, Cd, stages=S, fill=fill, tile=tile)
                torch.cuda.synchronize()
                full = full_rows(Cd)
                assert np.all(full[:, N:] == SENTINEL), (what, tile, fill, S)
                C = np.ascontiguousarray(full[:, :N])
                if ref is None:
                    check16(C, A, B, fmt, what=f"{what} {tile}")
                    ref = C
                else:
                    assert same_bits(C, ref), (what, tile, fill, S)


@pytest.mark.parametrize("case", CASES)
def test_attention_random(case):
    rng = _rng(200 + case)
    fmt = ("bf16", "f16")[case % 2]
    D = (64, 128)[(case // 2) % 2]
    B, H = (int(x) for x in rng.integers(1, 3, size=2))
    Sq, Sk = int(rng.integers(1, 300)), int(rng.integers(1, 400))
    scale = float(rng.uniform(-2.0, 2.0))
    layout = ("bhsd", "bshd")[int(rng.integers(0, 2))]
    offset = 2 * int(rng.integers(0, 5))
    Q, K, V = (dev_qkv(500 + 10 * case + s, B, H, n, D, fmt, layout=layout, offset=offset)
               for s, n in ((0, Sq), (1, Sk), (2, Sk)))
    what = f"case {case} {fmt} D{D}: B{B} H{H} Sq{Sq} Sk{Sk} scale {scale:.3f} {layout} offset {offset}"
    ref = None
    for fill in ("sync", "piped"):
        for S in (1, 2, 3, 4):
            if fill == "sync" and S == 4:
                continue
            try:
                m.plan_attention(B, H, Sq, Sk, D, stages=S, fill=fill)
            except m.MgemmError:
                continue
            buf = torch.full((B, H, Sq, D + 3), SENTINEL, dtype=torch.float32, device="cuda")
            O = buf[..., :D]
            m.attention(Q, K, V, O, scale=scale, stages=S, fill=fill)
            torch.cuda.synchronize()
            assert bool(torch.all(buf[..., D:] == SENTINEL)), (what, fill, S)
            if ref is None:
                check_attention(O, Q, K, V, fmt, scale, what)
                ref = O.clone()
            else:
                assert torch.equal(O.view(torch.int32), ref.view(torch.int32)), (what, fill, S)


@pytest.mark.parametrize("case", CASES)
def test_tile_copy_random(case):
    rng = _rng(300 + case)
    rows, cols = (int(x) for x in rng.integers(1, 900, size=2))
    ps, pd = (int(x) for x in rng.integers(0, 9, size=2))
    os_, od = (int(x) for x in rng.integers(0, 4, size=2))
    x = datagen.matrix("normal", 600 + case, rows, cols)
    src = padded_device(x, cols + ps, offset=os_)
    want = oracle.copy_f32(x)
    for S in (1, 2, 3, 4, 5, 6):
        dst = out_device(rows, cols, cols + pd, offset=od)
        m.tile_copy(src, dst, stages=S)
        torch.cuda.synchronize()
        full = full_rows(dst)
        assert same_bits(np.ascontiguousarray(full[:, :cols]), want), (case, rows, cols, S)
        assert np.all(full[:, cols:] == SENTINEL), (case, rows, cols, S)


@pytest.mark.parametrize("case", PLAIN_CASES)
def test_plain_copy_random(case):
    """The plain copy (the tile copy's ceiling) moves the same bytes, on
    aligned (16-byte lanes) and misaligned (4-byte lanes) layouts, and
    leaves dst's padding alone."""
    rng = _rng(700 + case)
    rows, cols = (int(x) for x in rng.integers(1, 900, size=2))
    if case % 2 == 0:
        cols = 4 * ((cols + 3) // 4)
    ps, pd = (int(x) for x in rng.integers(0, 9, size=2)) if case % 2 else (4 * (case % 3), 8)
    os_, od = (int(x) for x in rng.integers(0, 4, size=2)) if case % 2 else (0, 0)
    x = datagen.matrix("normal", 800 + case, rows, cols)
    src = padded_device(x, cols + ps, offset=os_)
    dst = out_device(rows, cols, cols + pd, offset=od)
    m.plain_copy(src, dst)
    torch.cuda.synchronize()
    full = full_rows(dst)
    assert same_bits(np.ascontiguousarray(full[:, :cols]), oracle.copy_f32(x)), (case, rows, cols)
    assert np.all(full[:, cols:] == SENTINEL), (case, rows, cols)
