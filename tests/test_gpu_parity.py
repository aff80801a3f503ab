"""Parity of the HIP path with the oracle, through the C ABI, on the GPU.

Bars: every GPU result lies within |C - C_ref| <= 4 K 2^-24 (|A||B|)_ij of the
fp64 oracle; for a fixed (compute, tile) every fill mode, stage count and
loader width gives bit-identical C ("pipelined_gemm.cu": the piped output must
be memcmp-equal to the sync one before anything is timed); on inputs whose
every partial sum is exact the result equals the oracle bit for bit; C cells
outside M x N are never written; and the tile copy returns its input bytes.
"""
import numpy as np
import pytest
import torch

import async_global_shared_amd as m
import datagen
import oracle
from tests.gpu_util import (ring_fits, FILLS, SENTINEL, STAGES, TILES, check_bound, full_rows, out_device, padded_device, run,
                            same_bits)

pytestmark = pytest.mark.gpu


def _inputs(kind, M, N, K, seed=0):
    A = datagen.matrix(kind, datagen.SEED_A + seed, M, K)
    B = datagen.matrix(kind, datagen.SEED_B + seed, K, N)
    return A, B


# ---- config: 256^3, 64x64x16 tile, 4x4 micro-tile, sync S=1 vs piped S=2 ------

def test_page_kernel_shape_256():
    M = N = K = 256
    A, B = _inputs("uniform", M, N, K)
    Ad, Bd = padded_device(A), padded_device(B)
    p = m.plan(M, N, K)
    assert (p["bm"], p["bn"], p["bk"], p["threads"]) == (64, 64, 16, 256)
    cs = full_rows(run(Ad, Bd, out_device(M, N), compute="valu", tile="64x64", fill="sync", stages=1))
    cp = full_rows(run(Ad, Bd, out_device(M, N), compute="valu", tile="64x64", fill="piped", stages=2))
    check_bound(cs, A, B, what="sync S=1")
    assert same_bits(cs, cp), "piped S=2 differs from sync S=1"


# ---- config: 1024^3, stages 1..3 x {sync, piped}, bit identity --------------------

@pytest.mark.parametrize("compute", ["valu", "mfma"])
def test_1024_all_stages_and_fills(compute):
    M = N = K = 1024
    A, B = _inputs("uniform", M, N, K)
    Ad, Bd = padded_device(A), padded_device(B)
    outs = {}
    for fill in FILLS:
        for S in STAGES:
            outs[(fill, S)] = full_rows(run(Ad, Bd, out_device(M, N), compute=compute, tile="auto", fill=fill,
                                            stages=S))
    ref = outs[("sync", 1)]
    worst = check_bound(ref, A, B, what=f"{compute} sync S=1")
    assert worst <= 1.0
    for k, v in outs.items():
        assert same_bits(v, ref), f"{compute} {k} differs from sync S=1"


# ---- every variant on ragged shapes, aligned and misaligned layouts -------------

LAYOUTS = {
    # M, N, K, lda, ldb, ldc, base offsets (A, B, C) in floats
    "aligned": (300, 260, 200, 200, 260, 260, (0, 0, 0)),
    "padded_ld": (300, 260, 200, 204, 268, 264, (0, 0, 0)),
    "misaligned": (301, 259, 203, 207, 263, 267, (1, 3, 2)),
    "tiny_k": (130, 70, 5, 9, 70, 75, (0, 0, 0)),
    # more than 256 64x64 tiles: the MFMA 64x64 tile's 32-k slice (fewer: 64-k)
    "many_tiles": (1090, 1030, 83, 87, 1030, 1034, (0, 0, 0)),
}


@pytest.mark.parametrize("layout", sorted(LAYOUTS))
def test_every_variant_ragged(layout):
    M, N, K, lda, ldb, ldc, (oa, ob, oc) = LAYOUTS[layout]
    A, B = _inputs("uniform", M, N, K, seed=10)
    Ad = padded_device(A, lda, offset=oa)
    Bd = padded_device(B, ldb, offset=ob)
    loaders = ["auto", "b32"]
    for compute, tile in TILES:
        ref = None
        for fill in FILLS:
            for S in STAGES:
                for ld in loaders:
                    Cd = out_device(M, N, ldc, offset=oc)
                    full = full_rows(run(Ad, Bd, Cd, compute=compute, tile=tile, fill=fill, stages=S, loader=ld))
                    assert np.all(full[:, N:] == SENTINEL), f"{layout} {compute} {tile}: wrote C padding"
                    C = full[:, :N]
                    if ref is None:
                        check_bound(C, A, B, what=f"{layout} {compute} {tile} {fill} S={S} {ld}")
                        ref = C
                    else:
                        assert same_bits(C, ref), f"{layout} {compute} {tile} {fill} S={S} {ld} != first variant"


@pytest.mark.parametrize("layout", ["aligned", "misaligned", "many_tiles"])
def test_tiles_agree_bitwise(layout):
    """For one compute kind every block tile gives the same bits: each C
    element is one fma chain over k ascending (VALU) or one MFMA sequence in
    the absolute k order (MFMA), however the tile and its K slice cut the
    problem; so the automatic tile choice never changes a result."""
    M, N, K, lda, ldb, ldc, (oa, ob, oc) = LAYOUTS[layout]
    A, B = _inputs("uniform", M, N, K, seed=12)
    Ad = padded_device(A, lda, offset=oa)
    Bd = padded_device(B, ldb, offset=ob)
    for compute in ("valu", "mfma"):
        ref = None
        for c, tile in TILES:
            if c != compute:
                continue
            for fill, S in (("sync", 1), ("piped", 2)):
                C = full_rows(run(Ad, Bd, out_device(M, N, ldc, offset=oc), compute=compute, tile=tile, fill=fill,
                                  stages=S))[:, :N]
                if ref is None:
                    ref = C
                else:
                    assert same_bits(C, ref), f"{layout} {compute} {tile} {fill} S={S} differs from the first tile"


def test_long_k_many_slices():
    """K far beyond any ring (65573: 4099 slices of 16 k, 1025 of 64, the last
    one ragged) on a ragged 70 x 130 C: every tile, fill and depth that fits,
    within the bound and bit-identical per (compute, tile); C padding untouched."""
    M, N, K = 70, 130, 65573
    A, B = _inputs("uniform", M, N, K, seed=7)
    Ad, Bd = padded_device(A), padded_device(B)
    for compute, tile in TILES:
        ref = None
        for fill in FILLS:
            for S in STAGES:
                if not ring_fits(M, N, K, compute=compute, tile=tile, fill=fill, stages=S):
                    continue
                full = full_rows(run(Ad, Bd, out_device(M, N), compute=compute, tile=tile, fill=fill, stages=S))
                assert np.all(full[:, N:] == SENTINEL), f"long K {compute} {tile}: wrote C padding"
                C = full[:, :N]
                if ref is None:
                    check_bound(C, A, B, what=f"long K {compute} {tile} {fill} S={S}")
                    ref = C
                else:
                    assert same_bits(C, ref), f"long K {compute} {tile} {fill} S={S} != first variant"


@pytest.mark.parametrize("layout", ["padded_ld", "misaligned"])
def test_deep_piped_rings(layout):
    """Rings of 4-6 stages (the lesson's exercise sweeps the depth) give the
    same bits as the synchronous fill, for every compute tile and loader."""
    M, N, K, lda, ldb, ldc, (oa, ob, oc) = LAYOUTS[layout]
    K = 517  # 33 slices: the tail of every deep ring is exercised
    A, B = _inputs("uniform", M, N, K, seed=70)
    Ad = padded_device(A, K + 3, offset=oa)
    Bd = padded_device(B, ldb, offset=ob)
    for compute, tile in TILES:
        ref = full_rows(run(Ad, Bd, out_device(M, N, ldc, offset=oc), compute=compute, tile=tile, fill="sync",
                            stages=1))
        check_bound(ref[:, :N], A, B, what=f"{layout} {compute} {tile} sync S=1")
        for S in (4, 5, 6):
            if not ring_fits(M, N, K, stages=S, fill="piped", compute=compute, tile=tile, lda=K + 3, ldb=ldb, ldc=ldc):
                with pytest.raises(m.MgemmError):  # refused, never run on a ring the LDS cannot hold
                    run(Ad, Bd, out_device(M, N, ldc, offset=oc), compute=compute, tile=tile, fill="piped", stages=S)
                continue
            for ld in ("auto", "b32"):
                C = full_rows(run(Ad, Bd, out_device(M, N, ldc, offset=oc), compute=compute, tile=tile,
                                  fill="piped", stages=S, loader=ld))
                assert same_bits(C, ref), (layout, compute, tile, S, ld)


@pytest.mark.parametrize("layout", ["aligned", "misaligned", "tiny_k"])
def test_warp_specialised_ring(layout):
    """Dedicated filling waves with per-slot LDS counters give the same bits as
    the synchronous fill, for every compute tile, depth and loader."""
    M, N, K, lda, ldb, ldc, (oa, ob, oc) = LAYOUTS[layout]
    A, B = _inputs("uniform", M, N, K, seed=80)
    Ad = padded_device(A, lda, offset=oa)
    Bd = padded_device(B, ldb, offset=ob)
    for compute, tile in TILES:
        ref = full_rows(run(Ad, Bd, out_device(M, N, ldc, offset=oc), compute=compute, tile=tile, fill="sync",
                            stages=1))
        check_bound(ref[:, :N], A, B, what=f"{layout} {compute} {tile} sync S=1")
        for S in range(1, 7):
            if not ring_fits(M, N, K, stages=S, fill="piped_ws", compute=compute, tile=tile, lda=lda, ldb=ldb, ldc=ldc):
                continue
            for ld in ("auto", "b32"):
                C = full_rows(run(Ad, Bd, out_device(M, N, ldc, offset=oc), compute=compute, tile=tile,
                                  fill="piped_ws", stages=S, loader=ld))
                assert not np.isnan(C[:, :N]).any(), ("ring reported broken", layout, compute, tile, S, ld)
                assert same_bits(C, ref), (layout, compute, tile, S, ld)


def test_deep_ring_copy():
    x = datagen.matrix("normal", datagen.SEED_COPY, 700, 900)
    src = padded_device(x, 904)
    for S in (4, 5, 6):
        dst = out_device(700, 900, 905)
        m.tile_copy(src, dst, stages=S)
        torch.cuda.synchronize()
        full = full_rows(dst)
        assert same_bits(np.ascontiguousarray(full[:, :900]), x) and np.all(full[:, 900:] == SENTINEL), S


def test_blocks_per_cu_query():
    """Deeper rings hold more LDS per block; the query reports what fits."""
    occ = [m.blocks_per_cu(8192, 8192, 8192, stages=S, compute="mfma", tile="128x128") for S in range(1, 7)]
    assert all(1 <= o <= 8 for o in occ)
    assert occ == sorted(occ, reverse=True)  # never more resident blocks with a deeper ring
    with pytest.raises(m.MgemmError):
        m.blocks_per_cu(64, 64, 64, stages=4, fill="sync")


def test_residency_cap():
    """Where every CU would take exactly one block more than the 3 or 4 it
    holds, the launch holds half as many per CU, rounded up; elsewhere the
    kernel's own residency stands. (Bit identity across residencies is the
    4096^3 full-size test's.)"""
    q = lambda M, N, K, **kw: m.blocks_per_cu(M, N, K, compute="mfma", tile="128x128", **kw)
    assert q(8192, 8192, 8192, stages=3) == 3             # 16 blocks per CU: no cap
    assert q(3072, 4096, 4096, stages=3) == 3             # 3 per CU: one round, no cap
    assert q(4096, 4096, 4096, stages=3) == 2             # 4 per CU against 3 resident: two rounds of 2
    assert q(3584, 4096, 4096, stages=3) == 2             # 896 blocks: up to 4 per CU
    assert q(4608, 4096, 4096, stages=2, fill="sync") == 3  # 5 per CU against 4 resident
    assert q(4096, 4096, 4096, stages=2, fill="sync") == 4  # 4 per CU: one round
    # the 64x64 VALU tile keeps its residency (3 at six stages, 4 blocks per CU at N = 2048)
    assert m.blocks_per_cu(2048, 2048, 2048, stages=6, compute="valu", tile="64x64") == 3


def test_b128_and_b32_loaders_agree_when_both_apply():
    M, N, K = 384, 256, 320
    A, B = _inputs("uniform", M, N, K, seed=20)
    Ad, Bd = padded_device(A), padded_device(B)
    for compute, tile in TILES:
        a = full_rows(run(Ad, Bd, out_device(M, N), compute=compute, tile=tile, fill="piped", stages=3,
                          loader="b128"))
        b = full_rows(run(Ad, Bd, out_device(M, N), compute=compute, tile=tile, fill="piped", stages=3,
                          loader="b32"))
        assert same_bits(a, b), (compute, tile)


# ---- exactness pins ---------------------------------------------------------------

@pytest.mark.parametrize("shape", [(200, 136, 520), (1024, 1024, 1024)])
def test_coarse_grid_is_exact_for_every_variant(shape):
    """Inputs on the 2^-4 grid make every fp32 partial sum exact, so every
    variant, MFMA included, must equal the oracle rounded to fp32, bit for bit."""
    M, N, K = shape
    A, B = _inputs("coarse", M, N, K, seed=30)
    want = oracle.gemm_f64(A, B).astype(np.float32)
    Ad, Bd = padded_device(A), padded_device(B)
    for compute, tile in TILES:
        for fill, S in (("sync", 1), ("piped", 2), ("piped", 3)):
            C = full_rows(run(Ad, Bd, out_device(M, N), compute=compute, tile=tile, fill=fill, stages=S))
            assert same_bits(C, want), (shape, compute, tile, fill, S)


@pytest.mark.parametrize("K", [1000, 1537, 16, 17, 32, 47, 48, 64, 80, 96])
def test_slice_sentinels(K):
    """A = 1, B[k, j] = floor(k/16) (and the mirror) give C = 16 T(T-1)/2 + rT
    exactly; a slice computed from the wrong ring slot changes the sum."""
    T, r = K // 16, K % 16
    want = np.float32(16 * T * (T - 1) // 2 + r * T)
    M, N = 192, 160
    pairs = [(np.ones((M, K), np.float32), datagen.slice_sentinel(K, N, axis=0)),
             (datagen.slice_sentinel(M, K, axis=1), np.ones((K, N), np.float32))]
    for A, B in pairs:
        Ad, Bd = padded_device(A), padded_device(B)
        for compute, tile in TILES:
            for fill in FILLS:
                for S in STAGES:
                    C = full_rows(run(Ad, Bd, out_device(M, N), compute=compute, tile=tile, fill=fill, stages=S))
                    assert np.all(C == want), (K, compute, tile, fill, S)


def test_closed_forms_identity_and_permutation():
    M = K = 192
    N = 136
    B = datagen.matrix("uniform", 41, K, N)
    I = np.eye(M, dtype=np.float32)
    perm = np.random.default_rng(5).permutation(M)
    P = np.zeros((M, M), np.float32)
    P[np.arange(M), perm] = 1.0
    Bd = padded_device(B)
    for A, want in ((I, B), (P, B[perm])):
        Ad = padded_device(A)
        for compute, tile in TILES:
            for fill, S in (("sync", 1), ("piped", 3)):
                C = full_rows(run(Ad, Bd, out_device(M, N), compute=compute, tile=tile, fill=fill, stages=S))
                C = np.where(C == 0, 0.0, C).astype(np.float32)  # -0 and +0 compare equal
                assert np.array_equal(C, want), (compute, tile, fill, S)


def test_page_input_pattern_relative_tolerance():
    """The day-74 program's own inputs and its relative 1e-4 check, at the
    program's three sizes ("pipelined_gemm.cu", main: kSizes)."""
    for n in (512, 1024, 2048):
        A = datagen.page_pattern_a(n * n).reshape(n, n)
        B = datagen.page_pattern_b(n * n).reshape(n, n)
        ref = oracle.gemm_f64(A, B)
        Ad, Bd = padded_device(A), padded_device(B)
        for compute in ("valu", "mfma"):
            C = full_rows(run(Ad, Bd, out_device(n, n), compute=compute, tile="auto", fill="piped", stages=2))
            scale = np.where(ref == 0, 1.0, np.abs(ref))
            assert np.all(np.abs(C - ref) <= 1e-4 * scale), (n, compute)
            check_bound(C, A, B, what=f"page pattern {n} {compute}")


# ---- edge cases ---------------------------------------------------------------------

def test_k_zero_writes_zeros_only_inside():
    M, N, ldc = 70, 50, 53
    Ad = torch.empty((M, 0), device="cuda")
    Bd = torch.empty((0, N), device="cuda")
    Cd = out_device(M, N, ldc)
    m.sgemm(Ad, Bd, Cd, stages=2, fill="piped")
    torch.cuda.synchronize()
    full = full_rows(Cd)
    assert np.all(full[:, :N] == 0) and not np.any(np.signbit(full[:, :N]))
    assert np.all(full[:, N:] == SENTINEL)


def test_empty_m_or_n_is_a_noop():
    Cd = out_device(4, 4)
    A = torch.ones((0, 8), device="cuda")
    B = torch.ones((8, 4), device="cuda")
    m.sgemm(A, B, torch.empty((0, 4), device="cuda"))
    torch.cuda.synchronize()
    assert torch.all(Cd == SENTINEL)


@pytest.mark.parametrize("shape", [(1, 1, 1), (1, 1000, 37), (999, 1, 64), (65, 65, 15), (2, 3, 1)])
def test_small_and_degenerate(shape):
    M, N, K = shape
    A, B = _inputs("uniform", M, N, K, seed=50)
    Ad, Bd = padded_device(A), padded_device(B)
    for compute, tile in TILES:
        ref = None
        for fill in FILLS:
            for S in STAGES:
                C = full_rows(run(Ad, Bd, out_device(M, N), compute=compute, tile=tile, fill=fill, stages=S))
                if ref is None:
                    check_bound(C, A, B, what=f"{shape} {compute} {tile}")
                    ref = C
                assert same_bits(C, ref), (shape, compute, tile, fill, S)


def test_errors_through_the_abi_on_device():
    A = torch.ones((64, 64), device="cuda")
    B = torch.ones((64, 64), device="cuda")
    with pytest.raises(m.MgemmError) as e:
        m.sgemm(A, B, A)  # C overlaps A
    assert e.value.status == m.ERR_ALIAS
    Bm = torch.ones(64 * 64 + 1, device="cuda")[1:].view(64, 64)  # misaligned base
    with pytest.raises(m.MgemmError) as e:
        m.sgemm(A, Bm, loader="b128")
    assert e.value.status == m.ERR_ARG


def test_runs_on_a_non_default_stream():
    M = N = K = 512
    A, B = _inputs("uniform", M, N, K, seed=60)
    Ad, Bd = padded_device(A), padded_device(B)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        Cd = out_device(M, N)
        m.sgemm(Ad, Bd, Cd, stages=3, fill="piped", compute="mfma")
    s.synchronize()
    check_bound(full_rows(Cd), A, B, what="side stream")


# ---- tile copy ---------------------------------------------------------------------

def test_copy_page_example_pattern():
    """The TVM cp.async page copies (arange(4096) % 97) as 128 x 32 through
    shared memory and asserts array equality; the same pattern in fp32."""
    x = (np.arange(4096) % 97).astype(np.float32).reshape(128, 32)
    src = padded_device(x)
    for S in STAGES:
        dst = out_device(128, 32)
        m.tile_copy(src, dst, stages=S)
        torch.cuda.synchronize()
        assert same_bits(full_rows(dst), x)


@pytest.mark.parametrize("case", [
    (1000, 777, 781, 790, 0, 0), (64, 64, 64, 64, 0, 0), (130, 200, 200, 204, 1, 0), (5, 3, 3, 3, 0, 1),
    (257, 1024, 1024, 1024, 0, 0), (130, 300, 300, 303, 0, 2), (65, 1000, 1001, 1000, 3, 0)])
def test_copy_ragged(case):
    rows, cols, lds, ldd, os_, od = case
    x = datagen.matrix("normal", datagen.SEED_COPY, rows, cols)
    src = padded_device(x, lds, offset=os_)
    for S in STAGES:
        dst = out_device(rows, cols, ldd, offset=od)
        m.tile_copy(src, dst, stages=S)
        torch.cuda.synchronize()
        full = full_rows(dst)
        assert same_bits(np.ascontiguousarray(full[:, :cols]), x), (case, S)
        assert np.all(full[:, cols:] == SENTINEL), (case, S)
