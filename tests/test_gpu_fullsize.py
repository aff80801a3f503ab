"""Parity at the full benchmark sizes, in the launch configurations the
benchmark times: sampled rows against the oracle (computed one row at a time),
and properties that hold at any size (bit identity across fills and stages,
closed forms). Inputs: A, B ~ U[-1, 1) from the seeded generator."""
import numpy as np
import pytest
import torch

import async_global_shared_amd as m
import datagen
import oracle
from tests.gpu_util import check_bound, same_bits

pytestmark = pytest.mark.gpu


def _dev_uniform(seed, rows, cols):
    return datagen.uniform_pm1_torch(seed, rows * cols, device="cuda").view(rows, cols)


def _sample_rows(M, n=12):
    rows = sorted(set([0, 1, M // 3, M // 2, M - 2, M - 1] + list(np.linspace(0, M - 1, n).astype(int))))
    return np.array(rows)


def _host_rows(Ad, rows):
    return Ad[torch.as_tensor(rows, device=Ad.device)].cpu().numpy()


@pytest.mark.parametrize("n", [4096, 8192])
def test_square_full_size(n):
    M = N = K = n
    Ad = _dev_uniform(datagen.SEED_A, M, K)
    Bd = _dev_uniform(datagen.SEED_B, K, N)
    # the generator's GPU twin equals the CPU one (integer arithmetic)
    assert torch.equal(Ad[:2, :100].cpu(), torch.from_numpy(datagen.uniform_pm1(datagen.SEED_A, 2 * K)
                                                              .reshape(2, K)[:, :100]))
    B = Bd.cpu().numpy()
    rows = _sample_rows(M)
    A_rows = _host_rows(Ad, rows)
    for compute in ("mfma", "valu"):
        ref = torch.empty((M, N), device="cuda")
        m.sgemm(Ad, Bd, ref, stages=3, fill="piped", compute=compute, tile="128x128")
        torch.cuda.synchronize()
        C_rows = ref[torch.as_tensor(rows, device="cuda")].cpu().numpy()
        check_bound(C_rows, A_rows, B, what=f"{n}^3 {compute} piped S=3 (sampled rows)")
        other = torch.empty_like(ref)
        variants = [("sync", 1), ("piped", 2)] if compute == "valu" and n == 8192 else \
            [("sync", 1), ("sync", 2), ("sync", 3), ("piped", 1), ("piped", 2), ("piped", 4), ("piped", 6),
             ("piped_ws", 2), ("piped_ws", 3)]
        for fill, S in variants:
            other.fill_(float("nan"))
            m.sgemm(Ad, Bd, other, stages=S, fill=fill, compute=compute, tile="128x128")
            torch.cuda.synchronize()
            assert torch.equal(other.view(torch.int32), ref.view(torch.int32)), (n, compute, fill, S)
        del ref, other


def test_whole_output_8192_against_oracle():
    """The benchmark's timed configuration (MFMA compute tile, 128x128,
    piped S=2) on the full 8192^3 problem: every element of C against the
    oracle's bound, as the pages' program checks every element against its
    CPU product ("pipelined_gemm.cu", main). The oracle runs the whole fp64
    product and |A||B| on the host cores (about 30 s)."""
    n = 8192
    Ad = _dev_uniform(datagen.SEED_A, n, n)
    Bd = _dev_uniform(datagen.SEED_B, n, n)
    C = torch.empty((n, n), device="cuda")
    m.sgemm(Ad, Bd, C, stages=2, fill="piped", compute="mfma", tile="128x128")
    torch.cuda.synchronize()
    print("8192^3 timed variant done; oracle on the whole product", flush=True)
    check_bound(C.cpu().numpy(), Ad.cpu().numpy(), Bd.cpu().numpy(), what="8192^3 MFMA piped S=2 (whole output)")


@pytest.mark.parametrize("M", [3584, 4608])
def test_residency_capped_grids(M):
    """Grids where the launch caps residency (896 tiles: piped S=3 holds 2
    blocks per CU instead of 3; 1152 tiles: sync S=2 holds 3 instead of 4):
    every fill and depth stays bit-identical and within the bound on sampled
    rows."""
    N, K = 4096, 512
    Ad = _dev_uniform(datagen.SEED_A, M, K)
    Bd = _dev_uniform(datagen.SEED_B, K, N)
    capped = {3584: ("piped", 3, 2), 4608: ("sync", 2, 3)}[M]
    assert m.blocks_per_cu(M, N, K, stages=capped[1], fill=capped[0], compute="mfma", tile="128x128") == capped[2]
    rows = _sample_rows(M)
    for compute in ("mfma", "valu"):
        ref = torch.empty((M, N), device="cuda")
        m.sgemm(Ad, Bd, ref, stages=1, fill="sync", compute=compute, tile="128x128")
        torch.cuda.synchronize()
        check_bound(ref[torch.as_tensor(rows, device="cuda")].cpu().numpy(), _host_rows(Ad, rows), Bd.cpu().numpy(),
                    what=f"{M}x{N}x{K} {compute} sync S=1 (sampled rows)")
        other = torch.empty_like(ref)
        for fill, S in (("sync", 2), ("sync", 3), ("piped", 1), ("piped", 2), ("piped", 3), ("piped", 4)):
            other.fill_(float("nan"))
            m.sgemm(Ad, Bd, other, stages=S, fill=fill, compute=compute, tile="128x128")
            torch.cuda.synchronize()
            assert torch.equal(other.view(torch.int32), ref.view(torch.int32)), (M, compute, fill, S)


def test_ragged_full_size():
    """M = 4099, N = 3001, K = 1537 with lda = 1537 and ldb = ldc = 3001: no
    leading dimension is a multiple of 4, so every fill takes 4-byte loads,
    and the last K slice holds one valid k."""
    M, N, K = 4099, 3001, 1537
    Ad = _dev_uniform(datagen.SEED_A, M, K)
    Bd = _dev_uniform(datagen.SEED_B, K, N)
    assert m.plan(M, N, K, lda=K, ldb=N, ldc=N)["load_bytes"] == 4
    B = Bd.cpu().numpy()
    rows = _sample_rows(M)
    A_rows = _host_rows(Ad, rows)
    for compute in ("valu", "mfma"):
        ref = torch.empty((M, N), device="cuda")
        m.sgemm(Ad, Bd, ref, stages=3, fill="piped", compute=compute)
        torch.cuda.synchronize()
        check_bound(ref[torch.as_tensor(rows, device="cuda")].cpu().numpy(), A_rows, B,
                    what=f"ragged {compute}")
        other = torch.empty_like(ref)
        for fill, S in (("sync", 1), ("piped", 2)):
            m.sgemm(Ad, Bd, other, stages=S, fill=fill, compute=compute)
            torch.cuda.synchronize()
            assert torch.equal(other.view(torch.int32), ref.view(torch.int32)), (compute, fill, S)


def test_tall_skinny_full_size():
    M, N, K = 16384, 64, 4096
    Ad = _dev_uniform(datagen.SEED_A, M, K)
    Bd = _dev_uniform(datagen.SEED_B, K, N)
    B = Bd.cpu().numpy()
    rows = _sample_rows(M, 24)
    A_rows = _host_rows(Ad, rows)
    for compute in ("valu", "mfma"):
        ref = torch.empty((M, N), device="cuda")
        m.sgemm(Ad, Bd, ref, stages=3, fill="piped", compute=compute)
        torch.cuda.synchronize()
        check_bound(ref[torch.as_tensor(rows, device="cuda")].cpu().numpy(), A_rows, B,
                    what=f"tall-skinny {compute}")
        other = torch.empty_like(ref)
        m.sgemm(Ad, Bd, other, stages=1, fill="sync", compute=compute)
        torch.cuda.synchronize()
        assert torch.equal(other.view(torch.int32), ref.view(torch.int32)), compute


def test_sentinel_full_size_8192():
    """A = 1, B[k, j] = floor(k/16): C = 16 T (T-1) / 2 exactly (T = 512,
    2093056 < 2^24, every partial sum an exact integer), on the whole 8192^3
    output of the timed configuration."""
    n = 8192
    Ad = torch.ones((n, n), device="cuda")
    Bd = (torch.arange(n, device="cuda", dtype=torch.int64) // 16).to(torch.float32)[:, None].expand(n, n).contiguous()
    want = 16 * 512 * 511 // 2
    C = torch.empty((n, n), device="cuda")
    for compute in ("mfma", "valu"):
        for fill, S in (("piped", 3), ("piped", 2), ("sync", 1)):
            C.fill_(float("nan"))
            m.sgemm(Ad, Bd, C, stages=S, fill=fill, compute=compute, tile="128x128")
            torch.cuda.synchronize()
            assert bool(torch.all(C == want)), (compute, fill, S)


@pytest.mark.parametrize("S", [1, 2, 3])
@pytest.mark.parametrize("shape", [(16384, 16384), (4194304, 64)], ids=["16384x16384", "4194304x64"])
def test_copy_one_gib(S, shape):
    """The 1 GiB copy in both views the benchmark times (2^28 fp32), every
    byte compared; then the plain copy, its ceiling."""
    src = datagen.normal01_torch(datagen.SEED_COPY, 1 << 28, device="cuda").view(*shape)
    dst = torch.full_like(src, float("nan"))
    m.tile_copy(src, dst, stages=S)
    torch.cuda.synchronize()
    assert torch.equal(dst.view(torch.int32), src.view(torch.int32))
    if S == 1:
        dst.fill_(float("nan"))
        m.plain_copy(src, dst)
        torch.cuda.synchronize()
        assert torch.equal(dst.view(torch.int32), src.view(torch.int32))


def test_largest_leading_dimension():
    """The largest leading dimension the library takes, 2^21 - 4 words (8 MiB
    rows): a 256-row tile's panel then spans nearly the 2^31-byte range its
    buffer descriptor covers. A (300 x 70) sits in a NaN-poisoned buffer of
    that row pitch, 2.4 GiB, and C has the same pitch. Every fp32 tile, both
    fills at depths 1 and 2, within the bound and bit-identical per tile; the
    tile copy (S = 1-3) and the plain copy between views of that pitch, byte
    for byte; the 16-bit GEMM on the same bytes (2 (2^21 - 4) elements per
    row) within the bound and bit-identical."""
    M, N, K = 300, 130, 70
    ld = (1 << 21) - 4
    A = datagen.matrix("uniform", 41, M, K)
    B = datagen.matrix("uniform", 42, K, N)
    abuf = torch.full(((M + 2) * ld,), float("nan"), dtype=torch.float32, device="cuda")
    Ad = abuf[:M * ld].view(M, ld)[:, :K]
    Ad.copy_(torch.from_numpy(A))
    Bd = torch.from_numpy(B).cuda()
    cbuf = torch.full(((M + 1) * ld,), -1.0, dtype=torch.float32, device="cuda")
    Cd = cbuf[:M * ld].view(M, ld)[:, :N]
    for compute, tile in [("valu", "64x64"), ("valu", "128x128"), ("mfma", "64x64"), ("mfma", "128x128"),
                          ("mfma", "256x128")]:
        ref = None
        for fill in ("sync", "piped"):
            for S in (1, 2):
                Cd.fill_(float("nan"))
                m.sgemm(Ad, Bd, Cd, stages=S, fill=fill, compute=compute, tile=tile)
                torch.cuda.synchronize()
                C = Cd.cpu().numpy()
                if ref is None:
                    check_bound(C, A, B, what=f"ld 2^21-4 {compute} {tile}")
                    ref = C
                else:
                    assert same_bits(C, ref), (compute, tile, fill, S)
    assert bool(torch.all(cbuf[:M * ld].view(M, ld)[:, N:N + 64] == -1.0)), "C written past N"
    # the tile copy and the plain copy between views of that pitch
    src = abuf[:M * ld].view(M, ld)[:, :N]
    src.copy_(datagen.normal01_torch(45, M * N, device="cuda").view(M, N))
    for S in (1, 2, 3, 0):
        Cd.fill_(float("nan"))
        if S:
            m.tile_copy(src, Cd, stages=S)
        else:
            m.plain_copy(src, Cd)
        torch.cuda.synchronize()
        assert torch.equal(Cd.view(torch.int32), src.view(torch.int32)), f"copy S={S} at ld 2^21-4"
    assert bool(torch.all(cbuf[:M * ld].view(M, ld)[:, N:N + 64] == -1.0)), "copy wrote past the columns"
    del abuf, Ad, cbuf, Cd, src

    fmt = "bf16"
    A16 = datagen.matrix16(43, M, K, fmt)
    B16 = datagen.matrix16(44, K, N, fmt)
    ld16 = 2 * ld
    a16 = torch.full(((M + 2) * ld16,), float("nan"), dtype=torch.bfloat16, device="cuda")
    Ad16 = a16[:M * ld16].view(M, ld16)[:, :K]
    Ad16.copy_(torch.from_numpy(A16.view(np.int16)).view(torch.bfloat16))
    Bd16 = torch.from_numpy(B16.view(np.int16)).cuda().view(torch.bfloat16)
    ref = None
    for tile in ("128x128", "256x128", "256x256"):
        for fill, S in (("sync", 1), ("piped", 2)):
            C16 = m.gemm16(Ad16, Bd16, stages=S, fill=fill, tile=tile)
            torch.cuda.synchronize()
            C = C16.cpu().numpy()
            if ref is None:
                want = oracle.gemm16_f64(A16, B16, fmt)
                bnd = oracle.bound(K, oracle.gemm16_f64(A16, B16, fmt, absolute=True))
                assert np.all(np.abs(C.astype(np.float64) - want) <= bnd), f"16-bit ld 2(2^21-4) {tile}"
                ref = C
            else:
                assert same_bits(C, ref), (tile, fill, S)
