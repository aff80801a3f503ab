"""Parity of the 16-bit (bfloat16 / binary16) MFMA GEMM with the oracle, through
the C ABI: within |C - C_ref| <= 4 K 2^-24 (|A||B|)_ij (products of 16-bit
values are exact in fp32; the sums are fp32), bit-identical across fills,
stages and loaders, exact on the 2^-4 grid, C padding untouched."""
import numpy as np
import pytest
import torch

import async_global_shared_amd as m
import datagen
import oracle
from tests.gpu_util import SENTINEL, check_bound, full_rows, out_device, same_bits

pytestmark = pytest.mark.gpu

TORCH16 = {"bf16": torch.bfloat16, "f16": torch.float16}
NAN16 = {"bf16": 0x7FC0, "f16": 0x7E00}


def dev16(bits: np.ndarray, fmt: str, ld: int | None = None, offset: int = 0, extra_rows: int = 2):
    """Device view (torch 16-bit) of a uint16 pattern matrix with leading
    dimension ld; padding, trailing rows and the offset hold NaN patterns."""
    rows, cols = bits.shape
    ld = cols if ld is None else ld
    buf = np.full(offset + (rows + extra_rows) * ld, NAN16[fmt], dtype=np.uint16)
    buf[offset:offset + rows * ld].reshape(rows, ld)[:, :cols] = bits
    t = torch.from_numpy(buf.view(np.int16)).to("cuda").view(TORCH16[fmt])
    return t[offset:offset + rows * ld].view(rows, ld)[:, :cols]


TILES16 = ("128x128", "256x128", "256x256")


def fits(tile, S):
    """The ring of this tile and depth fits the CU's LDS."""
    st, _ = m.mgemm_plan_gemm16(1024, 1024, 1024, 1 << 32, 1024, 1 << 36, 1024, 1 << 40, 1024, m.DTYPE_BF16, S,
                                m.FILL_PIPED, m._TILE[tile])
    return st == m.OK


def check16(C, A, B, fmt, rows=None, what=""):
    if rows is not None:
        A = np.ascontiguousarray(A[rows])
        C = C[rows]
    ref = oracle.gemm16_f64(A, B, fmt)
    bnd = oracle.bound(A.shape[1], oracle.gemm16_f64(A, B, fmt, absolute=True))
    bad = ~(np.abs(C.astype(np.float64) - ref) <= bnd)
    assert not bad.any(), f"{what}: {bad.sum()} outside the bound"


LAYOUTS = {
    # M, N, K, lda, ldb, ldc, offsets (elements; A and B offsets keep 4-byte alignment)
    "aligned": (256, 256, 256, 256, 256, 256, (0, 0, 0)),
    "ragged": (300, 258, 198, 198, 258, 261, (0, 0, 0)),
    "ragged_b128": (300, 264, 200, 208, 272, 267, (0, 0, 0)),
    "padded_ld": (130, 200, 330, 340, 208, 203, (0, 0, 0)),
    "misaligned": (131, 194, 202, 206, 198, 199, (2, 6, 1)),
    "tiny_k": (70, 66, 2, 2, 66, 66, (0, 0, 0)),
}


@pytest.mark.parametrize("fmt", ["bf16", "f16"])
@pytest.mark.parametrize("layout", sorted(LAYOUTS))
def test_every_variant(fmt, layout):
    M, N, K, lda, ldb, ldc, (oa, ob, oc) = LAYOUTS[layout]
    A = datagen.matrix16(1, M, K, fmt)
    B = datagen.matrix16(2, K, N, fmt)
    Ad = dev16(A, fmt, lda, oa)
    Bd = dev16(B, fmt, ldb, ob)
    W = m.plan16(M, N, K, dtype=fmt, lda=lda, ldb=ldb, ldc=ldc, a_ptr=Ad.data_ptr(), b_ptr=Bd.data_ptr(),
                 c_ptr=out_device(M, N, ldc, offset=oc).data_ptr())["load_bytes"]
    assert W == (16 if layout in ("aligned", "ragged_b128") else 4)
    for tile in TILES16:
        ref = None
        for fill in ("sync", "piped"):
            for S in (1, 2, 3, 4):
                if not fits(tile, S) or (fill == "sync" and S == 4):
                    continue
                Cd = out_device(M, N, ldc, offset=oc)
                m.gemm16(Ad, Bd, Cd, stages=S, fill=fill, tile=tile)
                torch.cuda.synchronize()
                full = full_rows(Cd)
                assert np.all(full[:, N:] == SENTINEL), (fmt, layout, tile, fill, S)
                C = full[:, :N]
                if ref is None:
                    check16(C, A, B, fmt, what=f"{fmt} {layout} {tile}")
                    ref = C
                else:
                    assert same_bits(C, ref), (fmt, layout, tile, fill, S)


@pytest.mark.parametrize("K", [8, 64, 72, 128, 136, 192, 256, 320])
def test_few_slices(K):
    """1 to 5 K slices with 16-byte loads: the split ring's first iteration
    (no tail yet), its last ones (a tail but no refill) and the tail after
    the loop; the two-set synchronous ring's grouped loop with and without
    its masked last load (odd and even slice counts). Every tile, fill and
    depth; exact on the 2^-4 grid and bit-identical across variants."""
    fmt, M, N = "bf16", 300, 264
    A = datagen.matrix16(5, M, K, fmt, kind="coarse")
    B = datagen.matrix16(6, K, N, fmt, kind="coarse")
    want = oracle.gemm16_f64(A, B, fmt).astype(np.float32)
    Ad, Bd = dev16(A, fmt), dev16(B, fmt)
    assert m.plan16(M, N, K, a_ptr=Ad.data_ptr(), b_ptr=Bd.data_ptr())["load_bytes"] == 16
    for tile in TILES16:
        for fill in ("sync", "piped"):
            for S in (1, 2, 3, 4):
                if not fits(tile, S) or (fill == "sync" and S == 4):
                    continue
                Cd = out_device(M, N, N + 3)
                m.gemm16(Ad, Bd, Cd, stages=S, fill=fill, tile=tile)
                torch.cuda.synchronize()
                full = full_rows(Cd)
                assert np.all(full[:, N:] == SENTINEL), (K, tile, fill, S)
                assert same_bits(full[:, :N], want), (K, tile, fill, S)


@pytest.mark.parametrize("fmt", ["bf16", "f16"])
def test_long_k(fmt):
    """K = 32776 (513 slices of 64, the last one ragged) on a ragged 96 x 130 C:
    every tile, fill and depth that fits, within the bound and bit-identical."""
    M, N, K = 96, 130, 32776
    A = datagen.matrix16(11, M, K, fmt)
    B = datagen.matrix16(12, K, N, fmt)
    Ad, Bd = dev16(A, fmt), dev16(B, fmt)
    for tile in TILES16:
        ref = None
        for fill in ("sync", "piped"):
            for S in (1, 2, 3, 4):
                if not fits(tile, S) or (fill == "sync" and S == 4):
                    continue
                Cd = out_device(M, N, N + 2)
                m.gemm16(Ad, Bd, Cd, stages=S, fill=fill, tile=tile)
                torch.cuda.synchronize()
                full = full_rows(Cd)
                assert np.all(full[:, N:] == SENTINEL), (fmt, tile, fill, S)
                C = full[:, :N]
                if ref is None:
                    check16(C, A, B, fmt, what=f"{fmt} long K {tile}")
                    ref = C
                else:
                    assert same_bits(C, ref), (fmt, tile, fill, S)


@pytest.mark.parametrize("fmt", ["bf16", "f16"])
def test_coarse_grid_exact(fmt):
    M, N, K = 384, 256, 1024
    A = datagen.matrix16(3, M, K, fmt, kind="coarse")
    B = datagen.matrix16(4, K, N, fmt, kind="coarse")
    want = oracle.gemm16_f64(A, B, fmt).astype(np.float32)
    Ad, Bd = dev16(A, fmt), dev16(B, fmt)
    for tile in TILES16:
        for fill, S in (("sync", 1), ("piped", 2), ("piped", 3), ("piped", 4)):
            if not fits(tile, S):
                continue
            C = m.gemm16(Ad, Bd, stages=S, fill=fill, tile=tile)
            torch.cuda.synchronize()
            assert same_bits(C.cpu().numpy(), want), (fmt, tile, fill, S)


def test_ones_and_zero_k():
    fmt = "bf16"
    A = datagen.matrix16(0, 200, 512, fmt, kind="ones")
    B = datagen.matrix16(0, 512, 136, fmt, kind="ones")
    C = m.gemm16(dev16(A, fmt), dev16(B, fmt))
    torch.cuda.synchronize()
    assert torch.all(C == 512)
    Cd = out_device(10, 12, 13)
    m.gemm16(torch.empty((10, 0), dtype=torch.bfloat16, device="cuda"),
             torch.empty((0, 12), dtype=torch.bfloat16, device="cuda"), Cd)
    torch.cuda.synchronize()
    full = full_rows(Cd)
    assert np.all(full[:, :12] == 0) and np.all(full[:, 12:] == SENTINEL)


def test_odd_sizes_are_refused():
    A = torch.ones((8, 7), dtype=torch.bfloat16, device="cuda")
    B = torch.ones((7, 8), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(m.MgemmError) as e:
        m.gemm16(A, B)
    assert e.value.status == m.ERR_ARG


def test_whole_output_8192_bf16_against_oracle():
    """The benchmark's 16-bit row (bfloat16, default plan: 256x256 piped S=2)
    on the full 8192^3 problem: every element of C against the oracle's
    bound, the whole fp64 product and |A||B| computed on the host cores."""
    n = 8192
    A = datagen.matrix16(1, n, n, "bf16")
    B = datagen.matrix16(2, n, n, "bf16")
    Ad, Bd = dev16(A, "bf16", extra_rows=0), dev16(B, "bf16", extra_rows=0)
    assert m.plan16(n, n, n)["tile"] == m._TILE["256x256"]
    C = m.gemm16(Ad, Bd, stages=2, fill="piped")
    torch.cuda.synchronize()
    print("bf16 8192^3 default plan done; oracle on the whole product", flush=True)
    # every bfloat16 value is exact in fp32, so the fp32 GEMM oracle on the
    # inputs decoded once (by the oracle's own decoder, tabulated) forms the
    # same fp64 sums as its 16-bit GEMM, in the same order, at the fp32
    # oracle's speed
    table = np.array([oracle.decode16(b, "bf16") for b in range(1 << 16)])
    Af, Bf = table[A].astype(np.float32), table[B].astype(np.float32)
    assert np.array_equal(Af, table[A]) and np.array_equal(Bf, table[B])
    check_bound(C.cpu().numpy(), Af, Bf, what="bf16 8192^3 piped S=2 (whole output)")


@pytest.mark.parametrize("fmt", ["bf16", "f16"])
def test_full_size_8192(fmt):
    n = 8192
    A = datagen.matrix16(1, n, n, fmt)
    B = datagen.matrix16(2, n, n, fmt)
    Ad, Bd = dev16(A, fmt, extra_rows=0), dev16(B, fmt, extra_rows=0)
    ref = m.gemm16(Ad, Bd, stages=2, fill="piped")
    other = torch.empty_like(ref)
    for fill, S, tile in (("sync", 1, "auto"), ("sync", 2, "auto"), ("piped", 3, "256x128"), ("piped", 1, "256x128"),
                          ("sync", 1, "128x128")):
        other.fill_(float("nan"))
        m.gemm16(Ad, Bd, other, stages=S, fill=fill, tile=tile)
        torch.cuda.synchronize()
        assert torch.equal(other.view(torch.int32), ref.view(torch.int32)), (fmt, fill, S, tile)
    rows = np.unique(np.r_[0, 1, n // 2, n - 1, np.linspace(0, n - 1, 8).astype(int)])
    check16(ref[torch.as_tensor(rows, device="cuda")].cpu().numpy(), A[rows], B, fmt,
            what=f"{fmt} 8192^3 sampled rows")
