"""Every entry point under HIP graph capture (torch.cuda.CUDAGraph), through
the C ABI. The launch path makes kernel launches on the caller's stream and
nothing else (no allocation, memset or synchronisation), so one captured call
can be replayed. Each graph is replayed several times with new input values
written between replays, eager work and synchronisations in between, and
every replay must equal an eager call on the same inputs, bit for bit."""
import pytest
import torch

import async_global_shared_amd as m
import datagen

pytestmark = pytest.mark.gpu

REPLAYS = 4


def _check_replays(call, out, refill):
    """Capture call() (which writes `out`), then for each replay: refill the
    inputs, run call() eagerly, copy its result aside, poison `out`, replay,
    and compare."""
    side = torch.cuda.Stream()  # first call outside capture, as torch warms up graphs
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for r in range(REPLAYS):
        refill(r)
        call()
        want = out.clone()
        torch.cuda.synchronize()
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int32), want.view(torch.int32)), r
        assert not torch.isnan(out).any(), r


def _uniform(seed, rows, cols):
    return datagen.uniform_pm1_torch(seed, rows * cols, device="cuda").view(rows, cols)


@pytest.mark.parametrize("compute,tile,fill,S", [("mfma", "128x128", "piped", 2), ("valu", "64x64", "sync", 3),
                                                  ("mfma", "256x128", "piped", 3)])
def test_sgemm_graph(compute, tile, fill, S):
    M, N, K = 700, 600, 530
    A, B = _uniform(1, M, K), _uniform(2, K, N)
    C = torch.empty((M, N), device="cuda")

    def refill(r):
        A.copy_(_uniform(10 + r, M, K))
        B.copy_(_uniform(20 + r, K, N))

    _check_replays(lambda: m.sgemm(A, B, C, stages=S, fill=fill, compute=compute, tile=tile), C, refill)


def test_gemm16_graph():
    M, N, K = 520, 776, 264
    dt = torch.bfloat16
    A = _uniform(3, M, K).to(dt)
    B = _uniform(4, K, N).to(dt)
    C = torch.empty((M, N), device="cuda")

    def refill(r):
        A.copy_(_uniform(30 + r, M, K).to(dt))
        B.copy_(_uniform(40 + r, K, N).to(dt))

    _check_replays(lambda: m.gemm16(A, B, C, stages=2, fill="piped", tile="auto"), C, refill)


def test_attention_graph():
    Bt, H, Sq, Sk, D = 1, 2, 200, 330, 128
    dt = torch.bfloat16

    def qkv(seed, S):
        return datagen.uniform_pm1_torch(seed, Bt * H * S * D, device="cuda").view(Bt, H, S, D).to(dt)

    Q, K, V = qkv(5, Sq), qkv(6, Sk), qkv(7, Sk)
    O = torch.empty((Bt, H, Sq, D), device="cuda")

    def refill(r):
        Q.copy_(qkv(50 + r, Sq))
        K.copy_(qkv(60 + r, Sk))
        V.copy_(qkv(70 + r, Sk))

    _check_replays(lambda: m.attention(Q, K, V, O, scale=D ** -0.5, stages=2, fill="piped"), O, refill)


def test_tile_copy_graph():
    rows, cols = 1000, 777
    src = _uniform(8, rows, cols)
    dst = torch.empty_like(src)

    def refill(r):
        src.copy_(_uniform(80 + r, rows, cols))

    _check_replays(lambda: m.tile_copy(src, dst, stages=3), dst, refill)
