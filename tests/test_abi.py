"""Host-side tests of libmgemm: exports, argument validation, launch plans,
the ring schedule and the loader map the kernels execute, and evidence in
the generated gfx950 ISA. No GPU is touched: every call here returns before any HIP call."""
import os
import re

import numpy as np
import pytest

import async_global_shared_amd as m

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mgemm.h")

A0, B0, C0 = 0x100000, 0x40000000, 0x80000000  # fake, aligned, disjoint device addresses


def test_exports_every_declared_symbol():
    src = open(HEADER).read()
    names = set(re.findall(r"^\s*(?:const\s+)?[a-z_]+\s*\*?\s*(mgemm_[a-z_]+)\s*\(", src, re.M))
    assert {"mgemm_sgemm", "mgemm_sgemm_ex", "mgemm_tile_copy", "mgemm_status_string", "mgemm_version",
            "mgemm_plan_sgemm", "mgemm_ring_trace", "mgemm_fill_trace"} <= names
    L = m.lib()
    for n in names:
        assert hasattr(L, n), n


def test_no_undefined_kernel_symbols():
    """Every kernel the dispatch tables name has its host launch stub."""
    import subprocess
    out = subprocess.run(["nm", "-D", m.LIB_PATH], capture_output=True, text=True, check=True).stdout
    undefined = [l for l in out.splitlines() if " U _ZN5mgemm" in l]
    assert not undefined, undefined[:5]


def test_version_and_status_strings():
    assert m.mgemm_version() == m.MGEMM_VERSION
    for s in (m.OK, m.ERR_ARG, m.ERR_ALIAS, m.ERR_ARCH, m.ERR_LAUNCH, m.ERR_UNSUPPORTED):
        assert m.mgemm_status_string(s) not in ("", "unknown status")
    assert m.mgemm_status_string(12345) == "unknown status"


def sg(M=64, N=64, K=64, A=A0, lda=None, B=B0, ldb=None, C=C0, ldc=None, stages=2, fill=1, compute=0, tile=0,
       loader=0):
    lda = K if lda is None else lda
    ldb = N if ldb is None else ldb
    ldc = N if ldc is None else ldc
    return m.mgemm_sgemm_ex(M, N, K, A, lda, B, ldb, C, ldc, stages, fill, compute, tile, loader, None)


@pytest.mark.parametrize("kw,want", [
    (dict(M=-1), m.ERR_ARG), (dict(N=-1), m.ERR_ARG), (dict(K=-1), m.ERR_ARG),
    (dict(stages=0), m.ERR_ARG), (dict(stages=7), m.ERR_ARG), (dict(stages=4, fill=0), m.ERR_ARG),
    (dict(fill=3), m.ERR_ARG),
    (dict(compute=2), m.ERR_ARG), (dict(tile=4), m.ERR_ARG), (dict(tile=3, compute=0), m.ERR_ARG), (dict(loader=3), m.ERR_ARG),
    (dict(lda=63), m.ERR_ARG), (dict(ldb=10), m.ERR_ARG), (dict(ldc=63), m.ERR_ARG),
    (dict(A=0), m.ERR_ARG), (dict(B=0), m.ERR_ARG), (dict(C=0), m.ERR_ARG),
    (dict(C=A0), m.ERR_ALIAS), (dict(C=B0 + 4 * 100), m.ERR_ALIAS),
    (dict(lda=1 << 21), m.ERR_UNSUPPORTED), (dict(M=1 << 20, K=4096), m.ERR_UNSUPPORTED),
    (dict(A=A0 + 4, loader=1), m.ERR_ARG), (dict(K=62, loader=1), m.ERR_ARG),
])
def test_validation_before_any_device_call(kw, want):
    assert sg(**kw) == want


def test_largest_leading_dimension_is_planned():
    # 256-row tiles at ld = 2^21 - 4 words: the last in-block byte offset,
    # 255 * ld * 4 + ..., still fits below 2^31 (planner only: no device access)
    ld = (1 << 21) - 4
    A, B, C = 1 << 32, 1 << 36, 1 << 40
    st, p = m.mgemm_plan_sgemm(256, 64, 64, A, ld, B, 64, C, 64, 2, 1, 1, 3, 0)
    assert st == m.OK and p.bm == 256 and 255 * ld * 4 + 64 * 4 < 1 << 31
    st, p = m.mgemm_plan_gemm16(256, 64, 64, A, 2 * ld, B, 64, C, 64, 1, 2, 1, 3)
    assert st == m.OK and p.bm == 256
    st, _ = m.mgemm_plan_gemm16(256, 64, 64, A, 2 * ld + 8, B, 64, C, 64, 1, 2, 1, 3)
    assert st == m.ERR_UNSUPPORTED


def test_empty_operands_need_no_pointers():
    # M == 0 or N == 0 is a no-op that touches nothing; NULL is fine there
    assert m.mgemm_sgemm(0, 5, 5, 0, 5, B0, 5, 0, 5, 2, 1, None) == m.OK
    assert m.mgemm_sgemm(5, 0, 5, A0, 5, 0, 0, 0, 0, 2, 1, None) == m.OK


def test_copy_validation():
    f = m.mgemm_tile_copy
    assert f(10, 10, A0, 10, B0, 10, 0, None) == m.ERR_ARG
    assert f(10, 10, A0, 10, B0, 10, 7, None) == m.ERR_ARG
    assert f(10, 10, A0, 9, B0, 10, 2, None) == m.ERR_ARG
    assert f(10, 10, A0, 10, A0 + 40, 10, 2, None) == m.ERR_ALIAS
    assert f(10, 10, 0, 10, B0, 10, 2, None) == m.ERR_ARG
    assert f(0, 10, 0, 10, 0, 10, 2, None) == m.OK


def test_plain_copy_validation():
    f = m.mgemm_plain_copy
    assert f(10, 10, A0, 9, B0, 10, None) == m.ERR_ARG
    assert f(10, 10, A0, 10, B0, 9, None) == m.ERR_ARG
    assert f(10, 10, A0, 10, A0 + 40, 10, None) == m.ERR_ALIAS
    assert f(10, 10, 0, 10, B0, 10, None) == m.ERR_ARG
    assert f(-1, 10, A0, 10, B0, 10, None) == m.ERR_ARG
    assert f(0, 10, 0, 10, 0, 10, None) == m.OK
    assert f(1 << 20, 4096, A0, 4096, B0, 4096, None) == m.ERR_UNSUPPORTED


def test_plan_tiles_loaders_and_lds():
    p = m.plan(256, 256, 256)
    assert (p["bm"], p["bn"], p["bk"], p["threads"], p["blocks"]) == (64, 64, 16, 256, 16)
    assert p["load_bytes"] == 16 and p["slices"] == 16
    p = m.plan(4096, 4096, 4096, compute="mfma", stages=3, tile="128x128")
    assert (p["bm"], p["blocks"], p["lds_bytes"], p["loads_per_slice"], p["max_vmcnt"]) == (128, 1024, 49152, 4, 4)
    p = m.plan(4096, 4096, 4096, compute="mfma", stages=3)  # automatic: 256x128 on the 2+ stage ring
    assert (p["bm"], p["bn"], p["blocks"], p["lds_bytes"], p["loads_per_slice"], p["max_vmcnt"]) == \
        (256, 128, 512, 73728, 6, 6)
    # ragged, misaligned leading dimensions -> 4-byte loads
    p = m.plan(4099, 3001, 1537, stages=3, tile="128x128", lda=1537, ldb=3001, ldc=3001)
    assert p["load_bytes"] == 4 and p["bm"] == 128 and p["blocks"] == 33 * 24 and p["slices"] == 97
    assert p["loads_per_slice"] == 16 and p["max_vmcnt"] == 16
    # tall-skinny keeps enough blocks with 64 x 64 tiles
    p = m.plan(16384, 64, 4096)
    assert p["bm"] == 64 and p["blocks"] == 256
    # misaligned base
    st, pl = m.mgemm_plan_sgemm(64, 64, 64, A0 + 4, 64, B0, 64, C0, 64, 2, 1, 0, 0, 0)
    assert st == m.OK and pl.load_bytes == 4
    for S in range(1, 7):
        for b in ("64x64", "128x128"):
            for ld in ("b128", "b32"):
                p = m.plan(512, 512, 512, stages=S, tile=b, loader=ld)
                assert p["max_vmcnt"] == min(63, max(0, S - 2) * p["loads_per_slice"])
    # deep rings fit the 160 KiB of LDS: 6 stages of 256x128x16 fp32 tiles
    p = m.plan(8192, 8192, 8192, stages=6, compute="mfma", tile="256x128")
    assert p["lds_bytes"] == 6 * (256 + 128) * 16 * 4 <= 160 * 1024


# (M, N, K) -> automatic fp32 tile edge, for both compute tiles: the cases
# measured on MI355X (ragged and tall-skinny, where 128x128 would leave CUs
# with a partial last round or a lone block, and the large squares).
AUTO_FP32 = {(4099, 3001, 1537): 64, (16384, 64, 4096): 64, (2048, 2048, 2048): 64, (256, 256, 256): 64,
             (4096, 4096, 4096): 128, (8192, 8192, 8192): 128}


@pytest.mark.parametrize("compute", ["valu", "mfma"])
def test_auto_fp32_tile(compute):
    for (M, N, K), edge in AUTO_FP32.items():
        for fill in ("sync", "piped"):
            for S in (1, 2, 3):
                p = m.plan(M, N, K, stages=S, fill=fill, compute=compute)
                want = (edge, edge)
                # MFMA on the asynchronous ring of 2 or 3 stages: 256x128 where
                # 128x128 would be chosen and every CU gets an even number of
                # 256x128 tiles (both shapes here: 2 and 8 per CU)
                if compute == "mfma" and fill == "piped" and S >= 2 and edge == 128:
                    want = (256, 128)
                assert (p["bm"], p["bn"]) == want, (compute, fill, M, N, K, S)
    # the warp-specialised ring, deeper rings and odd or uneven 256x128 tile
    # counts per CU keep 128x128 (N = K = 8192: 256x128 tiles per CU = M / 1024)
    p = m.plan(8192, 8192, 8192, stages=2, fill="piped_ws", compute="mfma")
    assert (p["bm"], p["bn"]) == (128, 128)
    if compute == "mfma":
        assert m.plan(8192, 8192, 8192, stages=4, compute="mfma")["bm"] == 128
        for M, bm in ((6144, 256), (10240, 256), (5120, 128), (7168, 128), (8704, 128), (9728, 128)):
            assert m.plan(M, 8192, 8192, stages=2, compute="mfma")["bm"] == bm, M
    # the ABI's plain entry point plans with the VALU tile and the same choice
    st, pl = m.mgemm_plan_sgemm(4099, 3001, 1537, A0, 1537, B0, 3001, C0, 3001, 2, 1, 0, 0, 0)
    assert st == m.OK and pl.bm == 64


def test_plan_warp_specialised():
    p = m.plan(8192, 8192, 8192, stages=3, fill="piped_ws", compute="mfma")
    assert p["threads"] == 512 and p["fill_mode"] == 2
    assert p["lds_bytes"] == 3 * 16384 + 13 * 4 and p["max_vmcnt"] == 4
    assert m.lib().mgemm_ring_trace(0, 2, 2, 3, None, 0) == m.ERR_ARG


def test_lds_per_stage_matches_the_pages_budget():
    """The day-74 lesson reports ptxas shared memory per block for its 64x64x16
    kernel; every stage holds one 64x16 A tile and one 16x64 B tile (8 KiB),
    plus the libcu++ pipeline's own state. Our ring needs no such state, so the
    page's totals minus ours leave exactly a per-stage-growing remainder."""
    rows = [l.split() for l in open(os.path.join(ROOT, "tests", "golden", "day74_smem_per_block.txt"))
            if l.strip() and not l.startswith("#")]
    page = {int(s): int(b) for s, b in rows}
    for S in (2, 3):
        ours = m.plan(512, 512, 512, stages=S)["lds_bytes"]
        assert ours == S * 8192
        assert page[S] - ours == 8 + 16 * S  # 8 B header + 16 B per stage
    assert page[4] - 4 * 8192 == 8 + 16 * 4 and page[5] - 5 * 8192 == 8 + 16 * 5


# ---- the ring schedule the kernels execute ---------------------------------

def simulate_piped(events, S, T, split=False):
    """Check an asynchronous-ring trace: every slice issued once in order; a
    slot is refilled only after a barrier that follows the compute on its
    previous slice; compute(t) follows a wait that leaves slice t complete and
    a barrier after it; in flight never exceeds S-1 during compute (S for S=1).
    With split computes, head(t) (the first LDS reads) obeys the same rules as
    compute(t) and comes right before it, apart from tail(t-1); tail(t) (no
    LDS access) follows compute(t), in order, and every slice gets one."""
    issued, done = [], set()
    slot_of = {}
    tails, headed = [], None
    slot_busy = {}  # slot -> slice computed-from but not yet released by a barrier
    last_compute_released = True
    computed = []
    waited_since_issue = {}
    barrier_after_wait = set()
    for op, a, b in events:
        if op == 1:  # issue a -> slot b
            assert a == len(issued), "slices issued out of order"
            assert 0 <= b < S
            # slot b must not hold an uncomputed slice or one computed without a barrier since
            for s, sl in slot_of.items():
                if sl == b and s not in computed:
                    raise AssertionError(f"slot {b} refilled before slice {s} was computed")
            assert slot_busy.get(b) is None, f"slot {b} refilled before a barrier released it"
            issued.append(a)
            slot_of[a] = b
        elif op == 2:  # wait: at most a slices in flight
            inflight = [s for s in issued if s not in done]
            keep = inflight[len(inflight) - a:] if a else []
            for s in inflight:
                if s not in keep:
                    done.add(s)
        elif op == 3:  # barrier
            for s in list(done):
                barrier_after_wait.add(s)
            slot_busy.clear()
        elif op in (4, 7):  # compute (or head) of slice a from slot b
            assert split == (op == 7 or headed is not None), "head and compute must pair up"
            assert a == len(computed), "compute out of order"
            assert a in barrier_after_wait, f"slice {a} read before wait+barrier"
            assert slot_of[a] == b
            inflight = [s for s in issued if s not in done]
            assert len(inflight) <= max(S - 1, 0)
            if op == 7:
                assert headed is None
                headed = a
            else:
                assert not split or headed == a, f"compute of slice {a} without its head"
                headed = None
                computed.append(a)
            slot_busy[b] = a
        elif op == 8 and split:  # tail of slice a: registers only
            assert a == len(tails) and a in computed, f"tail of slice {a} out of order"
            tails.append(a)
        else:
            raise AssertionError(f"unexpected op {op}")
    assert issued == list(range(T)) and computed == list(range(T))
    assert not split or tails == list(range(T))


def simulate_sync(events, S, T):
    """Check a synchronous-ring trace: each slice loaded once, in order, into a
    register set that is free; stored from the set holding it into the slot it
    is computed from; a barrier separates store and compute; a slot is
    overwritten only after a barrier that follows the compute on it. A load
    of a slice past the last (the masked load that keeps the loop body free
    of branches) comes after every real one and its set is never stored."""
    R = max(S - 1, 1)
    sets = {}
    loaded = []
    masked = []
    slot_holds = {}
    visible = set()
    slot_busy = {}
    computed = []
    for op, a, b in events:
        if op == 6 and a >= T:  # masked load into set b
            assert len(loaded) == T and 0 <= b < R, "masked load before the last real one"
            assert sets.get(b) is None, f"register set {b} reused before its store"
            sets[b] = "masked"
            masked.append(a)
        elif op == 6:  # load slice a into set b
            assert a == len(loaded) and 0 <= b < R
            assert sets.get(b) is None or sets[b] == "masked", f"register set {b} reused before its store"
            sets[b] = a
            loaded.append(a)
        elif op == 5:  # store set a -> slot b
            assert sets.get(a) is not None, "store of an empty register set"
            assert sets[a] != "masked", "store of a masked load"
            assert slot_busy.get(b) is None, f"slot {b} overwritten before a barrier released it"
            assert slot_holds.get(b) is None or slot_holds[b] in computed, f"slot {b} overwritten before use"
            s = sets.pop(a)
            slot_holds[b] = s
            visible.discard(s)
            slot_busy[b] = "written"
        elif op == 3:
            for sl, s in slot_holds.items():
                visible.add(s)
            slot_busy.clear()
        elif op == 4:
            assert a == len(computed)
            assert slot_holds.get(b) == a and a in visible, f"slice {a} not visible in slot {b}"
            computed.append(a)
            slot_busy[b] = "read"
        else:
            raise AssertionError(op)
    assert loaded == list(range(T)) and computed == list(range(T))
    assert len(masked) <= R - 1 if S > 1 else not masked
    return masked


@pytest.mark.parametrize("S,fill", [(S, 1) for S in range(1, 7)] + [(S, 0) for S in (1, 2, 3)])
def test_ring_schedule(S, fill):
    for T in list(range(0, 14)) + [31, 40, 97]:
        ev = m.mgemm_ring_trace(0, S, fill, T)
        if fill == 1:
            simulate_piped(ev, S, T)
            waits = [a for op, a, b in ev if op == 2]
            assert all(0 <= w <= max(S - 2, 0) for w in waits)
            # the waits are exact: each leaves in flight exactly the slices issued after the awaited one
            if S >= 2:
                assert waits == [min(T - 1, t + S - 2) - t for t in range(T)]
        else:
            masked = simulate_sync(ev, S, T)
            # two register sets: the grouped loop's one masked load when T is odd
            assert masked == ([T] if S == 3 and T >= 3 and T % 2 else [])
    if fill == 1:
        assert m.mgemm_ring_trace(1, S, 1, 5) == m.mgemm_ring_trace(0, S, 1, 5)


@pytest.mark.parametrize("S", range(1, 7))
def test_split_ring_schedule(S):
    """The 16-bit GEMM's ring: the piped schedule with each compute split into
    head / body / tail, the previous slice's tail after the next one's head."""
    for T in list(range(0, 14)) + [31, 97]:
        ev = m.mgemm_ring_trace(2, S, 1, T)
        simulate_piped(ev, S, T, split=True)
        # removing heads and tails leaves exactly the unsplit ring
        assert [e for e in ev if e[0] not in (7, 8)] == m.mgemm_ring_trace(0, S, 1, T)
        # the overlap itself: tail(t-1) sits between head(t) and compute(t),
        # and so does the refill issued after the barrier (S >= 2), which
        # tail_issue spreads over the tail's matrix instructions
        for t in range(1, T):
            k = ev.index((7, t, t % S if S > 1 else 0))
            refill = S > 1 and t + S - 1 < T
            between = ev[k + 1:k + 2 + refill]
            assert (8, t - 1, 0) in between and ev[k + 2 + refill][0] == 4
            assert not refill or between[0] == (1, t + S - 1, (t + S - 1) % S)
    # a tail before its compute, or a missing head, is caught
    ev = m.mgemm_ring_trace(2, S, 1, 4)
    bad = list(ev)
    t0 = bad.pop(bad.index((8, 0, 0)))
    bad.insert(bad.index((4, 0, 0)), t0)
    with pytest.raises(AssertionError):
        simulate_piped(bad, S, 4, split=True)
    with pytest.raises(AssertionError):
        simulate_piped([e for e in ev if e[:2] != (7, 2)], S, 4, split=True)


FILL_KINDS = {0: "fp32 VALU 64", 1: "fp32 VALU 128", 2: "fp32 MFMA 64 (32-k slice)", 3: "fp32 MFMA 128",
              4: "fp32 MFMA 256x128", 5: "16-bit 128", 6: "16-bit 256x128", 7: "16-bit 256x256", 8: "attention D64",
              9: "attention D128", 10: "tile copy, 8 waves", 11: "fp32 MFMA 64 (64-k slice)",
              12: "tile copy, 16 waves"}


@pytest.mark.parametrize("kind", sorted(FILL_KINDS))
@pytest.mark.parametrize("W", [16, 4])
@pytest.mark.parametrize("fill", [0, 1])
def test_fill_map_covers_the_slot_once(kind, W, fill):
    """One slice's loader map, from the kernels' own operand types and
    filling-wave rules: every byte of the LDS slot is written exactly once,
    every element of each operand's slice is fetched exactly once, and each
    lands where the compute side's layout reads it."""
    if kind in (10, 12) and fill == 0:
        assert m.lib().mgemm_fill_trace(kind, W, fill, None, 0) == m.ERR_ARG
        return
    (slot, r0, c0, r1, c1), ev = m.mgemm_fill_trace(kind, W, fill)
    written = np.zeros(slot, np.int32)
    fetched = [np.zeros((r0, c0), np.int32), np.zeros((r1, c1), np.int32)]
    words = W // 4
    for op, wave, lds, r, c, want in ev:
        assert 0 <= lds and lds + W <= slot, (FILL_KINDS[kind], op, wave, lds)
        written[lds:lds + W] += 1
        assert lds == want, (FILL_KINDS[kind], op, wave, r, c, lds, want)
        fetched[op][r, c:c + words] += 1
    assert np.all(written == 1), (FILL_KINDS[kind], int((written != 1).sum()))
    for op in (0, 1):
        assert np.all(fetched[op] == 1), (FILL_KINDS[kind], op)
    waves = {w for _, w, *_ in ev}
    if kind == 7 and fill == 1 and W == 16:
        assert waves == {0, 1, 2, 3}  # the 8-wave tile's asynchronous ring fills from one wave per SIMD
    elif kind in (10, 12):
        assert waves == set(range(4 if kind == 10 else 8))  # the copy's filling waves: the block's first half
    else:
        assert waves == set(range(8 if kind in (7, 8, 9) else 4))


def test_fill_map_catches_a_misplaced_unit():
    """The fill-map test above rejects a loader that writes one unit of one wave
    at its neighbour's place."""
    (slot, *_), ev = m.mgemm_fill_trace(7, 16, 1)
    bad = [(op, w, lds + 1024 if (w, op) == (1, 0) and i % 97 == 0 else lds, r, c, want)
           for i, (op, w, lds, r, c, want) in enumerate(ev)]
    written = np.zeros(slot + 2048, np.int32)
    ok = True
    for op, w, lds, r, c, want in bad:
        written[lds:lds + 16] += 1
        ok &= lds == want
    assert not ok and np.any(written[:slot] != 1)


def test_ring_trace_rejects_bad_arguments():
    assert m.lib().mgemm_ring_trace(0, 7, 1, 3, None, 0) == m.ERR_ARG
    assert m.lib().mgemm_ring_trace(0, 4, 0, 3, None, 0) == m.ERR_ARG
    assert m.lib().mgemm_ring_trace(1, 2, 0, 3, None, 0) == m.ERR_ARG
    assert m.lib().mgemm_ring_trace(3, 2, 1, 3, None, 0) == m.ERR_ARG
    assert m.lib().mgemm_ring_trace(2, 2, 0, 3, None, 0) == m.ERR_ARG


def test_simulators_catch_planted_schedule_bugs():
    """The ring simulators above reject the classic ring mistakes."""
    good = m.mgemm_ring_trace(0, 3, 1, 6)
    # compute before waiting: drop the first wait
    bad = list(good)
    bad.remove(next(e for e in bad if e[0] == 2))
    with pytest.raises(AssertionError):
        simulate_piped(bad, 3, 6)
    # wrong slot index for a compute
    bad = [(4, a, (b + 1) % 3) if op == 4 and a == 2 else (op, a, b) for op, a, b in good]
    with pytest.raises(AssertionError):
        simulate_piped(bad, 3, 6)
    # refill a slot before the barrier that releases it: swap barrier and issue in one iteration
    i = next(k for k in range(1, len(good)) if good[k][0] == 1 and good[k - 1][0] == 3 and good[k][1] >= 3)
    bad = list(good)
    bad[i - 1], bad[i] = bad[i], bad[i - 1]
    with pytest.raises(AssertionError):
        simulate_piped(bad, 3, 6)
    # sync ring: drop the barrier between store and compute
    good = m.mgemm_ring_trace(0, 2, 0, 5)
    bad = list(good)
    del bad[next(k for k, e in enumerate(bad) if e[0] == 3)]
    with pytest.raises(AssertionError):
        simulate_sync(bad, 2, 5)


# ---- evidence in our own gfx950 ISA -----------------------------------------

def _kernels(isa):
    out = {}
    cur = None
    for line in isa.splitlines():
        mm = re.match(r"^(_ZN5mgemm\w+):", line)
        if mm:
            cur = mm.group(1)
            out[cur] = []
        elif cur is not None:
            if line.startswith(".Lfunc_end"):
                cur = None
            else:
                out[cur].append(line)
    return out


def _mangled(cfg):
    """Itanium-mangled config name: "CfgX" or "CfgX<n>" (an int template)."""
    mm = re.fullmatch(r"(\w+)<(\d+)>", cfg)
    if mm:
        return f"{len(mm[1])}{mm[1]}ILi{mm[2]}EE"
    return f"{len(cfg)}{cfg}"


def _name(cfg, S, piped, W):
    return f"_ZN5mgemm12sgemm_kernelINS_{_mangled(cfg)}ELi{S}ELb{int(piped)}ELi{W}EEEvNS_8GemmArgsE"


@pytest.fixture(scope="module")
def isa():
    if not os.path.exists(m.ISA_PATH):
        pytest.skip("ISA not built")
    return _kernels(open(m.ISA_PATH).read())


CFGS = ["CfgValu64", "CfgValu128", "CfgMfma64K<32>", "CfgMfma64K<64>", "CfgMfma128", "CfgMfma256x128"]
# a problem each config is planned for: (M, N, K, tile, compute)
CFG_PLAN = {"CfgValu64": (1024, 1024, 1024, "64x64", "valu"), "CfgValu128": (1024, 1024, 1024, "128x128", "valu"),
            "CfgMfma64K<32>": (2048, 2048, 1024, "64x64", "mfma"), "CfgMfma64K<64>": (1024, 1024, 1024, "64x64", "mfma"),
            "CfgMfma128": (1024, 1024, 1024, "128x128", "mfma"), "CfgMfma256x128": (1024, 1024, 1024, "256x128", "mfma")}


def _cfg_plan(cfg, S, fill="piped", W=16):
    """The plan of cfg's problem at depth S, or None where the ring exceeds the LDS."""
    M, N, K, tile, compute = CFG_PLAN[cfg]
    try:
        p = m.plan(M, N, K, stages=S, fill=fill, tile=tile, compute=compute, loader="b128" if W == 16 else "b32")
    except m.MgemmError as e:
        assert e.status == m.ERR_UNSUPPORTED
        return None
    assert p["bk"] == (int(cfg[-3:-1]) if "<" in cfg else 16)
    return p


def test_every_config_and_depth_that_fits_is_planned():
    """Rings within the 160 KiB of LDS are planned; deeper ones are refused
    (their kernels are empty) rather than run."""
    for cfg in CFGS:
        for S in range(1, 7):
            p = _cfg_plan(cfg, S)
            slot = (CFG_PLAN[cfg][3], int(cfg[-3:-1]) if "<" in cfg else 16)
            bm, bn = (int(x) for x in slot[0].split("x"))
            fits = S * (bm + bn) * slot[1] * 4 <= 160 * 1024
            assert (p is not None) == fits, (cfg, S)


@pytest.mark.parametrize("cfg", CFGS)
def test_isa_fill_instructions(isa, cfg):
    """Piped kernels fill LDS with buffer_load ... lds and no ds_write; sync
    kernels fill through VGPRs (ds_write) and have no LDS-direct load."""
    for S in range(1, 7):
        for W in (16, 4):
            if _cfg_plan(cfg, S) is None:
                continue
            body = "\n".join(isa[_name(cfg, S, True, W)])
            width = "dwordx4" if W == 16 else "dword"
            assert re.search(rf"buffer_load_{width} .* lds", body), (cfg, S, W)
            assert "ds_write" not in body, (cfg, S, W)
            assert "v_pk_fma_f32" not in body
            if S > 3:
                assert _name(cfg, S, False, W) not in isa  # no register-staged ring that deep
                continue
            sbody = "\n".join(isa[_name(cfg, S, False, W)])
            assert " lds" not in sbody.replace("lds_", "") or not re.search(r"buffer_load\S* .* lds", sbody)
            assert "ds_write" in sbody
            assert "v_pk_fma_f32" not in body and "v_pk_fma_f32" not in sbody


def _cfg(lines):
    """Basic blocks of one kernel's assembly: list of (label, instructions,
    successor labels), following labels and s_branch / s_cbranch_*."""
    blocks, cur, body = [], "entry", []
    def close(nxt):
        blocks.append([cur, body, nxt])
    for raw in lines:
        l = raw.split(";")[0].rstrip()
        if not l.strip() or l.strip().startswith("."):
            mm = re.match(r"^(\.LBB\w+):", raw)
            if mm:
                close(None)
                cur, body = mm.group(1), []
            continue
        ins = l.strip()
        body.append(ins)
        op = ins.split()[0]
        if op == "s_branch" or op.startswith("s_cbranch") or op in ("s_endpgm", "s_setpc_b64"):
            blocks.append([cur, body, ins])
            cur, body = cur + "+", []
    blocks.append([cur, body, None])
    out = []
    for i, (lab, ins, term) in enumerate(blocks):
        succ = []
        op = term.split()[0] if isinstance(term, str) else None
        if op and (op == "s_branch" or op.startswith("s_cbranch")):
            succ.append(term.split()[1])
        if op not in ("s_branch", "s_endpgm", "s_setpc_b64") and i + 1 < len(blocks):
            succ.append(blocks[i + 1][0])
        out.append((lab, ins, succ))
    return out


def _drain_before_compute(lines, op):
    """True if some path from a ring barrier reaches the compute instruction
    `op` through an s_waitcnt vmcnt(0)."""
    blocks = _cfg(lines)
    index = {lab: i for i, (lab, _, _) in enumerate(blocks)}
    # states: (block index, position, drained?)
    starts = [(i, k + 1) for i, (_, ins, _) in enumerate(blocks) for k, x in enumerate(ins) if x == "s_barrier"]
    seen, stack = set(), [(i, k, False) for i, k in starts]
    found_compute = False
    while stack:
        i, k, drained = stack.pop()
        if (i, k, drained) in seen:
            continue
        seen.add((i, k, drained))
        lab, ins, succ = blocks[i]
        stop = False
        for x in ins[k:]:
            if x == "s_barrier":
                stop = True
                break
            if "vmcnt(0)" in x:
                drained = True
            if x.startswith(op):
                found_compute = True
                if drained:
                    return True, True
                stop = True
                break
        if not stop:
            for sname in succ:
                if sname in index:
                    stack.append((index[sname], 0, drained))
    return False, found_compute


@pytest.mark.parametrize("cfg", CFGS)
def test_isa_compute_does_not_drain_the_prefetch(isa, cfg):
    """In the piped S >= 2 kernels no path through the control-flow graph goes
    from a ring barrier through s_waitcnt vmcnt(0) to the arithmetic: the
    compute runs while the next slices are still in flight."""
    op = "v_mfma_f32_32x32x2_f32" if "Mfma" in cfg else "v_fmac_f32"
    for S in range(2, 7):
        for W in (16, 4):
            p = _cfg_plan(cfg, S, W=W)
            if p is None:
                continue
            lines = isa[_name(cfg, S, True, W)]
            drained, reached = _drain_before_compute(lines, op)
            assert reached, (cfg, S, W)
            assert not drained, (cfg, S, W)
            if S >= 3:
                body = "\n".join(lines)
                assert f"s_waitcnt vmcnt({p['max_vmcnt']})" in body, (cfg, S, W, p["max_vmcnt"])


def test_isa_drain_checker_sees_a_drain():
    """The path checker flags a vmcnt(0) between barrier and compute."""
    lines = ["s_barrier", ".LBB0_1:", "s_waitcnt vmcnt(0)", "v_fmac_f32_e32 v1, v2, v3", "s_endpgm"]
    assert _drain_before_compute(lines, "v_fmac_f32") == (True, True)
    lines = ["s_waitcnt vmcnt(0)", "s_barrier", "s_cbranch_scc1 .LBB0_2", "s_waitcnt vmcnt(0)", ".LBB0_2:",
             "v_fmac_f32_e32 v1, v2, v3", "s_endpgm"]
    assert _drain_before_compute(lines, "v_fmac_f32") == (True, True)
    lines = ["s_waitcnt vmcnt(0)", "s_barrier", "s_waitcnt lgkmcnt(0)", "v_fmac_f32_e32 v1, v2, v3"]
    assert _drain_before_compute(lines, "v_fmac_f32") == (False, True)


@pytest.mark.parametrize("cfg", CFGS)
def test_isa_warp_specialised(isa, cfg):
    """The warp-specialised kernels synchronise through LDS counters: one
    start-up barrier only, polls with s_sleep, ds_add arrivals, and the
    asynchronous fill."""
    for S in range(1, 7):
        for W in (16, 4):
            if _cfg_plan(cfg, S, fill="piped_ws") is None:
                continue
            name = f"_ZN5mgemm15sgemm_ws_kernelINS_{_mangled(cfg)}ELi{S}ELi{W}EEEvNS_8GemmArgsE"
            body = "\n".join(isa[name])
            assert body.count("s_barrier") == 1, (cfg, S, W)
            assert "ds_add_u32" in body and "s_sleep" in body
            assert re.search(r"buffer_load_dword\S* .* lds", body)
            assert "flat_atomic" not in body and "flat_load" not in body


# ---- 16-bit (bfloat16 / binary16) GEMM: validation, plans, ISA ----------------

def g16(M=64, N=64, K=64, A=A0, lda=None, B=B0, ldb=None, C=C0, ldc=None, dtype=1, stages=2, fill=1, tile=0):
    lda = K if lda is None else lda
    ldb = N if ldb is None else ldb
    ldc = N if ldc is None else ldc
    return m.mgemm_plan_gemm16(M, N, K, A, lda, B, ldb, C, ldc, dtype, stages, fill, tile)[0]


@pytest.mark.parametrize("kw,want", [
    (dict(dtype=0), m.ERR_ARG), (dict(dtype=3), m.ERR_ARG), (dict(stages=0), m.ERR_ARG), (dict(stages=5), m.ERR_ARG),
    (dict(stages=4, fill=0), m.ERR_ARG),
    (dict(fill=2), m.ERR_ARG), (dict(tile=1), m.ERR_ARG), (dict(tile=5), m.ERR_ARG),
    (dict(K=63, lda=64), m.ERR_ARG), (dict(N=63, ldb=64, ldc=64), m.ERR_ARG), (dict(lda=65), m.ERR_ARG),
    (dict(ldb=65), m.ERR_ARG), (dict(A=A0 + 2), m.ERR_ARG), (dict(B=B0 + 6), m.ERR_ARG), (dict(lda=62), m.ERR_ARG),
    (dict(ldc=63), m.ERR_ARG), (dict(A=0), m.ERR_ARG), (dict(C=0), m.ERR_ARG),
    (dict(C=A0), m.ERR_ALIAS), (dict(C=B0 + 2 * 64 * 63), m.ERR_ALIAS), (dict(C=A0 + 2 * 64 * 64), m.OK),
    (dict(lda=1 << 22), m.ERR_UNSUPPORTED),
    (dict(A=A0 + 4), m.OK), (dict(B=B0 + 4, ldb=66), m.OK), (dict(stages=3, fill=0, tile=3), m.OK),
    (dict(tile=4), m.OK),
])
def test_gemm16_validation(kw, want):
    assert g16(**kw) == want
    if want != m.OK:
        # the launching entry point refuses the same arguments before any HIP call
        a = dict(M=64, N=64, K=64, A=A0, B=B0, C=C0, dtype=1, stages=2, fill=1, tile=0)
        a.update(kw)
        a.setdefault("lda", a["K"]), a.setdefault("ldb", a["N"]), a.setdefault("ldc", a["N"])
        assert m.mgemm_gemm16(a["M"], a["N"], a["K"], a["A"], a["lda"], a["B"], a["ldb"], a["C"], a["ldc"],
                              a["dtype"], a["stages"], a["fill"], a["tile"], None) == want


def test_gemm16_empty_operands_ignore_layout():
    # an operand with no elements is never read: its base and ld are free
    assert g16(M=10, K=0, lda=1, N=12, B=0, ldb=1, ldc=13) == m.OK
    assert g16(M=0, K=64, A=0, lda=1) == m.OK
    assert m.mgemm_gemm16(0, 8, 8, 0, 1, B0, 8, 0, 8, 1, 2, 1, 0, None) == m.OK


def test_gemm16_plans():
    bk = m.plan16(64, 64, 64)["bk"]
    assert bk in (32, 64)
    p = m.plan16(8192, 8192, 8192)
    assert (p["bm"], p["bn"], p["threads"], p["blocks"]) == (256, 256, 512, 32 * 32)
    assert m.plan16(4096, 4096, 4096)["bn"] == 256 and m.plan16(4096, 2048, 64)["bn"] == 128
    assert m.plan16(2048, 2048, 2048)["bm"] == 128
    # 240 blocks of 256x256 (one round of the 256 CUs) beat 960 of 128x128 (four rounds)
    assert (m.plan16(3000, 5000, 4000)["bm"], m.plan16(3000, 5000, 4000)["bn"]) == (256, 256)
    assert m.plan16(3000, 5000, 4000, lda=4002, ldb=5002)["bn"] == 128  # 4-byte loads: never the 8-wave tile
    # the asynchronous ring of the 8-wave tile fills from 4 waves; the register-staged one from all 8
    assert p["lds_bytes"] == 2 * (256 + 256) * bk * 2 and p["loads_per_slice"] == (256 + 256) * bk * 2 // 1024 // 4
    assert m.plan16(8192, 8192, 8192, fill="sync")["loads_per_slice"] == (256 + 256) * bk * 2 // 1024 // 8
    # rings beyond the 160 KiB of LDS are refused
    st, _ = m.mgemm_plan_gemm16(8192, 8192, 8192, A0, 8192, B0, 8192, C0, 8192, 1, 3, 1, 4)
    assert st == (m.ERR_UNSUPPORTED if 3 * (256 + 256) * bk * 2 > 160 * 1024 else m.OK)
    if bk != 64:
        return
    p = m.plan16(8192, 8192, 8192, tile="256x128")
    assert (p["bm"], p["bn"], p["bk"], p["blocks"], p["load_bytes"]) == (256, 128, 64, 32 * 64, 16)
    assert p["slices"] == 128 and p["lds_bytes"] == 2 * (256 + 128) * 64 * 2 and p["compute"] == m.COMPUTE_MFMA
    # one slice: (256 x 64 + 64 x 128) 16-bit elements = 48 KiB = 12 dwordx4 per lane of each of 4 waves
    assert p["loads_per_slice"] == 12 and p["max_vmcnt"] == 0
    assert m.plan16(8192, 8192, 8192, stages=3, tile="256x128")["max_vmcnt"] == 12
    assert m.plan16(8192, 8192, 8192, stages=3, tile="256x128")["lds_bytes"] == 3 * 49152 <= 160 * 1024
    p = m.plan16(1024, 1024, 1024, dtype="f16")
    assert (p["bm"], p["blocks"]) == (128, 64)
    # ragged K or a leading dimension off the 8-element grid -> 4-byte loads (pairs of elements)
    p = m.plan16(300, 258, 198, stages=3)
    assert p["load_bytes"] == 4 and p["slices"] == 4 and p["loads_per_slice"] == 32 and p["max_vmcnt"] == 32
    assert m.plan16(300, 264, 200, lda=208, ldb=272)["load_bytes"] == 16
    assert m.plan16(64, 64, 64, a_ptr=0x10004)["load_bytes"] == 4
    # misaligned big problems keep 4-byte loads and the 4-wave 256 x 128 tile
    p = m.plan16(8192, 8192, 8192, a_ptr=0x10004)
    assert (p["load_bytes"], p["bm"], p["bn"]) == (4, 256, 128)


def _name16(cfg, bf16, S, piped, W):
    return f"_ZN5mgemm12sgemm_kernelINS_{len(cfg)}{cfg}ILb{int(bf16)}EEELi{S}ELb{int(piped)}ELi{W}EEEvNS_8GemmArgsE"


H16_CFGS = ["CfgH128", "CfgH256x128", "CfgH256x256"]
H16_TILE = {"CfgH128": "128x128", "CfgH256x128": "256x128", "CfgH256x256": "256x256"}


def _fits16(cfg, S):
    st, _ = m.mgemm_plan_gemm16(1024, 1024, 1024, A0, 1024, B0, 1024, C0, 1024, 1, S, 1,
                                {"CfgH128": 2, "CfgH256x128": 3, "CfgH256x256": 4}[cfg])
    return st == m.OK


@pytest.mark.parametrize("cfg", H16_CFGS)
@pytest.mark.parametrize("bf16", [True, False])
def test_isa_gemm16(isa, cfg, bf16):
    """The 16-bit kernels multiply on v_mfma_f32_32x32x16_{bf16,f16}, read B
    through the transposing LDS read, fill LDS asynchronously (piped) or
    through VGPRs (sync), and never drain the prefetch before the MFMAs."""
    mfma = "v_mfma_f32_32x32x16_" + ("bf16" if bf16 else "f16")
    bk = m.plan16(64, 64, 64)["bk"]
    per_slice = {"CfgH128": 4, "CfgH256x128": 8, "CfgH256x256": 8}[cfg] * bk // 16  # WTM*WTN x k steps
    for S in (1, 2, 3, 4):
        if not _fits16(cfg, S):
            continue
        for W in (16, 4):
            for piped in ((True, False) if S < 4 else (True,)):
                lines = isa[_name16(cfg, bf16, S, piped, W)]
                body = "\n".join(lines)
                assert body.count(mfma) >= per_slice, (cfg, S, W, piped)
                assert "v_mfma_f32_32x32x2_f32" not in body
                assert "ds_read_b64_tr_b16" in body and "ds_read_b128" in body
                width = "dwordx4" if W == 16 else "dword"
                if piped:
                    assert re.search(rf"buffer_load_{width} .* lds", body) and "ds_write" not in body
                    if S >= 2:
                        drained, reached = _drain_before_compute(lines, mfma)
                        assert reached and not drained, (cfg, S, W)
                else:
                    assert "ds_write" in body and not re.search(r"buffer_load\S* .* lds", body)
                assert "v_pk_fma_f32" not in body and "v_pk_add_f32" not in body and "v_pk_mul_f32" not in body


def _store_waits(lines):
    """The vmcnt each ds_write waits for: groups of consecutive ds_writes,
    each write carrying the last s_waitcnt vmcnt(N) of its group (None if
    the group has had none)."""
    out, cur, last = [], None, None
    for raw in lines:
        x = raw.strip()
        if not x or x.startswith(";"):
            continue
        mm = re.match(r"s_waitcnt .*vmcnt\((\d+)\)", x)
        if mm:
            last = int(mm.group(1))
            continue
        if x.startswith("ds_write"):
            cur = [] if cur is None else cur
            cur.append(last)
        elif cur is not None and not x.startswith("s_waitcnt"):
            out.append(cur)
            cur, last = None, None
        if x.startswith(("buffer_load", "s_barrier")):
            last = None
    if cur:
        out.append(cur)
    return out


SYNC3 = ([(c, lambda c=c: _name(c, 3, False, 16)) for c in CFGS]
         + [(c, lambda c=c: _name16(c, True, 3, False, 16)) for c in ("CfgH128", "CfgH256x128")]
         + [(f"attention D{D}", lambda D=D: _attn_name(D, True, 3, False, 16)) for D in (64, 128)])


@pytest.mark.parametrize("what,name", SYNC3, ids=[w for w, _ in SYNC3])
def test_isa_sync_ring_keeps_the_newer_slice_in_flight(isa, what, name):
    """The two-register-set synchronous ring stores slice t+1 while slice
    t+2's loads are still in flight: its two steps' ds_writes wait with
    vmcnt >= L, the loads of one set (the prologue's store of slice 0 has L
    writes). Branches in the loop body used to make these waits drain to
    vmcnt(0..L-1)."""
    groups = _store_waits(isa[name()])
    L = len(groups[0])
    overlapped = 0
    for g in groups[1:]:
        w = None
        for x in g:
            w = x if x is not None else w
            overlapped += w is not None and w >= L
    assert overlapped >= 2 * L, (what, L, groups)


def _regs(operand):
    """VGPR indices named by one operand ('v7', 'v[30:33]'), else empty."""
    mm = re.fullmatch(r"v(\d+)", operand) or re.fullmatch(r"v\[(\d+):(\d+)\]", operand)
    if not mm:
        return set()
    lo = int(mm.group(1))
    hi = int(mm.group(2)) if mm.lastindex == 2 else lo
    return set(range(lo, hi + 1))


def _early_uses_of_lds_results(lines):
    """Instructions that read or overwrite the destination of an LDS read on
    some control-flow path before an s_waitcnt lgkmcnt(0): the wait the LDS
    reads issued from inline asm depend on. A forward may-analysis over the
    basic blocks of `_cfg` (pending registers join at block entries)."""
    blocks = _cfg(lines)
    index = {lab: i for i, (lab, _, _) in enumerate(blocks)}
    entry = {0: frozenset()}
    work, bad = [0], []
    while work:
        i = work.pop()
        pending = set(entry[i])
        for ins in blocks[i][1]:
            op, _, rest = ins.partition(" ")
            ops = [o.strip() for o in rest.split(",")]
            if op == "s_waitcnt" and "lgkmcnt(0)" in rest:
                pending.clear()
                continue
            used = set().union(*(_regs(o.split()[0]) for o in ops if o)) if ops else set()
            if used & pending and ins not in bad:
                bad.append(ins)
            if op.startswith("ds_read"):
                pending |= _regs(ops[0])
        for succ in blocks[i][2]:
            j = index.get(succ)
            if j is None:
                continue
            new = frozenset(pending) | entry.get(j, frozenset())
            if j not in entry or new != entry[j]:
                entry[j] = new
                work.append(j)
    return bad


def test_isa_guard_sees_an_early_use():
    lines = ["ds_read_b128 v[4:7], v1", "v_mov_b32_e32 v9, v5", "s_waitcnt lgkmcnt(0)", "v_mov_b32_e32 v9, v5"]
    assert _early_uses_of_lds_results(lines) == ["v_mov_b32_e32 v9, v5"]
    assert _early_uses_of_lds_results(lines[:1] + lines[2:]) == []
    # a use reached only over a branch that skips the wait is caught ...
    lines = ["ds_read_b128 v[4:7], v1", "s_cbranch_scc1 .LBB0_2", "s_waitcnt lgkmcnt(0)", ".LBB0_2:",
             "v_mov_b32_e32 v9, v6", "s_endpgm"]
    assert _early_uses_of_lds_results(lines) == ["v_mov_b32_e32 v9, v6"]
    # ... and code laid out after an unconditional branch is not on the read's path
    lines = [".LBB0_1:", "s_waitcnt lgkmcnt(0)", "ds_read_b128 v[4:7], v1", "s_branch .LBB0_1",
             ".LBB0_3:", "v_mov_b32_e32 v9, v6", "s_endpgm"]
    assert _early_uses_of_lds_results(lines) == []


@pytest.mark.parametrize("cfg", H16_CFGS)
def test_isa_gemm16_reads_are_waited_for(isa, cfg):
    """No instruction touches an LDS read's destination before the wait."""
    for bf16 in (True, False):
        for S in (1, 2, 3):
            for W in (16, 4):
                for piped in (True, False):
                    bad = _early_uses_of_lds_results(isa[_name16(cfg, bf16, S, piped, W)])
                    assert not bad, (cfg, bf16, S, W, piped, bad[:3])


# ---- attention: validation, plans, ISA -----------------------------------------

def att(B=2, H=3, Sq=100, Sk=90, D=64, Q=A0, K=B0, V=B0 + (1 << 24), O=C0, q=None, k=None, v=None, o=None,
        dtype=1, stages=2, fill=1):
    """(status, plan) for contiguous (B, H, S, D) views unless strides are given."""
    q = q or (H * Sq * D, Sq * D, D)
    k = k or (H * Sk * D, Sk * D, D)
    v = v or (H * Sk * D, Sk * D, D)
    o = o or (H * Sq * D, Sq * D, D)
    return m.mgemm_plan_attention(B, H, Sq, Sk, D, Q, *q, K, *k, V, *v, O, *o, dtype, stages, fill)


@pytest.mark.parametrize("kw,want", [
    (dict(D=96), m.ERR_ARG), (dict(D=0), m.ERR_ARG), (dict(B=-1), m.ERR_ARG), (dict(Sk=0), m.ERR_ARG),
    (dict(dtype=0), m.ERR_ARG), (dict(stages=0), m.ERR_ARG), (dict(stages=5), m.ERR_ARG),
    (dict(stages=4, fill=0), m.ERR_ARG), (dict(fill=2), m.ERR_ARG), (dict(Q=0), m.ERR_ARG), (dict(O=0), m.ERR_ARG),
    (dict(Q=A0 + 2), m.ERR_ARG), (dict(k=(3 * 90 * 64, 90 * 64, 63)), m.ERR_ARG), (dict(v=(3 * 90 * 64, 90 * 64, 65)), m.ERR_ARG),
    (dict(o=(3 * 100 * 64, 100 * 64, 63)), m.ERR_ARG), (dict(O=A0), m.ERR_ALIAS), (dict(O=B0 + 64), m.ERR_ALIAS),
    (dict(q=(0, 0, 1 << 22)), m.ERR_UNSUPPORTED),
    (dict(Sk=0, Sq=0), m.OK), (dict(B=0, Q=0, K=0, V=0, O=0), m.OK), (dict(Q=A0 + 4), m.OK), (dict(stages=4), m.OK),
])
def test_attention_validation(kw, want):
    st, _ = att(**kw)
    assert st == want
    if want != m.OK:
        a = dict(B=2, H=3, Sq=100, Sk=90, D=64, Q=A0, K=B0, V=B0 + (1 << 24), O=C0, q=None, k=None, v=None, o=None,
                 dtype=1, stages=2, fill=1)
        a.update(kw)
        q = a["q"] or (a["H"] * a["Sq"] * a["D"], a["Sq"] * a["D"], a["D"])
        k = a["k"] or (a["H"] * a["Sk"] * a["D"], a["Sk"] * a["D"], a["D"])
        v = a["v"] or (a["H"] * a["Sk"] * a["D"], a["Sk"] * a["D"], a["D"])
        o = a["o"] or (a["H"] * a["Sq"] * a["D"], a["Sq"] * a["D"], a["D"])
        # the launching entry point refuses the same arguments before any HIP call
        assert m.mgemm_attention(a["B"], a["H"], a["Sq"], a["Sk"], a["D"], a["Q"], *q, a["K"], *k, a["V"], *v,
                                 a["O"], *o, 0.125, a["dtype"], a["stages"], a["fill"], None) == want


@pytest.mark.parametrize("o,want", [
    ((3 * 100 * 64, 0, 64), m.ERR_ALIAS),           # every head writes the same rows
    ((0, 100 * 64, 64), m.ERR_ALIAS),               # every batch writes the same rows
    ((3 * 100 * 64, 100 * 64, 32), m.ERR_ARG),      # rows overlap (ld < head_dim)
    ((3 * 100 * 64, 99 * 64, 64), m.ERR_ALIAS),     # a head's last row is the next head's first
    ((100 * 3 * 64, 64, 3 * 64), m.OK),             # (batch, seq, head, dim) storage
    ((3 * 64, 64, 2 * 3 * 64), m.OK),               # batch innermost of the rows: still disjoint
    ((3 * (100 * 64 + 5) + 7, 100 * 64 + 5, 64), m.OK),  # padded strides
    ((3 * 100 * 64 + 7, 100 * 64 + 5, 64), m.ERR_ALIAS),  # padded heads spill into the next batch
])
def test_attention_refuses_an_output_that_overlaps_itself(o, want):
    st, _ = att(o=o)
    assert st == want
    if want != m.OK:  # refused by the launching entry point too, before any HIP call
        assert m.mgemm_attention(2, 3, 100, 90, 64, A0, 3 * 100 * 64, 100 * 64, 64, B0, 3 * 90 * 64, 90 * 64, 64,
                                 B0 + (1 << 24), 3 * 90 * 64, 90 * 64, 64, C0, *o, 0.125, 1, 2, 1, None) == want


def test_overlapping_tensor_views_reach_the_ld_check():
    """The binding passes a row stride below the width (an expanded row,
    stride 0) through as the leading dimension, so the library refuses the
    view (ld < cols) before any launch; a single row keeps its width."""
    import torch
    row = torch.ones(1, 8)
    assert m._ld(row.expand(5, 8)) == 0
    assert m._ld(torch.ones(6, 8).as_strided((3, 8), (4, 1))) == 4
    assert m._ld(row) == 8 and m._ld(torch.ones(4, 8)[:, :5]) == 8
    assert sg(lda=0) == m.ERR_ARG and sg(lda=4, K=8, M=3) == m.ERR_ARG and sg(ldc=0) == m.ERR_ARG
    assert m.mgemm_tile_copy(5, 8, A0, 0, B0, 8, 2, None) == m.ERR_ARG
    assert m.mgemm_gemm16(5, 8, 8, A0, 0, B0, 8, C0, 8, 1, 2, 1, 0, None) == m.ERR_ARG


def test_attention_rejects_nonfinite_scale():
    for s in (float("nan"), float("inf"), float("-inf")):
        assert m.mgemm_attention(1, 1, 8, 8, 64, A0, 512, 512, 64, B0, 512, 512, 64, B0 + 4096, 512, 512, 64,
                                 C0, 512, 512, 64, s, 1, 2, 1, None) == m.ERR_ARG


def test_attention_plans():
    p = m.plan_attention(16, 16, 4096, 4096, 128)
    assert (p["bm"], p["bn"], p["bk"], p["threads"], p["blocks"]) == (256, 128, 64, 512, 16 * 16 * 16)
    assert p["slices"] == 64 and p["load_bytes"] == 16 and p["lds_bytes"] == 2 * 2 * 64 * 128 * 2
    # one slice: a 64 x 128 K tile and a V tile, 32 KiB = 4 dwordx4 per lane of each of 8 waves
    assert p["loads_per_slice"] == 4 and p["max_vmcnt"] == 0
    assert m.plan_attention(16, 16, 4096, 4096, 128, stages=4)["max_vmcnt"] == 8
    p = m.plan_attention(1, 3, 200, 300, 64, stages=3, fill="sync", align=4)
    assert p["load_bytes"] == 4 and p["blocks"] == 3 * 1 and p["slices"] == 5 and p["loads_per_slice"] == 8
    # the (batch, seq, head, dim) layout keeps 16-byte loads when its strides allow
    st, p = att(B=2, H=4, Sq=64, Sk=64, D=128, q=(64 * 4 * 128, 128, 4 * 128), k=(64 * 4 * 128, 128, 4 * 128),
                v=(64 * 4 * 128, 128, 4 * 128))
    assert st == m.OK and p.load_bytes == 16


def _attn_name(D, bf16, S, piped, W):
    return f"_ZN5mgemm16attention_kernelILi{D}ELb{int(bf16)}ELi{S}ELb{int(piped)}ELi{W}EEEvNS_8AttnArgsE"


@pytest.mark.parametrize("D", [64, 128])
def test_isa_attention(isa, D):
    """The attention kernels score and accumulate on the 16-bit MFMA (two
    products per slice), exponentiate with v_exp_f32, pair lanes with
    v_permlane32_swap, read V through the transposing LDS read, fill the ring
    asynchronously (piped) or through VGPRs (sync), never drain the prefetch
    before the MFMAs and never touch an LDS read's result before its wait."""
    for bf16 in (True, False):
        mfma = "v_mfma_f32_32x32x16_" + ("bf16" if bf16 else "f16")
        per_slice = (D // 16) * 2 + (64 // 16) * (D // 32)
        for S in (1, 2, 3, 4):
            for W in (16, 4):
                for piped in ((True, False) if S < 4 else (True,)):
                    lines = isa[_attn_name(D, bf16, S, piped, W)]
                    body = "\n".join(lines)
                    assert body.count(mfma) >= per_slice, (D, bf16, S, W, piped)
                    assert body.count("v_exp_f32") >= 33 and "v_permlane32_swap" in body
                    assert "ds_read_b64_tr_b16" in body and "ds_read_b128" in body
                    width = "dwordx4" if W == 16 else "dword"
                    if piped:
                        assert re.search(rf"buffer_load_{width} .* lds", body) and "ds_write" not in body
                        if S >= 2:
                            drained, reached = _drain_before_compute(lines, mfma)
                            assert reached and not drained, (D, S, W)
                    else:
                        assert "ds_write" in body and not re.search(r"buffer_load\S* .* lds", body)
                    assert not _early_uses_of_lds_results(lines), (D, bf16, S, W, piped)
                    assert "v_pk_fma_f32" not in body and "v_pk_add_f32" not in body and "v_pk_mul_f32" not in body


def test_isa_no_kernel_spills():
    """No kernel spills registers to scratch: a scratch reload would count in
    vmcnt, and the compiler would then drain the in-flight fills before it.
    Documented exceptions, none ever chosen automatically: the
    warp-specialised ring with the 8 x 8 VALU tile (512-thread blocks cap
    every wave at 256 registers, which that tile and both roles' state
    exceed); the register-staged 16-bit rings of the 256-row tiles with
    4-byte loads (a slice's 32 single-dword loads per register set beside 128
    accumulators), which only misaligned inputs with an explicit synchronous
    fill reach; and the 8-wave 256 x 256 tile with 4-byte loads at two stages
    (three dwords over the 256-VGPR cap of 512-thread blocks), which only an
    explicit tile request with misaligned inputs reaches."""
    if not os.path.exists(m.ISA_PATH):
        pytest.skip("ISA not built")
    txt = open(m.ISA_PATH).read()
    sizes = re.findall(r"^(_ZN5mgemm\w+):.*?; ScratchSize: (\d+)", txt, re.M | re.S)
    names = re.findall(r"^(_ZN5mgemm\w+):", txt, re.M)
    assert len(names) >= 200
    spilled = []
    for name in names:
        i = txt.index("; Kernel info:", txt.index(name + ":"))
        size = int(re.search(r"; ScratchSize: (\d+)", txt[i:i + 600]).group(1))
        allowed = name.startswith("_ZN5mgemm15sgemm_ws_kernelINS_10CfgValu128E") or \
            re.fullmatch(r"_ZN5mgemm12sgemm_kernelINS_\d+CfgH256x(128|256)ILb[01]EEELi[23]ELb0ELi4EEEvNS_8GemmArgsE", name) or \
            re.fullmatch(r"_ZN5mgemm12sgemm_kernelINS_11CfgH256x256ILb[01]EEELi2ELb1ELi4EEEvNS_8GemmArgsE", name)
        if size and not allowed:
            spilled.append((name, size))
    assert not spilled, spilled[:5]
