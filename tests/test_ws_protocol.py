"""CPU model of the warp-specialised ring's protocol (sgemm_ws_kernel).

Four filling waves and four computing waves share S ring slots and two
cumulative LDS counters per slot. The model follows the kernel's steps in the
same order and runs them under random interleavings, with each filling wave's
asynchronous fills completing in order after a random delay (its vmcnt). It
checks that no interleaving deadlocks, that a computing wave only reads a slot
once every filling wave's part of the right slice has landed there, and that
no fill lands in a slot a computing wave has not yet released.
"""
import random

import pytest

NF = NC = 4


class Broken(Exception):
    pass


def run(S, T, seed, *, bug=None):
    rng = random.Random(seed)
    D = S - 2 if S >= 2 else 0
    ready = [0] * S
    consumed = [0] * S
    slot_holds = {}                      # (slot, wave f) -> slice whose part landed there
    inflight = {f: [] for f in range(NF)}  # issued, not yet landed (in order)
    reading = {}

    def filler(f):
        signalled = 0
        for t in range(T):
            slot = t % S
            if t >= S:
                need = NC * (t // S)
                if bug == "no_release_wait":
                    need = 0
                while consumed[slot] < need:
                    yield "wait"
            inflight[f].append(t)        # issue(t, slot)
            if t >= D:
                while len(inflight[f]) > (D if bug != "loose_vmcnt" else D + 1):
                    yield "wait"         # s_waitcnt vmcnt(D * L)
                ready[signalled % S] += 1
                signalled += 1
            yield "step"
        while inflight[f]:
            yield "wait"
        while signalled < T:
            ready[signalled % S] += 1
            signalled += 1
            yield "step"

    def computer(c):
        for t in range(T):
            slot = t % S
            need = NF * (t // S + 1)
            if bug == "early_compute":
                need -= 1
            while ready[slot] < need:
                yield "wait"
            reading[c] = slot
            for f in range(NF):
                if slot_holds.get((slot, f)) != t:
                    raise Broken(f"compute wave {c} read slice {slot_holds.get((slot, f))} for {t} (fill wave {f})")
            yield "step"                 # the reads take time
            for f in range(NF):
                if slot_holds.get((slot, f)) != t:
                    raise Broken(f"slot {slot} overwritten while wave {c} read slice {t}")
            del reading[c]
            consumed[slot] += 1
            yield "step"

    agents = {("f", f): filler(f) for f in range(NF)}
    agents.update({("c", c): computer(c) for c in range(NC)})
    live = dict(agents)
    idle_rounds = 0
    while live or any(inflight.values()):
        # a random pending fill may land (in order per filling wave)
        if rng.random() < 0.5:
            ws = [f for f in range(NF) if inflight[f]]
            if ws:
                f = rng.choice(ws)
                u = inflight[f].pop(0)
                for c, sl in reading.items():
                    if sl == u % S:
                        raise Broken(f"fill of slice {u} landed in slot {sl} while wave {c} read it")
                slot_holds[(u % S, f)] = u
                idle_rounds = 0
                continue
        if not live:
            continue
        key = rng.choice(list(live))
        try:
            r = next(live[key])
            idle_rounds = 0 if r == "step" else idle_rounds + 1
        except StopIteration:
            del live[key]
            idle_rounds = 0
        if idle_rounds > 5000 and not any(inflight.values()):
            raise Broken(f"deadlock: {sorted(live)} waiting, ready={ready} consumed={consumed}")


@pytest.mark.parametrize("S", [1, 2, 3, 4, 5, 6])
def test_protocol_random_interleavings(S):
    for T in (1, 2, 3, S, S + 1, 2 * S + 3, 17):
        for seed in range(25):
            run(S, T, seed * 1000 + T)


@pytest.mark.parametrize("bug", ["no_release_wait", "loose_vmcnt", "early_compute"])
def test_model_catches_planted_protocol_bugs(bug):
    caught = False
    for S in (2, 3, 4):
        for seed in range(60):
            try:
                run(S, 12, seed, bug=bug)
            except Broken:
                caught = True
                break
        if caught:
            break
    assert caught, bug
