"""Host replay of the GEMM main loop's LDS ring schedule (no GPU).

The kernel streams operand tiles into a ring of 5 LDS slots by DMA and publishes them
with one workgroup barrier per 32-deep step. Its correctness rests on bookkeeping that no
GPU test can observe directly: which loads a `s_waitcnt vmcnt(N)` has retired (loads
retire in issue order), that every slot is rewritten only after the barrier that follows
its last read, and, in the persistent schedule, that the next tile's first steps and the
epilogue's LDS areas never share a slot. This file restates the schedule step by step,
as the kernel issues it, at the granularity of one DMA instruction per thread:

  prologue  W0; X0, X1 (paired); W1; W2; X2, X3 (paired); wait 9; barrier
  step kt   read X blocks 4..7 of kt | W of kt+3 | wait 5 (odd kt) or 8 (even kt);
            barrier | read W and X blocks 0..3 of kt+1; odd kt: X of kt+3 and kt+4
  end       wait 0; barrier; epilogue in the three slots after the next tile's two
  resume    W2; X2, X3 (paired) of the next tile, ring rotated by KT mod 5

and replays it for many depths and tile sequences, asserting the invariants. Planted
schedule mistakes (a wait one load too short, loads issued a step late or shifted by a
step, an epilogue area on a prefetched slot) must make it fail.

Every vector-memory instruction of the loop is counted by the waits, whatever its
destination: the DMA loads into LDS, and any load whose data returns into a VGPR. Such a
load writes its register when the data arrives, not when it issues; the hardware does
not hold back other writers of that register, so it must stay reserved until a wait has
retired the load. A load issued from inline asm with the register as an asm output is
done, as far as the compiler knows, when the asm statement ends: the register may be
reassigned right away (to an address, say) and then be overwritten by the late data. An
L2 prefetch of future depth steps written that way (one 4-byte load per lane into a
dummy "+v" operand, its loads counted in the waits) faulted the GPU; the model shows the
cause: the waits retire the prefetch loads a step later, long after their register was
given back. The main loop itself issues no load with a register destination."""
import itertools

import pytest

NS = 5     # LDS slots
NEXT = 2   # depth steps of the next tile loaded during the current tile's tail


class ScheduleError(AssertionError):
    pass


def check(cond, msg):
    if not cond:
        raise ScheduleError(msg)


class Ring:
    """One thread's view; every thread runs the same schedule, and a barrier makes what
    each thread has waited for visible to all."""

    def __init__(self):
        self.pending = []                        # DMA instructions in flight, issue order
        self.landed = {p: {} for p in range(NS)}  # slot -> {(half, j): (tile, step) or 'zero'}
        self.epoch = 0                           # barriers passed
        self.last_read = {p: -1 for p in range(NS)}
        self.retired_epoch = {}                  # (slot, tile, step, half, j) -> epoch it landed in

    def barrier(self):
        self.epoch += 1

    def wait(self, n):
        while len(self.pending) > n:
            ld = self.pending.pop(0)
            if ld["slot"] is None:     # a load into a register: nothing lands in LDS
                continue
            self.landed[ld["slot"]][(ld["half"], ld["j"])] = ld["what"]
            self.retired_epoch[(ld["slot"], ld["what"], ld["half"], ld["j"])] = self.epoch

    def issue(self, slot, what, half, j):
        check(self.last_read[slot] < self.epoch,
              f"DMA into slot {slot} ({what}) in the barrier interval of its last read")
        self.pending.append(dict(slot=slot, what=what, half=half, j=j))

    def issue_to_vgpr(self, reg):
        """A load whose data returns into VGPR `reg` (counted by the waits like a DMA)."""
        self.pending.append(dict(slot=None, reg=reg))

    def release(self, reg):
        """The compiler may hand `reg` to another value from here on: no load into it may
        still be in flight."""
        check(all(ld.get("reg") != reg for ld in self.pending),
              f"VGPR {reg} given back while a load into it is in flight")

    def retire_reg(self, reg):
        """The wait a compiler inserts before it reuses `reg`: every load into it retired."""
        last = max((i for i, ld in enumerate(self.pending) if ld.get("reg") == reg), default=-1)
        self.wait(len(self.pending) - 1 - last)

    def wait_for_step(self, what):
        """The shortest wait that retires every pending load of step `what`: the vmcnt a
        schedule with extra loads would have to use."""
        last = max((i for i, ld in enumerate(self.pending) if ld["slot"] is not None and ld["what"] == what),
                   default=-1)
        self.wait(len(self.pending) - 1 - last)

    def read(self, slot, what, halves):
        """A read of step `what` needs every thread's loads of it retired before the last
        barrier (each thread waited for its own, then the barrier)."""
        for half in halves:
            for j in (0, 1):
                got = self.landed[slot].get((half, j))
                check(got == what, f"read of {what} {half}{j} from slot {slot}, which holds {got}")
                check(self.retired_epoch[(slot, what, half, j)] < self.epoch,
                      f"read of {what} {half}{j} before the barrier that publishes it")
        self.last_read[slot] = self.epoch

    def touch(self, slot):
        """A read of a slot whose contents are not used (the last step reads one past the end)."""
        self.last_read[slot] = self.epoch


def run(KTs, waits=(8, 5), prologue_wait=9, pair_ahead=3, w_ahead=3, epi_shift=NEXT, prefetch=None):
    """Replay one workgroup walking tiles of depths KTs (a single entry: the per-tile
    schedule). waits = (even step, odd step) vmcnt limits; step kt loads W of kt + w_ahead
    and, on odd steps, X of kt + pair_ahead and the step after it.

    prefetch (not in the kernel: the rejected variant and its repair) adds one load per
    step into a VGPR after the barrier, with every wait lengthened to retire exactly the
    loads it needs: "asm" gives the register back right after the issuing statement;
    "reserved" keeps it until a wait has retired the load (the wait a compiler inserts
    before it reuses a register that a tracked load writes)."""
    R = Ring()
    rot = 0

    def phys(logical):
        return (logical + rot) % NS

    def load(tile, KT, has_next, logical, kk, half, j):
        if has_next and KT <= kk < KT + NEXT:
            what = (tile + 1, kk - KT)
        elif kk >= KT:
            what = "zero"
        else:
            what = (tile, kk)
        R.issue(phys(logical), what, half, j)

    def pair(tile, KT, has_next, kk):  # X of kk and kk+1, the two row halves back to back
        for j in (0, 1):
            load(tile, KT, has_next, kk % NS, kk, "X", j)
            load(tile, KT, has_next, (kk + 1) % NS, kk + 1, "X", j)

    def wload(tile, KT, has_next, kk):
        for j in (0, 1):
            load(tile, KT, has_next, kk % NS, kk, "W", j)

    KT = KTs[0]
    has_next = len(KTs) > 1
    wload(0, KT, has_next, 0)
    pair(0, KT, has_next, 0)
    wload(0, KT, has_next, 1)
    wload(0, KT, has_next, 2)
    pair(0, KT, has_next, 2)
    R.wait(prologue_wait)
    R.barrier()
    for tile, KT in enumerate(KTs):
        has_next = tile + 1 < len(KTs)
        R.read(phys(0), (tile, 0), "WX")            # W and X blocks 0..3 of step 0
        for kt in range(KT):
            S = kt % NS
            odd = kt % 2 == 1
            R.read(phys(S), (tile, kt), "X")        # X blocks 4..7 of kt
            wload(tile, KT, has_next, kt + w_ahead)  # W of kt+3 into the slot of kt-2
            if prefetch:
                R.wait_for_step((tile, kt + 1) if kt + 1 < KT else None)
            else:
                R.wait(waits[1] if odd else waits[0])
            R.barrier()
            nxt = phys((S + 1) % NS)
            if kt + 1 < KT:
                R.read(nxt, (tile, kt + 1), "WX")
            else:
                R.touch(nxt)
            if odd:
                pair(tile, KT, has_next, kt + pair_ahead)  # X of kt+3, kt+4 into the slots of kt-2, kt-1
            if prefetch == "reserved":
                R.retire_reg("pf")                  # the register is reused: its last load is waited for
                R.release("pf")
            if prefetch:
                R.issue_to_vgpr("pf")               # an L2 prefetch of a later step
                if prefetch == "asm":
                    R.release("pf")                 # the asm output is dead to the compiler
        R.wait(0)
        if prefetch:
            R.release("pf")
        R.barrier()
        e = (rot + KT % NS + epi_shift) % NS
        epi = {e, (e + 1) % NS, (e + 2) % NS}
        nxt_slots = {(rot + KT) % NS, (rot + KT + 1) % NS}
        check(not (epi & nxt_slots), f"epilogue areas {epi} overlap the next tile's steps {nxt_slots}")
        if has_next:
            for s, p in enumerate(sorted(nxt_slots, key=lambda p: (p - rot - KT) % NS)):
                for half, j in itertools.product("XW", (0, 1)):
                    check(R.landed[p].get((half, j)) == (tile + 1, s),
                          f"next tile's step {s} {half}{j} missing from slot {p}")
        for p in epi:
            check(R.last_read[p] < R.epoch, f"epilogue area {p} still read")
            R.touch(p)
            R.landed[p] = {}
        if not has_next:
            break
        rot = (rot + KT) % NS
        R.barrier()
        wload(tile + 1, KTs[tile + 1], tile + 2 < len(KTs), 2)
        pair(tile + 1, KTs[tile + 1], tile + 2 < len(KTs), 2)
    return True


def test_per_tile_schedule_every_depth():
    for KT in range(1, 70):
        run([KT])


@pytest.mark.parametrize("n", [2, 3, 5])
def test_persistent_schedule_every_depth(n):
    # the persistent schedule needs at least 4 depth steps per tile
    for KT in range(4, 60):
        run([KT] * n)


def test_persistent_schedule_mixed_depths():
    for KTs in ([4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14], [13, 4, 9, 5, 448, 4, 17], [5, 4, 7, 4, 9, 6]):
        run(KTs)


@pytest.mark.parametrize("plant", [
    dict(waits=(8, 6)),          # odd steps: one load too many left in flight
    dict(waits=(9, 5)),          # even steps: the same
    dict(prologue_wait=10),      # prologue: step 0 not waited for
    dict(pair_ahead=2),          # X pairs issued a step late: not landed when published
    dict(w_ahead=2),             # W issued a step late
    dict(pair_ahead=4),          # X pairs shifted a step: step 4's X is never loaded
    dict(epi_shift=0),           # epilogue on the slots of the next tile's first steps
])
def test_planted_schedule_mistakes_fail(plant):
    with pytest.raises(ScheduleError):
        for KTs in ([9], [12, 12], [7, 10, 5], [4] * 4, [13] * 3):
            run(KTs, **plant)


def test_register_destination_loads():
    """An L2 prefetch into a register, every wait lengthened to count it: with the
    register kept until a wait retires the load the schedule holds; with the register
    given back at the end of the issuing asm statement (the rejected variant) a later
    load lands in a register that may already hold something else."""
    for KTs in ([1], [2], [9], [30], [12, 12], [7, 10, 5]):
        run(KTs, prefetch="reserved")
    for KTs in ([9], [12, 12]):
        with pytest.raises(ScheduleError, match="in flight"):
            run(KTs, prefetch="asm")
