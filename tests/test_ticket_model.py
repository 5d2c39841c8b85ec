"""A host-side model of how gla_fwd's workgroups take their work (no GPU).

The bf16 forward kernel's workgroup i runs on XCD i % 8 and takes a ticket
from that XCD's counter with an atomic increment that wraps at gsize - 1
(gsize = workgroups per XCD); a ticket t >= gsize reads as gsize - 1; ticket
t of XCD x is segment t % nseg of unit x * per_xcd + t // nseg (units past
the last one are padding).  With one segment per scan no workgroup waits for
another and the kernel takes no ticket: t = i // 8, the launch index, and the
counters are never touched.  This model replays that logic exactly as the
kernel states it, over counters holding any value (zero-filled, a rotation,
byte-pattern garbage) and random start orders, and checks that

  * every (unit, segment) is taken by exactly one workgroup -- so no o rows
    are skipped and no segment is left without its workgroup, whatever the
    workspace held;
  * a launch leaves each counter where it found it, or (after garbage) at
    gsize - 1, so later launches stay bijective;
  * with zero-filled counters, every segment starts after all earlier
    segments of its scan (the order the waits rely on).
"""
import random

import pytest

MASK = 0xFFFFFFFF


def atomic_inc(mem, idx, val):
    """The hardware's wrapping increment: old = mem; mem = old >= val ? 0 : old + 1."""
    old = mem[idx]
    mem[idx] = 0 if old >= val else (old + 1) & MASK
    return old


def launch(counters, units, nseg, rng):
    per_xcd = (units + 7) // 8
    grid = 8 * per_xcd * nseg
    gsize = grid // 8
    arrival = list(range(grid))
    rng.shuffle(arrival)
    taken = {}
    start = {}
    for pos, wg in enumerate(arrival):
        xcd = wg & 7
        if nseg == 1:
            t = wg >> 3
        else:
            t = atomic_inc(counters, xcd, gsize - 1)
            if t >= gsize:
                t = gsize - 1
        unit = xcd * per_xcd + t // nseg
        seg = t % nseg
        if unit >= units:
            continue
        assert (unit, seg) not in taken, f"(unit {unit}, segment {seg}) taken twice"
        taken[(unit, seg)] = wg
        start[(unit, seg)] = pos
    return taken, start, gsize


@pytest.mark.parametrize("units,nseg", [(128, 2), (16, 16), (192, 1), (12, 21), (8, 8), (3, 5), (257, 1)])
@pytest.mark.parametrize("init", ["zero", "rotated", "garbage", "max"])
def test_tickets_are_a_bijection(units, nseg, init):
    rng = random.Random(units * 31 + nseg)
    per_xcd = (units + 7) // 8
    gsize = per_xcd * nseg
    counters = {"zero": [0] * 8,
                "rotated": [rng.randrange(gsize) for _ in range(8)],
                "garbage": [0x5A5A5A5A] * 8,
                "max": [MASK] * 8}[init]
    before = list(counters)
    for rep in range(3):
        taken, start, gs = launch(counters, units, nseg, rng)
        assert gs == gsize
        assert set(taken) == {(u, s) for u in range(units) for s in range(nseg)}
        for x in range(8):
            if nseg == 1 or before[x] < gsize:
                assert counters[x] == before[x]
            else:
                assert counters[x] == gsize - 1
        before = list(counters)
        if init == "zero":
            for (u, s), pos in start.items():
                for s2 in range(s):
                    assert start[(u, s2)] < pos, "a segment started before an earlier one of its scan"
