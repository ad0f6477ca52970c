"""The row kernel's dynamic tail, as a protocol: the grid's last `takers`
workgroups each claim from one count with a wrapping increment (the
semantics of atomicInc: old >= limit wraps to 0, else old + 1) at their
start, run their own unit, and then, while the claim in hand is below
`tail`, run unit tail_first + claim and claim again.  Simulated on the CPU
over random interleavings of the takers, including claims that come back
past the tail while others are still running, it must give every tail
unit to exactly one workgroup, make exactly tail + takers claims, and
leave the count at 0 for the next launch."""
from __future__ import annotations

import numpy as np
import pytest


def atomic_inc(cell, limit):
    old = cell[0]
    cell[0] = 0 if old >= limit else old + 1
    return old


def run_launch(rng, tail, takers, tail_first, cell):
    """One launch: takers interleaved at random; returns the units each ran."""
    limit = tail + takers - 1
    # each taker: [state, claim in hand, units run]; state 0 = own unit next
    ts = [{"claim": atomic_inc(cell, limit), "ran": [tail_first - takers + i], "done": False}
          for i in range(takers)]
    claims = takers
    live = list(range(takers))
    while live:
        i = live[rng.integers(len(live))]
        t = ts[i]
        c = t["claim"]
        if c >= tail:
            t["done"] = True
            live.remove(i)
            continue
        t["ran"].append(tail_first + c)
        t["claim"] = atomic_inc(cell, limit)
        claims += 1
    return ts, claims


@pytest.mark.parametrize("tail,takers", [(256, 256), (128, 256), (512, 256), (8, 8), (24, 16),
                                         (1000, 7)])
def test_every_tail_unit_once_and_count_back_at_zero(tail, takers):
    rng = np.random.default_rng(tail * 1000 + takers)
    units = 4 * takers + tail
    tail_first = units - tail
    cell = [0]
    for launch in range(5):               # the count carries over between launches
        ts, claims = run_launch(rng, tail, takers, tail_first, cell)
        ran = sorted(u for t in ts for u in t["ran"][1:])
        assert ran == list(range(tail_first, units)), "a tail unit run twice or never"
        assert claims == tail + takers
        assert cell[0] == 0, "count not back at 0 after the launch"


def test_a_count_left_nonzero_is_caught():
    # the invariant the launches rely on: a count that does not start at 0
    # hands out a tail unit twice or skips one (the header makes the caller
    # zero the array once; every call then leaves it at 0)
    rng = np.random.default_rng(5)
    tail, takers = 64, 32
    tail_first = 200
    cell = [17]
    ts, _ = run_launch(rng, tail, takers, tail_first, cell)
    ran = sorted(u for t in ts for u in t["ran"][1:])
    assert ran != list(range(tail_first, tail_first + tail))
