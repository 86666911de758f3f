"""Host model of the persistent 256-row GEMM's run-time tile claims.

On one XCD, the workgroups of the grid (g8 of them) each start with their own
slot j = b and then claim j = g8 + c from a counter, where c is the counter's
value before an atomic increment, until j passes the nx slots; the claim that
returns nx - 1 puts the counter back to zero. The kernel issues a claim after
its current tile's last MFMA step and acts on it after the tile. This model
runs the workgroups in random interleavings (each step: one workgroup takes
its next action) and checks that every slot is processed exactly once, that
a launch makes exactly nx claims, and that the counter ends at zero, also
when it is reused by the next launch.
"""
import random

import pytest


def run_launch(g8, nx, counter, rng):
    """One launch on one XCD; returns (slots processed in order, claims made,
    counter after the launch)."""
    assert counter[0] == 0, "a launch must find its counter at zero"
    done = []
    claims = 0
    # per workgroup: current slot (None once finished)
    cur = [b if b < nx else None for b in range(g8)]
    while any(c is not None for c in cur):
        b = rng.choice([i for i, c in enumerate(cur) if c is not None])
        done.append(cur[b])             # process the tile of slot cur[b]
        c = counter[0]                  # atomicAdd returns the old value
        counter[0] += 1
        claims += 1
        if c == nx - 1:
            counter[0] = 0              # the last claim of the launch
        j = g8 + c
        cur[b] = j if j < nx else None
    return done, claims, counter[0]


@pytest.mark.parametrize("g8,nx", [(1, 1), (1, 7), (32, 1), (32, 31), (32, 32), (32, 33), (32, 460), (5, 64),
                                   (32, 0)])
def test_every_slot_once_and_counter_back_to_zero(g8, nx):
    rng = random.Random(g8 * 1000 + nx)
    counter = [0]
    for _ in range(20):                 # launches in a row reuse the counter
        done, claims, after = run_launch(g8, nx, counter, rng)
        assert sorted(done) == list(range(nx))
        assert claims == nx
        assert after == 0
