"""Host model of the fused step's per-XCD queue: every dependency can be met.

The persistent launch of tp_mlp_step drains, on each XCD, a queue of units
over the XCD's own row blocks in this order: fc1 forward tiles (F1) of every
shard, fc2 forward partial tiles (F2), fc2 data-gradient tiles (D2), the
forward sum slices (S1), fc1 data-gradient partial tiles (D1) and the dX sum
slices (S2). A unit waits for a count of completed units of its row block:

  F2(i, j)  needs all n1 F1 tiles of shard i, row block j (its A operand Y_i)
  D2(i, j)  needs the same (it reads U_i in its GeLU' epilogue)
  S1(j)     needs all p * n2 F2 tiles of row block j
  D1(i, j)  needs all n1 D2 tiles of shard i, row block j (its A operand dU_i)
  S2(j)     needs all p * n2 D1 tiles of row block j

These checks model that queue on the host. Every unit depends only on units
with smaller tickets, so blocks that take tickets in order never wait on a
unit no block holds. An event simulation then drains the queue with any
number of resident blocks and random unit durations and finds no deadlock.
"""
import heapq
import random

import pytest

PHASES = ("F1", "F2", "D2", "S1", "D1", "S2")
# A launch runs the whole queue, or only its forward or its backward units (in
# the same order); in a backward-only launch fc2's data gradient (D2) waits for
# nothing, fc1's forward having run in an earlier launch. When the weight
# gradients follow in the same call, the launch leaves the dX sum (S2) to
# their launch.
QUEUES = {"step": PHASES, "fwd": ("F1", "F2", "S1"), "bwd": ("D2", "D1", "S2"),
          "step_no_dx_sum": PHASES[:-1], "bwd_no_dx_sum": ("D2", "D1")}


def queue(p, R, n1, n2, SS, phases=PHASES):
    """Units of one XCD in ticket order: (kind, shard, row block, column)."""
    units = []
    for kind in phases:
        if kind in ("F1", "D2"):
            units += [(kind, i, j, n) for i in range(p) for j in range(R) for n in range(n1)]
        elif kind in ("F2", "D1"):
            units += [(kind, i, j, n) for i in range(p) for j in range(R) for n in range(n2)]
        else:
            units += [(kind, 0, j, n) for j in range(R) for n in range(SS)]
    return units


def producers(unit, p, n1, n2, d2_waits=True):
    """The counter a unit waits for: (kind produced, shards, row block), needed count."""
    kind, i, j, _ = unit
    if kind == "D2" and not d2_waits:
        return None, 0
    if kind in ("F2", "D2"):
        return ("F1", (i,), j), n1
    if kind == "S1":
        return ("F2", tuple(range(p)), j), p * n2
    if kind == "D1":
        return ("D2", (i,), j), n1
    if kind == "S2":
        return ("D1", tuple(range(p)), j), p * n2
    return None, 0


# shapes of the workloads' queues: (p, row blocks per XCD, n1, n2, sum slices)
SHAPES = [
    (2, 2, 12, 6, 16),    # GPT-2-small MLP, 256 x 128 tiles
    (4, 3, 8, 8, 16),     # the ~350M layer's MLP, 256 x 128 tiles
    (2, 4, 12, 6, 8),     # GPT-2-small MLP, 128 x 128 tiles
    (1, 1, 1, 1, 8),      # the smallest queue
    (3, 2, 2, 5, 8),
]


@pytest.mark.parametrize("which", sorted(QUEUES))
@pytest.mark.parametrize("p,R,n1,n2,SS", SHAPES)
def test_every_dependency_has_an_earlier_ticket(p, R, n1, n2, SS, which):
    units = queue(p, R, n1, n2, SS, QUEUES[which])
    tickets = {u: t for t, u in enumerate(units)}
    size = {"F1": p * R * n1, "D2": p * R * n1, "F2": p * R * n2, "D1": p * R * n2,
            "S1": R * SS, "S2": R * SS}
    assert len(tickets) == len(units) == sum(size[k] for k in QUEUES[which])
    for t, u in enumerate(units):
        (src, need) = producers(u, p, n1, n2, d2_waits=not which.startswith("bwd"))
        if src is None:
            continue
        kind, shards, j = src
        deps = [v for v in units if v[0] == kind and v[1] in shards and v[2] == j]
        assert len(deps) == need, (u, len(deps), need)
        assert max(tickets[v] for v in deps) < t, u


def drain(units, p, n1, n2, blocks, rng, d2_waits=True):
    """Event simulation: `blocks` blocks take tickets in order, wait for their
    unit's count, run it for a random time, count it done. Returns the number
    of completed units (all of them unless the queue deadlocks)."""
    done = {}
    nxt = 0
    clock = 0.0
    running = []  # (finish time, unit)
    waiting = []  # units whose count is not complete yet, each holding a block
    free = blocks
    finished = 0

    def ready(u):
        src, need = producers(u, p, n1, n2, d2_waits)
        if src is None:
            return True
        kind, shards, j = src
        return sum(done.get((kind, i, j), 0) for i in shards) >= need

    while True:
        # start every waiting unit whose count is complete
        still = []
        for u in waiting:
            if ready(u):
                heapq.heappush(running, (clock + rng.uniform(0.5, 2.0), u))
            else:
                still.append(u)
        waiting = still
        # free blocks take the next tickets
        while free > 0 and nxt < len(units):
            u = units[nxt]
            nxt += 1
            free -= 1
            if ready(u):
                heapq.heappush(running, (clock + rng.uniform(0.5, 2.0), u))
            else:
                waiting.append(u)
        if not running:
            return finished
        clock, u = heapq.heappop(running)
        key = (u[0], u[1], u[2])
        done[key] = done.get(key, 0) + 1
        finished += 1
        free += 1


@pytest.mark.parametrize("which", sorted(QUEUES))
@pytest.mark.parametrize("p,R,n1,n2,SS", SHAPES)
@pytest.mark.parametrize("blocks", [1, 2, 3, 7, 32, 64])
def test_queue_drains_with_any_number_of_blocks(p, R, n1, n2, SS, blocks, which):
    units = queue(p, R, n1, n2, SS, QUEUES[which])
    rng = random.Random(1000 * blocks + p * 97 + R)
    assert drain(units, p, n1, n2, blocks, rng, d2_waits=not which.startswith("bwd")) == len(units)


def test_model_detects_a_queue_that_could_deadlock():
    # the same model on a queue with the sums moved ahead of the products they
    # read: one block takes the first sum's ticket and waits for ever
    p, R, n1, n2, SS = 2, 1, 2, 2, 2
    units = queue(p, R, n1, n2, SS)
    bad = [u for u in units if u[0] == "S1"] + [u for u in units if u[0] != "S1"]
    assert drain(bad, p, n1, n2, 1, random.Random(0)) < len(bad)
