"""The flag-ordered persistent ring's waiting rule, simulated on the CPU.

The kernel (ring_persistent_flags_kernel) gives workgroup b of a grid of G
the tiles b, b + G, ... of every step; tile t = r * T + seg is rank r's
piece seg of its chunk (T tiles per chunk, N * T tiles in all).  After a
step a workgroup publishes the number of steps it has completed; before
step s it waits until the workgroup holding the upstream tile
(r - 1, seg) of each of its tiles has published s, or, with more than 64
tiles per step, until every workgroup has.

This restates that rule in Python and runs the grid under an adversarial
scheduler that always picks a random runnable workgroup.  It checks what the
kernel's comments claim: no schedule deadlocks (the workgroup with the
lowest next step can always run), and every tile's step s starts only after
the tile it receives from has finished step s - 1, which is what the ring
needs ([RING] §1: a rank's step consumes what its upstream neighbour sent
at the step before).  The GPU parity tests check the kernel itself.
"""

import random

import pytest


def upstream_blocks(b, g, n, tpc, whole_grid):
    """The workgroups block b waits on before a step (the kernel's
    flags_upstream and flags_wait, restated)."""
    ntiles = n * tpc
    if whole_grid:
        return {w for w in range(g) if w != b}
    ups = set()
    for t in range(b, ntiles, g):
        u = (t - tpc) % ntiles  # tile (r-1, seg)
        w = u % g
        if w != b:
            ups.add(w)
    return ups


def simulate(n, tpc, g, nsteps, first_step, seed, force_whole_grid=False):
    """Run the grid to completion (or to a deadlock) under a scheduler that
    always picks a random runnable workgroup; a workgroup runs one whole
    step at a time and then publishes it.  Returns each workgroup's next
    step, and the event index at which every (tile, step) started and
    finished."""
    ntiles = n * tpc
    assert g <= ntiles
    blocks = range(g)
    whole = {b: force_whole_grid or len(range(b, ntiles, g)) > 64 for b in blocks}
    ups = {b: upstream_blocks(b, g, n, tpc, whole[b]) for b in blocks}
    dependents = {b: [] for b in blocks}
    for b in blocks:
        for w in ups[b]:
            dependents[w].append(b)
    flag = [0] * g                         # published: steps completed (the kernel's flag word)
    next_step = [first_step] * g
    done_at, started_at = {}, {}
    clock = 0
    rng = random.Random(seed)

    def runnable(b):
        s = next_step[b]
        return s < nsteps and (s == first_step or all(flag[w] >= s for w in ups[b]))

    ready = {b for b in blocks if runnable(b)}
    while ready:
        b = rng.choice(sorted(ready)) if len(ready) < 64 else rng.choice(tuple(ready))
        s = next_step[b]
        clock += 1
        for t in range(b, ntiles, g):
            started_at[(t, s)] = clock
        clock += 1
        for t in range(b, ntiles, g):
            done_at[(t, s)] = clock
        flag[b] = s + 1                    # flags_publish: after every tile of the step
        next_step[b] = s + 1
        for x in [b] + dependents[b]:
            if runnable(x):
                ready.add(x)
            else:
                ready.discard(x)
    return next_step, started_at, done_at


CASES = [
    # n, tiles per chunk, grid, steps, first step
    (2, 1, 2, 2, 0),
    (3, 1, 3, 4, 0),
    (8, 128, 256, 14, 0),        # N = 8, M = 2^24 float32: 4 tiles per workgroup
    (8, 512, 256, 14, 0),        # N = 8, M = 2^26: every upstream tile is the workgroup's own
    (8, 100, 256, 14, 0),        # 100 tiles per chunk: 3 or 4 tiles per workgroup
    (16, 3, 40, 30, 0),
    (64, 4, 256, 126, 0),
    (256, 1, 256, 510, 0),       # N = 256, M = 2^22 float32
    (5, 7, 13, 5, 1),            # an in-place AllGather: its placement step is skipped
    (8, 2048, 256, 14, 0),       # 64 tiles per workgroup: still the upstream rule
    (8, 2056, 256, 14, 0),       # up to 65 tiles per workgroup: the whole grid for some
]


@pytest.mark.parametrize("n,tpc,g,nsteps,first", CASES)
@pytest.mark.parametrize("seed", [1, 2])
def test_no_deadlock_and_every_step_follows_its_upstream(n, tpc, g, nsteps, first, seed):
    next_step, started, done = simulate(n, tpc, g, nsteps, first, seed)
    assert all(s == nsteps for s in next_step), "a workgroup never reached the last step"
    ntiles = n * tpc
    for t in range(ntiles):
        up = (t - tpc) % ntiles
        for s in range(first + 1, nsteps):
            assert done[(up, s - 1)] < started[(t, s)], (t, s)


@pytest.mark.parametrize("seed", [3, 4])
def test_whole_grid_wait_is_also_safe(seed):
    next_step, started, done = simulate(8, 24, 16, 14, 0, seed, force_whole_grid=True)
    assert all(s == 14 for s in next_step)
    for t in range(8 * 24):
        for s in range(1, 14):
            assert done[((t - 24) % (8 * 24), s - 1)] < started[(t, s)]


def test_a_rule_without_the_upstream_wait_is_caught():
    """The check has teeth: waiting on the downstream neighbour instead
    (tile + T) lets some tile start a step before its upstream finished."""
    n, tpc, g, nsteps = 8, 3, 8, 14
    ntiles = n * tpc

    def wrong_upstream(b, *_):
        return {((t + tpc) % ntiles) % g for t in range(b, ntiles, g)} - {b}

    saved = globals()["upstream_blocks"]
    globals()["upstream_blocks"] = wrong_upstream
    try:
        caught = False
        for seed in range(20):
            next_step, started, done = simulate(n, tpc, g, nsteps, 0, seed)
            if any(s < nsteps for s in next_step):
                caught = True
                break
            if any(done[((t - tpc) % ntiles, s - 1)] >= started[(t, s)]
                   for t in range(ntiles) for s in range(1, nsteps)):
                caught = True
                break
        assert caught
    finally:
        globals()["upstream_blocks"] = saved
