"""The flag-ordered persistent ring's waiting rule, simulated on the CPU.

The kernel (ring_persistent_flags_kernel) gives workgroup b of a grid of G
the tiles f(b), f(b) + G, ... of every step, where f is the identity or,
with the XCD placement, f(b) = (b mod 8)·G/8 + b/8; tile t = r * T + seg is
rank r's piece seg of its chunk (T tiles per chunk, N * T tiles in all).
After a step a workgroup publishes the number of steps it has completed;
before step s it waits until the workgroups holding the upstream tiles
(r - 1, seg) of its own tiles have published s.  The kernel finds those
workgroups without walking its tiles: the holder of a tile depends only on
the tile's index modulo G, so the upstream tiles of b's tiles from T on all
sit on one workgroup and those of its tiles below T on one other.

This restates that rule in Python, checks it against the per-tile
definition of the upstream workgroups, and runs the grid under an
adversarial scheduler that always picks a random runnable workgroup.  It
checks what the kernel's comments claim: no schedule deadlocks (the
workgroup with the lowest next step can always run), and every tile's step
s starts only after the tile it receives from has finished step s - 1,
which is what the ring needs ([RING] §1: a rank's step consumes what its
upstream neighbour sent at the step before).  The GPU parity tests check
the kernel itself.
"""

import random

import pytest


def first_tile(b, g, xcd_map):
    return (b % 8) * (g // 8) + b // 8 if xcd_map else b


def holder(t, g, xcd_map):
    """The workgroup holding tile t: the inverse of first_tile on t mod G."""
    m = t % g
    return (m % (g // 8)) * 8 + m // (g // 8) if xcd_map else m


def tiles_of(b, g, ntiles, xcd_map):
    return range(first_tile(b, g, xcd_map), ntiles, g)


def upstream_by_tile(b, g, n, tpc, xcd_map=False):
    """The definition: the holders of the upstream tile of each of b's tiles,
    b itself left out."""
    ntiles = n * tpc
    return {holder((t - tpc) % ntiles, g, xcd_map) for t in tiles_of(b, g, ntiles, xcd_map)} - {b}


def upstream_blocks(b, g, n, tpc, xcd_map=False):
    """The kernel's rule (flags_upstream), restated: at most two workgroups,
    from the offsets the host reduces modulo G."""
    ntiles = n * tpc
    f = first_tile(b, g, xcd_map)
    up_back, up_wrap, ntiles_mod = (g - tpc % g) % g, (ntiles - tpc) % g, ntiles % g
    last = ntiles - 1 - (ntiles_mod + g - 1 - f) % g          # b's last tile
    ups = set()
    if last >= tpc:                                          # some tile is not rank 0's
        ups.add(holder(f + up_back, g, xcd_map))
    if f < tpc:                                              # some tile is rank 0's
        ups.add(holder(f + up_wrap, g, xcd_map))
    return ups - {b}


def simulate(n, tpc, g, nsteps, first_step, seed, xcd_map=False, rule=None):
    """Run the grid to completion (or to a deadlock) under a scheduler that
    always picks a random runnable workgroup; a workgroup runs one whole
    step at a time and then publishes it.  Returns each workgroup's next
    step, and the event index at which every (tile, step) started and
    finished."""
    ntiles = n * tpc
    assert g <= ntiles and (not xcd_map or g % 8 == 0)
    blocks = range(g)
    rule = rule or upstream_blocks
    ups = {b: rule(b, g, n, tpc, xcd_map) for b in blocks}
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
        for t in tiles_of(b, g, ntiles, xcd_map):
            started_at[(t, s)] = clock
        clock += 1
        for t in tiles_of(b, g, ntiles, xcd_map):
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
    # n, tiles per chunk, grid, steps, first step, XCD placement
    (2, 1, 2, 2, 0, False),
    (3, 1, 3, 4, 0, False),
    (8, 128, 256, 14, 0, False),     # N = 8, M = 2^24 float32: 4 tiles per workgroup
    (8, 512, 256, 14, 0, False),     # N = 8, M = 2^26: every upstream tile is the workgroup's own
    (8, 100, 256, 14, 0, False),     # 100 tiles per chunk: 3 or 4 tiles per workgroup
    (16, 3, 40, 30, 0, False),
    (64, 4, 256, 126, 0, False),
    (256, 1, 256, 510, 0, False),    # N = 256, M = 2^22 float32
    (5, 7, 13, 5, 1, False),         # an in-place AllGather: its placement step is skipped
    (8, 2056, 256, 14, 0, False),    # up to 65 tiles per workgroup
    (3, 1000, 256, 4, 0, False),     # about 12 tiles per workgroup, two upstream workgroups for some
    (64, 3, 192, 126, 0, True),      # the XCD placement: 3 tiles per chunk, 24 workgroups per XCD
    (256, 2, 256, 510, 0, True),     # N = 256, M = 6,553,600 bf16: two ragged tiles per chunk
    (16, 5, 80, 30, 0, True),
    (7, 3, 16, 12, 1, True),
]


@pytest.mark.parametrize("n,tpc,g,nsteps,first,xcd", CASES)
@pytest.mark.parametrize("seed", [1, 2])
def test_no_deadlock_and_every_step_follows_its_upstream(n, tpc, g, nsteps, first, xcd, seed):
    next_step, started, done = simulate(n, tpc, g, nsteps, first, seed, xcd_map=xcd)
    assert all(s == nsteps for s in next_step), "a workgroup never reached the last step"
    ntiles = n * tpc
    for t in range(ntiles):
        up = (t - tpc) % ntiles
        for s in range(first + 1, nsteps):
            assert done[(up, s - 1)] < started[(t, s)], (t, s)


def test_two_workgroup_rule_equals_the_per_tile_definition():
    """The kernel's two candidates are exactly the holders of the upstream
    tiles of every tile of the workgroup, on every workgroup of many grids,
    with and without the XCD placement, at up to thousands of tiles per
    workgroup."""
    rng = random.Random(7)
    shapes = [(n, tpc, g) for n in (2, 3, 8, 16, 256) for tpc in (1, 2, 3, 7, 8, 100, 512, 2048, 8192)
              for g in (8, 16, 40, 96, 256) if g <= n * tpc]
    shapes += [(rng.randint(2, 300), rng.randint(1, 600), 8 * rng.randint(1, 64)) for _ in range(300)]
    checked = 0
    for n, tpc, g in shapes:
        if g > n * tpc:
            continue
        for xcd_map in (False, True):
            for b in range(g):
                assert upstream_blocks(b, g, n, tpc, xcd_map) == upstream_by_tile(b, g, n, tpc, xcd_map), \
                    (n, tpc, g, xcd_map, b)
            checked += 1
    assert checked > 300
    # and the number of candidates never exceeds two
    assert all(len(upstream_by_tile(b, 256, 8, 8192, False)) <= 2 for b in range(256))


def test_a_rule_without_the_upstream_wait_is_caught():
    """The check has teeth: waiting on the downstream neighbour instead
    (tile + T) lets some tile start a step before its upstream finished."""
    n, tpc, g, nsteps = 8, 3, 8, 14
    ntiles = n * tpc

    def wrong_upstream(b, g, n, tpc, xcd_map):
        return {holder((t + tpc) % ntiles, g, xcd_map) for t in tiles_of(b, g, ntiles, xcd_map)} - {b}

    caught = False
    for seed in range(20):
        next_step, started, done = simulate(n, tpc, g, nsteps, 0, seed, rule=wrong_upstream)
        if any(s < nsteps for s in next_step):
            caught = True
            break
        if any(done[((t - tpc) % ntiles, s - 1)] >= started[(t, s)]
               for t in range(ntiles) for s in range(1, nsteps)):
            caught = True
            break
    assert caught


def test_the_rule_check_catches_a_dropped_wrap():
    """Leaving out the second candidate (the workgroup holding the upstream
    tiles of rank 0's tiles) is caught by the definition check."""
    def no_wrap(b, g, n, tpc, xcd_map=False):
        ntiles = n * tpc
        f = first_tile(b, g, xcd_map)
        return {holder(f + (g - tpc % g) % g, g, xcd_map)} - {b}

    assert any(no_wrap(b, 40, 16, 3) != upstream_by_tile(b, 40, 16, 3) for b in range(40))
