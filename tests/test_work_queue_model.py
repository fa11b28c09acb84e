"""A model of the backward's launch-counter queues (take_work_item in
depth_augmented_attention_amd/csrc/moda_bwd.hpp), run on the CPU under random
interleavings of the workgroups' atomic steps: one queue per (b, kv head)
pair with per_pair tiles; a workgroup fetch-adds its home pair's counter
(blockIdx % npairs) and, while the value it gets is past the end, the
following pairs' counters in turn.  With exactly one workgroup per tile,
every workgroup must find a tile within npairs attempts and every tile must
be taken exactly once, whatever the order of the steps."""
from __future__ import annotations

import random


def simulate(npairs: int, per_pair: int, seed: int):
    rng = random.Random(seed)
    grid = npairs * per_pair
    counters = [0] * npairs
    # state per workgroup: (queue to try next, attempts made, result)
    state = {w: [w % npairs, 0, None] for w in range(grid)}
    pending = list(range(grid))
    while pending:
        w = pending[rng.randrange(len(pending))]   # any workgroup may take the next atomic step
        q, k, _ = state[w]
        it = counters[q]
        counters[q] += 1                           # fetch-add
        if it < per_pair:
            state[w][2] = (q, it)
            pending.remove(w)
        else:
            state[w][1] = k + 1
            assert state[w][1] < npairs, f"workgroup {w} found no tile"
            state[w][0] = q + 1 if q + 1 < npairs else 0
    return [state[w][2] for w in range(grid)]


def test_every_tile_taken_once_under_random_interleavings():
    for npairs in (1, 2, 3, 9, 15):
        for per_pair in (1, 2, 7, 64):
            for seed in range(20):
                got = simulate(npairs, per_pair, seed)
                assert sorted(got) == [(q, i) for q in range(npairs) for i in range(per_pair)]


def test_home_pair_first():
    # taken one after another in blockIdx order, each workgroup gets its home pair's tiles
    npairs, per_pair = 4, 5
    counters = [0] * npairs
    for w in range(npairs * per_pair):
        q = w % npairs
        assert counters[q] < per_pair
        counters[q] += 1
    assert counters == [per_pair] * npairs
