"""The selection protocol's arithmetic (step tags, walk parities, clearing,
watchdog) under random interleavings, on the CPU model in protocol_model."""
import random

import pytest

from protocol_model import Memory, run_walk, random_keys


@pytest.mark.parametrize("G", [1, 5, 16, 37, 64])
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_every_worker_sees_the_maximum(G, seed):
    rng = random.Random(1000 * G + seed)
    mem = Memory(G)
    for walk in range(3):                     # walks back to back: parities alternate
        keys = random_keys(rng, 5, G, ties=(walk == 1))
        seen = run_walk(mem, keys, rng)
        assert mem.err is None
        for t in range(5):
            assert all(s == max(keys[t]) for s in seen[t]), (walk, t)
        assert mem.epoch == walk + 1


def _stale_sequence(G):
    # walk k (2 steps, large keys) leaves step tags 1 and 2 in the lines of its
    # parity; walk k+1 (4 steps) uses the other parity; walk k+2 (2 steps,
    # small keys) uses walk k's lines again with the same tags.  A worker whose
    # leader polls before it publishes exposes walk k's key unless the lines
    # were cleared in between.
    big = [[(1 << 49) + g for g in range(G)] for _ in range(2)]
    mid = [[7 + g for g in range(G)] for _ in range(4)]
    small = [[1 + g for g in range(G)] for _ in range(2)]
    return big, mid, small


@pytest.mark.parametrize("seed", range(10))
def test_stale_lines_of_two_walks_back_are_never_taken(seed):
    rng = random.Random(seed)
    G = 32
    mem = Memory(G)
    for keys in _stale_sequence(G):
        seen = run_walk(mem, keys, rng)
        assert all(s == max(keys[t]) for t in range(len(keys)) for s in seen[t])


def test_without_clearing_stale_keys_leak():
    # the same sequences with the clearing left out of the model: some worker
    # takes a key of two walks back, so the clearing is necessary
    leaked = False
    for seed in range(10):
        rng = random.Random(seed)
        G = 32
        mem = Memory(G)
        big, mid, small = _stale_sequence(G)
        run_walk(mem, big, rng, skip_clear=True)
        run_walk(mem, mid, rng, skip_clear=True)
        seen = run_walk(mem, small, rng, skip_clear=True)
        leaked = leaked or any(s != max(small[t]) for t in range(2) for s in seen[t] if s is not None)
    assert leaked


def test_a_worker_that_never_arrives_times_everyone_out():
    rng = random.Random(3)
    G = 40
    mem = Memory(G)
    keys = random_keys(rng, 4, G)
    seen = run_walk(mem, keys, rng, watchdog=200, never_arrive=(21, 2))
    assert mem.err == "timeout"
    # steps before the missing arrival complete correctly; nobody completes step 2
    for t in range(2):
        assert all(s == max(keys[t]) for s in seen[t])
    assert all(s is None for s in seen[2])
    assert mem.epoch == 0                       # the walk never completes
