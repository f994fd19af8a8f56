"""Pins of the expert-cache oracle (oracle/lru.py): least-recently-used replacement.

Each test ties the oracle to something other than itself: fault counts worked
by hand for textbook reference strings (tests/golden/), the stack-distance
characterisation of LRU computed by brute force, the inclusion property, and
the cold-miss count of a cache that holds everything.
"""
import os
import random

import pytest

from oracle.lru import layer_accesses, lru_run

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _reference_strings():
    with open(os.path.join(GOLD, "lru_reference_strings.txt")) as f:
        for ln in f:
            if ln.strip() and not ln.startswith("#"):
                frames, faults, seq = ln.split()
                yield int(frames), int(faults), [int(v) for v in seq.split(",")]


def test_textbook_fault_counts():
    rows = list(_reference_strings())
    assert len(rows) == 3
    for frames, faults, seq in rows:
        hits, _ = lru_run(seq, frames)
        assert hits.count(False) == faults, (frames, seq)


def test_final_contents_hand_worked():
    # the last line of the hand-worked trace: [7 0 1], least recently used first
    _, cache = lru_run([7, 0, 1, 2, 0, 3, 0, 4, 2, 3, 0, 3, 2, 1, 2, 0, 1, 7, 0, 1], 3)
    assert list(cache) == [7, 0, 1]


def _stack_distance_hits(seq, capacity):
    """LRU hits by definition (Mattson et al., 1970): an access hits iff its key
    was seen before and fewer than `capacity` distinct keys, itself included,
    were touched since (and including) its previous access."""
    out = []
    for i, key in enumerate(seq):
        prev = [j for j in range(i) if seq[j] == key]
        if not prev:
            out.append(False)
            continue
        distinct = set(seq[prev[-1]:i])
        out.append(len(distinct) <= capacity)
    return out


@pytest.mark.parametrize("seed", range(6))
def test_stack_distance_brute_force(seed):
    rng = random.Random(seed)
    n_keys = rng.choice([3, 5, 9, 17])
    seq = [rng.randrange(n_keys) for _ in range(120)]
    for capacity in range(1, n_keys + 2):
        hits, cache = lru_run(seq, capacity)
        assert hits == _stack_distance_hits(seq, capacity), capacity
        assert len(cache) == min(capacity, len(set(seq)))


@pytest.mark.parametrize("seed", range(4))
def test_inclusion_and_cold_misses(seed):
    rng = random.Random(100 + seed)
    seq = [rng.randrange(40) for _ in range(400)]
    faults = [lru_run(seq, c)[0].count(False) for c in range(1, 45)]
    assert all(a >= b for a, b in zip(faults, faults[1:]))  # more frames never cost more
    assert faults[-1] == len(set(seq))  # everything fits: cold misses only
    assert faults[0] == 1 + sum(1 for a, b in zip(seq, seq[1:]) if a != b)  # one frame


def test_continued_run_equals_one_run():
    rng = random.Random(7)
    seq = [rng.randrange(12) for _ in range(200)]
    whole, cache_whole = lru_run(seq, 5)
    first, state = lru_run(seq[:77], 5)
    second, state = lru_run(seq[77:], 5, state)
    assert first + second == whole and list(state) == list(cache_whole)


def test_layer_access_order():
    # token order, then rank order; keys distinguish layers
    assert layer_accesses(2, [[5, 1], [1, 7]], 8) == [21, 17, 17, 23]
    hits, _ = lru_run(layer_accesses(0, [[5, 1], [1, 7]], 8), 4)
    assert hits == [False, False, True, False]  # a repeat inside one call hits
