"""Pins of the oracle's pinned-RAM expert cache (CPU only).

"LFM2.5-24B-A2B -- Packed MXFP4 Inference", "Bounded pinned RAM expert cache":
CPU-backed expert triplets are kept in a packed RAM cache with LRU eviction
under a memory limit.  The oracle's LRU is pinned by a hand-worked sequence,
by the closed forms of cyclic access (capacity + 1 keys in a cycle always
miss; at most capacity keys miss only on their first pass), and by an
independent characterisation of LRU: a request hits exactly when fewer than
`capacity` distinct other keys were requested since the same key's previous
request (the LRU stack distance), which also gives the inclusion property
(a larger cache never turns a hit into a miss).
"""
import numpy as np
import pytest


def test_lru_hand_example(orc):
    # capacity 3: 1 2 3 miss; 1 hits (order 1 3 2); 4 misses and drops 2;
    # 2 misses and drops 3; 5 misses and drops 1; 1 misses
    assert orc.lru([1, 2, 3, 1, 4, 2, 5, 1], 3).tolist() == [0, 0, 0, 1, 0, 0, 0, 0]
    # capacity 4 keeps 2 alive: 2 and 1 hit
    assert orc.lru([1, 2, 3, 1, 4, 2, 5, 1], 4).tolist() == [0, 0, 0, 1, 0, 1, 0, 1]


@pytest.mark.parametrize("cap", [1, 2, 5, 64])
def test_lru_cyclic_closed_forms(orc, cap):
    cyc_over = list(range(cap + 1)) * 7
    assert orc.lru(cyc_over, cap).sum() == 0
    cyc_fit = list(range(cap)) * 7
    h = orc.lru(cyc_fit, cap)
    assert h[:cap].sum() == 0 and h[cap:].all()
    same = [42] * 10
    assert orc.lru(same, cap).tolist() == [0] + [1] * 9


def _stack_distance_hits(keys, cap):
    last = {}
    out = []
    for i, k in enumerate(keys):
        if k in last:
            between = set(keys[last[k] + 1:i])
            out.append(1 if len(between) < cap else 0)
        else:
            out.append(0)
        last[k] = i
    return out


def test_lru_matches_stack_distance_and_inclusion(orc):
    rng = np.random.default_rng(4)
    for trial in range(40):
        n = int(rng.integers(1, 300))
        universe = int(rng.integers(1, 40))
        # skewed keys, as routed experts are
        keys = (rng.zipf(1.3, n) % universe).tolist()
        prev = None
        for cap in (1, 2, 3, 7, 16, 50):
            h = orc.lru(keys, cap)
            assert h.tolist() == _stack_distance_hits(keys, cap), (trial, cap)
            if prev is not None:
                assert np.all(h >= prev)
            prev = h


def test_lru_requests_order(orc):
    ids = np.array([[5, 3, 9, 1], [3, 7, 5, 2]])
    cpu = np.zeros(16, bool)
    cpu[[3, 5, 7, 9]] = True
    assert orc.lru_requests(ids, cpu) == [5, 3, 9, 7]
    with pytest.raises(ValueError):
        orc.lru([1, 2], 0)
