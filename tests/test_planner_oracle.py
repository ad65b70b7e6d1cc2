"""Pins for the reference planner: hand-worked cases and the invariants any
valid split plan must satisfy (every block covered exactly once, pieces in
order, per-part load within the cap, consistent split counts)."""
import numpy as np
import pytest

import oracle
from oracle.planner import blocks_of


def check_plan_valid(seqlens, sched, num_splits, num_parts=None, fixed_overhead=0, greedy=True):
    n = blocks_of(seqlens)
    b = len(n)
    assert num_splits.shape == (b + 1,) and num_splits[0] == 0
    pieces = oracle.pieces_of(sched, seqlens)
    covered = [np.zeros(nb, dtype=np.int32) for nb in n]
    seen_pieces = [[] for _ in range(b)]
    for (p, r, lo, hi, k) in pieces:
        assert 0 <= lo <= hi <= n[r]
        covered[r][lo:hi] += 1
        seen_pieces[r].append((k, lo, hi))
    for r in range(b):
        assert np.all(covered[r] == 1), f"request {r} not covered exactly once"
        ks = sorted(seen_pieces[r])
        assert [k for k, _, _ in ks] == list(range(len(ks))), "piece indices must be 0..n-1"
        assert num_splits[r + 1] - num_splits[r] == len(ks)
        ends = [lo for _, lo, _ in ks] + [n[r]]
        for (k, lo, hi), nxt in zip(ks, ends[1:]):
            assert hi == nxt, "pieces must tile the request in order"
        if n[r] > 0:
            assert all(hi > lo for _, lo, hi in ks), "only empty requests have empty pieces"
    if greedy and num_parts is not None:
        assert sched.shape[0] <= num_parts
        F = fixed_overhead
        total = sum(nb + F for nb in n)
        payload = -(-total // num_parts) + F
        for p in range(sched.shape[0] - 1):
            load = sum(hi - lo + F for (pp, r, lo, hi, k) in pieces if pp == p)
            assert load <= payload


def test_hand_worked_two_parts():
    # L = {100, 257} -> 2 and 5 blocks; 2 parts, F = 0: payload = ceil(7/2) = 4.
    # Part 0 takes request 0 whole (2) and 2 blocks of request 1; part 1 takes the rest.
    sched, ns = oracle.plan([100, 257], num_parts=2, fixed_overhead=0)
    assert sched.tolist() == [[0, 1, 0, 2, 0, 2, 0, 0], [1, 1, 2, 5, 1, 2, 0, 0]]   # column 5: most pieces (2)
    assert ns.tolist() == [0, 1, 3]


def test_hand_worked_fixed_overhead():
    # n = {2, 5}, F = 1, 3 parts: total = 3 + 6 = 9, payload = 3 + 1 = 4.
    # Part 0: request 0 costs 3 (fits, cap 1 left), request 1 needs 6 > 1 and
    # 1 - F = 0 blocks can be taken -> part ends.  Part 1: request 1 costs 6 > 4,
    # take 4 - 1 = 3 blocks.  Part 2 (last): the remaining 2 blocks.
    sched, ns = oracle.plan([100, 257], num_parts=3, fixed_overhead=1)
    assert sched.tolist() == [[0, 0, 0, 2, 0, 2, 0, 0], [1, 1, 0, 3, 0, 2, 0, 0],
                              [1, 1, 3, 5, 1, 2, 0, 0]]
    assert ns.tolist() == [0, 1, 3]


def test_forced_two_splits_tiny_config():
    sched, ns = oracle.plan([100, 257], num_parts=1, force_splits=2)
    assert sched.tolist() == [[0, 0, 0, 1, 0, 2, 0, 0], [0, 0, 1, 2, 1, 2, 0, 0],
                              [1, 1, 0, 3, 0, 2, 0, 0], [1, 1, 3, 5, 1, 2, 0, 0]]
    assert ns.tolist() == [0, 2, 4]


def test_empty_requests_are_placed():
    sched, ns = oracle.plan([0, 130, 0, 0], num_parts=2, fixed_overhead=0)
    check_plan_valid([0, 130, 0, 0], sched, ns, 2, 0)
    # n = {0, 3, 0, 0}, payload = ceil(3/2) = 2: request 1 is cut 2 + 1 blocks.
    assert ns.tolist() == [0, 1, 3, 4, 5]
    assert sched.tolist() == [[0, 1, 0, 2, 0, 2, 0, 0], [1, 3, 2, 0, 1, 2, 0, 0]]


@pytest.mark.parametrize("seed", range(40))
def test_random_plans_are_valid(seed):
    rng = np.random.default_rng(seed)
    b = int(rng.integers(1, 140))
    kind = seed % 4
    if kind == 0:
        seqlens = rng.integers(0, 20000, size=b)
    elif kind == 1:
        seqlens = rng.integers(1, 200, size=b)
    elif kind == 2:
        seqlens = np.full(b, 64 * int(rng.integers(1, 100)))
    else:
        seqlens = np.where(rng.random(b) < 0.1, rng.integers(50000, 140000, size=b),
                           rng.integers(1, 3000, size=b))
    P = int(rng.integers(1, 300))
    F = int(rng.integers(0, 6))
    sched, ns = oracle.plan(seqlens, num_parts=P, fixed_overhead=F)
    check_plan_valid(seqlens, sched, ns, P, F)
    fk = int(rng.integers(1, 5))
    sched, ns = oracle.plan(seqlens, num_parts=P, force_splits=fk)
    check_plan_valid(seqlens, sched, ns, greedy=False)
