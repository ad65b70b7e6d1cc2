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


def test_hand_worked_even_runs_at_h128_geometry():
    # 4 requests of 64 blocks, 16 parts, F = 4: total = 4 * 68 = 272, payload = 17 + 4 = 21.
    # The walk gives every request 17 + 17 + 17 + 13 blocks (the 13-block rest costs 17 <= 21
    # and leaves 4, too little for 4 - F = 0 blocks of the next request).  Each request's four
    # parts hold it alone, so the evening step deals its 64 blocks out as 4 x 16.
    raw, ns_raw = oracle.plan([64 * 64] * 4, num_parts=16, fixed_overhead=4, even=False)
    assert [(int(r[2]), int(r[3])) for r in raw[:4]] == [(0, 17), (17, 34), (34, 51), (51, 64)]
    sched, ns = oracle.plan([64 * 64] * 4, num_parts=16, fixed_overhead=4)
    assert sched.tolist() == [[r, r, 16 * i, 16 * i + 16, i, 4, 0, 0] for r in range(4) for i in range(4)]
    assert ns.tolist() == ns_raw.tolist() == [0, 4, 8, 12, 16]


def test_hand_worked_even_run_after_a_shared_part():
    # n = {1, 9}, 3 parts, F = 0: payload = ceil(10 / 3) = 4.  Part 0 takes request 0 (1 block)
    # and blocks 0..2 of request 1; part 1 takes 4 more (3..6), the last part the rest (7, 8).
    # Part 0 holds two requests and keeps its cut; parts 1 and 2 hold request 1 alone and
    # share its blocks 3..8 evenly: 3..5 and 6..8.
    raw, _ = oracle.plan([64, 576], num_parts=3, even=False)
    assert raw.tolist() == [[0, 1, 0, 3, 0, 3, 0, 0], [1, 1, 3, 7, 1, 3, 0, 0], [1, 1, 7, 9, 2, 3, 0, 0]]
    sched, ns = oracle.plan([64, 576], num_parts=3)
    assert sched.tolist() == [[0, 1, 0, 3, 0, 3, 0, 0], [1, 1, 3, 6, 1, 3, 0, 0], [1, 1, 6, 9, 2, 3, 0, 0]]
    assert ns.tolist() == [0, 1, 4]


def check_even_against_walk(seqlens, P, F):
    """The evening step moves only block boundaries between consecutive parts that hold one
    request alone; inside such a run the sizes are the even split, longest first."""
    raw, ns_raw = oracle.plan(seqlens, num_parts=P, fixed_overhead=F, even=False)
    sched, ns = oracle.plan(seqlens, num_parts=P, fixed_overhead=F)
    assert sched.shape == raw.shape and ns.tolist() == ns_raw.tolist()
    assert (sched[:, [0, 1, 4, 5, 6, 7]] == raw[:, [0, 1, 4, 5, 6, 7]]).all()
    alone = raw[:, 0] == raw[:, 1]
    assert (sched[~alone] == raw[~alone]).all()
    p = 0
    while p < len(raw):
        q = p + 1
        while alone[p] and q < len(raw) and alone[q] and raw[q, 0] == raw[p, 0]:
            q += 1
        sizes = (sched[p:q, 3] - sched[p:q, 2]).tolist()
        assert sched[p, 2] == raw[p, 2] and sched[q - 1, 3] == raw[q - 1, 3]
        assert (sched[p + 1:q, 2] == sched[p:q - 1, 3]).all()
        assert max(sizes) - min(sizes) <= 1 and sizes == sorted(sizes, reverse=True)
        assert max(sizes) <= max((raw[p:q, 3] - raw[p:q, 2]).tolist())
        p = q


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
    check_even_against_walk(seqlens, P, F)
    fk = int(rng.integers(1, 5))
    sched, ns = oracle.plan(seqlens, num_parts=P, force_splits=fk)
    check_plan_valid(seqlens, sched, ns, greedy=False)
