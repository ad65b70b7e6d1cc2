"""Reference split-KV tile planner (integer work).

TEST INFRASTRUCTURE ONLY: only ``tests/``, ``__graft_entry__.smoke()`` and
``bench.py``'s ``cpu_baseline`` leg may use anything under ``oracle/``.

Follows the tile-scheduler description on the FlashMLA new-kernel deep-dive
page (nxmr.cn, section "Tile Scheduler"): count each request's KV blocks
from its sequence length, set a per-part work cap
payload = ceil(total / num_parts) + fixed_overhead, then walk the requests
in order filling each part greedily, cutting a request across parts when it
does not fit, and record how many pieces (splits) each request ends up in so
the combine step can find them.

Readings taken where the page is silent:
  * "total" counts every request's blocks plus one fixed overhead per
    request, and every piece a part takes costs its blocks plus the fixed
    overhead;
  * the last part takes whatever is left, so every block is always covered;
  * a request with no blocks (L = 0) is still placed in a part as an empty
    piece, so that its output (zeros, lse = -inf) is written;
  * ``force_splits = k > 0`` replaces the greedy walk: each request is cut
    into min(k, n_b) page-aligned pieces (at least one), earlier pieces one
    block longer when n_b is not a multiple, one part per piece.

After the walk, a step that is not on the page (the GPU library's planner
takes it too, because it measured faster on MI355X): the walk leaves a long
request in pieces of payload - F blocks and one shorter last piece.  Each
maximal run of consecutive parts that hold a piece of one request and nothing
else has its blocks dealt out again as evenly as possible, earlier parts one
block longer when the count does not divide (``_even_runs``).  Parts, piece
indices and split counts are the walk's; only block boundaries inside a run
move, so no part's load grows past the longest piece the walk made.

Output layout (shared with the GPU library's planner, which must agree bit
for bit): one row of 8 int32 per part
  [begin_req, end_req (inclusive), begin_block (in begin_req),
   end_block (exclusive, in end_req), begin_piece (index of begin_req's piece
   in this part among that request's pieces), 0, 0, 0]
and ``num_splits`` as an exclusive prefix sum over requests, length b + 1:
request b owns partial slots [num_splits[b], num_splits[b+1]).
"""
from __future__ import annotations

import numpy as np

PAGE = 64
SCHED_INTS = 8


def blocks_of(seqlens) -> list[int]:
    return [(int(L) + PAGE - 1) // PAGE for L in seqlens]


def plan(seqlens, num_parts: int, fixed_overhead: int = 0, force_splits: int = 0, even: bool = True):
    """Return (sched int32 [parts, 8], num_splits int32 [b + 1]).

    ``even=False`` returns the page's walk alone, without the evening step.

    A row is [begin_req, end_req, begin_block, end_block, begin_piece,
    max_pieces, 0, 0]; max_pieces (the same in every row) is the largest
    number of pieces any request was cut into."""
    n = blocks_of(seqlens)
    b = len(n)
    if b == 0 or num_parts <= 0:
        raise ValueError("need at least one request and one part")
    if force_splits > 0:
        return _plan_forced(n, force_splits)
    F = int(fixed_overhead)
    total = sum(nb + F for nb in n)
    payload = -(-total // num_parts) + F            # ceil_div + fixed overhead
    parts = []
    pieces = [0] * b
    req, blk = 0, 0
    for p in range(num_parts):
        if req >= b:
            break
        last_part = p == num_parts - 1
        cap = payload
        begin = (req, blk, pieces[req])
        end_req, end_blk = -1, -1
        while req < b:
            rem = n[req] - blk
            if last_part or rem + F <= cap:         # rest of the request fits
                cap -= rem + F
                pieces[req] += 1
                end_req, end_blk = req, n[req]
                req, blk = req + 1, 0
                continue
            take = cap - F
            if take > 0:                             # cut the request here
                blk += take
                pieces[req] += 1
                end_req, end_blk = req, blk
            break
        if end_req < 0:                              # nothing fitted: close the walk
            continue
        parts.append([begin[0], end_req, begin[1], end_blk, begin[2], 0, 0, 0])
    if even:
        _even_runs(parts)
    num_splits = np.zeros(b + 1, dtype=np.int32)
    num_splits[1:] = np.cumsum(pieces)
    return _with_max_pieces(np.array(parts, dtype=np.int32).reshape(-1, SCHED_INTS), pieces), num_splits


def _even_runs(parts) -> None:
    """Deal the blocks of each run of single-request parts out evenly (in place)."""
    alone = [row[0] == row[1] for row in parts]
    p = 0
    while p < len(parts):
        if not alone[p]:
            p += 1
            continue
        q = p + 1
        while q < len(parts) and alone[q] and parts[q][0] == parts[p][0]:
            q += 1
        start, end, k = parts[p][2], parts[q - 1][3], q - p
        sizes = [(end - start) // k + (1 if i < (end - start) % k else 0) for i in range(k)]
        at = start
        for i in range(k):
            parts[p + i][2], parts[p + i][3] = at, at + sizes[i]
            at += sizes[i]
        p = q


def _with_max_pieces(sched: np.ndarray, pieces) -> np.ndarray:
    """Column 5 of every row: the largest number of pieces of any request
    (table layout only: it tells the merge how many partials a row can have)."""
    sched[:, 5] = max(pieces) if len(pieces) else 0
    return sched


def _plan_forced(n, k):
    parts = []
    pieces = []
    for r, nb in enumerate(n):
        cnt = max(1, min(k, nb))
        q, extra = divmod(nb, cnt)
        start = 0
        for i in range(cnt):
            size = q + (1 if i < extra else 0)
            parts.append([r, r, start, start + size, i, 0, 0, 0])
            start += size
        pieces.append(cnt)
    num_splits = np.zeros(len(n) + 1, dtype=np.int32)
    num_splits[1:] = np.cumsum(pieces)
    return _with_max_pieces(np.array(parts, dtype=np.int32).reshape(-1, SCHED_INTS), pieces), num_splits


def pieces_of(sched: np.ndarray, seqlens):
    """Expand a plan into (part, request, block_begin, block_end, piece) tuples."""
    n = blocks_of(seqlens)
    out = []
    for p, row in enumerate(np.asarray(sched)):
        br, er, bb, eb, bp = (int(x) for x in row[:5])
        for r in range(br, er + 1):
            lo = bb if r == br else 0
            hi = eb if r == er else n[r]
            out.append((p, r, lo, hi, bp if r == br else 0))
    return out
