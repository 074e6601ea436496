"""Work lists of the jagged tile scheduler, written from its rules (test infrastructure only).

Padding jagged sequences to a common length wastes compute, and without padding the naive grid
leaves compute units idle once short sequences finish (aihot.vn GEM page, "Jagged Sequence Flash
Attention"); after padding is gone the bottleneck moves to tile scheduling and load balance
(vibekk.com GEM page, section on moving from padding to jagged kernels). The planner therefore
emits one work item per tile of useful work, splits items that alone exceed a fair share, and
orders the list longest first so that greedy in-order dispatch approximates longest-processing-
time scheduling. These are the rules, restated here independently of the C++ planner so that the
two can be compared entry by entry:

query-tile lists (forward and dQ), tile BM queries x BN keys:
  for b, h, t in lexicographic order with t < ceil(Lq_b / BM):
      n_kv = ceil(Lkv_b / BN)
      cost = min(ceil((t + 1) BM / BN), n_kv) under the causal mask, else n_kv
      item covers key tiles [0, cost)
key-tile lists (dK/dV), tile BNk keys x BMq queries:
  for b, h, kt in lexicographic order with kt < ceil(Lkv_b / BNk):
      n_q = ceil(Lq_b / BMq);  first = floor(kt BNk / BMq) under the causal mask, else 0
      cost = max(0, n_q - first);  item covers query tiles [first, first + cost)
with a window W or block size B (the visibility of oracle.attention), the ranges shrink to the
tiles that hold a visible pair: the keys seen by rows r0..r1 = t BM .. min((t+1) BM, Lq_b) - 1
form the interval [max(0, r0 - W + 1, B floor(r0 / B)), min(Lkv_b - 1, r1 (causal),
r1 + W - 1 (no mask), B floor(r1 / B) + B - 1)] (each bound only when its mode is on), and the
rows that see keys c0..c1 = kt BNk .. min((kt+1) BNk, Lkv_b) - 1 form
[max(c0 (causal), c0 - W + 1 (no mask), B floor(c0 / B)), min(Lq_b - 1, c1 + W - 1,
B floor(c1 / B) + B - 1)]; the item covers the tiles from the one holding the lower bound through
the one holding the upper bound (none when the interval is empty: key tiles [0, 0), query tiles
[lo, lo)). Without a window or block the rules above apply unchanged.
splitting (both lists), given the number of concurrent workgroups ``slots``:
  target = max(1, ceil(sum(cost) / slots)); when sum(cost) > slots, an item with cost > target becomes
  R = ceil(cost / target) pieces, piece r covering [lo + floor(r cost / R), lo + floor((r+1) cost / R))
  (with less than one tile of work per slot nothing is split: merging the pieces would cost a launch
  of its own, more than the tiles it saves);
  split groups are numbered in the lexicographic order above and own partial slots
  slot0 .. slot0 + R - 1 (piece r -> slot0 + r); unsplit items carry slot -1
order: by (piece length descending, b, h, tile, range start) ascending.
shared queries (one set of query rows for every sequence, dQ summed over sequences), dQ list only:
  after the rules above every piece owns a partial slot; slots are numbered by (h, tile, b, range
  start) ascending, and one group per (h, tile) - written (0, h, tile, slot0, R) - sums its R pieces
  in slot order.

Each item is the tuple (b, h, tile, lo, hi, slot); each split group is (b, h, tile, slot0, R).
"""
from __future__ import annotations


def _ceil_div(a: int, b: int) -> int:
    return -(-a // b)


def _finish(raw, slots: int, split: bool):
    total = sum(hi - lo for (_, _, _, lo, hi) in raw)
    target = max(1, _ceil_div(total, max(1, slots)))
    items, groups = [], []
    next_slot = 0
    for (b, h, t, lo, hi) in raw:
        cost = hi - lo
        if split and total > max(1, slots) and cost > target:
            R = _ceil_div(cost, target)
            groups.append((b, h, t, next_slot, R))
            for r in range(R):
                items.append((b, h, t, lo + (r * cost) // R, lo + ((r + 1) * cost) // R, next_slot + r))
            next_slot += R
        else:
            items.append((b, h, t, lo, hi, -1))
    items.sort(key=lambda it: (-(it[4] - it[3]), it[0], it[1], it[2], it[3]))
    return items, groups, next_slot


def _key_range(t, Lq, Lkv, causal, BM, BN, window, block):
    """Key tiles [lo, hi) holding a visible pair for query tile t under a window or block."""
    r0, r1 = t * BM, min((t + 1) * BM, Lq) - 1
    lo_key, hi_key = 0, Lkv - 1
    if window:
        lo_key = max(lo_key, r0 - window + 1)
        if not causal:
            hi_key = min(hi_key, r1 + window - 1)
    if causal:
        hi_key = min(hi_key, r1)
    if block:
        lo_key = max(lo_key, (r0 // block) * block)
        hi_key = min(hi_key, (r1 // block) * block + block - 1)
    if hi_key < lo_key:
        return 0, 0
    return lo_key // BN, hi_key // BN + 1


def _query_range(kt, Lq, Lkv, causal, BMq, BNk, window, block):
    """Query tiles [lo, hi) holding a visible pair for key tile kt under a window or block."""
    c0, c1 = kt * BNk, min((kt + 1) * BNk, Lkv) - 1
    lo_row, hi_row = 0, Lq - 1
    if causal:
        lo_row = c0
    if window:
        hi_row = min(hi_row, c1 + window - 1)
        if not causal:
            lo_row = max(lo_row, c0 - window + 1)
    if block:
        lo_row = max(lo_row, (c0 // block) * block)
        hi_row = min(hi_row, (c1 // block) * block + block - 1)
    lo = lo_row // BMq
    if hi_row < lo_row:
        return lo, lo
    return lo, hi_row // BMq + 1


def query_tile_items(lq, lkv, H: int, causal: bool, BM: int, BN: int, slots: int, split: bool = True,
                     window: int = 0, block: int = 0):
    """(items, groups, n_partial_slots) for a kernel that owns query tiles and loops over keys."""
    raw = []
    for b in range(len(lq)):
        n_kv = _ceil_div(int(lkv[b]), BN)
        for h in range(H):
            for t in range(_ceil_div(int(lq[b]), BM)):
                if window or block:
                    lo, hi = _key_range(t, int(lq[b]), int(lkv[b]), causal, BM, BN, window, block)
                else:
                    lo, hi = 0, (min(_ceil_div((t + 1) * BM, BN), n_kv) if causal else n_kv)
                raw.append((b, h, t, lo, hi))
    return _finish(raw, slots, split)


def key_tile_items(lq, lkv, H: int, causal: bool, BMq: int, BNk: int, slots: int, split: bool = True,
                   window: int = 0, block: int = 0):
    """(items, groups, n_partial_slots) for a kernel that owns key tiles and loops over queries."""
    raw = []
    for b in range(len(lq)):
        n_q = _ceil_div(int(lq[b]), BMq)
        for h in range(H):
            for kt in range(_ceil_div(int(lkv[b]), BNk)):
                if window or block:
                    lo, hi = _query_range(kt, int(lq[b]), int(lkv[b]), causal, BMq, BNk, window, block)
                else:
                    lo = (kt * BNk) // BMq if causal else 0
                    hi = lo + max(0, n_q - lo)
                raw.append((b, h, kt, lo, hi))
    return _finish(raw, slots, split)


def dispatch_order(items, n_xcd: int = 8):
    """The items of one list in the order the kernel's workgroups take them.

    Workgroup p of a launch runs on XCD p mod n_xcd, and every XCD has its own L2, so items that
    read the same sequence's K/V (or Q/dO) are kept on one XCD:
      a group is (b, h); its cost is the sum of (hi - lo) over its items;
      groups are ranked by cost, largest first, ties by (b, h) ascending;
      in rank order each group joins the XCD with the smallest total cost so far (lowest index
      on ties);
      an XCD's queue holds its items by group rank, then by position in the list;
      position p takes the next item of queue p mod n_xcd, or, when that queue is empty, of the
      queue with the most items left (lowest index on ties).
    """
    cost = {}
    for (b, h, _t, lo, hi, _s) in items:
        cost[(b, h)] = cost.get((b, h), 0) + (hi - lo)
    ranked = sorted(cost, key=lambda g: (-cost[g], g))
    load = [0] * n_xcd
    home, rank = {}, {}
    for r, g in enumerate(ranked):
        x = min(range(n_xcd), key=lambda y: (load[y], y))
        home[g], rank[g] = x, r
        load[x] += cost[g]
    queues = [[] for _ in range(n_xcd)]
    for i, it in enumerate(items):
        queues[home[(it[0], it[1])]].append(i)
    for q in queues:
        q.sort(key=lambda i: (rank[(items[i][0], items[i][1])], i))
    taken = [0] * n_xcd
    out = []
    for p in range(len(items)):
        x = p % n_xcd
        if taken[x] == len(queues[x]):
            x = max((y for y in range(n_xcd) if taken[y] < len(queues[y])),
                    key=lambda y: (len(queues[y]) - taken[y], -y))
        out.append(items[queues[x][taken[x]]])
        taken[x] += 1
    return out


def share_query_slots(items):
    """(items, groups, n_partial_slots) of a dQ list under shared queries (see the module rules)."""
    order = sorted(range(len(items)), key=lambda i: (items[i][1], items[i][2], items[i][0], items[i][3]))
    slot = {}
    groups = []
    for n, i in enumerate(order):
        b, h, t = items[i][:3]
        if not groups or tuple(groups[-1][1:3]) != (h, t):
            groups.append([0, h, t, n, 0])
        groups[-1][4] += 1
        slot[i] = n
    new_items = [(b, h, t, lo, hi, slot[i]) for i, (b, h, t, lo, hi, _s) in enumerate(items)]
    return new_items, [tuple(g) for g in groups], len(items)
