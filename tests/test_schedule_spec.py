"""Pins of the schedule spec (CPU): exact once-only coverage, longest-first order, LPT bound."""
import heapq

import numpy as np
import pytest

import jfa_inputs as ji
from oracle import schedule as S


def _visible_blocks(lq, lkv, H, causal, BQ, BK, window=0, block=0):
    """Brute force: every (b, h, query tile, key tile) holding at least one visible (i, j) pair."""
    out = set()
    for b in range(len(lq)):
        Lq, Lk = int(lq[b]), int(lkv[b])
        if Lq == 0 or Lk == 0:
            continue
        i = np.arange(Lq)[:, None]
        j = np.arange(Lk)[None, :]
        vis = (j <= i) if causal else np.ones((Lq, Lk), dtype=bool)
        if window:  # |i - j| < window, looking back only under the causal mask
            vis = vis & (np.abs(i - j) < window)
        if block:
            vis = vis & ((i // block) == (j // block))
        ii, jj = np.nonzero(vis)
        blocks = set(zip((ii // BQ).tolist(), (jj // BK).tolist()))
        for h in range(H):
            for (a, c) in blocks:
                out.add((b, h, a, c))
    return out


def _expand(items):
    cover = []
    for (b, h, t, lo, hi, _) in items:
        for x in range(lo, hi):
            cover.append((b, h, t, x))
    return cover


CASES = [
    ([5, 130, 0, 257, 64], [5, 130, 0, 257, 64], True),
    ([1, 40, 3, 64], [300, 17, 0, 1000], False),
    ([700, 129, 1], [700, 129, 1], True),
]


@pytest.mark.parametrize("case", range(len(CASES)))
@pytest.mark.parametrize("slots", [1, 7, 64])
def test_query_tile_items_cover_each_visible_block_once(case, slots):
    lq, lkv, causal = CASES[case]
    items, groups, nslots = S.query_tile_items(lq, lkv, 2, causal, 128, 64, slots)
    cover = _expand(items)
    assert len(cover) == len(set(cover))
    assert set(cover) == _visible_blocks(lq, lkv, 2, causal, 128, 64)
    # every q tile of every non-empty query sequence appears, also with no keys
    tiles = {(b, h, t) for (b, h, t, *_rest) in items}
    expect = {(b, h, t) for b in range(len(lq)) for h in range(2) for t in range(-(-lq[b] // 128))}
    assert tiles == expect
    _check_order_and_groups(items, groups, nslots, slots)


@pytest.mark.parametrize("case", range(len(CASES)))
@pytest.mark.parametrize("slots", [1, 5, 64])
def test_key_tile_items_cover_each_visible_block_once(case, slots):
    lq, lkv, causal = CASES[case]
    items, groups, nslots = S.key_tile_items(lq, lkv, 3, causal, 64, 128, slots)
    cover = _expand(items)
    assert len(cover) == len(set(cover))
    # key-tile items are (b, h, key tile, query tile)
    assert {(b, h, x, t) for (b, h, t, x) in cover} == _visible_blocks(lq, lkv, 3, causal, 64, 128)
    tiles = {(b, h, t) for (b, h, t, *_rest) in items}
    expect = {(b, h, t) for b in range(len(lq)) for h in range(3) for t in range(-(-lkv[b] // 128))}
    assert tiles == expect
    _check_order_and_groups(items, groups, nslots, slots)


def _check_order_and_groups(items, groups, nslots, slots):
    lengths = [hi - lo for (_, _, _, lo, hi, _) in items]
    assert lengths == sorted(lengths, reverse=True)
    total = sum(lengths)
    target = max(1, -(-total // slots))
    used = sorted(s for (*_x, s) in items if s >= 0)
    assert used == list(range(nslots))
    for (b, h, t, s0, R) in groups:
        pieces = sorted((it for it in items if it[5] in range(s0, s0 + R)), key=lambda it: it[5])
        assert len(pieces) == R and all(p[:3] == (b, h, t) for p in pieces)
        for a, c in zip(pieces, pieces[1:]):
            assert a[4] == c[3]
        assert all(p[4] - p[3] <= target for p in pieces)


@pytest.mark.parametrize("name", ["causal_bucket", "target_attn", "gdpa_silu"])
def test_lpt_makespan_bound(name):
    """Greedy in-order dispatch of a longest-first list is LPT: makespan <= 4/3 of the optimum."""
    w = ji.WORKLOADS[name]
    lq, lkv = ji.lengths(w)
    slots = 512
    items, _, _ = S.query_tile_items(lq, lkv, w.H, w.mask == "causal", 128, 64, slots)
    loads = [0] * slots
    heapq.heapify(loads)
    for (_, _, _, lo, hi, _) in items:
        heapq.heappush(loads, heapq.heappop(loads) + (hi - lo))
    makespan = max(loads)
    total = sum(hi - lo for (_, _, _, lo, hi, _) in items)
    lower = max(total / slots, max(hi - lo for (_, _, _, lo, hi, _) in items))
    assert makespan <= (4 / 3) * lower + 1e-9
    # splitting pays: the efficiency mean/makespan is high on every workload
    assert total / slots / makespan > 0.9


def test_splitting_matches_the_worked_counts():
    # asymmetric workload at 64x64 tiles: 2,048 q-tile items, of which the longest get split
    w = ji.WORKLOADS["target_attn"]
    lq, lkv = ji.lengths(w)
    items, groups, _ = S.query_tile_items(lq, lkv, w.H, False, 64, 64, 512, split=False)
    assert len(items) == 2048
    items2, groups2, nslots = S.query_tile_items(lq, lkv, w.H, False, 64, 64, 512)
    assert sum(hi - lo for (*_a, lo, hi, _s) in items2) == sum(hi - lo for (*_a, lo, hi, _s) in items)
    assert len(groups2) > 0 and nslots == sum(R for (*_g, R) in groups2)


BAND_CASES = [
    ([5, 130, 0, 257, 64, 700], [5, 130, 0, 257, 64, 700], True, 100, 0),
    ([5, 130, 0, 257, 64, 700], [5, 130, 0, 257, 64, 700], True, 1, 0),
    ([5, 130, 0, 257, 64, 700], [5, 130, 0, 257, 64, 700], True, 0, 200),
    ([5, 130, 0, 257, 64, 700], [5, 130, 0, 257, 64, 700], True, 300, 256),
    ([1, 40, 3, 64, 300], [300, 17, 0, 1000, 90], False, 70, 0),
    ([1, 40, 3, 64, 300], [300, 17, 0, 1000, 90], False, 0, 50),
    ([700, 129, 1], [700, 129, 1], False, 64, 128),
]


@pytest.mark.parametrize("case", range(len(BAND_CASES)))
def test_band_ranges_cover_each_visible_block_once(case):
    """Window / block masks: query- and key-tile ranges are exactly the tiles with a visible pair."""
    lq, lkv, causal, window, block = BAND_CASES[case]
    items, groups, nslots = S.query_tile_items(lq, lkv, 2, causal, 128, 64, 7, window=window, block=block)
    cover = _expand(items)
    assert len(cover) == len(set(cover))
    assert set(cover) == _visible_blocks(lq, lkv, 2, causal, 128, 64, window, block)
    tiles = {(b, h, t) for (b, h, t, *_rest) in items}
    assert tiles == {(b, h, t) for b in range(len(lq)) for h in range(2) for t in range(-(-lq[b] // 128))}
    _check_order_and_groups(items, groups, nslots, 7)
    items, groups, nslots = S.key_tile_items(lq, lkv, 2, causal, 64, 128, 5, window=window, block=block)
    cover = _expand(items)
    assert len(cover) == len(set(cover))
    assert {(b, h, x, t) for (b, h, t, x) in cover} == _visible_blocks(lq, lkv, 2, causal, 64, 128, window, block)
    tiles = {(b, h, t) for (b, h, t, *_rest) in items}
    assert tiles == {(b, h, t) for b in range(len(lq)) for h in range(2) for t in range(-(-lkv[b] // 128))}
    _check_order_and_groups(items, groups, nslots, 5)


def test_band_without_limits_is_the_plain_schedule():
    lq = [5, 130, 0, 257, 64, 700]
    for causal in (True, False):
        a = S.query_tile_items(lq, lq, 2, causal, 128, 64, 9)
        b = S.query_tile_items(lq, lq, 2, causal, 128, 64, 9, window=10**6, block=10**6)
        assert a == b
        a = S.key_tile_items(lq, lq, 2, causal, 64, 128, 9)
        b = S.key_tile_items(lq, lq, 2, causal, 64, 128, 9, window=10**6, block=10**6)
        assert a == b
