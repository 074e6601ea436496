"""Useful-work accounting: visible (query, key) pairs and the FLOPs credited to them.

Only unpadded, unmasked pairs count (the pages' point is that padding to the longest sequence
wastes compute; aihot.vn GEM page, "Jagged Sequence Flash Attention"). Per visible pair and head
the forward pass is credited 4 D FLOPs (two matrix products) and the backward pass 10 D (the
usual 2.5x of the forward, recomputation included).
"""
from __future__ import annotations

import numpy as np


def visible_pairs(q_offsets, kv_offsets, causal: bool, window: int = 0, block: int = 0) -> int:
    """Number of visible (i, j) pairs of one head summed over sequences.

    With a window W or block size Bk, query i sees the keys j with i - j < W (and j - i < W without
    the causal limit) and i // Bk == j // Bk: per row an interval of keys, counted row by row.
    """
    qo = np.asarray(q_offsets, dtype=np.int64)
    ko = np.asarray(kv_offsets, dtype=np.int64)
    lq, lkv = np.diff(qo), np.diff(ko)
    if window or block:
        total = 0
        for nq, nk in zip(lq.tolist(), lkv.tolist()):
            i = np.arange(nq, dtype=np.int64)
            lo = np.zeros(nq, dtype=np.int64)
            hi = np.full(nq, nk - 1, dtype=np.int64)
            if causal:
                hi = np.minimum(hi, i)
            if window:
                lo = np.maximum(lo, i - window + 1)
                if not causal:
                    hi = np.minimum(hi, i + window - 1)
            if block:
                lo = np.maximum(lo, (i // block) * block)
                hi = np.minimum(hi, (i // block) * block + block - 1)
            total += int(np.maximum(hi - lo + 1, 0).sum())
        return total
    if not causal:
        return int((lq * lkv).sum())
    n = np.minimum(lq, lkv)
    return int((n * (n + 1) // 2 + np.maximum(lq - lkv, 0) * lkv).sum())


def useful_flops(q_offsets, kv_offsets, H: int, D: int, causal: bool, backward: bool = True, window: int = 0,
                 block: int = 0) -> tuple[int, int]:
    """(forward FLOPs, backward FLOPs) credited to the useful pairs of one batch."""
    pairs = visible_pairs(q_offsets, kv_offsets, causal, window, block) * H
    return 4 * D * pairs, (10 * D * pairs if backward else 0)
