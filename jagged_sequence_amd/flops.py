"""Useful-work accounting: visible (query, key) pairs and the FLOPs credited to them.

Only unpadded, unmasked pairs count (the pages' point is that padding to the longest sequence
wastes compute; aihot.vn GEM page, "Jagged Sequence Flash Attention"). Per visible pair and head
the forward pass is credited 4 D FLOPs (two matrix products) and the backward pass 10 D (the
usual 2.5x of the forward, recomputation included).
"""
from __future__ import annotations

import numpy as np


def visible_pairs(q_offsets, kv_offsets, causal: bool) -> int:
    """Number of visible (i, j) pairs of one head summed over sequences."""
    qo = np.asarray(q_offsets, dtype=np.int64)
    ko = np.asarray(kv_offsets, dtype=np.int64)
    lq, lkv = np.diff(qo), np.diff(ko)
    if not causal:
        return int((lq * lkv).sum())
    n = np.minimum(lq, lkv)
    return int((n * (n + 1) // 2 + np.maximum(lq - lkv, 0) * lkv).sum())


def useful_flops(q_offsets, kv_offsets, H: int, D: int, causal: bool, backward: bool = True) -> tuple[int, int]:
    """(forward FLOPs, backward FLOPs) credited to the useful pairs of one batch."""
    pairs = visible_pairs(q_offsets, kv_offsets, causal) * H
    return 4 * D * pairs, (10 * D * pairs if backward else 0)
