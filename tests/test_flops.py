"""Useful-pair accounting (CPU): closed forms and a brute-force count under window / block limits."""
import numpy as np
import pytest

import jfa_inputs as ji
from jagged_sequence_amd.flops import useful_flops, visible_pairs
from oracle import attention as A


def _brute(lq, lkv, causal, window, block):
    n = 0
    for a, c in zip(lq, lkv):
        i, j = np.meshgrid(np.arange(a), np.arange(c), indexing="ij")
        n += int(A.visible(i, j, "causal" if causal else "none", window, block).sum())
    return n


@pytest.mark.parametrize("causal,window,block", [(True, 0, 0), (False, 0, 0), (True, 7, 0), (True, 0, 16),
                                                  (True, 100, 64), (False, 5, 0), (False, 0, 33), (False, 9, 20)])
def test_visible_pairs_brute_force(causal, window, block):
    lq = [0, 1, 37, 130, 257]
    lkv = lq if causal else [5, 300, 0, 64, 129]
    got = visible_pairs(ji.offsets(lq), ji.offsets(lkv), causal, window, block)
    assert got == _brute(lq, lkv, causal, window, block)


def test_closed_forms_and_workload_counts():
    assert visible_pairs(ji.offsets([4]), ji.offsets([4]), True) == 10
    assert visible_pairs(ji.offsets([3]), ji.offsets([5]), False) == 15
    # window 1 under causal: each row sees itself only
    assert visible_pairs(ji.offsets([50, 7]), ji.offsets([50, 7]), True, 1) == 57
    w = ji.WORKLOADS["causal_bucket"]
    lq, _ = ji.lengths(w)
    off = ji.offsets(lq)
    assert visible_pairs(off, off, True) * w.H == 165_926_884
    fw, bw = useful_flops(off, off, w.H, w.D, True)
    assert (fw, bw) == (4 * 128 * 165_926_884, 10 * 128 * 165_926_884)
