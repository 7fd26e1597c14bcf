"""Host-side pins of the workload definitions: the visible-pair counts that bench.py turns into
FLOPs agree with a brute-force count over the oracle's visibility rule."""
import numpy as np
import pytest

import oracle
from workloads import visible_pairs, workload


@pytest.mark.parametrize("causal,window", [(True, 0), (True, 1), (True, 7), (True, 50), (False, 0), (False, 1),
                                           (False, 7), (False, 50)])
def test_visible_pairs_brute_force(causal, window):
    lengths = (1, 13, 40, 0)
    brute = 0
    for L in lengths:
        i = np.arange(L)[:, None]
        j = np.arange(L)[None, :]
        brute += int(oracle.visible(i, j, causal, window).sum())
    assert visible_pairs(lengths, causal, window) == brute


def test_workload_table():
    assert visible_pairs(workload("causal4k").lengths, True, 0) == 4096 * 4097 // 2
    w = workload("band4k")
    assert not w.causal and w.window == 128
    # interior rows see 2W - 1 keys; the first and last W - 1 rows see fewer
    assert visible_pairs(w.lengths, False, 128) == 4096 * 255 - 2 * sum(range(1, 128))
