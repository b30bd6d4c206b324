"""bench.py's host-side bookkeeping (CPU only): the attended-pair count behind its FLOP figures,
against counts of the oracle's element-wise mask."""
import numpy as np
import pytest

import bench
import oracle


@pytest.mark.parametrize("S,Sq,causal,window,sink", [
    (64, 64, False, 0, 0), (300, 300, True, 0, 0), (300, 300, True, 40, 0), (300, 100, True, 40, 0),
    (300, 1, True, 0, 0), (257, 100, True, 0, 0), (50, 7, True, 64, 0), (130, 70, False, 0, 0),
    (512, 512, True, 1, 0), (300, 300, True, 40, 4), (300, 100, True, 40, 64), (300, 1, True, 16, 3),
    (90, 90, True, 8, 200), (512, 512, True, 1, 1),
])
def test_attended_pairs(S, Sq, causal, window, sink):
    exact = oracle.visible_mask(np.arange(Sq), np.arange(S), causal, window, S - Sq, sink).sum()
    got = bench.attended_pairs(S, causal, window, Sq, sink)
    if causal and window == 0:
        # the S^2/2 convention: the exact count less half a pair per query row (the diagonal)
        assert got == exact - Sq / 2.0
    else:
        assert got == exact
