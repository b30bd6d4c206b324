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


def test_cpu_sample_is_bounded():
    """The CPU-oracle sample keeps whole KV groups while it fits, then one group, one head and
    finally the last query rows, never above bench.CPU_SAMPLE_PAIRS attended pairs (documents aside)."""
    from causal_attention_fa2_amd.workloads import WORKLOADS
    # the S = 4096 headline: all 64 heads, every row (5.4e8 pairs)
    assert bench.cpu_sample(WORKLOADS["gqa64x8-s4096-d128"], 64)[:3] == (64, 8, 4096)
    # S = 32768: one query head of the first KV group, every row
    h, g, rows, pairs = bench.cpu_sample(WORKLOADS["gqa64x8-s32768-d128"], 64)
    assert (h, g, rows) == (1, 1, 32768) and pairs == 32768 * 32768 / 2  # S^2/2, the FLOP convention
    # whole groups are kept when they fit; --cpu-heads rounds to whole groups
    assert bench.cpu_sample(WORKLOADS["small-mha-causal-bf16"], 64)[:3] == (16, 16, 1024)
    assert bench.cpu_sample(WORKLOADS["gqa64x8-s4096-d128"], 20)[:3] == (16, 2, 4096)
    for name, w in WORKLOADS.items():
        if w.docs or w.paged or w.decode:
            continue
        h, g, rows, pairs = bench.cpu_sample(w, 64)
        assert 1 <= rows <= w.n_q and 1 <= h <= w.Hq and 1 <= g <= w.Hkv, name
        assert w.B * h * pairs <= bench.CPU_SAMPLE_PAIRS or rows <= 64, name
        assert pairs == bench.attended_pairs(w.S, w.causal, w.window, rows, w.sink), name
