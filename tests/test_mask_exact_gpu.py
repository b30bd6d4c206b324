"""Bit-exact checks of the kernels' mask and index logic, and run-to-run determinism.

These hold exactly (integer compares or bitwise equality), whatever the floating-point order:
  * Q = 0: every visible score is 0, so the row sum is exactly the number of visible keys and
    round(exp(lse_i)) equals it;
  * keys a row cannot see (future, or outside the window) can be changed arbitrarily without
    changing that row's O, lse or dQ by a single bit;
  * a one-hot dO (one row of one head) gives exactly zero dK / dV for every key that row cannot
    see and exactly zero dQ for every other row;
  * f32 path with Q = 0 and V[j, 0] = j: O_i[0] is the mean of the visible key indices, so
    round(2 O_i[0] - i) is the first visible key;
  * two runs give bitwise identical outputs (no atomics anywhere).
"""
import math

import numpy as np
import pytest

from causal_attention_fa2_amd.workloads import random_tensor, to_elem
from gpu_util import run_hip, say

pytestmark = pytest.mark.gpu


def _count(S, causal, window):
    i = np.arange(S)
    if not causal:
        return np.full(S, S)
    return i + 1 if window == 0 else np.minimum(i + 1, window)


@pytest.mark.parametrize("dtype,S,D,window", [
    ("bf16", 300, 128, 0), ("bf16", 300, 64, 1), ("bf16", 300, 128, 63), ("bf16", 300, 64, 64),
    ("bf16", 300, 128, 65), ("f32", 200, 64, 0), ("f32", 257, 128, 100),
    ("bf16", 4096, 128, 0), ("bf16", 8192, 64, 1024),
])
def test_zero_queries_count_visible_keys(dtype, S, D, window):
    say(f"zero-Q counts {dtype} S={S} D={D} W={window}")
    q = np.zeros((1, 2, S, D), np.float32)
    k = random_tensor((1, 1, S, D), dtype, 1)
    v = random_tensor((1, 1, S, D), dtype, 2)
    got = run_hip(q, k, v, None, dtype, True, window, 1.0 / math.sqrt(D), want_bwd=False)
    want = _count(S, True, window)
    for h in range(2):
        assert np.array_equal(np.rint(np.exp(got["LSE"][0, h])).astype(np.int64), want)


@pytest.mark.parametrize("dtype,S,D,window,lo,hi", [
    ("bf16", 300, 128, 0, 0, 150), ("bf16", 300, 64, 0, 100, 131), ("bf16", 400, 128, 70, 200, 260),
    ("f32", 260, 64, 33, 90, 97), ("bf16", 1000, 64, 128, 700, 703),
])
def test_hidden_keys_are_bitwise_irrelevant(dtype, S, D, window, lo, hi):
    """Rows lo..hi cannot see keys > hi nor keys < lo - window + 1: change those K and V rows."""
    say(f"hidden keys {dtype} S={S} D={D} W={window} rows {lo}..{hi}")
    q = random_tensor((1, 4, S, D), dtype, 3)
    k = random_tensor((1, 2, S, D), dtype, 4)
    v = random_tensor((1, 2, S, D), dtype, 5)
    do = random_tensor((1, 4, S, D), dtype, 6)
    a = run_hip(q, k, v, do, dtype, True, window)
    k2, v2 = k.copy(), v.copy()
    hidden = np.arange(S) > hi
    if window:
        hidden |= np.arange(S) < lo - window + 1
    k2[:, :, hidden] = random_tensor(k2[:, :, hidden].shape, dtype, 7, std=3.0)
    v2[:, :, hidden] = to_elem(random_tensor(v2[:, :, hidden].shape, dtype, 8) - 4, dtype)
    b = run_hip(q, k2, v2, do, dtype, True, window)
    rows = slice(lo, hi + 1)
    for n in ("O", "LSE", "dQ"):
        assert np.array_equal(a[n][:, :, rows], b[n][:, :, rows]), n


@pytest.mark.parametrize("dtype,S,D,window,h0,i0", [
    ("bf16", 300, 128, 0, 3, 200), ("bf16", 300, 64, 40, 1, 150), ("f32", 200, 64, 0, 0, 77),
    ("bf16", 129, 128, 1, 2, 128),
])
def test_one_hot_dout(dtype, S, D, window, h0, i0):
    say(f"one-hot dO {dtype} S={S} D={D} W={window} head {h0} row {i0}")
    Hq, Hkv = 4, 2
    q = random_tensor((1, Hq, S, D), dtype, 9)
    k = random_tensor((1, Hkv, S, D), dtype, 10)
    v = random_tensor((1, Hkv, S, D), dtype, 11)
    do = np.zeros((1, Hq, S, D), np.float32)
    do[0, h0, i0] = random_tensor((D,), dtype, 12)
    got = run_hip(q, k, v, do, dtype, True, window)
    g0 = h0 // (Hq // Hkv)
    j = np.arange(S)
    seen = (j <= i0) & ((window == 0) | (i0 - j < window))
    assert np.all(got["dK"][0, g0, ~seen] == 0) and np.all(got["dV"][0, g0, ~seen] == 0)
    other = [g for g in range(Hkv) if g != g0]
    assert np.all(got["dK"][0, other] == 0) and np.all(got["dV"][0, other] == 0)
    mask = np.ones((Hq, S), bool)
    mask[h0, i0] = False
    assert np.all(got["dQ"][0][mask] == 0)
    assert np.any(got["dV"][0, g0, seen] != 0)


@pytest.mark.parametrize("S,D,window", [(300, 64, 0), (1000, 128, 77), (4096, 64, 0), (513, 128, 1)])
def test_f32_first_visible_index(S, D, window):
    say(f"f32 index mean S={S} D={D} W={window}")
    q = np.zeros((1, 1, S, D), np.float32)
    k = random_tensor((1, 1, S, D), "f32", 13)
    v = random_tensor((1, 1, S, D), "f32", 14)
    v[0, 0, :, 0] = np.arange(S, dtype=np.float32)
    got = run_hip(q, k, v, None, "f32", True, window, want_bwd=False)
    i = np.arange(S)
    lo = np.zeros(S, np.int64) if window == 0 else np.maximum(0, i - window + 1)
    assert np.array_equal(np.rint(2 * got["O"][0, 0, :, 0] - i).astype(np.int64), lo)


@pytest.mark.parametrize("dtype,B,Hq,Hkv,S,D,window", [
    ("bf16", 1, 8, 2, 700, 128, 0), ("bf16", 2, 4, 4, 333, 64, 100), ("f32", 1, 2, 1, 200, 64, 0),
])
def test_deterministic(dtype, B, Hq, Hkv, S, D, window):
    q = random_tensor((B, Hq, S, D), dtype, 15)
    k = random_tensor((B, Hkv, S, D), dtype, 16)
    v = random_tensor((B, Hkv, S, D), dtype, 17)
    do = random_tensor((B, Hq, S, D), dtype, 18)
    a = run_hip(q, k, v, do, dtype, True, window)
    b = run_hip(q, k, v, do, dtype, True, window)
    for n in a:
        assert np.array_equal(a[n], b[n]), n
