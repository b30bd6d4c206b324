"""Parity of the HIP path (through the C ABI) with the fp64 oracle, on the GPU.

* Small cases: the oracle computes every output; shapes span several tiles with ragged tails,
  grouped heads, D = 64 / 128, f32 and bf16, windows around tile sizes, S = 1.
* Full-size workloads: the GPU runs the whole problem in the configuration the bench times; the
  oracle checks sampled rows (O, LSE, dQ) and sampled key columns (dK, dV) one by one, plus
  identities that hold at any size.
"""
import math

import numpy as np
import pytest

import oracle
from causal_attention_fa2_amd.workloads import WORKLOADS, make_inputs, random_tensor
from gpu_util import assert_parity, run_hip, say

pytestmark = pytest.mark.gpu

SMALL_CASES = [
    # dtype, B, Hq, Hkv, S, D, causal, window
    ("f32", 1, 2, 2, 64, 64, True, 0),       # the tiny f32 workload itself
    ("f32", 2, 4, 2, 300, 128, True, 0),
    ("f32", 1, 2, 1, 257, 64, True, 65),
    ("f32", 1, 2, 2, 130, 64, False, 0),
    ("bf16", 1, 2, 2, 1, 64, True, 0),
    ("bf16", 1, 2, 2, 63, 128, True, 0),
    ("bf16", 1, 2, 2, 65, 64, True, 0),
    ("bf16", 1, 2, 2, 130, 128, True, 0),
    ("bf16", 2, 4, 2, 300, 128, True, 0),
    ("bf16", 1, 8, 2, 300, 64, True, 0),
    ("bf16", 1, 4, 4, 263, 128, True, 1),
    ("bf16", 1, 4, 2, 384, 64, True, 63),
    ("bf16", 1, 4, 2, 384, 128, True, 64),
    ("bf16", 1, 4, 2, 385, 64, True, 65),
    ("bf16", 1, 2, 2, 500, 128, True, 200),
    ("bf16", 1, 2, 1, 190, 128, False, 0),
    # more than 1024 visible keys per row on average: the 8-wave (256-row) forward and dQ workgroups
    # (the cases above run the 4-wave ones)
    ("bf16", 1, 4, 2, 2200, 128, True, 0),
    ("bf16", 1, 2, 2, 2113, 64, True, 0),
    ("bf16", 1, 2, 1, 2600, 128, True, 1500),
    ("bf16", 1, 2, 2, 1100, 64, False, 0),
    # D = 64 dK/dV streams 128-row query tiles: windows and lengths either side of 128
    ("bf16", 1, 4, 2, 643, 64, True, 127),
    ("bf16", 2, 8, 2, 515, 64, True, 129),
    ("bf16", 1, 4, 1, 257, 64, True, 128),
    # enough heads x rows for the forward / dQ workgroups to take several query heads of a KV group
    # (at least 256 workgroups after packing): 4-wave and 8-wave workgroups, a ragged last tile, a
    # window, and a group of 16 heads split into several packed chunks
    ("f32", 8, 32, 4, 300, 64, True, 0),
    ("bf16", 8, 32, 4, 300, 128, True, 0),
    ("bf16", 2, 16, 2, 2200, 128, True, 0),
    ("bf16", 4, 32, 2, 1000, 64, True, 300),
]


def _small_inputs(dtype, B, Hq, Hkv, S, D, seed):
    q = random_tensor((B, Hq, S, D), dtype, seed)
    k = random_tensor((B, Hkv, S, D), dtype, seed + 1)
    v = random_tensor((B, Hkv, S, D), dtype, seed + 2)
    do = random_tensor((B, Hq, S, D), dtype, seed + 3)
    return q, k, v, do


@pytest.mark.parametrize("case", SMALL_CASES, ids=lambda c: "-".join(map(str, c)))
def test_small_full_parity(case):
    dtype, B, Hq, Hkv, S, D, causal, window = case
    say(f"case {case}")
    q, k, v, do = _small_inputs(dtype, B, Hq, Hkv, S, D, seed=S * 7 + D)
    scale = 1.0 / math.sqrt(D)
    got = run_hip(q, k, v, do, dtype, causal, window, scale)
    ref = oracle.forward_backward(q, k, v, do, causal, window, scale)
    assert_parity(got, ref, dtype, tag=str(case))


def test_small_mha_workload_full():
    """B=4, Hq=Hkv=16, S=1024, D=64 bf16, causal: every output against the oracle."""
    w = WORKLOADS["small-mha-causal-bf16"]
    q, k, v, do = make_inputs(w)
    got = run_hip(q, k, v, do, w.dtype, w.causal, w.window, w.scale)
    ref = oracle.forward_backward(q, k, v, do, w.causal, w.window, w.scale)
    assert_parity(got, ref, w.dtype, tag=w.name)


def _sampled_check(w, q, k, v, do, got, rows_by_head, cols_by_group, tag):
    """Oracle on sampled rows (O, LSE, dQ) and sampled key columns (dK, dV)."""
    go, gl, gq, gk, gv, ro, rl, rq, rk, rv = ([] for _ in range(10))
    for (b, h), rows in rows_by_head.items():
        rows = np.asarray(sorted(set(rows)))
        O, L = oracle.rows_forward(q, k, v, b, h, rows, w.causal, w.window, w.scale)
        dq = oracle.rows_dq(q, k, v, do, b, h, rows, w.causal, w.window, w.scale)
        go.append(got["O"][b, h, rows]); ro.append(O)
        gl.append(got["LSE"][b, h, rows]); rl.append(L)
        gq.append(got["dQ"][b, h, rows]); rq.append(dq)
    for (b, g), cols in cols_by_group.items():
        cols = np.asarray(sorted(set(cols)))
        dk, dv = oracle.cols_dkdv(q, k, v, do, b, g, cols, w.causal, w.window, w.scale)
        gk.append(got["dK"][b, g, cols]); rk.append(dk)
        gv.append(got["dV"][b, g, cols]); rv.append(dv)
    cat = np.concatenate
    assert_parity({"O": cat(go), "LSE": cat(gl), "dQ": cat(gq), "dK": cat(gk), "dV": cat(gv)},
                  {"O": cat(ro), "LSE": cat(rl), "dQ": cat(rq), "dK": cat(rk), "dV": cat(rv)},
                  w.dtype, tag=tag + " (sampled)")


def _identities(w, do, got, tag):
    """sum_j dK_j = 0 and sum_j dV_j = sum over the group of sum_i dO_i, for every (b, KV head)."""
    B, Hkv, S, D = got["dK"].shape
    G = w.Hq // w.Hkv
    sk = got["dK"].sum(axis=2)
    ek = np.sqrt(np.sum(sk ** 2)) / np.sqrt(np.sum(got["dK"] ** 2))
    sv = got["dV"].sum(axis=2)
    want = do.astype(np.float64).reshape(B, Hkv, G, S, D).sum(axis=(2, 3))
    ev = np.sqrt(np.sum((sv - want) ** 2)) / np.sqrt(np.sum(got["dV"] ** 2))
    say(f"  identities {tag}: |sum dK|/|dK|={ek:.2e} |sum dV - sum dO|/|dV|={ev:.2e}")
    assert ek <= 2e-2 and ev <= 2e-2


def _rows_sample(rng, S, tile=128):
    base = [0, 1, 31, 32, tile - 1, tile, S // 2, S - 2, S - 1]
    return [r for r in base if 0 <= r < S] + list(rng.integers(0, S, size=12))


@pytest.mark.parametrize("name", ["gqa64x8-s4096-d128", "swa-w1024-s8192"])
def test_workload_full_size_sampled(name):
    w = WORKLOADS[name]
    say(f"workload {name}: generating inputs")
    q, k, v, do = make_inputs(w)
    say(f"workload {name}: GPU forward + backward")
    got = run_hip(q, k, v, do, w.dtype, w.causal, w.window, w.scale)
    rng = np.random.default_rng(5)
    heads = [(0, 0), (0, w.Hq - 1), (0, w.Hq // 2 + 1)]
    rows = {bh: _rows_sample(rng, w.S) for bh in heads}
    groups = [(0, 0), (0, w.Hkv - 1)]
    cols = {bg: [0, 1, 63, 64, 127, 128, w.S // 2, w.S - 1] + list(rng.integers(0, w.S, size=6))
            for bg in groups}
    say(f"workload {name}: oracle on samples")
    _sampled_check(w, q, k, v, do, got, rows, cols, name)
    _identities(w, do, got, name)


def test_long_context_workload_sampled():
    """B=1, Hq=64, Hkv=8, S=32768, D=128 with per-head U(0.5, 2) factors on Q and K."""
    w = WORKLOADS["gqa64x8-s32768-d128"]
    say("long-context workload: generating inputs")
    q, k, v, do = make_inputs(w)
    say("long-context workload: GPU forward + backward")
    got = run_hip(q, k, v, do, w.dtype, w.causal, w.window, w.scale)
    rng = np.random.default_rng(6)
    rows = {(0, h): _rows_sample(rng, w.S) for h in (0, 37, 63)}
    # a key column j needs every row i >= j: sample the last key tiles so the oracle stays cheap
    cols = {(0, g): [w.S - 1, w.S - 2, w.S - 33, w.S - 64, w.S - 100, w.S - 128]
            for g in (0, 5)}
    say("long-context workload: oracle on samples")
    _sampled_check(w, q, k, v, do, got, rows, cols, w.name)
    _identities(w, do, got, w.name)


@pytest.mark.timeout(900)
def test_long_context_early_key_columns():
    """The same workload: dK / dV of the first keys, element by element. Key tile 0 sums its
    gradient over every query tile of all 8 heads of a group (the longest fp32 accumulation of the
    pass); keys 0, 1, 127, 128 (key tiles 0 and 1), 4095 and 16384 of KV heads 0 and 5. The oracle
    needs every query row here (a whole group's softmax over 32768 keys)."""
    w = WORKLOADS["gqa64x8-s32768-d128"]
    say("long-context early keys: generating inputs")
    q, k, v, do = make_inputs(w)
    say("long-context early keys: GPU forward + backward")
    got = run_hip(q, k, v, do, w.dtype, w.causal, w.window, w.scale)
    cols = np.array([0, 1, 127, 128, 4095, 16384])

    for g in (0, 5):
        def progress(done, total):
            if done % 16 == 0 or done == total:
                say(f"  oracle, KV head {g}: {done}/{total} row blocks")
        dk, dv = oracle.cols_dkdv(q, k, v, do, 0, g, cols, w.causal, w.window, w.scale, progress=progress)
        assert_parity({"dK": got["dK"][0, g, cols], "dV": got["dV"][0, g, cols]}, {"dK": dk, "dV": dv},
                      w.dtype, tag=w.name + f" (keys 0..16384 of KV head {g})")
