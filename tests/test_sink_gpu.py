"""Sink keys beside the sliding window on the GPU (attn_fwd_qk / attn_bwd_qk with sink > 0).

* Small cases: every output against the fp64 oracle -- sink counts below, at and above a key tile,
  windows shorter and longer than a tile, S_q < S_k, grouped heads, f32 and bf16.
* Q = 0: round(exp(lse_i)) is exactly the size of the union of the window and the sink keys.
* Keys outside both the window and the sink range are bitwise irrelevant to a row.
* The full-size sliding-window workload with 4 sinks: sampled rows and key columns against the
  oracle, plus the dK / dV sum identities.
"""
import math

import numpy as np
import pytest

import oracle
from causal_attention_fa2_amd.workloads import WORKLOADS, make_inputs, random_tensor
from gpu_util import assert_parity, run_hip, say

pytestmark = pytest.mark.gpu

CASES = [
    # dtype, B, Hq, Hkv, Sq, Sk, D, window, sink
    ("f32", 1, 2, 2, 200, 200, 64, 16, 4),
    ("f32", 1, 4, 2, 90, 300, 128, 33, 40),
    ("bf16", 1, 2, 2, 300, 300, 128, 1, 1),
    ("bf16", 1, 4, 2, 384, 384, 64, 64, 4),
    ("bf16", 1, 4, 2, 400, 400, 128, 65, 63),
    ("bf16", 1, 4, 4, 500, 500, 64, 100, 64),
    ("bf16", 1, 2, 1, 700, 700, 128, 128, 65),
    ("bf16", 2, 4, 2, 640, 640, 128, 70, 130),
    ("bf16", 1, 8, 2, 1000, 1000, 64, 200, 256),
    ("bf16", 1, 4, 2, 120, 600, 128, 50, 8),
    ("bf16", 1, 8, 2, 1, 900, 128, 64, 4),
    ("bf16", 1, 4, 2, 65, 1100, 64, 300, 300),
]


def _inputs(dtype, B, Hq, Hkv, Sq, Sk, D, seed):
    q = random_tensor((B, Hq, Sq, D), dtype, seed)
    k = random_tensor((B, Hkv, Sk, D), dtype, seed + 1)
    v = random_tensor((B, Hkv, Sk, D), dtype, seed + 2)
    do = random_tensor((B, Hq, Sq, D), dtype, seed + 3)
    return q, k, v, do


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(map(str, c)))
def test_sink_small_parity(case):
    dtype, B, Hq, Hkv, Sq, Sk, D, window, sink = case
    say(f"sink case {case}")
    q, k, v, do = _inputs(dtype, B, Hq, Hkv, Sq, Sk, D, seed=Sq * 3 + sink)
    scale = 1.0 / math.sqrt(D)
    got = run_hip(q, k, v, do, dtype, True, window, scale, sink=sink)
    ref = oracle.forward_backward(q, k, v, do, True, window, scale, sink=sink)
    assert_parity(got, ref, dtype, tag=str(case))
    # keys that no query sees (after the sinks, before every window): exact zeros
    first_window_key = Sk - Sq - window + 1
    if first_window_key > sink:
        for name in ("dK", "dV"):
            assert np.all(got[name][:, :, sink:first_window_key] == 0.0), name


@pytest.mark.parametrize("dtype,Sq,Sk,D,window,sink", [
    ("bf16", 300, 300, 128, 16, 4), ("bf16", 300, 300, 64, 1, 64), ("bf16", 257, 257, 128, 64, 65),
    ("f32", 200, 200, 64, 33, 100), ("bf16", 100, 700, 128, 50, 3), ("bf16", 8192, 8192, 64, 1024, 4),
])
def test_sink_zero_queries_count_visible_keys(dtype, Sq, Sk, D, window, sink):
    say(f"sink zero-Q counts {dtype} Sq={Sq} Sk={Sk} D={D} W={window} sink={sink}")
    q = np.zeros((1, 2, Sq, D), np.float32)
    k = random_tensor((1, 1, Sk, D), dtype, 1)
    v = random_tensor((1, 1, Sk, D), dtype, 2)
    got = run_hip(q, k, v, None, dtype, True, window, 1.0 / math.sqrt(D), want_bwd=False, sink=sink)
    p = np.arange(Sq) + Sk - Sq
    lo = np.maximum(0, p - window + 1)
    want = (p - lo + 1) + np.minimum(sink, lo)
    for h in range(2):
        assert np.array_equal(np.rint(np.exp(got["LSE"][0, h])).astype(np.int64), want)


def test_sink_hidden_keys_are_bitwise_irrelevant():
    """Rows 500..520 with W = 100 and 5 sinks see keys 0..4 and 401..520 only: change every other
    K / V row and their O, lse and dQ keep every bit."""
    dtype, S, D, W, n = "bf16", 700, 128, 100, 5
    say("sink hidden keys")
    q = random_tensor((1, 4, S, D), dtype, 3)
    k = random_tensor((1, 2, S, D), dtype, 4)
    v = random_tensor((1, 2, S, D), dtype, 5)
    do = random_tensor((1, 4, S, D), dtype, 6)
    a = run_hip(q, k, v, do, dtype, True, W, sink=n)
    k2, v2 = k.copy(), v.copy()
    hidden = np.r_[np.arange(n, 401), np.arange(521, S)]
    k2[:, :, hidden] = random_tensor((1, 2, hidden.size, D), dtype, 7)
    v2[:, :, hidden] = random_tensor((1, 2, hidden.size, D), dtype, 8)
    b = run_hip(q, k2, v2, do, dtype, True, W, sink=n)
    rows = slice(500, 521)
    for name in ("O", "LSE", "dQ"):
        assert np.array_equal(a[name][:, :, rows], b[name][:, :, rows]), name


def test_sink_workload_full_size_sampled():
    w = WORKLOADS["swa-w1024-sink4-s8192"]
    say(f"workload {w.name}: generating inputs")
    q, k, v, do = make_inputs(w)
    say(f"workload {w.name}: GPU forward + backward")
    got = run_hip(q, k, v, do, w.dtype, w.causal, w.window, w.scale, sink=w.sink)
    rng = np.random.default_rng(9)
    S = w.S
    base = [0, 1, 3, 4, 63, 64, 1023, 1024, 1027, 1028, S // 2, S - 2, S - 1]
    rows = {bh: base + list(rng.integers(0, S, size=8)) for bh in [(0, 0), (0, w.Hq - 1), (0, 7)]}
    # sink key columns need every later row: keep their count small
    cols = {bg: [0, 3, 4, 5, 1000, S // 2, S - 1] for bg in [(0, 0), (0, w.Hkv - 1)]}
    say(f"workload {w.name}: oracle on samples")
    go, gl, gq, gk, gv, ro, rl, rq, rk, rv = ([] for _ in range(10))
    for (b, h), rr in rows.items():
        rr = np.asarray(sorted(set(rr)))
        O, L = oracle.rows_forward(q, k, v, b, h, rr, True, w.window, w.scale, sink=w.sink)
        dq = oracle.rows_dq(q, k, v, do, b, h, rr, True, w.window, w.scale, sink=w.sink)
        go.append(got["O"][b, h, rr]); ro.append(O)
        gl.append(got["LSE"][b, h, rr]); rl.append(L)
        gq.append(got["dQ"][b, h, rr]); rq.append(dq)
    for (b, g), cc in cols.items():
        cc = np.asarray(sorted(set(cc)))
        dk, dv = oracle.cols_dkdv(q, k, v, do, b, g, cc, True, w.window, w.scale, sink=w.sink)
        gk.append(got["dK"][b, g, cc]); rk.append(dk)
        gv.append(got["dV"][b, g, cc]); rv.append(dv)
    cat = np.concatenate
    assert_parity({"O": cat(go), "LSE": cat(gl), "dQ": cat(gq), "dK": cat(gk), "dV": cat(gv)},
                  {"O": cat(ro), "LSE": cat(rl), "dQ": cat(rq), "dK": cat(rk), "dV": cat(rv)},
                  w.dtype, tag=w.name + " (sampled)")
    B, Hkv, _, D = got["dK"].shape
    G = w.Hq // w.Hkv
    ek = np.sqrt(np.sum(got["dK"].sum(axis=2) ** 2)) / np.sqrt(np.sum(got["dK"] ** 2))
    want = do.astype(np.float64).reshape(B, Hkv, G, S, D).sum(axis=(2, 3))
    ev = np.sqrt(np.sum((got["dV"].sum(axis=2) - want) ** 2)) / np.sqrt(np.sum(got["dV"] ** 2))
    say(f"  identities {w.name}: |sum dK|/|dK|={ek:.2e} |sum dV - sum dO|/|dV|={ev:.2e}")
    assert ek <= 2e-2 and ev <= 2e-2


SPLIT_CASES = [
    # B, Hq, Hkv, S, D, window, sink: head group split in 4 / two batch rows / S not a multiple of 128
    # (D = 64 streams 128-row query tiles, D = 128 64-row tiles)
    (1, 8, 2, 1024, 128, 128, 4),
    (2, 4, 2, 768, 64, 64, 2),
    (1, 4, 4, 600, 128, 100, 1),
    (1, 4, 2, 1000, 64, 96, 3),
]


@pytest.mark.parametrize("case", SPLIT_CASES, ids=lambda c: "-".join(map(str, c)))
def test_sink_split_matches_unsplit(case):
    """The sink split of the dK/dV pass (workspace sized by attn_bwd_qk_workspace_bytes_for) against
    the unsplit pass (workspace of attn_bwd_qk_workspace_bytes) and the oracle. dQ and the dK/dV
    rows past the first 128-key tile do not depend on the split (bit-identical); the first tile's
    rows differ only in the order of their fp32 partial sums."""
    import torch
    import causal_attention_fa2_amd as fa
    from gpu_util import download, upload
    B, Hq, Hkv, S, D, window, sink = case
    dtype = "bf16"
    base = fa.attn_bwd_qk_workspace_bytes(B, Hq, Hkv, S, S, D)
    full = fa.attn_bwd_qk_workspace_bytes_for(B, Hq, Hkv, S, S, D, True, window, sink)
    assert full > base  # these shapes split
    say(f"sink split {case}: {base} / {full} bytes")
    q, k, v, do = _inputs(dtype, B, Hq, Hkv, S, S, D, seed=77 + S)
    scale = 1.0 / math.sqrt(D)
    tq, tk, tv, tdo = (upload(x, dtype) for x in (q, k, v, do))
    o, lse = fa.forward(tq, tk, tv, True, window, scale, sink=sink)
    res = {}
    for name, nbytes in (("unsplit", base), ("split", full)):
        ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        dq, dk, dv = fa.backward(tq, tk, tv, o, lse, tdo, True, window, scale, workspace=ws, sink=sink)
        torch.cuda.synchronize()
        res[name] = {"dQ": download(dq), "dK": download(dk), "dV": download(dv)}
    ref = oracle.forward_backward(q, k, v, do, True, window, scale, sink=sink)
    for name, got in res.items():
        assert_parity(got, ref, dtype, names=("dQ", "dK", "dV"), tag=name)
    assert np.array_equal(res["split"]["dQ"], res["unsplit"]["dQ"])
    for n in ("dK", "dV"):
        a, b = res["split"][n], res["unsplit"][n]
        assert np.array_equal(a[:, :, 128:], b[:, :, 128:]), n
        # first tile: the same fp32 sums in another order, then one rounding to bf16
        assert np.allclose(a[:, :, :128], b[:, :, :128], rtol=2.0 ** -7, atol=1e-6 * np.abs(b).max()), n
