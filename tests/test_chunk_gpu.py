"""Fewer queries than keys (S_q < S_k, the queries being the last S_q positions) on the GPU,
through attn_fwd_qk / attn_bwd_qk.

* Small cases: every output against the fp64 oracle (ragged tails, grouped heads, windows,
  one-token decode, f32 and bf16).
* A chunk is a slice of the square problem: O, lse and dQ of the last S_q rows equal, bit for bit,
  what the square call over all S_k positions gives for those rows; dK and dV equal the square
  call's with dO zero on the other rows, bit for bit when the chunk starts on a query-tile
  boundary (the same tiles then accumulate in the same order, the extra ones adding exact zeros).
* Q = 0: round(exp(lse_i)) is exactly the number of keys visible from position i + S_k - S_q.
* Full-size prefill-chunk and decode workloads: sampled rows / key columns against the oracle.
"""
import math

import numpy as np
import pytest

import oracle
from causal_attention_fa2_amd.workloads import WORKLOADS, make_inputs, random_tensor
from gpu_util import assert_parity, download, run_hip, say, upload

pytestmark = pytest.mark.gpu

CASES = [
    # dtype, B, Hq, Hkv, Sq, Sk, D, causal, window
    ("f32", 1, 2, 2, 40, 64, 64, True, 0),
    ("f32", 1, 4, 2, 100, 300, 128, True, 0),
    ("f32", 1, 2, 1, 1, 257, 64, True, 0),
    ("f32", 1, 2, 2, 70, 130, 64, False, 0),
    ("f32", 1, 2, 2, 33, 200, 64, True, 50),
    ("bf16", 1, 2, 2, 1, 1, 64, True, 0),
    ("bf16", 1, 2, 2, 1, 300, 128, True, 0),
    ("bf16", 1, 8, 2, 1, 513, 64, True, 0),
    ("bf16", 2, 4, 2, 1, 300, 128, True, 100),
    ("bf16", 1, 4, 2, 63, 64, 128, True, 0),
    ("bf16", 1, 4, 2, 65, 300, 64, True, 0),
    ("bf16", 2, 4, 2, 128, 384, 128, True, 0),
    ("bf16", 1, 8, 2, 200, 1000, 128, True, 0),
    ("bf16", 1, 4, 4, 257, 700, 64, True, 64),
    ("bf16", 1, 4, 2, 300, 900, 128, True, 129),
    ("bf16", 1, 4, 2, 100, 1000, 64, True, 1),
    ("bf16", 1, 2, 2, 90, 400, 128, False, 0),
]


def _inputs(dtype, B, Hq, Hkv, Sq, Sk, D, seed):
    q = random_tensor((B, Hq, Sq, D), dtype, seed)
    k = random_tensor((B, Hkv, Sk, D), dtype, seed + 1)
    v = random_tensor((B, Hkv, Sk, D), dtype, seed + 2)
    do = random_tensor((B, Hq, Sq, D), dtype, seed + 3)
    return q, k, v, do


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(map(str, c)))
def test_chunk_small_parity(case):
    dtype, B, Hq, Hkv, Sq, Sk, D, causal, window = case
    say(f"chunk case {case}")
    q, k, v, do = _inputs(dtype, B, Hq, Hkv, Sq, Sk, D, seed=Sq * 13 + Sk)
    scale = 1.0 / math.sqrt(D)
    got = run_hip(q, k, v, do, dtype, causal, window, scale)
    ref = oracle.forward_backward(q, k, v, do, causal, window, scale)
    assert_parity(got, ref, dtype, tag=str(case))
    if causal and window and Sk - Sq >= window:
        # keys no query can see: exact zeros
        first = Sk - Sq - window + 1
        assert np.all(got["dK"][:, :, :first] == 0.0) and np.all(got["dV"][:, :, :first] == 0.0)


@pytest.mark.parametrize("dtype,Hq,Hkv,Sq,Sk,D,window", [
    ("bf16", 4, 2, 128, 512, 128, 0),    # chunk on a query-tile boundary
    ("bf16", 4, 2, 100, 450, 64, 0),     # ragged: not on a tile boundary
    ("bf16", 4, 2, 256, 1024, 128, 200),
    ("bf16", 8, 2, 1, 700, 128, 0),
    # S_k = 2000: the rows' mean key count (1000) picks 4-wave workgroups; the chunk alone would
    # average 1950 keys per row, so the choice must not look at S_q
    ("bf16", 4, 2, 100, 2000, 128, 0),
    ("bf16", 4, 2, 1, 2000, 64, 0),
    ("f32", 2, 2, 96, 320, 64, 0),
    ("f32", 2, 1, 50, 260, 128, 70),
])
def test_chunk_is_bitwise_slice_of_square(dtype, Hq, Hkv, Sq, Sk, D, window):
    import torch
    import causal_attention_fa2_amd as fa
    say(f"chunk vs square {dtype} Hq={Hq} Hkv={Hkv} Sq={Sq} Sk={Sk} D={D} W={window}")
    off = Sk - Sq
    qf = random_tensor((1, Hq, Sk, D), dtype, 41)
    k = random_tensor((1, Hkv, Sk, D), dtype, 42)
    v = random_tensor((1, Hkv, Sk, D), dtype, 43)
    dof = random_tensor((1, Hq, Sk, D), dtype, 44)
    dof[:, :, :off] = 0.0
    tqf, tk, tv, tdof = (upload(x, dtype) for x in (qf, k, v, dof))
    tq = tqf[:, :, off:].contiguous()
    tdo = tdof[:, :, off:].contiguous()
    o_f, l_f = fa.forward(tqf, tk, tv, True, window)
    dq_f, dk_f, dv_f = fa.backward(tqf, tk, tv, o_f, l_f, tdof, True, window)
    o_c, l_c = fa.forward(tq, tk, tv, True, window)
    dq_c, dk_c, dv_c = fa.backward(tq, tk, tv, o_c, l_c, tdo, True, window)
    torch.cuda.synchronize()
    assert torch.equal(o_c, o_f[:, :, off:]), "O"
    assert torch.equal(l_c, l_f[:, :, off:]), "lse"
    assert torch.equal(dq_c, dq_f[:, :, off:]), "dQ"
    br = 64 if dtype == "bf16" else 32  # query rows per tile of the dK/dV pass
    if off % br == 0:
        assert torch.equal(dk_c, dk_f) and torch.equal(dv_c, dv_f), "dK / dV"
    else:
        for name, a, b in (("dK", dk_c, dk_f), ("dV", dv_c, dv_f)):
            e = (torch.linalg.vector_norm((a - b).double()) / torch.linalg.vector_norm(b.double())).item()
            say(f"  {name} chunk vs square rel-L2 {e:.2e}")
            assert e <= (1e-2 if dtype == "bf16" else 1e-5), name


@pytest.mark.parametrize("dtype,Sq,Sk,D,window", [
    ("bf16", 1, 300, 128, 0), ("bf16", 1, 300, 64, 40), ("bf16", 77, 300, 128, 0),
    ("bf16", 200, 1000, 64, 129), ("f32", 64, 257, 64, 0), ("bf16", 1000, 4096, 128, 0),
    ("bf16", 1, 8192, 64, 1024),
])
def test_chunk_zero_queries_count_visible_keys(dtype, Sq, Sk, D, window):
    say(f"chunk zero-Q counts {dtype} Sq={Sq} Sk={Sk} D={D} W={window}")
    q = np.zeros((1, 2, Sq, D), np.float32)
    k = random_tensor((1, 1, Sk, D), dtype, 1)
    v = random_tensor((1, 1, Sk, D), dtype, 2)
    got = run_hip(q, k, v, None, dtype, True, window, 1.0 / math.sqrt(D), want_bwd=False)
    p = np.arange(Sq) + Sk - Sq
    want = p + 1 if window == 0 else np.minimum(p + 1, window)
    for h in range(2):
        assert np.array_equal(np.rint(np.exp(got["LSE"][0, h])).astype(np.int64), want)


def test_qk_entry_point_equals_square_entry_point():
    """attn_fwd_qk / attn_bwd_qk with Sq == Sk give the same bits as attn_fwd / attn_bwd."""
    import torch
    import causal_attention_fa2_amd as fa
    dtype, Hq, Hkv, S, D = "bf16", 4, 2, 300, 128
    q, k, v, do = (upload(x, dtype) for x in _inputs(dtype, 1, Hq, Hkv, S, S, D, seed=5))
    o1, l1 = torch.empty_like(q), torch.empty((1, Hq, S), dtype=torch.float32, device="cuda")
    o2, l2 = torch.empty_like(o1), torch.empty_like(l1)
    fa.attn_fwd(q, k, v, o1, l1, True, 37)
    fa.attn_fwd_qk(q, k, v, o2, l2, True, 37)
    ws = torch.empty(fa.attn_bwd_qk_workspace_bytes(1, Hq, Hkv, S, S, D), dtype=torch.uint8,
                     device="cuda")
    g1 = [torch.empty_like(t) for t in (q, k, v)]
    g2 = [torch.empty_like(t) for t in (q, k, v)]
    fa.attn_bwd(q, k, v, o1, l1, do, *g1, ws, True, 37)
    fa.attn_bwd_qk(q, k, v, o1, l1, do, *g2, ws, True, 37)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)


def _sampled(w, q, k, v, do, got, rows_by_head, cols_by_group):
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
                  w.dtype, tag=w.name + " (sampled)")


@pytest.mark.parametrize("name", ["gqa64x8-q1024-k4096-d128", "gqa64x8-q1-k4096-d128"])
def test_chunk_workload_full_size_sampled(name):
    w = WORKLOADS[name]
    say(f"workload {name}: generating inputs")
    q, k, v, do = make_inputs(w)
    say(f"workload {name}: GPU forward + backward")
    got = run_hip(q, k, v, do, w.dtype, w.causal, w.window, w.scale)
    Sq, Sk = w.n_q, w.S
    rng = np.random.default_rng(8)
    base = [0, 1, 31, 32, 63, 64, Sq // 2, Sq - 2, Sq - 1]
    rows = {bh: [r for r in base if 0 <= r < Sq] + list(rng.integers(0, Sq, size=8))
            for bh in [(0, 0), (0, w.Hq - 1), (0, 29)]}
    cols = {bg: [0, 1, 127, 128, Sk - Sq - 1, Sk - Sq, Sk // 2, Sk - 1] + list(rng.integers(0, Sk, size=6))
            for bg in [(0, 0), (0, w.Hkv - 1)]}
    cols = {bg: [c for c in cs if 0 <= c < Sk] for bg, cs in cols.items()}
    say(f"workload {name}: oracle on samples")
    _sampled(w, q, k, v, do, got, rows, cols)
    # sum_j dK_j = 0 and sum_j dV_j = sum over the group of sum_i dO_i at any size
    B, Hkv, _, D = got["dK"].shape
    G = w.Hq // w.Hkv
    ek = np.sqrt(np.sum(got["dK"].sum(axis=2) ** 2)) / np.sqrt(np.sum(got["dK"] ** 2))
    want = do.astype(np.float64).reshape(B, Hkv, G, Sq, D).sum(axis=(2, 3))
    ev = np.sqrt(np.sum((got["dV"].sum(axis=2) - want) ** 2)) / np.sqrt(np.sum(got["dV"] ** 2))
    say(f"  identities {name}: |sum dK|/|dK|={ek:.2e} |sum dV - sum dO|/|dV|={ev:.2e}")
    assert ek <= 2e-2 and ev <= 2e-2
