"""Packed documents on the GPU (attn_fwd_varlen / attn_bwd_varlen).

* Every output against the fp64 oracle: documents of 1 .. 600 tokens, empty documents, boundaries
  inside and on key / query tiles, grouped heads, a window, f32 and bf16, rows of one batch with
  different document counts.
* One document spanning the row gives the same bits as attn_fwd / attn_bwd.
* Q = 0: round(exp(lse_i)) counts the keys from the document start (or the window start) to i.
* The full-size packed workload (6 documents in 8192 tokens): sampled rows / key columns against
  the oracle and the dK / dV sum identities.
"""
import math

import numpy as np
import pytest

import oracle
from causal_attention_fa2_amd.workloads import WORKLOADS, document_boundaries, make_inputs, random_tensor
from gpu_util import assert_parity, download, say, upload

pytestmark = pytest.mark.gpu


def _cu(lengths_per_row, S):
    n = max(len(x) for x in lengths_per_row)
    rows = []
    for lens in lengths_per_row:
        c = list(np.concatenate([[0], np.cumsum(lens)]))
        assert c[-1] == S
        rows.append(c + [S] * (n - len(lens)))
    return np.array(rows, dtype=np.int32)


def run_varlen(q, k, v, do, cu, dtype, window=0, scale=None, want_bwd=True):
    import torch
    import causal_attention_fa2_amd as fa
    tq, tk, tv = upload(q, dtype), upload(k, dtype), upload(v, dtype)
    tcu = torch.from_numpy(cu).cuda()
    B, Hq, S, D = q.shape
    o = torch.empty_like(tq)
    lse = torch.empty((B, Hq, S), dtype=torch.float32, device="cuda")
    fa.attn_fwd_varlen(tq, tk, tv, o, lse, tcu, window, scale)
    out = {}
    if want_bwd:
        tdo = upload(do, dtype)
        ws = torch.empty(max(1, fa.attn_bwd_workspace_bytes(B, Hq, k.shape[1], S, D)), dtype=torch.uint8,
                         device="cuda")
        dq, dk, dv = torch.empty_like(tq), torch.empty_like(tk), torch.empty_like(tv)
        fa.attn_bwd_varlen(tq, tk, tv, o, lse, tdo, dq, dk, dv, ws, tcu, window, scale)
        torch.cuda.synchronize()
        out.update(dQ=download(dq), dK=download(dk), dV=download(dv))
    torch.cuda.synchronize()
    out.update(O=download(o), LSE=lse.double().cpu().numpy())
    return out


CASES = [
    # dtype, Hq, Hkv, S, D, window, per-row document lengths
    ("f32", 2, 2, 200, 64, 0, [[50, 1, 99, 50]]),
    ("f32", 4, 2, 130, 128, 16, [[64, 66], [1, 1, 128]]),
    ("bf16", 4, 2, 300, 128, 0, [[100, 1, 199], [300]]),
    ("bf16", 4, 4, 513, 64, 0, [[64, 64, 0, 128, 257]]),
    ("bf16", 8, 2, 700, 128, 100, [[255, 1, 2, 3, 439]]),
    ("bf16", 2, 1, 640, 128, 0, [[7] * 80 + [80]]),
    ("bf16", 4, 2, 1024, 64, 0, [[512, 512], [1, 1023], [600, 424]]),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(map(str, c[:6])) + f"-{len(c[6][0])}docs")
def test_varlen_small_parity(case):
    dtype, Hq, Hkv, S, D, window, lens = case
    say(f"varlen case {case[:6]} docs {lens}")
    B = len(lens)
    cu = _cu(lens, S)
    q = random_tensor((B, Hq, S, D), dtype, S + 1)
    k = random_tensor((B, Hkv, S, D), dtype, S + 2)
    v = random_tensor((B, Hkv, S, D), dtype, S + 3)
    do = random_tensor((B, Hq, S, D), dtype, S + 4)
    scale = 1.0 / math.sqrt(D)
    got = run_varlen(q, k, v, do, cu, dtype, window, scale)
    ref = oracle.forward_backward(q, k, v, do, True, window, scale, cu_seqlens=cu)
    assert_parity(got, ref, dtype, tag=str(case[:6]))


def test_varlen_one_document_is_bitwise_plain():
    import torch
    import causal_attention_fa2_amd as fa
    dtype, Hq, Hkv, S, D = "bf16", 8, 2, 777, 128
    say("varlen one document vs plain")
    q, k, v, do = (random_tensor(shp, dtype, 80 + i) for i, shp in enumerate(
        [(1, Hq, S, D), (1, Hkv, S, D), (1, Hkv, S, D), (1, Hq, S, D)]))
    a = run_varlen(q, k, v, do, np.array([[0, S]], dtype=np.int32), dtype, 0)
    tq, tk, tv, tdo = upload(q, dtype), upload(k, dtype), upload(v, dtype), upload(do, dtype)
    o, lse = fa.forward(tq, tk, tv, True, 0)
    # the plain workspace: dQ recomputes the score tiles, as the packed-document pass always does
    # (a workspace with room for the stored dS changes dQ's rounding, not dK / dV)
    ws = torch.empty(fa.attn_bwd_workspace_bytes(1, Hq, Hkv, S, D), dtype=torch.uint8, device="cuda")
    dq, dk, dv = fa.backward(tq, tk, tv, o, lse, tdo, True, 0, workspace=ws)
    torch.cuda.synchronize()
    for name, t in (("O", o), ("LSE", lse), ("dQ", dq), ("dK", dk), ("dV", dv)):
        b = t.double().cpu().numpy()
        assert np.array_equal(a[name], b), name


@pytest.mark.parametrize("window", [0, 1, 40])
def test_varlen_zero_queries_count(window):
    dtype, S, D = "bf16", 900, 128
    say(f"varlen zero-Q counts W={window}")
    lens = [[1, 130, 0, 64, 300, 5, 400]]
    cu = _cu(lens, S)
    q = np.zeros((1, 2, S, D), np.float32)
    k = random_tensor((1, 1, S, D), dtype, 1)
    v = random_tensor((1, 1, S, D), dtype, 2)
    got = run_varlen(q, k, v, None, cu, dtype, window, 1.0 / math.sqrt(D), want_bwd=False)
    p = np.arange(S)
    start = cu[0][oracle.document_of(p, cu[0])]
    if window:
        start = np.maximum(start, p - window + 1)
    for h in range(2):
        assert np.array_equal(np.rint(np.exp(got["LSE"][0, h])).astype(np.int64), p - start + 1)


def test_varlen_workload_full_size_sampled():
    w = WORKLOADS["docs-gqa64x8-s8192-d128"]
    say(f"workload {w.name}: generating inputs")
    q, k, v, do = make_inputs(w)
    cu = document_boundaries(w)
    say(f"workload {w.name}: GPU forward + backward, documents {cu[0].tolist()}")
    got = run_varlen(q, k, v, do, cu, w.dtype, w.window, w.scale)
    rng = np.random.default_rng(11)
    S = w.S
    edges = [int(c) for c in cu[0][1:-1]]
    base = [0, 1, 63, 64] + [e - 1 for e in edges] + [e for e in edges] + [e + 1 for e in edges] + [S - 1]
    rows = {bh: base + list(rng.integers(0, S, size=6)) for bh in [(0, 0), (0, w.Hq - 1), (0, 21)]}
    cols = {bg: [0, 5] + [e - 1 for e in edges] + edges + [S - 1] for bg in [(0, 0), (0, w.Hkv - 1)]}
    say(f"workload {w.name}: oracle on samples")
    go, gl, gq, gk, gv, ro, rl, rq, rk, rv = ([] for _ in range(10))
    for (b, h), rr in rows.items():
        rr = np.asarray(sorted(set(rr)))
        O, L = oracle.rows_forward(q, k, v, b, h, rr, True, w.window, w.scale, cu_seqlens=cu)
        dqr = oracle.rows_dq(q, k, v, do, b, h, rr, True, w.window, w.scale, cu_seqlens=cu)
        go.append(got["O"][b, h, rr]); ro.append(O)
        gl.append(got["LSE"][b, h, rr]); rl.append(L)
        gq.append(got["dQ"][b, h, rr]); rq.append(dqr)
    for (b, g), cc in cols.items():
        cc = np.asarray(sorted(set(cc)))
        dk, dv = oracle.cols_dkdv(q, k, v, do, b, g, cc, True, w.window, w.scale, cu_seqlens=cu)
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
