"""Pins for the fp64 oracle: checks against facts the mathematics fixes, independent of the
oracle's own code. Each pin takes the oracle module `A` (oracle.attention, or a copy with a
planted mistake) and raises AssertionError when the oracle disagrees.

Kinds of pin used (each chosen so a plausible mistake -- a dropped term, a wrong sign or index,
a transposed operand, an off-by-one mask -- fails at least one of them):
  * central finite differences of L = sum(O * dO) (the backward is the derivative of the forward);
  * a scalar brute force on tiny inputs that takes the softmax derivative through its full
    Jacobian instead of the rowsum(dO * O) shortcut;
  * torch's own float64 scaled_dot_product_attention and autograd on the CPU (a library routine);
  * closed forms: constant V, identical keys, window 1, zero queries, a hand-derived three-token case;
  * invariants: probability rows sum to 1, sum_j dS_ij = 0, sum_j dV_j = sum_i dO_i, keys outside
    a row's visible set cannot change that row;
  * fewer queries than keys (S_q < S_k): a chunk of queries equals the last S_q rows of the square
    problem over all S_k positions (gradients with dO zero on the other rows), torch's own
    lower-right causal bias, and a single decode query that sees every key (or the last W);
  * sink keys with a window: a decode query equals plain attention over the sink keys and the last
    W keys cut out and concatenated; sinks covering every key give plain causal attention; zero-query
    counts are the size of the union of the window and the sink range;
  * paged caches: an identity block layout reproduces the dense result exactly, shuffling the
    physical blocks (with the table) changes no bit, sequences of different lengths equal their
    own dense problems, and blocks shared by two sequences serve both;
  * packed documents: the packed result equals each document run as its own sequence (all five
    tensors), one document equals plain attention, one-token documents give O = V, and zero-query
    counts restart at every boundary.
"""
from __future__ import annotations

import math
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))


def _rng_inputs(seed, B, Hq, Hkv, S, D, std=1.0, Sk=None):
    """Q / dO have S rows, K / V have Sk (default S)."""
    Sk = S if Sk is None else Sk
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, Hq, S, D)) * std
    k = rng.standard_normal((B, Hkv, Sk, D)) * std
    v = rng.standard_normal((B, Hkv, Sk, D))
    do = rng.standard_normal((B, Hq, S, D))
    return q, k, v, do


def _loss(A, q, k, v, do, causal, window, scale):
    O, _ = A.forward(q, k, v, causal, window, scale)
    return float(np.sum(O * do))


# ---------------------------------------------------------------- finite differences
def pin_fd_every_entry(A, Hq=2, Hkv=2, S=16, D=8, window=0, seed=0, tol=1e-6):
    """Central differences on every entry of Q, K and V (h = 1e-6, float64)."""
    q, k, v, do = _rng_inputs(seed, 1, Hq, Hkv, S, D)
    scale = 1.0 / math.sqrt(D)
    dQ, dK, dV = A.backward(q, k, v, do, True, window, scale)
    h = 1e-6
    for name, x, g in (("Q", q, dQ), ("K", k, dK), ("V", v, dV)):
        fd = np.zeros_like(x)
        flat = x.reshape(-1)
        for idx in range(flat.size):
            old = flat[idx]
            flat[idx] = old + h
            lp = _loss(A, q, k, v, do, True, window, scale)
            flat[idx] = old - h
            lm = _loss(A, q, k, v, do, True, window, scale)
            flat[idx] = old
            fd.reshape(-1)[idx] = (lp - lm) / (2 * h)
        err = np.max(np.abs(fd - g)) / max(np.max(np.abs(fd)), 1e-30)
        assert err <= tol, f"finite differences vs d{name}: max rel err {err:.3e} > {tol}"


def pin_fd_sampled(A, seed=1, n_entries=256, n_dirs=16, tol=1e-6):
    """Tiny causal f32-workload shape (B=1, Hq=Hkv=2, S=64, D=64): central differences on a
    seeded sample of entries and along random directions, for each of Q, K, V."""
    q, k, v, do = _rng_inputs(seed, 1, 2, 2, 64, 64)
    scale = 1.0 / 8.0
    dQ, dK, dV = A.backward(q, k, v, do, True, 0, scale)
    rng = np.random.default_rng(seed + 100)
    h = 1e-6
    for name, x, g in (("Q", q, dQ), ("K", k, dK), ("V", v, dV)):
        flat = x.reshape(-1)
        gf = g.reshape(-1)
        idxs = rng.choice(flat.size, size=n_entries, replace=False)
        errs = []
        for idx in idxs:
            old = flat[idx]
            flat[idx] = old + h
            lp = _loss(A, q, k, v, do, True, 0, scale)
            flat[idx] = old - h
            lm = _loss(A, q, k, v, do, True, 0, scale)
            flat[idx] = old
            errs.append(abs((lp - lm) / (2 * h) - gf[idx]))
        gscale = np.max(np.abs(gf))
        err = max(errs) / gscale
        assert err <= tol, f"sampled finite differences d{name}: {err:.3e}"
        for _ in range(n_dirs):
            dirn = rng.standard_normal(x.shape)
            x0 = x.copy()
            x[...] = x0 + h * dirn
            lp = _loss(A, q, k, v, do, True, 0, scale)
            x[...] = x0 - h * dirn
            lm = _loss(A, q, k, v, do, True, 0, scale)
            x[...] = x0
            fd = (lp - lm) / (2 * h)
            an = float(np.sum(g * dirn))
            rel = abs(fd - an) / max(abs(an), 1e-12)
            assert rel <= 1e-5, f"directional derivative d{name}: rel err {rel:.3e}"


# ---------------------------------------------------------------- scalar brute force
def _brute(q, k, v, do, causal, window, scale, sink=0, cu=None):
    """Pure-Python loops; softmax derivative through the full Jacobian dP_k/dx_j = P_k (d_kj - P_j).
    With Sq queries and Sk keys, query i stands at position i + Sk - Sq."""
    B, Hq, S, D = q.shape
    Hkv, Sk = k.shape[1], k.shape[2]
    G = Hq // Hkv
    O = np.zeros(q.shape)
    L = np.zeros((B, Hq, S))
    dQ = np.zeros(q.shape)
    dK = np.zeros(k.shape)
    dV = np.zeros(v.shape)
    for b in range(B):
        for h in range(Hq):
            g = h // G
            for i in range(S):
                pos = i + Sk - S
                vis = [j for j in range(Sk)
                       if (not causal or j <= pos) and (window == 0 or pos - j < window or j < sink)]
                if cu is not None:  # same document: the last boundary at or before each position
                    doc = lambda t: max(c for c in range(len(cu[b]) - 1) if cu[b][c] <= t)  # noqa: E731
                    vis = [j for j in vis if doc(j) == doc(pos)]
                x = {j: scale * sum(q[b, h, i, d] * k[b, g, j, d] for d in range(D)) for j in vis}
                mx = max(x.values())
                z = sum(math.exp(x[j] - mx) for j in vis)
                p = {j: math.exp(x[j] - mx) / z for j in vis}
                L[b, h, i] = mx + math.log(z)
                for d in range(D):
                    O[b, h, i, d] = sum(p[j] * v[b, g, j, d] for j in vis)
                dp = {j: sum(do[b, h, i, d] * v[b, g, j, d] for d in range(D)) for j in vis}
                dx = {j: sum(dp[kk] * p[kk] * ((1.0 if kk == j else 0.0) - p[j]) for kk in vis)
                      for j in vis}
                for j in vis:
                    for d in range(D):
                        dQ[b, h, i, d] += scale * dx[j] * k[b, g, j, d]
                        dK[b, g, j, d] += scale * dx[j] * q[b, h, i, d]
                        dV[b, g, j, d] += p[j] * do[b, h, i, d]
    return O, L, dQ, dK, dV


def pin_bruteforce(A, tol=1e-12):
    for (B, Hq, Hkv, S, Sk, D, causal, window, seed, sink) in (
        (1, 2, 2, 7, 7, 3, True, 0, 3, 0), (2, 4, 2, 9, 9, 4, True, 3, 4, 0), (1, 3, 1, 6, 6, 2, False, 0, 5, 0),
        (1, 4, 4, 8, 8, 5, True, 1, 6, 0), (1, 2, 1, 5, 5, 3, True, 9, 7, 0),
        (1, 2, 1, 3, 8, 3, True, 0, 8, 0), (2, 4, 2, 4, 9, 2, True, 3, 9, 0), (1, 2, 2, 1, 6, 3, True, 0, 10, 0),
        (1, 2, 1, 1, 7, 2, True, 2, 14, 0), (1, 3, 3, 4, 6, 2, False, 0, 15, 0),
        (1, 2, 1, 9, 9, 3, True, 2, 16, 2), (2, 2, 2, 5, 10, 2, True, 3, 17, 1), (1, 4, 2, 10, 10, 2, True, 1, 18, 3),
        (1, 2, 1, 1, 9, 3, True, 2, 19, 3),
    ):
        q, k, v, do = _rng_inputs(seed, B, Hq, Hkv, S, D, Sk=Sk)
        scale = 0.7
        r = A.forward_backward(q, k, v, do, causal, window, scale, sink=sink)
        ref = _brute(q, k, v, do, causal, window, scale, sink)
        for name, x, y in zip(("O", "LSE", "dQ", "dK", "dV"),
                              (r["O"], r["LSE"], r["dQ"], r["dK"], r["dV"]), ref):
            err = np.max(np.abs(x - y)) / max(np.max(np.abs(y)), 1e-30)
            assert err <= tol, (f"brute force {name} (S={S}, Sk={Sk}, W={window}, causal={causal}, "
                                f"sink={sink}): {err:.3e}")


# ---------------------------------------------------------------- library routine
def pin_torch_sdpa(A, tol=1e-12):
    """torch.nn.functional.scaled_dot_product_attention in float64 on the CPU, K/V repeated
    over contiguous head groups, gradients through autograd."""
    import torch
    for (B, Hq, Hkv, S, D, causal, window, seed) in (
        (2, 4, 2, 33, 16, True, 0, 11), (1, 8, 2, 40, 8, True, 7, 12), (1, 2, 2, 24, 8, False, 0, 13),
    ):
        q, k, v, do = _rng_inputs(seed, B, Hq, Hkv, S, D)
        scale = 1.0 / math.sqrt(D)
        r = A.forward_backward(q, k, v, do, causal, window, scale)
        G = Hq // Hkv
        tq = torch.tensor(q, requires_grad=True)
        tk = torch.tensor(k, requires_grad=True)
        tv = torch.tensor(v, requires_grad=True)
        i = torch.arange(S)[:, None]
        j = torch.arange(S)[None, :]
        mask = torch.ones(S, S, dtype=torch.bool)
        if causal:
            mask &= j <= i
        if window:
            mask &= (i - j) < window
        o = torch.nn.functional.scaled_dot_product_attention(
            tq, tk.repeat_interleave(G, dim=1), tv.repeat_interleave(G, dim=1),
            attn_mask=mask, scale=scale)
        o.backward(torch.tensor(do))
        for name, x, y in (("O", r["O"], o.detach().numpy()), ("dQ", r["dQ"], tq.grad.numpy()),
                           ("dK", r["dK"], tk.grad.numpy()), ("dV", r["dV"], tv.grad.numpy())):
            err = np.max(np.abs(x - y)) / max(np.max(np.abs(y)), 1e-30)
            assert err <= tol, f"torch sdpa {name} (Hq={Hq}, Hkv={Hkv}, W={window}): {err:.3e}"


# ---------------------------------------------------------------- closed forms
def pin_three_token_closed_form(A, tol=1e-14):
    q = np.zeros((1, 1, 3, 2))
    q[..., 0] = 1.0
    k = np.zeros((1, 1, 3, 2))
    k[0, 0, :, 0] = np.log([1.0, 2.0, 3.0])
    v = np.array([[1.0, 0.0], [0.0, 1.0], [1.0, 1.0]]).reshape(1, 1, 3, 2)
    do = np.zeros((1, 1, 3, 2))
    do[..., 0] = 1.0
    r = A.forward_backward(q, k, v, do, True, 0, 2.0)
    n = 0
    with open(os.path.join(HERE, "golden", "three_token_closed_form.txt")) as f:
        for line in f:
            if not line.strip() or line.startswith("#"):
                continue
            name, idx, comp, expr = line.split(None, 3)
            want = float(eval(expr, {"math": math}))  # fixture expressions are plain arithmetic
            got = r[name][0, 0, int(idx)] if comp == "-" else r[name][0, 0, int(idx), int(comp)]
            assert abs(got - want) <= tol * max(1.0, abs(want)), f"{name}[{idx},{comp}]: {got} != {want}"
            n += 1
    assert n == 27


def pin_constant_v(A):
    q, k, v, do = _rng_inputs(21, 1, 4, 2, 37, 8)
    v[:] = np.array([0.5, -1.0, 2.0, 0.0, 3.0, 1.0, -2.0, 0.25])
    for window in (0, 1, 5):
        O, _ = A.forward(q, k, v, True, window, 0.4)
        assert np.max(np.abs(O - v[0, 0, 0])) <= 1e-14, f"constant V (W={window})"


def pin_identical_keys(A):
    """All keys equal => uniform weights over the visible set: O_i is the mean of the visible
    V rows and LSE_i = s<q_i, k> + ln(#visible)."""
    S, D = 50, 6
    q, k, v, do = _rng_inputs(22, 1, 2, 1, S, D)
    k[:] = k[0, 0, 0]
    scale = 0.3
    for window in (0, 1, 4, 64):
        O, LSE = A.forward(q, k, v, True, window, scale)
        for h in range(2):
            for i in range(S):
                lo = 0 if window == 0 else max(0, i - window + 1)
                want = v[0, 0, lo:i + 1].mean(axis=0)
                assert np.max(np.abs(O[0, h, i] - want)) <= 1e-13, f"identical keys O (W={window})"
                wl = scale * float(q[0, h, i] @ k[0, 0, 0]) + math.log(i + 1 - lo)
                assert abs(LSE[0, h, i] - wl) <= 1e-13, f"identical keys LSE (W={window})"


def pin_window_one(A):
    """W = 1: each query sees only its own key, so P = I, O_i = V_i, LSE_i = s<q_i, k_i>,
    dV_j = sum over the group of dO_j, and dQ = dK = 0."""
    q, k, v, do = _rng_inputs(23, 2, 4, 2, 19, 8)
    r = A.forward_backward(q, k, v, do, True, 1, 0.5)
    G = 2
    for h in range(4):
        g = h // G
        assert np.max(np.abs(r["O"][:, h] - v[:, g])) <= 1e-14
        lse = 0.5 * np.einsum("bsd,bsd->bs", q[:, h], k[:, g])
        assert np.max(np.abs(r["LSE"][:, h] - lse)) <= 1e-13
    dv = do.reshape(2, 2, G, 19, 8).sum(axis=2)
    assert np.max(np.abs(r["dV"] - dv)) <= 1e-13
    assert np.max(np.abs(r["dQ"])) <= 1e-13 and np.max(np.abs(r["dK"])) <= 1e-13


def pin_zero_queries(A):
    """Q = 0: every visible score is 0, so exp(LSE_i) is exactly the number of visible keys
    (p+1 causal, min(p+1, W) with a window, S_k without the causal mask, where p = i + S_k - S_q
    is the query's position) and O_i is their mean."""
    D = 4
    for S, Sk in ((70, 70), (20, 70), (1, 70)):
        q, k, v, do = _rng_inputs(24, 1, 2, 2, S, D, Sk=Sk)
        q[:] = 0.0
        for causal, window in ((True, 0), (True, 1), (True, 63), (True, 64), (True, 65), (False, 0)):
            O, LSE = A.forward(q, k, v, causal, window, 1.0)
            p = np.arange(S) + Sk - S
            if not causal:
                count = np.full(S, Sk)
            elif window == 0:
                count = p + 1
            else:
                count = np.minimum(p + 1, window)
            assert np.array_equal(np.rint(np.exp(LSE[0, 0])).astype(np.int64), count), (S, causal, window)
            hi = p + 1 if causal else np.full(S, Sk)
            lo = hi - count
            for i in (0, S // 2, S - 1):
                want = v[0, 0, lo[i]:hi[i]].mean(axis=0)
                assert np.max(np.abs(O[0, 0, i] - want)) <= 1e-14, (S, causal, window, i)


# ---------------------------------------------------------------- invariants
def pin_rows_sum_to_one(A):
    q, k, v, do = _rng_inputs(25, 1, 4, 2, 45, 8, std=2.0)
    for window in (0, 3, 17):
        for h in range(4):
            P = A.probabilities(q, k, 0, h, True, window, 0.5)
            assert np.max(np.abs(P.sum(axis=1) - 1.0)) <= 1e-14
            i = np.arange(45)[:, None]
            j = np.arange(45)[None, :]
            hidden = (j > i) | ((window > 0) & (i - j >= window))
            assert np.all(P[hidden] == 0.0) and np.all(P[~hidden] > 0.0)


def pin_gradient_identities(A):
    """sum_j dS_ij = 0 (softmax rows sum to a constant), hence sum_j dK_j = 0 per KV head;
    sum_j dV_j = sum over the group's heads and rows of dO (probability rows sum to 1)."""
    q, k, v, do = _rng_inputs(26, 2, 6, 2, 41, 8)
    r = A.forward_backward(q, k, v, do, True, 9, 0.35)
    assert np.max(np.abs(r["dK"].sum(axis=2))) <= 1e-12 * np.max(np.abs(r["dK"])) * 41
    want = do.reshape(2, 2, 3, 41, 8).sum(axis=(2, 3))
    assert np.max(np.abs(r["dV"].sum(axis=2) - want)) <= 1e-12
    qh = q[0, 1]
    t = A.head_rows(qh, k[0, 0], v[0, 0], np.arange(41), True, 9, 0.35, do[0, 1])
    assert np.max(np.abs(t["dS"].sum(axis=1))) <= 1e-15 * 41 * np.max(np.abs(t["dP"]))
    # delta_i equals <dO_i, O_i>
    assert np.max(np.abs(t["delta"] - np.sum(do[0, 1] * t["O"], axis=1))) <= 1e-13


def pin_gqa_is_repeated_mha(A):
    """Grouped heads equal full multi-head attention with K/V repeated over contiguous groups;
    dK/dV are the group sums of the multi-head dK/dV."""
    q, k, v, do = _rng_inputs(27, 1, 8, 2, 23, 8)
    r = A.forward_backward(q, k, v, do, True, 6, 0.5)
    kr = np.repeat(k, 4, axis=1)
    vr = np.repeat(v, 4, axis=1)
    m = A.forward_backward(q, kr, vr, do, True, 6, 0.5)
    for name in ("O", "LSE", "dQ"):
        assert np.max(np.abs(r[name] - m[name])) <= 1e-14, name
    assert np.max(np.abs(r["dK"] - m["dK"].reshape(1, 2, 4, 23, 8).sum(axis=2))) <= 1e-13
    assert np.max(np.abs(r["dV"] - m["dV"].reshape(1, 2, 4, 23, 8).sum(axis=2))) <= 1e-13


def pin_hidden_keys_do_not_matter(A):
    """Changing K_j, V_j for keys no query in a row set can see leaves those rows' O, LSE and dQ
    bitwise unchanged."""
    S = 40
    q, k, v, do = _rng_inputs(28, 1, 2, 2, S, 8)
    for window, i0 in ((0, 17), (5, 30)):
        r = A.forward_backward(q, k, v, do, True, window, 0.5)
        k2, v2 = k.copy(), v.copy()
        hidden = [j for j in range(S) if j > i0 or (window and i0 - j >= window)]
        k2[:, :, hidden] += 3.0
        v2[:, :, hidden] -= 5.0
        r2 = A.forward_backward(q, k2, v2, do, True, window, 0.5)
        assert np.array_equal(r["O"][:, :, i0], r2["O"][:, :, i0])
        assert np.array_equal(r["LSE"][:, :, i0], r2["LSE"][:, :, i0])
        assert np.array_equal(r["dQ"][:, :, i0], r2["dQ"][:, :, i0])


def pin_row_and_column_helpers(A):
    """The row/column helpers used for sampled checks at full size agree with the full pass."""
    q, k, v, do = _rng_inputs(29, 2, 4, 2, 60, 8)
    for window in (0, 11):
        r = A.forward_backward(q, k, v, do, True, window, 0.4, row_block=16)
        rows = np.array([0, 5, 31, 59])
        O, LSE = A.rows_forward(q, k, v, 1, 3, rows, True, window, 0.4)
        assert np.max(np.abs(O - r["O"][1, 3, rows])) <= 1e-14
        assert np.max(np.abs(LSE - r["LSE"][1, 3, rows])) <= 1e-14
        dq = A.rows_dq(q, k, v, do, 1, 3, rows, True, window, 0.4)
        assert np.max(np.abs(dq - r["dQ"][1, 3, rows])) <= 1e-13
        cols = np.array([0, 7, 58, 59])
        dk, dv = A.cols_dkdv(q, k, v, do, 1, 1, cols, True, window, 0.4, row_block=7)
        assert np.max(np.abs(dk - r["dK"][1, 1, cols])) <= 1e-13
        assert np.max(np.abs(dv - r["dV"][1, 1, cols])) <= 1e-13
    # the column helper with sink keys, fewer queries than keys, packed documents and no mask
    qc, kc, vc, dc = _rng_inputs(30, 1, 4, 2, 37, 8, Sk=60)
    cu = np.array([[0, 9, 9, 31, 60]])
    for qq, dd, causal, window, sink, docs in ((q, do, True, 9, 3, None), (qc, dc, True, 13, 2, None),
                                               (qc, dc, False, 0, 0, None), (q[:1], do[:1], True, 0, 0, cu)):
        kk, vv = (kc, vc) if qq is qc else (k[:qq.shape[0]], v[:qq.shape[0]])
        r = A.forward_backward(qq, kk, vv, dd, causal, window, 0.4, sink=sink, cu_seqlens=docs)
        cols = np.array([0, 2, 8, 9, 30, 31, 59])
        dk, dv = A.cols_dkdv(qq, kk, vv, dd, 0, 1, cols, causal, window, 0.4, row_block=5, sink=sink,
                             cu_seqlens=docs)
        assert np.max(np.abs(dk - r["dK"][0, 1, cols])) <= 1e-13, (causal, window, sink, docs)
        assert np.max(np.abs(dv - r["dV"][0, 1, cols])) <= 1e-13, (causal, window, sink, docs)


# ---------------------------------------------------------------- fewer queries than keys
def pin_chunk_is_suffix_of_square(A):
    """A chunk of the last S_q queries against all S_k keys is the square S_k x S_k problem seen
    on its last S_q rows: O, LSE and dQ equal those rows, and dK / dV equal the square problem's
    with dO zero on the first S_k - S_q rows (the other rows then contribute nothing)."""
    Sk, D = 29, 8
    qf, k, v, dof = _rng_inputs(31, 2, 4, 2, Sk, D)
    for S in (29, 17, 8, 1):
        for window in (0, 1, 6, 40):
            q, do = qf[:, :, Sk - S:], dof[:, :, Sk - S:]
            r = A.forward_backward(q, k, v, do, True, window, 0.45)
            dz = dof.copy()
            dz[:, :, :Sk - S] = 0.0
            full = A.forward_backward(qf, k, v, dz, True, window, 0.45)
            for name in ("O", "LSE", "dQ"):
                err = np.max(np.abs(r[name] - full[name][:, :, Sk - S:]))
                assert err <= 1e-13, f"chunk {name} (S_q={S}, W={window}): {err:.3e}"
            for name in ("dK", "dV"):
                err = np.max(np.abs(r[name] - full[name]))
                assert err <= 1e-13, f"chunk {name} (S_q={S}, W={window}): {err:.3e}"


def pin_torch_lower_right_causal(A, tol=1e-12):
    """torch's own lower-right causal bias (torch.nn.attention.bias.causal_lower_right) with
    float64 CPU scaled_dot_product_attention and autograd, for S_q < S_k without a window."""
    import torch
    from torch.nn.attention.bias import causal_lower_right
    for (B, Hq, Hkv, S, Sk, D, seed) in ((1, 4, 2, 11, 30, 8, 32), (2, 2, 1, 1, 17, 4, 33)):
        q, k, v, do = _rng_inputs(seed, B, Hq, Hkv, S, D, Sk=Sk)
        scale = 1.0 / math.sqrt(D)
        r = A.forward_backward(q, k, v, do, True, 0, scale)
        G = Hq // Hkv
        tq = torch.tensor(q, requires_grad=True)
        tk = torch.tensor(k, requires_grad=True)
        tv = torch.tensor(v, requires_grad=True)
        mask = causal_lower_right(S, Sk)._materialize(torch.device("cpu"))
        o = torch.nn.functional.scaled_dot_product_attention(
            tq, tk.repeat_interleave(G, dim=1), tv.repeat_interleave(G, dim=1),
            attn_mask=mask, scale=scale)
        o.backward(torch.tensor(do))
        for name, x, y in (("O", r["O"], o.detach().numpy()), ("dQ", r["dQ"], tq.grad.numpy()),
                           ("dK", r["dK"], tk.grad.numpy()), ("dV", r["dV"], tv.grad.numpy())):
            err = np.max(np.abs(x - y)) / max(np.max(np.abs(y)), 1e-30)
            assert err <= tol, f"torch lower-right causal {name} (S_q={S}, S_k={Sk}): {err:.3e}"


def pin_single_decode_query(A):
    """One query against S_k keys stands at the last position: causally it sees every key, so it
    equals attention without the causal mask; with a window W it equals attention over the last W
    keys alone."""
    Sk, D = 40, 8
    q, k, v, do = _rng_inputs(34, 1, 4, 2, 1, D, Sk=Sk)
    r = A.forward_backward(q, k, v, do, True, 0, 0.6)
    nc = A.forward_backward(q, k, v, do, False, 0, 0.6)
    for name in ("O", "LSE", "dQ", "dK", "dV"):
        assert np.max(np.abs(r[name] - nc[name])) <= 1e-14, f"decode {name}"
    for W in (1, 7, 39, 40, 64):
        r = A.forward_backward(q, k, v, do, True, W, 0.6)
        n = min(W, Sk)
        sub = A.forward_backward(q, k[:, :, Sk - n:], v[:, :, Sk - n:], do, False, 0, 0.6)
        for name in ("O", "LSE", "dQ"):
            assert np.max(np.abs(r[name] - sub[name])) <= 1e-14, f"decode W={W} {name}"
        for name in ("dK", "dV"):
            assert np.max(np.abs(r[name][:, :, Sk - n:] - sub[name])) <= 1e-14, f"decode W={W} {name}"
            assert np.all(r[name][:, :, :Sk - n] == 0.0), f"decode W={W} {name} outside the window"


def pin_chunk_helpers(A):
    """The row/column helpers agree with the full pass when S_q < S_k."""
    q, k, v, do = _rng_inputs(35, 1, 4, 2, 21, 8, Sk=50)
    for window in (0, 9):
        r = A.forward_backward(q, k, v, do, True, window, 0.4, row_block=8)
        rows = np.array([0, 3, 20])
        O, LSE = A.rows_forward(q, k, v, 0, 2, rows, True, window, 0.4)
        assert np.max(np.abs(O - r["O"][0, 2, rows])) <= 1e-14
        assert np.max(np.abs(LSE - r["LSE"][0, 2, rows])) <= 1e-14
        dq = A.rows_dq(q, k, v, do, 0, 2, rows, True, window, 0.4)
        assert np.max(np.abs(dq - r["dQ"][0, 2, rows])) <= 1e-13
        cols = np.array([0, 28, 29, 40, 49])
        dk, dv = A.cols_dkdv(q, k, v, do, 0, 1, cols, True, window, 0.4, row_block=5)
        assert np.max(np.abs(dk - r["dK"][0, 1, cols])) <= 1e-13
        assert np.max(np.abs(dv - r["dV"][0, 1, cols])) <= 1e-13


# ---------------------------------------------------------------- sink keys with a window
def pin_sink_decode_is_concatenation(A):
    """One decode query at the last position with a window W and n sink keys sees exactly keys
    0..n-1 and S_k-W..S_k-1: plain (unmasked) attention over those rows cut out of K and V and
    concatenated gives the same O, LSE, dQ, and dK / dV scattered back (zero elsewhere)."""
    Sk, D = 40, 8
    q, k, v, do = _rng_inputs(36, 1, 4, 2, 1, D, Sk=Sk)
    for n, W in ((1, 5), (3, 7), (4, 1), (6, 34)):
        idx = np.r_[np.arange(n), np.arange(Sk - W, Sk)]
        r = A.forward_backward(q, k, v, do, True, W, 0.6, sink=n)
        sub = A.forward_backward(q, k[:, :, idx], v[:, :, idx], do, False, 0, 0.6)
        for name in ("O", "LSE", "dQ"):
            assert np.max(np.abs(r[name] - sub[name])) <= 1e-14, f"sink decode n={n} W={W} {name}"
        for name in ("dK", "dV"):
            full = np.zeros_like(r[name])
            full[:, :, idx] = sub[name]
            assert np.max(np.abs(r[name] - full)) <= 1e-14, f"sink decode n={n} W={W} {name}"


def pin_sinks_covering_all_keys(A):
    """With at least as many sink keys as keys, the window no longer hides anything: the result is
    plain causal attention; with no sink keys it is the window alone."""
    q, k, v, do = _rng_inputs(37, 1, 4, 2, 30, 8)
    full = A.forward_backward(q, k, v, do, True, 0, 0.5)
    for W in (1, 4, 17):
        r = A.forward_backward(q, k, v, do, True, W, 0.5, sink=30)
        for name in ("O", "LSE", "dQ", "dK", "dV"):
            assert np.max(np.abs(r[name] - full[name])) <= 1e-14, f"sink=S W={W} {name}"
        r0 = A.forward_backward(q, k, v, do, True, W, 0.5, sink=0)
        w0 = A.forward_backward(q, k, v, do, True, W, 0.5)
        for name in ("O", "LSE", "dQ", "dK", "dV"):
            assert np.array_equal(r0[name], w0[name]), f"sink=0 W={W} {name}"


def pin_sink_zero_query_counts(A):
    """Q = 0: exp(LSE) is the number of visible keys, the size of the union of the window
    [p-W+1, p] and the sink keys [0, n-1] (those at or before p)."""
    D = 4
    for S, Sk in ((90, 90), (25, 90)):
        q, k, v, do = _rng_inputs(38, 1, 2, 1, S, D, Sk=Sk)
        q[:] = 0.0
        for W, n in ((1, 1), (8, 3), (8, 8), (8, 20), (33, 64), (64, 1)):
            _, LSE = A.forward(q, k, v, True, W, 1.0, sink=n)
            p = np.arange(S) + Sk - S
            lo = np.maximum(0, p - W + 1)                       # first key of the window
            extra = np.clip(np.minimum(n, p + 1) - 0, 0, None)  # sink keys at or before p ...
            extra = np.maximum(0, np.minimum(extra, lo))        # ... that lie before the window
            want = (p - lo + 1) + extra
            got = np.rint(np.exp(LSE[0, 0])).astype(np.int64)
            assert np.array_equal(got, want), (S, Sk, W, n)


def pin_sink_chunk_is_suffix_of_square(A):
    """Sinks with fewer queries than keys: still the last rows of the square problem."""
    Sk, D = 33, 8
    qf, k, v, dof = _rng_inputs(39, 1, 2, 2, Sk, D)
    for S, W, n in ((11, 4, 2), (1, 6, 3), (20, 9, 5)):
        q, do = qf[:, :, Sk - S:], dof[:, :, Sk - S:]
        r = A.forward_backward(q, k, v, do, True, W, 0.45, sink=n)
        dz = dof.copy()
        dz[:, :, :Sk - S] = 0.0
        full = A.forward_backward(qf, k, v, dz, True, W, 0.45, sink=n)
        for name in ("O", "LSE", "dQ"):
            assert np.max(np.abs(r[name] - full[name][:, :, Sk - S:])) <= 1e-13, (S, W, n, name)
        for name in ("dK", "dV"):
            assert np.max(np.abs(r[name] - full[name])) <= 1e-13, (S, W, n, name)


def pin_sink_helpers(A):
    """Row / column helpers agree with the full pass with sinks."""
    q, k, v, do = _rng_inputs(40, 1, 4, 2, 30, 8, Sk=45)
    r = A.forward_backward(q, k, v, do, True, 7, 0.4, row_block=8, sink=3)
    rows = np.array([0, 13, 29])
    O, LSE = A.rows_forward(q, k, v, 0, 1, rows, True, 7, 0.4, sink=3)
    assert np.max(np.abs(O - r["O"][0, 1, rows])) <= 1e-14
    assert np.max(np.abs(LSE - r["LSE"][0, 1, rows])) <= 1e-14
    dq = A.rows_dq(q, k, v, do, 0, 1, rows, True, 7, 0.4, sink=3)
    assert np.max(np.abs(dq - r["dQ"][0, 1, rows])) <= 1e-13
    cols = np.array([0, 2, 3, 20, 44])
    dk, dv = A.cols_dkdv(q, k, v, do, 0, 0, cols, True, 7, 0.4, row_block=5, sink=3)
    assert np.max(np.abs(dk - r["dK"][0, 0, cols])) <= 1e-13
    assert np.max(np.abs(dv - r["dV"][0, 0, cols])) <= 1e-13


# ---------------------------------------------------------------- paged K/V cache
def _pool_from_dense(kd, bs, extra, rng, perm=True):
    """Lay a dense [B, Hkv, S, D] tensor out as a pool of bs-token blocks (B * ceil(S/bs) blocks
    in a shuffled order, plus `extra` blocks of noise) and return (pool, table)."""
    B, Hkv, S, D = kd.shape
    nper = -(-S // bs)
    nb = B * nper + extra
    order = rng.permutation(nb) if perm else np.arange(nb)
    pool = rng.standard_normal((nb, Hkv, bs, D))
    table = np.full((B, nper + 2), -7, dtype=np.int64)  # trailing entries are never read
    for b in range(B):
        for t in range(nper):
            phys = order[b * nper + t]
            table[b, t] = phys
            n = min(bs, S - t * bs)
            pool[phys, :, :n, :] = kd[b, :, t * bs:t * bs + n, :]
    return pool, table


def pin_paged_matches_dense(A):
    """An identity layout and a shuffled layout of the same dense K/V both give the dense result."""
    import oracle.paged as PG
    rng = np.random.default_rng(41)
    q, k, v, _ = _rng_inputs(41, 2, 4, 2, 5, 8, Sk=37)
    O, L = A.forward(q, k, v, True, 9, 0.5, sink=2)
    for bs, perm in ((16, False), (16, True), (4, True), (64, True)):
        kp, table = _pool_from_dense(k, bs, 3, np.random.default_rng(bs), perm)
        vp, table2 = _pool_from_dense(v, bs, 3, np.random.default_rng(bs), perm)
        assert np.array_equal(table, table2)
        Op, Lp = PG.paged_forward(q, kp, vp, table, np.array([37, 37]), True, 9, 0.5, sink=2)
        assert np.array_equal(Op, O) and np.array_equal(Lp, L), (bs, perm)


def pin_paged_lengths_and_sharing(A):
    """Sequences of different lengths equal their own dense problems; two sequences whose tables
    share blocks read the same keys."""
    import oracle.paged as PG
    rng = np.random.default_rng(42)
    bs, D, Hkv = 8, 4, 2
    pool_k = rng.standard_normal((12, Hkv, bs, D))
    pool_v = rng.standard_normal((12, Hkv, bs, D))
    table = np.array([[3, 7, 1, 0], [3, 7, 9, 11]])  # the first 16 tokens are shared
    lens = np.array([21, 30])
    q = rng.standard_normal((2, 4, 3, D))
    O, L = PG.paged_forward(q, pool_k, pool_v, table, lens, True, 0, 0.7)
    for b in range(2):
        blocks = table[b]
        kd = np.concatenate([pool_k[p] for p in blocks], axis=1)[:, :lens[b]]
        vd = np.concatenate([pool_v[p] for p in blocks], axis=1)[:, :lens[b]]
        o, lse = A.forward(q[b:b + 1], kd[None], vd[None], True, 0, 0.7)
        assert np.array_equal(O[b], o[0]) and np.array_equal(L[b], lse[0]), b
    # changing a block only the second sequence uses leaves the first bitwise unchanged
    pool_k2 = pool_k.copy()
    pool_k2[9] += 1.0
    O2, L2 = PG.paged_forward(q, pool_k2, pool_v, table, lens, True, 0, 0.7)
    assert np.array_equal(O2[0], O[0]) and not np.array_equal(O2[1], O[1])


# ---------------------------------------------------------------- packed documents
def pin_docs_equal_separate_sequences(A):
    """Documents packed into one buffer behave exactly as if each were its own sequence: O, LSE
    and dQ of a document's rows and dK, dV of its keys equal the result of running the document
    alone (rows of other documents contribute nothing)."""
    q, k, v, do = _rng_inputs(43, 2, 4, 2, 40, 8)
    cu = np.array([[0, 7, 7, 25, 40], [0, 1, 2, 33, 40]])
    for window in (0, 5):
        r = A.forward_backward(q, k, v, do, True, window, 0.5, cu_seqlens=cu)
        for b in range(2):
            for d0, d1 in zip(cu[b][:-1], cu[b][1:]):
                if d1 == d0:
                    continue
                sl = slice(d0, d1)
                sub = A.forward_backward(q[b:b + 1, :, sl], k[b:b + 1, :, sl], v[b:b + 1, :, sl],
                                         do[b:b + 1, :, sl], True, window, 0.5)
                for name in ("O", "LSE", "dQ", "dK", "dV"):
                    got = r[name][b, :, sl]
                    assert np.max(np.abs(got - sub[name][0])) <= 1e-13, (b, d0, d1, window, name)


def pin_docs_special_cases(A):
    """One document is plain attention; one-token documents make every query see only its own
    key: O = V (group-repeated), LSE = s <q_i, k_i>, dQ = dK = 0, dV = group sum of dO."""
    q, k, v, do = _rng_inputs(44, 1, 4, 2, 12, 8)
    plain = A.forward_backward(q, k, v, do, True, 0, 0.5)
    one = A.forward_backward(q, k, v, do, True, 0, 0.5, cu_seqlens=np.array([[0, 12]]))
    for name in ("O", "LSE", "dQ", "dK", "dV"):
        assert np.array_equal(plain[name], one[name]), name
    r = A.forward_backward(q, k, v, do, True, 0, 0.5, cu_seqlens=np.arange(13)[None])
    for h in range(4):
        g = h // 2
        assert np.max(np.abs(r["O"][0, h] - v[0, g])) <= 1e-14
        assert np.max(np.abs(r["LSE"][0, h] - 0.5 * np.sum(q[0, h] * k[0, g], axis=1))) <= 1e-13
    assert np.max(np.abs(r["dQ"])) <= 1e-14 and np.max(np.abs(r["dK"])) <= 1e-14
    assert np.max(np.abs(r["dV"] - do.reshape(1, 2, 2, 12, 8).sum(axis=2))) <= 1e-13


def pin_docs_zero_query_counts(A):
    """Q = 0: exp(LSE) counts the keys from the document start (or the window start, if later)
    up to the query."""
    S = 60
    q, k, v, _ = _rng_inputs(45, 1, 2, 1, S, 4)
    q[:] = 0.0
    cu = np.array([[0, 5, 6, 30, 31, 60]])
    for W in (0, 1, 4, 20):
        _, LSE = A.forward(q, k, v, True, W, 1.0, cu_seqlens=cu)
        p = np.arange(S)
        start = np.array([max(c for c in cu[0][:-1] if c <= t) for t in p])
        if W:
            start = np.maximum(start, p - W + 1)
        assert np.array_equal(np.rint(np.exp(LSE[0, 0])).astype(np.int64), p - start + 1), W


def pin_docs_bruteforce(A, tol=1e-12):
    for (Hq, Hkv, S, D, window, cu, seed) in ((2, 1, 9, 3, 0, [[0, 4, 9]], 46), (4, 2, 10, 2, 3, [[0, 1, 5, 5, 10]], 47)):
        q, k, v, do = _rng_inputs(seed, 1, Hq, Hkv, S, D)
        cu = np.asarray(cu)
        r = A.forward_backward(q, k, v, do, True, window, 0.7, cu_seqlens=cu)
        ref = _brute(q, k, v, do, True, window, 0.7, 0, cu)
        for name, x, y in zip(("O", "LSE", "dQ", "dK", "dV"),
                              (r["O"], r["LSE"], r["dQ"], r["dK"], r["dV"]), ref):
            err = np.max(np.abs(x - y)) / max(np.max(np.abs(y)), 1e-30)
            assert err <= tol, f"docs brute force {name}: {err:.3e}"


ALL_PINS = [
    pin_fd_every_entry, pin_bruteforce, pin_torch_sdpa, pin_three_token_closed_form,
    pin_constant_v, pin_identical_keys, pin_window_one, pin_zero_queries, pin_rows_sum_to_one,
    pin_gradient_identities, pin_gqa_is_repeated_mha, pin_hidden_keys_do_not_matter,
    pin_row_and_column_helpers, pin_chunk_is_suffix_of_square, pin_torch_lower_right_causal,
    pin_single_decode_query, pin_chunk_helpers, pin_sink_decode_is_concatenation,
    pin_sinks_covering_all_keys, pin_sink_zero_query_counts, pin_sink_chunk_is_suffix_of_square,
    pin_sink_helpers, pin_paged_matches_dense, pin_paged_lengths_and_sharing,
    pin_docs_equal_separate_sequences, pin_docs_special_cases, pin_docs_zero_query_counts,
    pin_docs_bruteforce,
]
