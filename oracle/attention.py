"""fp64 CPU oracle for causal / sliding-window grouped-query attention, forward and backward.

TEST INFRASTRUCTURE. Only tests/, __graft_entry__.smoke() and bench.py's CPU-baseline leg may
import or call this module. The product path (the HIP library under causal_attention_fa2_amd/csrc
and its Python binding) never imports, links or calls it, and this module imports nothing from
the product package.

What it computes is plain materialised softmax attention and its exact gradient, in float64:

  * "KYNETRA FOUNDRY" page, FlashAttention paragraph: tiled attention with an online softmax is an
    IO reordering whose numerics are exact, so the plain materialised definition is the result the
    tiled kernels must reproduce; the backward pass recomputes probabilities rather than storing them.
  * Same page, decoder-block paragraph: the decoder mask enforces strict left-to-right causality
    (query i sees keys j <= i).
  * Same page, Grip (grouped-query attention) paragraph: the query heads are split into groups and
    each group shares one key/value head.
  * "CUDA-LLM: A GitHub Repository for Development", section "The custom CUDA kernel": one window
    parameter switches the same kernel between full-causal and sliding-window attention, and the
    backward recomputes the softmax probabilities from the saved log-sum-exp.
  * "From-scratch GPU LLM training", section "What is built": scaled-dot-product attention is one of
    the gradient kernels, checked tensor by tensor against a CPU reference.
  * "CUDA-LLM: A GitHub Repository for Development", section "The custom CUDA kernel": the kernel is
    generalised to fewer queries than keys (S_q <= S_k), so that one kernel serves a full prefill and
    a single-token decode against a cache.
  * "KYNETRA FOUNDRY" page, Vaultecho paragraph: besides the sliding window of recent tokens a few
    persistent "sink" tokens at the start of the sequence stay attended.
  * "Build a standalone, production grade system that trains a 4,..." (the page-4 prompt), its
    curriculum section: documents are concatenated contiguously into fixed-length buffers with
    document-boundary index arrays and boundary reset indicators, and the pipeline generates the
    matching attention block masks.

Readings where the pages leave a step open (each also listed in the design notes):
  * tensors are [B, H, S, D] contiguous, D fastest; K and V have Hkv heads, Q/O/dO have Hq heads;
  * query head h uses key/value head h // (Hq // Hkv) (contiguous groups); Hq % Hkv == 0;
  * window W == 0 means no window; W >= 1 makes key j visible to query i iff i - W < j <= i, so
    W counts the diagonal; a window without the causal mask is not defined by the pages and is
    rejected;
  * `scale` multiplies Q K^T before the softmax; the saved log-sum-exp is the natural log of the sum
    of exponentials of the *scaled* scores;
  * with S_q <= S_k the queries are the last S_q positions: query i sits at absolute position
    i + (S_k - S_q) for the causal mask and the window ("bottom-right" alignment; a single decode query
    sees every key); S_q > S_k is not defined by the pages and is rejected;
  * sinks: the first n_sink keys stay visible to every query at or after them even when the window
    has moved past them (key j visible iff causal allows it and (p - j < W or j < n_sink)); without a
    window every earlier key is visible anyway, so n_sink only matters when W > 0;
  * packed documents: cu_seqlens[b] = (0 = c_0 <= c_1 <= ... <= c_n = S) splits batch row b into
    documents [c_k, c_{k+1}); key j is visible to query i only if both lie in the same document
    (attention is reset at every boundary), on top of the causal mask and window;
  * every row has at least one visible key (its own position), so no empty-row convention is needed.

Rows are processed in blocks of `row_block` queries only to bound memory: each row's softmax is
normalised over that row alone, so a row's outputs depend only on that row; dK and dV sum the
per-row contributions block after block.
"""
from __future__ import annotations

import math

import numpy as np

__all__ = [
    "kv_head", "document_of", "visible_mask", "head_rows", "forward", "backward",
    "forward_backward", "probabilities", "rows_forward", "rows_dq", "cols_dkdv",
]


def _check(q, k, v, causal, window, sink=0):
    """Returns (B, Hq, Hkv, S_q, S_k, D)."""
    if sink < 0:
        raise ValueError("n_sink must be >= 0")
    if q.ndim != 4 or k.ndim != 4 or v.ndim != 4:
        raise ValueError("q, k, v must be [B, H, S, D]")
    B, Hq, Sq, D = q.shape
    Sk = k.shape[2]
    if k.shape[0] != B or k.shape[3] != D or v.shape != k.shape:
        raise ValueError("k and v must be [B, Hkv, S_k, D] with q's B and D")
    if Sq > Sk:
        raise ValueError("fewer keys than queries (S_q > S_k) is not defined")
    Hkv = k.shape[1]
    if Hkv < 1 or Hq % Hkv != 0:
        raise ValueError("Hq must be a multiple of Hkv")
    if window < 0:
        raise ValueError("window must be >= 0")
    if window > 0 and not causal:
        raise ValueError("a sliding window requires the causal mask")
    return B, Hq, Hkv, Sq, Sk, D


def kv_head(h: int, Hq: int, Hkv: int) -> int:
    """Key/value head shared by query head h: contiguous groups of Hq // Hkv query heads."""
    return h // (Hq // Hkv)


def document_of(pos, cu) -> np.ndarray:
    """Document index of each position: the k with cu[k] <= pos < cu[k+1]."""
    cu = np.asarray(cu, dtype=np.int64)
    return np.searchsorted(cu, np.asarray(pos, dtype=np.int64), side="right") - 1


def visible_mask(rows, cols, causal: bool, window: int, offset: int = 0, sink: int = 0,
                 docs=None) -> np.ndarray:
    """Boolean [len(rows), len(cols)]: with query i at position p = i + offset, key j is visible
    iff (not causal or j <= p) and (window == 0 or p - j < window or j < sink) and, when docs
    (one batch row's cu_seqlens) is given, p and j lie in the same document.
    offset = S_k - S_q; sink = number of sink keys."""
    i = np.asarray(rows, dtype=np.int64)[:, None] + offset
    j = np.asarray(cols, dtype=np.int64)[None, :]
    m = np.ones((i.shape[0], j.shape[1]), dtype=bool)
    if causal:
        m &= j <= i
    if window > 0:
        m &= ((i - j) < window) | (j < sink)
    if docs is not None:
        m &= document_of(i, docs) == document_of(j, docs)
    return m


def head_rows(qh, kh, vh, rows, causal, window, scale, doh=None, offset=0, sink=0, docs=None):
    """One head, a set of query rows, all S_k keys.

    qh [S_q, D], kh/vh [S_k, D], doh [S_q, D] or None (float64); query i at position i + offset.
    Returns a dict with P [R, S_k] (softmax probabilities, exactly 0 where masked), O [R, D],
    LSE [R], and when doh is given dP [R, S_k], delta [R] and dS [R, S_k]."""
    S = kh.shape[0]
    rows = np.asarray(rows, dtype=np.int64)
    mask = visible_mask(rows, np.arange(S), causal, window, offset, sink, docs)
    x = scale * (qh[rows] @ kh.T)                     # scaled scores
    x = np.where(mask, x, -np.inf)
    m = x.max(axis=1, keepdims=True)                  # finite: the row's own position is visible
    e = np.exp(x - m)                                 # exp(-inf) == 0 exactly for masked keys
    l = e.sum(axis=1, keepdims=True)
    p = e / l
    out = {"P": p, "O": p @ vh, "LSE": (m + np.log(l))[:, 0]}
    if doh is not None:
        dp = doh[rows] @ vh.T                         # dP_ij = <dO_i, V_j>
        delta = (p * dp).sum(axis=1)                  # softmax backward: sum_k P_ik dP_ik
        out["dP"] = dp
        out["delta"] = delta
        out["dS"] = p * (dp - delta[:, None])         # dS_ij = P_ij (dP_ij - delta_i)
    return out


def _f64(*xs):
    return tuple(np.asarray(x, dtype=np.float64) for x in xs)


def forward_backward(q, k, v, do=None, causal=True, window=0, scale=None, row_block=256, sink=0,
                     cu_seqlens=None):
    """Full attention forward (O, LSE) and, when do is given, backward (dQ, dK, dV).

    q, do [B,Hq,S_q,D]; k, v [B,Hkv,S_k,D] with S_q <= S_k; cu_seqlens [B, n+1] document
    boundaries (optional). Returns float64 arrays in a dict."""
    B, Hq, Hkv, S, Sk, D = _check(q, k, v, causal, window, sink)
    off = Sk - S
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    q, k, v = _f64(q, k, v)
    O = np.zeros((B, Hq, S, D))
    LSE = np.zeros((B, Hq, S))
    res = {"O": O, "LSE": LSE}
    if do is not None:
        (do,) = _f64(do)
        dQ = np.zeros_like(q)
        dK = np.zeros_like(k)
        dV = np.zeros_like(v)
        res.update(dQ=dQ, dK=dK, dV=dV, delta=np.zeros((B, Hq, S)))
    for b in range(B):
        for h in range(Hq):
            g = kv_head(h, Hq, Hkv)
            for r0 in range(0, S, row_block):
                rows = np.arange(r0, min(S, r0 + row_block))
                t = head_rows(q[b, h], k[b, g], v[b, g], rows, causal, window, scale,
                              None if do is None else do[b, h], off, sink,
                              None if cu_seqlens is None else cu_seqlens[b])
                O[b, h, rows] = t["O"]
                LSE[b, h, rows] = t["LSE"]
                if do is not None:
                    res["delta"][b, h, rows] = t["delta"]
                    dQ[b, h, rows] = scale * (t["dS"] @ k[b, g])      # dQ_i = s sum_j dS_ij K_j
                    dK[b, g] += scale * (t["dS"].T @ q[b, h, rows])  # dK_j = s sum_i dS_ij Q_i
                    dV[b, g] += t["P"].T @ do[b, h, rows]            # dV_j = sum_i P_ij dO_i
    return res


def forward(q, k, v, causal=True, window=0, scale=None, row_block=256, sink=0, cu_seqlens=None):
    """Returns (O, LSE) in float64."""
    r = forward_backward(q, k, v, None, causal, window, scale, row_block, sink, cu_seqlens)
    return r["O"], r["LSE"]


def backward(q, k, v, do, causal=True, window=0, scale=None, row_block=256, sink=0, cu_seqlens=None):
    """Returns (dQ, dK, dV) in float64: the exact gradient of sum(O * dO)."""
    r = forward_backward(q, k, v, do, causal, window, scale, row_block, sink, cu_seqlens)
    return r["dQ"], r["dK"], r["dV"]


def probabilities(q, k, b, h, causal=True, window=0, scale=None, sink=0):
    """Softmax probabilities P [S_q, S_k] of one (batch, query head)."""
    B, Hq, S, D = q.shape
    Hkv = k.shape[1]
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    qh, kh = _f64(q[b, h], k[b, kv_head(h, Hq, Hkv)])
    return head_rows(qh, kh, kh, np.arange(S), causal, window, scale, None, k.shape[2] - S, sink)["P"]


def rows_forward(q, k, v, b, h, rows, causal=True, window=0, scale=None, sink=0, cu_seqlens=None):
    """O[b, h, rows] and LSE[b, h, rows], each row computed on its own."""
    B, Hq, Hkv, S, Sk, D = _check(q, k, v, causal, window, sink)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    g = kv_head(h, Hq, Hkv)
    qh, kh, vh = _f64(q[b, h], k[b, g], v[b, g])
    t = head_rows(qh, kh, vh, rows, causal, window, scale, None, Sk - S, sink,
                  None if cu_seqlens is None else cu_seqlens[b])
    return t["O"], t["LSE"]


def rows_dq(q, k, v, do, b, h, rows, causal=True, window=0, scale=None, sink=0, cu_seqlens=None):
    """dQ[b, h, rows]: each row needs only its own probabilities and dP row."""
    B, Hq, Hkv, S, Sk, D = _check(q, k, v, causal, window, sink)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    g = kv_head(h, Hq, Hkv)
    qh, kh, vh, doh = _f64(q[b, h], k[b, g], v[b, g], do[b, h])
    t = head_rows(qh, kh, vh, rows, causal, window, scale, doh, Sk - S, sink,
                  None if cu_seqlens is None else cu_seqlens[b])
    return scale * (t["dS"] @ kh)


def cols_dkdv(q, k, v, do, b, g, cols, causal=True, window=0, scale=None, row_block=256, sink=0,
              cu_seqlens=None, progress=None):
    """dK[b, g, cols] and dV[b, g, cols]: sums over every query head of group g and every
    query row that can see at least one of `cols`.

    Per block of query rows only the span of keys that some row of the block can see is
    materialised (masked entries are exact zeros, so leaving them out changes no sum), and
    delta_i is taken from its definition <dO_i, O_i>, so the dP / dS entries are formed only in
    the requested columns. Each row's softmax still runs over all of its visible keys.
    progress(done, total), if given, is called after each block of rows."""
    B, Hq, Hkv, S, Sk, D = _check(q, k, v, causal, window, sink)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    cols = np.asarray(cols, dtype=np.int64)
    G = Hq // Hkv
    kh, vh = _f64(k[b, g], v[b, g])
    docs = None if cu_seqlens is None else cu_seqlens[b]
    off = Sk - S
    need = visible_mask(np.arange(S), cols, causal, window, off, sink, docs).any(axis=1)
    rows_all = np.nonzero(need)[0]
    dK = np.zeros((cols.size, D))
    dV = np.zeros((cols.size, D))
    heads = [_f64(q[b, h], do[b, h]) for h in range(g * G, (g + 1) * G)]
    n_blocks = (rows_all.size + row_block - 1) // row_block
    for n, r0 in enumerate(range(0, rows_all.size, row_block)):
        rows = rows_all[r0:r0 + row_block]
        mask = visible_mask(rows, np.arange(Sk), causal, window, off, sink, docs)
        seen = np.nonzero(mask.any(axis=0))[0]
        c_lo, c_hi = int(seen[0]), int(seen[-1]) + 1            # every visible key lies in [c_lo, c_hi)
        mask = mask[:, c_lo:c_hi]
        inside = (cols >= c_lo) & (cols < c_hi)
        for qh, doh in heads:
            x = scale * (qh[rows] @ kh[c_lo:c_hi].T)            # scaled scores of the span
            x = np.where(mask, x, -np.inf)
            m = x.max(axis=1, keepdims=True)
            e = np.exp(x - m)
            p = e / e.sum(axis=1, keepdims=True)                # P_ij (0 where masked)
            o = p @ vh[c_lo:c_hi]                               # O_i
            delta = np.sum(doh[rows] * o, axis=1)               # delta_i = <dO_i, O_i>
            pc = np.zeros((rows.size, cols.size))
            pc[:, inside] = p[:, cols[inside] - c_lo]           # P at the requested keys
            dpc = doh[rows] @ vh[cols].T                        # dP_ij = <dO_i, V_j>
            dsc = pc * (dpc - delta[:, None])                   # dS_ij = P_ij (dP_ij - delta_i)
            dK += scale * (dsc.T @ qh[rows])                    # dK_j = s sum_i dS_ij Q_i
            dV += pc.T @ doh[rows]                              # dV_j = sum_i P_ij dO_i
        if progress is not None:
            progress(n + 1, n_blocks)
    return dK, dV
