"""Planted mistakes in the oracle (CPU only): each plausible error must make at least two pins in
oracle_pins.py fail. This shows the pins constrain the oracle rather than restate it."""
import math

import numpy as np
import pytest

import oracle.attention as A
import oracle_pins as P

_real_head_rows = A.head_rows
_real_fb = A.forward_backward
_real_mask = A.visible_mask
import oracle.paged as PG  # noqa: E402
_real_gather = PG.gather_sequence


def _head_rows_mut(kind):
    def f(qh, kh, vh, rows, causal, window, scale, doh=None, offset=0, sink=0, docs=None):
        t = _real_head_rows(qh, kh, vh, rows, causal, window, scale, doh, offset, sink, docs)
        if doh is not None:
            if kind == "dropped_delta":          # dS = P * dP (rowsum term dropped)
                t["dS"] = t["P"] * t["dP"]
            elif kind == "dS_sign":
                t["dS"] = -t["dS"]
            elif kind == "delta_from_wrong_axis":  # sum over rows instead of keys
                d = (t["P"] * t["dP"]).sum(axis=0)[: len(rows)]
                d = np.pad(d, (0, len(rows) - d.size))
                t["dS"] = t["P"] * (t["dP"] - d[:, None])
        if kind == "unnormalised_P":
            t["P"] = t["P"] * 1.001
        return t
    return f


def _fb_mut(kind):
    def f(q, k, v, do=None, causal=True, window=0, scale=None, row_block=256, sink=0, cu_seqlens=None):
        r = _real_fb(q, k, v, do, causal, window, scale, row_block, sink, cu_seqlens)
        s = 1.0 / math.sqrt(q.shape[-1]) if scale is None else scale
        if kind == "lse_base2":
            r["LSE"] = r["LSE"] / math.log(2.0)
        if do is not None:
            if kind == "dq_missing_scale":
                r["dQ"] = r["dQ"] / s
            elif kind == "dk_transposed_groups":  # dK of KV heads swapped
                r["dK"] = r["dK"][:, ::-1].copy()
        return r
    return f


def _mask_mut(kind):
    def f(rows, cols, causal, window, offset=0, sink=0, docs=None):
        if kind == "offset_ignored":          # queries aligned top-left instead of bottom-right
            offset = 0
        elif kind == "offset_negated":
            offset = -offset
        i = np.asarray(rows, dtype=np.int64)[:, None] + offset
        j = np.asarray(cols, dtype=np.int64)[None, :]
        m = np.ones((i.shape[0], j.shape[1]), dtype=bool)
        if causal:
            m &= (j < i) | (j == i) if kind != "causal_transposed" else (j >= i)
        if window > 0:
            inw = ((i - j) <= window) if kind == "window_off_by_one" else ((i - j) < window)
            if kind == "sink_ignored":
                sk = inw
            elif kind == "sink_off_by_one":       # one sink key too many
                sk = inw | (j <= sink)
            elif kind == "sink_without_causal":   # sinks visible even to earlier queries
                sk = inw | (j < sink)
                m = (m | (j < sink)) if causal else m
            else:
                sk = inw | (j < sink)
            m &= sk
        if docs is not None and kind != "docs_ignored":
            di, dj = A.document_of(i, docs), A.document_of(j, docs)
            if kind == "doc_leaks_previous":      # a query also sees the document before its own
                m &= (di == dj) | (di == dj + 1)
            else:
                m &= di == dj
        return m
    return f


def _gather_mut(kind):
    def f(pool, block_table, b, n_tokens, block_size):
        nb, Hkv, bs, D = pool.shape
        out = np.empty((Hkv, n_tokens, D))
        for t in range(n_tokens):
            if kind == "paged_slot_reversed":
                phys, slot = int(block_table[b, t // bs]), bs - 1 - t % bs
            else:  # "paged_table_of_sequence_0"
                phys, slot = int(block_table[0, t // bs]), t % bs
            out[:, t, :] = pool[phys, :, slot, :]
        return out
    return f


MUTANTS = {
    "dropped_delta": ("head_rows", _head_rows_mut("dropped_delta")),
    "dS_sign": ("head_rows", _head_rows_mut("dS_sign")),
    "delta_from_wrong_axis": ("head_rows", _head_rows_mut("delta_from_wrong_axis")),
    "unnormalised_P": ("head_rows", _head_rows_mut("unnormalised_P")),
    "lse_base2": ("forward_backward", _fb_mut("lse_base2")),
    "dq_missing_scale": ("forward_backward", _fb_mut("dq_missing_scale")),
    "dk_transposed_groups": ("forward_backward", _fb_mut("dk_transposed_groups")),
    "kv_head_interleaved": ("kv_head", lambda h, Hq, Hkv: h % Hkv),
    "window_off_by_one": ("visible_mask", _mask_mut("window_off_by_one")),
    "causal_transposed": ("visible_mask", _mask_mut("causal_transposed")),
    "offset_ignored": ("visible_mask", _mask_mut("offset_ignored")),
    "offset_negated": ("visible_mask", _mask_mut("offset_negated")),
    "sink_ignored": ("visible_mask", _mask_mut("sink_ignored")),
    "sink_off_by_one": ("visible_mask", _mask_mut("sink_off_by_one")),
    "sink_without_causal": ("visible_mask", _mask_mut("sink_without_causal")),
    "doc_leaks_previous": ("visible_mask", _mask_mut("doc_leaks_previous")),
    "docs_ignored": ("visible_mask", _mask_mut("docs_ignored")),
    "paged_slot_reversed": ("paged.gather_sequence", _gather_mut("paged_slot_reversed")),
    "paged_table_of_sequence_0": ("paged.gather_sequence", _gather_mut("paged_table_of_sequence_0")),
}

# Pins that run quickly enough to try on every mutant.
FAST_PINS = [p for p in P.ALL_PINS if p is not P.pin_torch_sdpa] + [P.pin_torch_sdpa]


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    if attr.startswith("paged."):
        monkeypatch.setattr(PG, attr.split(".", 1)[1], fn)
    else:
        monkeypatch.setattr(A, attr, fn)
    if attr == "forward_backward":
        # forward/backward/... reach forward_backward through the module, so they see it too
        pass
    caught = []
    for pin in FAST_PINS:
        try:
            pin(A)
        except (AssertionError, ValueError, IndexError) as e:  # a pin rejected the oracle
            caught.append(f"{pin.__name__}: {str(e)[:80]}")
    # every planted mistake fails at least two independent pins
    assert len(caught) >= 2, f"planted mistake {name!r} caught only by {caught}"
