"""attn_bwd_qk_noalloc: the backward with its workspace in the library's static per-device scratch
array instead of a caller buffer. Through the C ABI it must give exactly the bits attn_bwd_qk gives
with an allocated workspace (same kernels, same decomposition, fixed summation order), call after
call: a later, smaller problem finds the array holding the previous call's values and must not
depend on them. Problems beyond the array are refused before anything is enqueued."""
import re

import pytest

from causal_attention_fa2_amd.workloads import random_tensor
from gpu_util import say, upload

pytestmark = pytest.mark.gpu


def _problem(dtype, B, Hq, Hkv, Sq, Sk, D, window, sink, seed):
    import causal_attention_fa2_amd as fa
    q = upload(random_tensor((B, Hq, Sq, D), dtype, seed), dtype)
    k = upload(random_tensor((B, Hkv, Sk, D), dtype, seed + 1), dtype)
    v = upload(random_tensor((B, Hkv, Sk, D), dtype, seed + 2), dtype)
    do = upload(random_tensor((B, Hq, Sq, D), dtype, seed + 3), dtype)
    o, lse = fa.forward(q, k, v, True, window, None, sink=sink)
    return q, k, v, o, lse, do


def _workspace_bytes(B, Hq, Hkv, Sq, Sk, D, window, sink):
    """The workspace the static array stands for: sized by attn_bwd_qk_workspace_bytes_for (sink
    split or stored dS on) when that fits in the array, else the plain size."""
    import causal_attention_fa2_amd as fa
    need = fa.attn_bwd_qk_workspace_bytes_for(B, Hq, Hkv, Sq, Sk, D, True, window, sink)
    return need if need <= fa.ATTN_NOALLOC_SCRATCH_BYTES else fa.attn_bwd_qk_workspace_bytes(B, Hq, Hkv, Sq, Sk, D)


def _with_workspace(p, window, sink):
    """attn_bwd_qk given an allocated workspace of _workspace_bytes(...)."""
    import torch
    import causal_attention_fa2_amd as fa
    q, k, v, o, lse, do = p
    B, Hq, Sq, D = q.shape
    Hkv, Sk = k.shape[1], k.shape[2]
    ws = torch.empty(_workspace_bytes(B, Hq, Hkv, Sq, Sk, D, window, sink), dtype=torch.uint8, device=q.device)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    fa.attn_bwd_qk(q, k, v, o, lse, do, dq, dk, dv, ws, True, window, None, None, sink)
    return dq, dk, dv


def _noalloc(p, window, sink):
    import torch
    import causal_attention_fa2_amd as fa
    q, k, v, o, lse, do = p
    dq, dk, dv = (torch.full_like(t, 3.0) for t in (q, k, v))
    fa.attn_bwd_qk_noalloc(q, k, v, o, lse, do, dq, dk, dv, True, window, None, None, sink)
    return dq, dk, dv


# Calls in this order, each smaller than the one before (bytes of workspace it uses):
#   the 64/8-head S=4096 D=128 bf16 backward with its head split (66 MiB of the 72 MiB array; its
#   stored dS would not fit, so dQ recomputes),
#   a sliding-window problem with 4 sink keys (sink split of key tile 0, chunk partials),
#   a bf16 prefill chunk (300 queries, 2100 keys) with its stored dS,
#   a small fp32 problem with fewer queries than keys.
CALLS = [
    ("bf16", 1, 64, 8, 4096, 4096, 128, 0, 0),
    ("bf16", 1, 8, 2, 2048, 2048, 64, 128, 4),
    ("bf16", 1, 4, 2, 300, 2100, 128, 0, 0),
    ("f32", 1, 4, 2, 300, 700, 64, 0, 0),
]


def test_noalloc_matches_workspace_call_in_sequence():
    import torch
    import causal_attention_fa2_amd as fa
    need = [_workspace_bytes(*c[1:9]) for c in CALLS]
    assert need[0] > need[1] > need[2] > need[3] > 0 and need[0] <= fa.ATTN_NOALLOC_SCRATCH_BYTES
    assert need[0] == fa.attn_bwd_qk_workspace_bytes(*CALLS[0][1:7])  # no room for its stored dS
    assert need[1] > fa.attn_bwd_qk_workspace_bytes(*CALLS[1][1:7])  # the sink split is in use
    assert need[2] > fa.attn_bwd_qk_workspace_bytes(*CALLS[2][1:7])  # the stored dS is in use
    for n, (dtype, B, Hq, Hkv, Sq, Sk, D, window, sink) in enumerate(CALLS):
        say(f"noalloc call {n}: {dtype} B={B} Hq={Hq} Hkv={Hkv} Sq={Sq} Sk={Sk} D={D} W={window} sink={sink}")
        p = _problem(dtype, B, Hq, Hkv, Sq, Sk, D, window, sink, 900 + 10 * n)
        want = _with_workspace(p, window, sink)
        got = _noalloc(p, window, sink)
        torch.cuda.synchronize()
        for name, g, w in zip(("dQ", "dK", "dV"), got, want):
            assert torch.isfinite(g.float()).all(), f"call {n} {name}: non-finite values"
            assert torch.equal(g, w), f"call {n} {name}: differs from attn_bwd_qk with a workspace"
        say(f"  call {n}: dQ, dK, dV bitwise equal to attn_bwd_qk")
        del p, want, got


def test_noalloc_repeat_after_larger_call():
    """The second call of a pair, on the smaller problem, repeated after a larger call has filled
    the array: identical bits each time."""
    import torch
    small = CALLS[2]
    p = _problem(*small, 950)
    first = _noalloc(p, small[7], small[8])
    big = CALLS[0]
    pb = _problem(*big, 960)
    _noalloc(pb, big[7], big[8])
    again = _noalloc(p, small[7], small[8])
    torch.cuda.synchronize()
    for a, b in zip(first, again):
        assert torch.equal(a, b)
    say("  small call after a large one: bitwise equal")


def test_noalloc_refuses_oversize_before_launch():
    import torch
    import causal_attention_fa2_amd as fa
    dtype, B, Hq, Hkv, S, D = "bf16", 1, 64, 8, 6144, 128
    assert fa.attn_bwd_qk_workspace_bytes(B, Hq, Hkv, S, S, D) > fa.ATTN_NOALLOC_SCRATCH_BYTES
    q = upload(random_tensor((B, Hq, S, D), dtype, 970), dtype)
    k = upload(random_tensor((B, Hkv, S, D), dtype, 971), dtype)
    v = upload(random_tensor((B, Hkv, S, D), dtype, 972), dtype)
    o, lse = fa.forward(q, k, v, True)
    dq, dk, dv = (torch.full_like(t, 5.0) for t in (q, k, v))
    with pytest.raises(fa.AttnError) as e:
        fa.attn_bwd_qk_noalloc(q, k, v, o, lse, q, dq, dk, dv, True)
    assert e.value.status == fa.ATTN_ERR_SCRATCH
    assert re.search("static scratch", str(e.value))
    torch.cuda.synchronize()
    for t in (dq, dk, dv):  # nothing was enqueued
        assert bool((t == 5.0).all())
    say("  S=6144 refused with ATTN_ERR_SCRATCH, outputs untouched")


def test_noalloc_in_graph_capture():
    """The call a capturing caller makes: captured once, replayed three times with the outputs
    overwritten between replays; every replay equals the eager call."""
    import torch
    import causal_attention_fa2_amd as fa
    p = _problem("bf16", 1, 8, 2, 1000, 1000, 128, 0, 0, 980)
    q, k, v, o, lse, do = p
    want = _with_workspace(p, 0, 0)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)

    def call():
        fa.attn_bwd_qk_noalloc(q, k, v, o, lse, do, dq, dk, dv, True)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    torch.cuda.synchronize()
    for rep in range(3):
        for t in (dq, dk, dv):
            t.fill_(7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, a, b in zip(("dQ", "dK", "dV"), (dq, dk, dv), want):
            assert torch.equal(a, b), f"replay {rep}: {name} differs"
    say("  captured noalloc backward: 3 replays bitwise equal")
