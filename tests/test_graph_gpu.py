"""The entry points enqueue kernels only (no allocation, memset or synchronisation), so a caller can
capture them in a HIP graph (torch.cuda.CUDAGraph). Each capture below is replayed several times,
with the outputs overwritten by eager work between replays, and every replay must reproduce the
eager call bit for bit (the kernels sum in a fixed order, so reruns are bitwise equal).

Covered: forward + backward with the head-split reduce, the same with the stored dS, the backward
with the sink split and its chunk reduce, and the key-split decode forward with its combine. A
last test runs two problems at once on two streams."""
import math

import numpy as np
import pytest

from causal_attention_fa2_amd.workloads import random_tensor
from gpu_util import say, upload

pytestmark = pytest.mark.gpu

REPLAYS = 3


def _inputs(dtype, B, Hq, Hkv, Sq, Sk, D, seed):
    q = upload(random_tensor((B, Hq, Sq, D), dtype, seed), dtype)
    k = upload(random_tensor((B, Hkv, Sk, D), dtype, seed + 1), dtype)
    v = upload(random_tensor((B, Hkv, Sk, D), dtype, seed + 2), dtype)
    do = upload(random_tensor((B, Hq, Sq, D), dtype, seed + 3), dtype)
    return q, k, v, do


def _replay_and_check(g, outs, want, tag):
    import torch
    for rep in range(REPLAYS):
        for t in outs:  # eager work between replays: the graph must rewrite every output
            t.fill_(7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, got, ref in zip(("out%d" % i for i in range(len(outs))), outs, want):
            assert torch.equal(got, ref), f"{tag}: replay {rep}, {name} differs from the eager call"
    say(f"  {tag}: {REPLAYS} replays bitwise equal to the eager call")


def _capture(fn):
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # one warm-up call on a side stream before capture
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def test_graph_forward_backward_head_split():
    """B=1, Hq=8, Hkv=2, S=1000, D=128 bf16 causal: 8 key-tile pairs give hs > 1, so the backward
    ends with the head-split reduce kernel."""
    import torch
    import causal_attention_fa2_amd as fa
    fa.attn_set_launch_hook(None)
    B, Hq, Hkv, S, D = 1, 8, 2, 1000, 128
    say("graph: forward + backward (head split)")
    q, k, v, do = _inputs("bf16", B, Hq, Hkv, S, S, D, 300)
    scale = 1.0 / math.sqrt(D)
    ws = torch.empty(fa.attn_bwd_workspace_bytes(B, Hq, Hkv, S, D), dtype=torch.uint8, device="cuda")
    o, lse = torch.empty_like(q), torch.empty((B, Hq, S), dtype=torch.float32, device="cuda")
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)

    def step():
        fa.attn_fwd(q, k, v, o, lse, True, 0, scale)
        fa.attn_bwd(q, k, v, o, lse, do, dq, dk, dv, ws, True, 0, scale)

    step()
    torch.cuda.synchronize()
    want = [t.clone() for t in (o, lse, dq, dk, dv)]
    g = _capture(step)
    _replay_and_check(g, [o, lse, dq, dk, dv], want, "fwd+bwd")


def test_graph_forward_backward_stored_ds():
    """S = 2100 with a workspace sized by attn_bwd_qk_workspace_bytes_for: the backward runs the delta
    rows, the dK/dV pass storing dS, and the dQ pass reading it (whose trailing workgroups add the
    head-split partials)."""
    import torch
    import causal_attention_fa2_amd as fa
    fa.attn_set_launch_hook(None)
    B, Hq, Hkv, S, D = 1, 8, 2, 2100, 128
    say("graph: forward + backward (stored dS, head split)")
    q, k, v, do = _inputs("bf16", B, Hq, Hkv, S, S, D, 305)
    scale = 1.0 / math.sqrt(D)
    need = fa.attn_bwd_qk_workspace_bytes_for(B, Hq, Hkv, S, S, D, True, 0, 0)
    assert need > fa.attn_bwd_workspace_bytes(B, Hq, Hkv, S, D)  # room for the stored dS
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    o, lse = torch.empty_like(q), torch.empty((B, Hq, S), dtype=torch.float32, device="cuda")
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)

    def step():
        fa.attn_fwd(q, k, v, o, lse, True, 0, scale)
        fa.attn_bwd(q, k, v, o, lse, do, dq, dk, dv, ws, True, 0, scale)

    step()
    torch.cuda.synchronize()
    want = [t.clone() for t in (o, lse, dq, dk, dv)]
    g = _capture(step)
    _replay_and_check(g, [o, lse, dq, dk, dv], want, "fwd+bwd stored dS")


def test_graph_backward_sink_split():
    """Sliding window with sink keys and a workspace sized by attn_bwd_qk_workspace_bytes_for: the
    backward splits key tile 0's query range into chunk items and ends with the chunk reduce."""
    import torch
    import causal_attention_fa2_amd as fa
    fa.attn_set_launch_hook(None)
    B, Hq, Hkv, S, D, W, sink = 1, 8, 2, 1024, 128, 128, 4
    say("graph: backward with the sink split")
    q, k, v, do = _inputs("bf16", B, Hq, Hkv, S, S, D, 310)
    scale = 1.0 / math.sqrt(D)
    need = fa.attn_bwd_qk_workspace_bytes_for(B, Hq, Hkv, S, S, D, True, W, sink)
    assert need > fa.attn_bwd_qk_workspace_bytes(B, Hq, Hkv, S, S, D)  # the split is planned
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    o, lse = torch.empty_like(q), torch.empty((B, Hq, S), dtype=torch.float32, device="cuda")
    fa.attn_fwd_qk(q, k, v, o, lse, True, W, scale, None, sink)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)

    def step():
        fa.attn_bwd_qk(q, k, v, o, lse, do, dq, dk, dv, ws, True, W, scale, None, sink)

    step()
    torch.cuda.synchronize()
    want = [t.clone() for t in (dq, dk, dv)]
    g = _capture(step)
    _replay_and_check(g, [dq, dk, dv], want, "bwd sink split")


def test_graph_decode_paged():
    """Key-split decode forward over a paged cache (sequences of different lengths)."""
    import torch
    import causal_attention_fa2_amd as fa
    fa.attn_set_launch_hook(None)
    B, Hq, Hkv, D, bs = 3, 16, 2, 128, 16
    lens = np.array([700, 70, 2000], dtype=np.int32)
    say("graph: paged decode")
    need = [-(-int(n) // bs) for n in lens]
    nb = sum(need) + 1
    rng = np.random.default_rng(320)
    order = rng.permutation(nb)
    table = np.full((B, max(need)), 0, np.int32)
    i = 0
    for b in range(B):
        for t in range(need[b]):
            table[b, t] = order[i]
            i += 1
    q = upload(random_tensor((B, Hq, 1, D), "bf16", 321), "bf16")
    kp = upload(random_tensor((nb, Hkv, bs, D), "bf16", 322), "bf16")
    vp = upload(random_tensor((nb, Hkv, bs, D), "bf16", 323), "bf16")
    tt, tl = torch.from_numpy(table).cuda(), torch.from_numpy(lens).cuda()
    ws = torch.empty(fa.attn_decode_workspace_bytes(B, Hq, Hkv, 1, table.shape[1] * bs, D),
                     dtype=torch.uint8, device="cuda")
    o, lse = torch.empty_like(q), torch.empty((B, Hq, 1), dtype=torch.float32, device="cuda")

    def step():
        fa.attn_decode_fwd(q, kp, vp, o, lse, ws, True, 0, None, None, 0, block_table=tt, seqlen_k=tl)

    step()
    torch.cuda.synchronize()
    want = [o.clone(), lse.clone()]
    g = _capture(step)
    _replay_and_check(g, [o, lse], want, "paged decode")


def test_two_streams_concurrently():
    """Two different problems enqueued at once on two non-default streams (each with its own
    workspace): the library keeps no per-call state, so each result equals the same call made
    alone, bit for bit."""
    import torch
    import causal_attention_fa2_amd as fa
    fa.attn_set_launch_hook(None)
    say("two streams")
    cases = [(1, 8, 2, 1000, 128, 0, 330), (2, 4, 4, 700, 64, 200, 340)]
    bufs = []
    for B, Hq, Hkv, S, D, W, seed in cases:
        q, k, v, do = _inputs("bf16", B, Hq, Hkv, S, S, D, seed)
        ws = torch.empty(fa.attn_bwd_workspace_bytes(B, Hq, Hkv, S, D), dtype=torch.uint8, device="cuda")
        outs = (torch.empty_like(q), torch.empty((B, Hq, S), dtype=torch.float32, device="cuda"),
                torch.empty_like(q), torch.empty_like(k), torch.empty_like(v))
        bufs.append((q, k, v, do, ws, outs, W, 1.0 / math.sqrt(D)))

    def run(buf, stream):
        q, k, v, do, ws, (o, lse, dq, dk, dv), W, scale = buf
        fa.attn_fwd(q, k, v, o, lse, True, W, scale, stream)
        fa.attn_bwd(q, k, v, o, lse, do, dq, dk, dv, ws, True, W, scale, stream)

    want = []
    for buf in bufs:  # alone, one after the other
        run(buf, torch.cuda.current_stream())
        torch.cuda.synchronize()
        want.append([t.clone() for t in buf[5]])
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for rep in range(3):
        for buf in bufs:
            for t in buf[5]:
                t.fill_(7)
        torch.cuda.synchronize()
        for buf, st in zip(bufs, streams):
            run(buf, st)
        torch.cuda.synchronize()
        for i, buf in enumerate(bufs):
            for got, ref in zip(buf[5], want[i]):
                assert torch.equal(got, ref), f"case {i}, repetition {rep}"
    say("  two streams: results equal to the serial calls")
