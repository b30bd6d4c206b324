"""Forward against a paged K/V cache on the GPU (attn_fwd_paged).

* Against the fp64 oracle (which gathers each sequence's K/V token by token through the table):
  block sizes 16 .. 256, sequences of different lengths in one batch, S_q = 1 decode and longer
  query chunks, grouped heads, windows and sinks, shuffled pools with unused noise blocks and
  table entries past a sequence's end set to out-of-range values (never read).
* Bit-exactness: the paged call reproduces attn_fwd_qk on the same keys laid out densely, bit
  for bit (the same key tiles are visited in the same order; only the addressing differs).
* Blocks shared by two sequences.
"""
import math

import numpy as np
import pytest

import oracle
from causal_attention_fa2_amd.workloads import random_tensor
from gpu_util import GATES, download, say, tdtype, upload

pytestmark = pytest.mark.gpu


def _layout(kd, vd, lens, bs, seed, extra=3):
    """Pools [nb, Hkv, bs, D] holding each sequence's first lens[b] keys of kd / vd in shuffled
    blocks, noise elsewhere; table [B, max_blocks] with -5 past each sequence's last block."""
    B, Hkv, S, D = kd.shape
    rng = np.random.default_rng(seed)
    need = [-(-int(n) // bs) for n in lens]
    nb = sum(need) + extra
    order = rng.permutation(nb)
    kp = rng.standard_normal((nb, Hkv, bs, D)).astype(np.float32)
    vp = rng.standard_normal((nb, Hkv, bs, D)).astype(np.float32)
    maxb = max(need) + 1
    table = np.full((B, maxb), -5, dtype=np.int32)
    i = 0
    for b in range(B):
        for t in range(need[b]):
            phys = order[i]
            i += 1
            table[b, t] = phys
            n = min(bs, int(lens[b]) - t * bs)
            kp[phys, :, :n] = kd[b, :, t * bs:t * bs + n]
            vp[phys, :, :n] = vd[b, :, t * bs:t * bs + n]
    return kp, vp, table


def _run_paged(q, kp, vp, table, lens, dtype, window=0, sink=0, scale=None):
    import torch
    import causal_attention_fa2_amd as fa
    tq, tk, tv = upload(q, dtype), upload(kp, dtype), upload(vp, dtype)
    tt = torch.from_numpy(table).cuda()
    tl = torch.from_numpy(np.asarray(lens, dtype=np.int32)).cuda()
    B, Hq, Sq, D = q.shape
    o = torch.empty_like(tq)
    lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device="cuda")
    fa.attn_fwd_paged(tq, tk, tv, tt, tl, o, lse, True, window, scale, None, sink)
    torch.cuda.synchronize()
    return o, lse


CASES = [
    # dtype, Hq, Hkv, Sq, lens, D, block size, window, sink
    ("bf16", 8, 2, 1, (300, 1000, 17), 128, 16, 0, 0),
    ("bf16", 4, 2, 64, (64, 700), 64, 32, 0, 0),
    ("bf16", 4, 4, 100, (513, 100), 128, 64, 50, 4),
    ("bf16", 8, 2, 5, (129, 2050, 640), 128, 128, 0, 0),
    ("bf16", 4, 2, 200, (1200, 4000), 128, 256, 0, 0),
    ("bf16", 8, 1, 1, (4096, 33), 64, 16, 256, 4),
    ("f32", 2, 1, 5, (90, 200), 64, 16, 0, 0),
    ("f32", 4, 2, 40, (40, 333), 128, 32, 20, 2),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(map(str, c)))
def test_paged_parity(case):
    dtype, Hq, Hkv, Sq, lens, D, bs, window, sink = case
    say(f"paged case {case}")
    B, Smax = len(lens), max(lens)
    q = random_tensor((B, Hq, Sq, D), dtype, 50 + Sq)
    kd = random_tensor((B, Hkv, Smax, D), dtype, 51)
    vd = random_tensor((B, Hkv, Smax, D), dtype, 52)
    kp, vp, table = _layout(kd, vd, lens, bs, seed=53)
    scale = 1.0 / math.sqrt(D)
    o, lse = _run_paged(q, kp, vp, table, lens, dtype, window, sink, scale)
    O, L = oracle.paged_forward(q, kp.astype(np.float64), vp.astype(np.float64), table, lens, True,
                                window, scale, sink=sink)
    got_o, got_l = download(o), lse.double().cpu().numpy()
    assert np.all(np.isfinite(got_o))
    e_o = oracle.rel_l2(got_o, O)
    e_l = oracle.rel_l2(got_l, L)
    say(f"  parity O={e_o:.2e} LSE={e_l:.2e}")
    assert e_o <= GATES[dtype]["O"] and e_l <= GATES[dtype]["LSE"]


@pytest.mark.parametrize("bs,Sq", [(16, 1), (32, 77), (64, 300), (256, 1)])
def test_paged_equals_dense_bitwise(bs, Sq):
    """Each sequence's paged result equals attn_fwd_qk on its keys laid out densely, bit for bit."""
    import torch
    import causal_attention_fa2_amd as fa
    dtype, Hq, Hkv, D = "bf16", 8, 2, 128
    lens = (1500, 700, 333)
    say(f"paged vs dense bs={bs} Sq={Sq}")
    B, Smax = len(lens), max(lens)
    q = random_tensor((B, Hq, Sq, D), dtype, 60)
    kd = random_tensor((B, Hkv, Smax, D), dtype, 61)
    vd = random_tensor((B, Hkv, Smax, D), dtype, 62)
    kp, vp, table = _layout(kd, vd, lens, bs, seed=63)
    o, lse = _run_paged(q, kp, vp, table, lens, dtype, 200, 3)
    for b, n in enumerate(lens):
        tq = upload(q[b:b + 1], dtype)
        tk = upload(np.ascontiguousarray(kd[b:b + 1, :, :n]), dtype)
        tv = upload(np.ascontiguousarray(vd[b:b + 1, :, :n]), dtype)
        od = torch.empty_like(tq)
        ld = torch.empty((1, Hq, Sq), dtype=torch.float32, device="cuda")
        fa.attn_fwd_qk(tq, tk, tv, od, ld, True, 200, None, None, 3)
        torch.cuda.synchronize()
        assert torch.equal(od[0], o[b]) and torch.equal(ld[0], lse[b]), b


def test_paged_shared_blocks():
    """Two sequences whose tables share their first blocks: each equals its own dense problem."""
    dtype, Hq, Hkv, D, bs = "bf16", 4, 2, 64, 16
    say("paged shared blocks")
    rng = np.random.default_rng(70)
    kp = random_tensor((10, Hkv, bs, D), dtype, 71)
    vp = random_tensor((10, Hkv, bs, D), dtype, 72)
    table = np.array([[4, 2, 8, 0], [4, 2, 1, 9]], dtype=np.int32)
    lens = (50, 64)
    q = random_tensor((2, Hq, 3, D), dtype, 73)
    o, lse = _run_paged(q, kp, vp, table, lens, dtype)
    O, L = oracle.paged_forward(q, kp.astype(np.float64), vp.astype(np.float64), table, lens, True, 0,
                                1.0 / math.sqrt(D))
    assert oracle.rel_l2(download(o), O) <= GATES[dtype]["O"]
    assert oracle.rel_l2(lse.double().cpu().numpy(), L) <= GATES[dtype]["LSE"]
