"""Key-split decode forward on the GPU (attn_decode_fwd), dense and paged K/V.

* Against the fp64 oracle: one query per sequence and short query chunks (up to 32 packed rows
  of a KV group), grouped heads, key counts not a multiple of 128, windows and sinks.
* Against the tiled forward (attn_fwd_qk / attn_fwd_paged) on the same inputs: the same outputs up
  to rounding (the key-split sums in a different order).
* Paged: sequences of different lengths through a shuffled pool.
* Determinism: two runs give the same bits.
"""
import math

import numpy as np
import pytest

import oracle
from causal_attention_fa2_amd.workloads import random_tensor
from gpu_util import GATES, download, say, upload

pytestmark = pytest.mark.gpu


def _decode(q, k, v, dtype, window=0, sink=0, scale=None, table=None, lens=None, max_keys=None):
    import torch
    import causal_attention_fa2_amd as fa
    tq, tk, tv = upload(q, dtype), upload(k, dtype), upload(v, dtype)
    B, Hq, Sq, D = q.shape
    Hkv = k.shape[1]
    paged = table is not None
    mk = max_keys if paged else k.shape[2]
    ws = torch.empty(fa.attn_decode_workspace_bytes(B, Hq, Hkv, Sq, mk, D), dtype=torch.uint8, device="cuda")
    o = torch.empty_like(tq)
    lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device="cuda")
    kw = {}
    if paged:
        kw = dict(block_table=torch.from_numpy(table).cuda(),
                  seqlen_k=torch.from_numpy(np.asarray(lens, dtype=np.int32)).cuda())
    fa.attn_decode_fwd(tq, tk, tv, o, lse, ws, True, window, scale, None, sink, **kw)
    torch.cuda.synchronize()
    return download(o), lse.double().cpu().numpy()


DENSE = [
    # Hq, Hkv, Sq, Sk, D, window, sink
    (8, 1, 1, 300, 128, 0, 0),
    (64, 8, 1, 4096, 128, 0, 0),
    (64, 8, 4, 1000, 128, 0, 0),
    (16, 2, 2, 777, 64, 0, 0),
    (8, 2, 8, 129, 128, 0, 0),
    (32, 4, 1, 2000, 128, 256, 4),
    (8, 8, 32, 500, 64, 100, 0),
    (4, 4, 1, 1, 128, 0, 0),
]


@pytest.mark.parametrize("case", DENSE, ids=lambda c: "-".join(map(str, c)))
def test_decode_dense_parity(case):
    Hq, Hkv, Sq, Sk, D, window, sink = case
    say(f"decode dense {case}")
    dtype = "bf16"
    q = random_tensor((2, Hq, Sq, D), dtype, 90 + Sq)
    k = random_tensor((2, Hkv, Sk, D), dtype, 91)
    v = random_tensor((2, Hkv, Sk, D), dtype, 92)
    scale = 1.0 / math.sqrt(D)
    O, L = _decode(q, k, v, dtype, window, sink, scale)
    ref_o, ref_l = oracle.forward(q, k, v, True, window, scale, sink=sink)
    eo, el = oracle.rel_l2(O, ref_o), oracle.rel_l2(L, ref_l)
    say(f"  parity O={eo:.2e} LSE={el:.2e}")
    assert eo <= GATES[dtype]["O"] and el <= GATES[dtype]["LSE"]


def test_decode_matches_tiled_forward_and_is_deterministic():
    import torch
    import causal_attention_fa2_amd as fa
    dtype, Hq, Hkv, Sq, Sk, D = "bf16", 64, 8, 1, 3000, 128
    say("decode vs tiled forward")
    q = random_tensor((2, Hq, Sq, D), dtype, 95)
    k = random_tensor((2, Hkv, Sk, D), dtype, 96)
    v = random_tensor((2, Hkv, Sk, D), dtype, 97)
    O1, L1 = _decode(q, k, v, dtype)
    O2, L2 = _decode(q, k, v, dtype)
    assert np.array_equal(O1, O2) and np.array_equal(L1, L2)
    tq, tk, tv = upload(q, dtype), upload(k, dtype), upload(v, dtype)
    o, lse = fa.forward(tq, tk, tv, True, 0)
    torch.cuda.synchronize()
    assert oracle.rel_l2(O1, download(o)) <= 1e-2
    assert np.max(np.abs(L1 - lse.double().cpu().numpy())) <= 1e-3


@pytest.mark.parametrize("bs,Sq,window,sink", [(16, 1, 0, 0), (64, 2, 0, 0), (256, 1, 0, 0), (16, 1, 300, 3),
                                               (32, 3, 1000, 0)])
def test_decode_paged_parity(bs, Sq, window, sink):
    """Sequences of 1500, 70, 4100 and 129 keys: the longer ones leave chunks that lie past the
    shorter ones' keys or (with a window) before every query's window; those chunks are skipped."""
    say(f"decode paged bs={bs} Sq={Sq} window={window} sink={sink}")
    dtype, Hq, Hkv, D = "bf16", 32, 4, 128
    lens = [1500, 70, 4100, 129]
    B, Smax = len(lens), max(lens)
    q = random_tensor((B, Hq, Sq, D), dtype, 100 + bs)
    kd = random_tensor((B, Hkv, Smax, D), dtype, 101)
    vd = random_tensor((B, Hkv, Smax, D), dtype, 102)
    rng = np.random.default_rng(bs)
    need = [-(-n // bs) for n in lens]
    nb = sum(need) + 2
    order = rng.permutation(nb)
    kp = np.zeros((nb, Hkv, bs, D), np.float32)
    vp = np.zeros((nb, Hkv, bs, D), np.float32)
    table = np.full((B, max(need) + 1), -3, np.int32)
    i = 0
    for b in range(B):
        for t in range(need[b]):
            ph = order[i]
            i += 1
            table[b, t] = ph
            n = min(bs, lens[b] - t * bs)
            kp[ph, :, :n] = kd[b, :, t * bs:t * bs + n]
            vp[ph, :, :n] = vd[b, :, t * bs:t * bs + n]
    scale = 1.0 / math.sqrt(D)
    O, L = _decode(q, kp, vp, dtype, window, sink, scale, table=table, lens=lens, max_keys=table.shape[1] * bs)
    ref_o, ref_l = oracle.paged_forward(q, kp.astype(np.float64), vp.astype(np.float64), table, lens, True,
                                        window, scale, sink=sink)
    eo, el = oracle.rel_l2(O, ref_o), oracle.rel_l2(L, ref_l)
    say(f"  parity O={eo:.2e} LSE={el:.2e}")
    assert eo <= GATES[dtype]["O"] and el <= GATES[dtype]["LSE"]
