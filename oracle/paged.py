"""Reading K and V out of a paged cache, for the fp64 oracle.

TEST INFRASTRUCTURE (same rules as oracle.attention: only tests/, __graft_entry__.smoke() and
bench.py's CPU-baseline leg use it; it imports nothing from the product package).

"KYNETRA FOUNDRY" page, paged-KV paragraph: a sequence's K/V cache is split into fixed-size
blocks that can sit anywhere in a global pool, and a per-sequence block table maps each logical
token position to its physical block, so attention reads K/V through that indirection.

Readings (also in the design notes): a pool is [num_blocks, Hkv, block_size, D]; token t of
sequence b is row t % block_size of pool block block_table[b, t // block_size]; sequence b holds
seqlen_k[b] tokens and its S_q queries are its last S_q positions. Attention itself is exactly
oracle.attention.forward on the gathered, contiguous K and V of each sequence.
"""
from __future__ import annotations

import numpy as np

from .attention import forward

__all__ = ["gather_sequence", "paged_forward"]


def gather_sequence(pool, block_table, b: int, n_tokens: int, block_size: int) -> np.ndarray:
    """[Hkv, n_tokens, D] float64: token by token, through the block table."""
    nb, Hkv, bs, D = pool.shape
    assert bs == block_size
    out = np.empty((Hkv, n_tokens, D))
    for t in range(n_tokens):
        phys = int(block_table[b, t // block_size])
        out[:, t, :] = pool[phys, :, t % block_size, :]
    return out


def paged_forward(q, k_pool, v_pool, block_table, seqlen_k, causal=True, window=0, scale=None, sink=0):
    """O [B, Hq, S_q, D] and LSE [B, Hq, S_q] (float64): sequence b attends over its own
    seqlen_k[b] keys gathered from the pools."""
    B, Hq, Sq, D = q.shape
    bs = k_pool.shape[2]
    O = np.zeros((B, Hq, Sq, D))
    LSE = np.zeros((B, Hq, Sq))
    for b in range(B):
        n = int(seqlen_k[b])
        K = gather_sequence(k_pool, block_table, b, n, bs)
        V = gather_sequence(v_pool, block_table, b, n, bs)
        o, lse = forward(q[b:b + 1], K[None], V[None], causal, window, scale, sink=sink)
        O[b], LSE[b] = o[0], lse[0]
    return O, LSE
