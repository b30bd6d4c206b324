"""Seeded synthetic inputs for causal / sliding-window grouped-query attention.

This module draws random tensors and rounds them to the element type; it holds none of
attention's arithmetic. Both the fp64 oracle (through the tests and the bench's CPU leg)
and the HIP path receive exactly the arrays produced here, so the two sides always see
the same rounded bits.

Workloads (shapes and distributions of the attention configurations this library is
measured and checked on; no dataset is involved, every input is synthetic):

  tiny-causal-f32        B=1, Hq=Hkv=2,  S=64,    D=64,  f32,  causal
  small-mha-causal-bf16  B=4, Hq=Hkv=16, S=1024,  D=64,  bf16, causal
  gqa64x8-s4096-d128     B=1, Hq=64, Hkv=8, S=4096,  D=128, bf16, causal, dO ~ N(0, 0.1^2)
  swa-w1024-s8192        B=1, Hq=Hkv=16, S=8192,  D=64,  bf16, causal, window 1024
  gqa64x8-s32768-d128    B=1, Hq=64, Hkv=8, S=32768, D=128, bf16, causal, Q and K
                         multiplied per head by factors drawn U(0.5, 2)
  gqa64x8-q1024-k4096-d128  a prefill chunk: the last 1024 of 4096 positions (Sq=1024 queries,
                         Sk=4096 keys), otherwise as gqa64x8-s4096-d128
  gqa64x8-q1-k4096-d128  one decode query against 4096 cached keys, otherwise as above
  swa-w1024-sink4-s8192  as swa-w1024-s8192 with the first 4 keys kept visible as sinks
  paged-decode-b16-gqa64x8  16 sequences of U[1024, 8192] cached keys in 16-token pool blocks,
                         one decode query each (forward only), Hq=64, Hkv=8, D=128, bf16
  paged-chunk-b4-q512-gqa64x8  4 sequences of U[2048, 8192] keys in 64-token blocks, a 512-query
                         prefill chunk each (forward only)
  docs-gqa64x8-s8192-d128  one 8192-token buffer of packed documents of U[64, 2048] tokens
                         (the last one cut to fit), Hq=64, Hkv=8, D=128, bf16, causal
  decode-b1-gqa64x8-k4096  gqa64x8-q1-k4096-d128 through the key-split decode forward
  decode-paged-b16-gqa64x8  paged-decode-b16-gqa64x8 through the key-split decode forward

Draw order per workload: numpy.random.default_rng(seed); Q, K, V, dO as float32
standard normals in that order (Q and dO with Sq rows, K and V with S rows) (dO then scaled by its standard deviation); then, for the
long-context workload only, one factor per query head and one per KV head. Every tensor
is then rounded once to the element type (round-to-nearest-even for bf16).
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    Hq: int
    Hkv: int
    S: int
    D: int
    dtype: str  # "f32" or "bf16"
    causal: bool
    window: int  # 0 = no window; W >= 1 = key j visible to query i iff i - W < j <= i
    seed: int
    do_std: float = 1.0
    head_factor: bool = False  # multiply Q and K per head by U(0.5, 2) factors
    Sq: int = 0  # query rows when fewer than the S keys (the last Sq positions); 0 = S
    sink: int = 0  # leading keys that stay visible beside the window
    paged: int = 0  # > 0: K/V in a paged pool of blocks of this many tokens (forward only)
    len_min: int = 0  # paged: sequence b holds U[len_min, S] keys
    docs: tuple = ()  # (min, max): packed documents of U[min, max] tokens per batch row
    decode: bool = False  # forward only, through the key-split decode forward

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.D)

    @property
    def n_q(self) -> int:
        return self.Sq or self.S

    def shapes(self):
        return ((self.B, self.Hq, self.n_q, self.D), (self.B, self.Hkv, self.S, self.D))


WORKLOADS = {
    w.name: w
    for w in (
        Workload("tiny-causal-f32", 1, 2, 2, 64, 64, "f32", True, 0, 1001),
        Workload("small-mha-causal-bf16", 4, 16, 16, 1024, 64, "bf16", True, 0, 1002),
        Workload("gqa64x8-s4096-d128", 1, 64, 8, 4096, 128, "bf16", True, 0, 1003, do_std=0.1),
        Workload("swa-w1024-s8192", 1, 16, 16, 8192, 64, "bf16", True, 1024, 1004),
        Workload("gqa64x8-s32768-d128", 1, 64, 8, 32768, 128, "bf16", True, 0, 1005,
                 head_factor=True),
        Workload("gqa64x8-q1024-k4096-d128", 1, 64, 8, 4096, 128, "bf16", True, 0, 1006,
                 do_std=0.1, Sq=1024),
        Workload("gqa64x8-q1-k4096-d128", 1, 64, 8, 4096, 128, "bf16", True, 0, 1007,
                 do_std=0.1, Sq=1),
        Workload("swa-w1024-sink4-s8192", 1, 16, 16, 8192, 64, "bf16", True, 1024, 1008, sink=4),
        Workload("paged-decode-b16-gqa64x8", 16, 64, 8, 8192, 128, "bf16", True, 0, 1009, Sq=1,
                 paged=16, len_min=1024),
        Workload("paged-chunk-b4-q512-gqa64x8", 4, 64, 8, 8192, 128, "bf16", True, 0, 1010, Sq=512,
                 paged=64, len_min=2048),
        Workload("docs-gqa64x8-s8192-d128", 1, 64, 8, 8192, 128, "bf16", True, 0, 1011, do_std=0.1,
                 docs=(64, 2048)),
        Workload("decode-b1-gqa64x8-k4096", 1, 64, 8, 4096, 128, "bf16", True, 0, 1007, do_std=0.1,
                 Sq=1, decode=True),
        Workload("decode-paged-b16-gqa64x8", 16, 64, 8, 8192, 128, "bf16", True, 0, 1009, Sq=1,
                 paged=16, len_min=1024, decode=True),
    )
}


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); returns float32
    arrays whose values are exactly representable in bfloat16. Inputs here are finite."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    r = ((u + bias) & np.uint32(0xFFFF0000)).astype(np.uint32)
    return r.view(np.float32)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Upper 16 bits of float32 values that are already bfloat16-representable."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    assert not np.any(u & np.uint32(0xFFFF)), "value is not bfloat16-representable"
    return (u >> np.uint32(16)).astype(np.uint16)


def to_elem(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "bf16":
        return round_to_bf16(x)
    raise ValueError(f"unknown element type {dtype!r}")


def make_inputs(w: Workload, *, seed: int | None = None, B: int | None = None,
                Hq: int | None = None, Hkv: int | None = None, S: int | None = None,
                D: int | None = None):
    """Draw (q, k, v, do) for workload `w` (optionally overriding its shape or seed).

    Returns float32 numpy arrays holding element-type-representable values:
    q, do [B,Hq,Sq,D]; k, v [B,Hkv,S,D], all contiguous with D fastest (Sq = S unless the
    workload has fewer queries than keys)."""
    B = w.B if B is None else B
    Hq = w.Hq if Hq is None else Hq
    Hkv = w.Hkv if Hkv is None else Hkv
    S = w.S if S is None else S
    D = w.D if D is None else D
    Sq = min(w.Sq, S) if w.Sq else S
    rng = np.random.default_rng(w.seed if seed is None else seed)
    q = rng.standard_normal((B, Hq, Sq, D), dtype=np.float32)
    k = rng.standard_normal((B, Hkv, S, D), dtype=np.float32)
    v = rng.standard_normal((B, Hkv, S, D), dtype=np.float32)
    do = rng.standard_normal((B, Hq, Sq, D), dtype=np.float32)
    if w.do_std != 1.0:
        do *= np.float32(w.do_std)
    if w.head_factor:
        cq = rng.uniform(0.5, 2.0, size=Hq).astype(np.float32)
        ck = rng.uniform(0.5, 2.0, size=Hkv).astype(np.float32)
        q *= cq[None, :, None, None]
        k *= ck[None, :, None, None]
    return tuple(to_elem(t, w.dtype) for t in (q, k, v, do))


def paged_layout(w: Workload, k: np.ndarray, v: np.ndarray):
    """Sequence lengths and a paged layout of k / v for a paged workload: (k_pool, v_pool, table,
    lens). Lengths are U[len_min, S] (seeded); the first lens[b] keys of sequence b go to
    ceil(lens[b] / block) pool blocks in a seeded random order; the table rows are padded with 0."""
    rng = np.random.default_rng(w.seed + 7919)
    lens = rng.integers(w.len_min, w.S + 1, size=w.B).astype(np.int32)
    lens = np.maximum(lens, w.n_q)
    bs = w.paged
    need = [-(-int(n) // bs) for n in lens]
    nb = sum(need)
    order = rng.permutation(nb)
    kp = np.zeros((nb, w.Hkv, bs, w.D), np.float32)
    vp = np.zeros((nb, w.Hkv, bs, w.D), np.float32)
    table = np.zeros((w.B, max(need)), np.int32)
    i = 0
    for b in range(w.B):
        for t in range(need[b]):
            phys = order[i]
            i += 1
            table[b, t] = phys
            n = min(bs, int(lens[b]) - t * bs)
            kp[phys, :, :n] = k[b, :, t * bs:t * bs + n]
            vp[phys, :, :n] = v[b, :, t * bs:t * bs + n]
    return kp, vp, table, lens


def document_boundaries(w: Workload) -> np.ndarray:
    """cu_seqlens [B, n + 1] int32 for a packed-document workload: per batch row, documents of
    U[docs[0], docs[1]] tokens (seeded) until S is filled, the last one cut to fit; rows with fewer
    documents repeat S at the end."""
    rng = np.random.default_rng(w.seed + 104729)
    rows = []
    for _ in range(w.B):
        cu = [0]
        while cu[-1] < w.S:
            cu.append(min(w.S, cu[-1] + int(rng.integers(w.docs[0], w.docs[1] + 1))))
        rows.append(cu)
    n = max(len(r) for r in rows)
    return np.array([r + [w.S] * (n - len(r)) for r in rows], dtype=np.int32)


def random_tensor(shape, dtype: str, seed: int, std: float = 1.0) -> np.ndarray:
    """One seeded N(0, std^2) tensor rounded to the element type (for ad-hoc test shapes)."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return to_elem(x, dtype)
