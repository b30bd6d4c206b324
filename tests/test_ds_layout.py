"""The stored-dS layout (DsMap in csrc/launch.h), compiled for the host: the blocks it holds for a
query block are exactly the 32-key blocks holding a pair the oracle's mask leaves visible; every
(batch x KV head, query head, query block, key block) gets its own 2 KB slot inside the region; and
the query heads of a KV group lie back to back for each 64-row query tile and key block (the
contiguous runs the dQ pass streams)."""
import os
import subprocess

import numpy as np
import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "causal_attention_fa2_amd", "csrc")

# Sq, Sk, causal, Hq, Hkv, B: ragged squares, fewer queries than keys at offsets that are not
# multiples of 32 or 64, one query row, odd query-block counts, no causal mask
CASES = [(1, 1, 1, 2, 1, 1), (31, 31, 1, 2, 2, 1), (32, 32, 1, 3, 1, 2), (33, 33, 1, 2, 1, 1),
         (64, 64, 1, 4, 2, 1), (65, 65, 1, 2, 1, 1), (200, 200, 1, 8, 2, 1), (300, 333, 1, 4, 2, 2),
         (1, 300, 1, 2, 1, 1), (33, 100, 1, 2, 2, 1), (97, 130, 1, 6, 2, 1), (130, 130, 0, 2, 1, 1),
         (33, 170, 0, 4, 2, 1), (257, 257, 1, 16, 2, 1)]


@pytest.fixture(scope="module")
def layout():
    exe = os.path.join(ROOT, "_build", "ds_layout_driver")
    os.makedirs(os.path.dirname(exe), exist_ok=True)
    subprocess.run(["g++", "-O2", "-std=c++17", "-I", CSRC,
                    os.path.join(ROOT, "tests", "native", "ds_layout_driver.cpp"), "-o", exe], check=True)
    inp = "".join(" ".join(map(str, c)) + "\n" for c in CASES)
    out = subprocess.run([exe], input=inp, capture_output=True, text=True, check=True).stdout
    res, cur = {}, None
    for line in out.splitlines():
        f = line.split()
        if f[0] == "CFG":
            cur = tuple(map(int, f[1:7]))
            res[cur] = {"bytes": int(f[7]), "blocks": {}}
        else:
            bg, hg, i, n = map(int, f[1:5])
            res[cur]["blocks"][(bg, hg, i)] = [int(x) for x in f[5:5 + n]]
    return res


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(map(str, c)))
def test_ds_layout(layout, case):
    Sq, Sk, causal, Hq, Hkv, B = case
    r = layout[case]
    G, nqb, nkb = Hq // Hkv, -(-Sq // 32), -(-Sk // 32)
    m = oracle.visible_mask(np.arange(Sq), np.arange(Sk), bool(causal), 0, Sk - Sq, 0)
    P = np.zeros((nqb * 32, nkb * 32), bool)
    P[:Sq, :Sk] = m
    needed = P.reshape(nqb, 32, nkb, 32).any(axis=(1, 3))
    seen = set()
    for bg in range(B * Hkv):
        for hg in range(G):
            for i in range(nqb):
                offs = r["blocks"][(bg, hg, i)]
                # exactly the key blocks holding a visible pair of this query block
                assert list(np.nonzero(needed[i])[0]) == list(range(len(offs))), (case, i)
                for o in offs:
                    assert o % 2048 == 0 and 0 <= o and o + 2048 <= r["bytes"], (case, bg, hg, i, o)
                    assert o not in seen, (case, bg, hg, i, o)
                    seen.add(o)
    # the heads of a group back to back: block (head hg + 1) = block (head hg) + 4 KB, and the two
    # 32-row halves of a 64-row tile 2 KB apart
    for bg in range(B * Hkv):
        for i in range(nqb):
            for j in range(len(r["blocks"][(bg, 0, i)])):
                for hg in range(G - 1):
                    assert r["blocks"][(bg, hg + 1, i)][j] == r["blocks"][(bg, hg, i)][j] + 4096, (case, bg, i, j)
                if i % 2 == 1 and j < len(r["blocks"][(bg, 0, i - 1)]):
                    assert r["blocks"][(bg, 0, i)][j] == r["blocks"][(bg, 0, i - 1)][j] + 2048, (case, bg, i, j)
