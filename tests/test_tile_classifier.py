"""The integer tile classifier (csrc/tiles.h), compiled for the host, against the oracle's
element-wise visibility mask: block classes must be exact and tile ranges tight."""
import os
import subprocess

import numpy as np
import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "causal_attention_fa2_amd", "csrc")


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    exe = str(tmp_path_factory.mktemp("tiles") / "tile_driver")
    subprocess.run(["g++", "-O2", "-std=c++17", "-I", CSRC,
                    os.path.join(ROOT, "tests", "native", "tile_driver.cpp"), "-o", exe], check=True)
    return exe


S_LIST = [1, 2, 31, 32, 33, 63, 64, 65, 100, 127, 128, 129, 200, 255, 256, 257, 300]
W_LIST = [0, 1, 2, 31, 32, 33, 63, 64, 65, 127, 128, 129, 1024]
TILES = [32, 64, 128]


def _configs():
    for S in S_LIST:
        for br in TILES:
            for bc in TILES:
                yield (S, br, bc, 0, 0)
                for W in W_LIST:
                    yield (S, br, bc, 1, W)


def test_tile_classifier_matches_mask(driver):
    cfgs = list(_configs())
    inp = "".join(" ".join(map(str, c)) + "\n" for c in cfgs)
    out = subprocess.run([driver], input=inp, capture_output=True, text=True, check=True).stdout
    lines = iter(out.splitlines())
    checked = 0
    for cfg in cfgs:
        S, br, bc, causal, W = cfg
        assert next(lines) == "CFG " + " ".join(map(str, cfg))
        nq, nk = -(-S // br), -(-S // bc)
        m = oracle.visible_mask(np.arange(S), np.arange(S), bool(causal), W)
        # pad to whole tiles: out-of-range rows / keys are never visible
        P = np.zeros((nq * br, nk * bc), bool)
        P[:S, :S] = m
        blocks = P.reshape(nq, br, nk, bc)
        any_vis = blocks.any(axis=(1, 3))
        inb = np.zeros((nq * br, nk * bc), bool)
        inb[:S, :S] = True
        all_vis = (blocks & inb.reshape(nq, br, nk, bc)).all(axis=(1, 3)) & \
            inb.reshape(nq, br, nk, bc).all(axis=(1, 3)) & blocks.all(axis=(1, 3))
        for qt in range(nq):
            tag, q, lo, hi = next(lines).split()
            assert (tag, int(q)) == ("R", qt)
            cols = np.nonzero(any_vis[qt])[0]
            assert (int(lo), int(hi)) == (cols.min(), cols.max()), (cfg, qt)
            assert np.all(any_vis[qt, cols.min():cols.max() + 1]), (cfg, qt)  # contiguous
        for kt in range(nk):
            tag, kk, lo, hi = next(lines).split()
            assert (tag, int(kk)) == ("C", kt)
            rows = np.nonzero(any_vis[:, kt])[0]
            assert (int(lo), int(hi)) == (rows.min(), rows.max()), (cfg, kt)
            assert np.all(any_vis[rows.min():rows.max() + 1, kt]), (cfg, kt)
        classes = next(lines).split()[1] if nq * nk else ""
        want = np.where(~any_vis, "E", np.where(all_vis, "F", "P")).reshape(-1)
        assert classes == "".join(want), cfg
        checked += 1
    assert checked == len(cfgs)
