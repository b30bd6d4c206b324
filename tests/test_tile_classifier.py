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
# fewer queries than keys: (S_q, S_k)
QK_LIST = [(1, 2), (1, 100), (1, 257), (5, 300), (31, 64), (33, 200), (64, 65), (100, 129),
           (127, 300), (128, 256), (200, 257), (255, 300)]
W_LIST = [0, 1, 2, 31, 32, 33, 63, 64, 65, 127, 128, 129, 1024]
TILES = [32, 64, 128]
# (window, sink) pairs for the sink configurations
SINK_LIST = [(1, 1), (2, 4), (31, 1), (33, 32), (64, 33), (65, 64), (100, 65), (1, 130), (128, 200), (32, 300)]


def _configs():
    for sq, sk in [(S, S) for S in S_LIST] + QK_LIST:
        for br in TILES:
            for bc in TILES:
                yield (sq, sk, br, bc, 0, 0, 0)
                for W in W_LIST:
                    yield (sq, sk, br, bc, 1, W, 0)
                if sk >= 64:
                    for W, n in SINK_LIST:
                        yield (sq, sk, br, bc, 1, W, n)


def test_tile_classifier_matches_mask(driver):
    cfgs = list(_configs())
    inp = "".join(" ".join(map(str, c)) + "\n" for c in cfgs)
    out = subprocess.run([driver], input=inp, capture_output=True, text=True, check=True).stdout
    lines = iter(out.splitlines())
    checked = 0
    for cfg in cfgs:
        Sq, Sk, br, bc, causal, W, n_sink = cfg
        assert next(lines) == "CFG " + " ".join(map(str, cfg))
        nq, nk = -(-Sq // br), -(-Sk // bc)
        m = oracle.visible_mask(np.arange(Sq), np.arange(Sk), bool(causal), W, Sk - Sq, n_sink)
        # pad to whole tiles: out-of-range rows / keys are never visible
        P = np.zeros((nq * br, nk * bc), bool)
        P[:Sq, :Sk] = m
        blocks = P.reshape(nq, br, nk, bc)
        any_vis = blocks.any(axis=(1, 3))
        inb = np.zeros((nq * br, nk * bc), bool)
        inb[:Sq, :Sk] = True
        all_vis = (blocks & inb.reshape(nq, br, nk, bc)).all(axis=(1, 3)) & \
            inb.reshape(nq, br, nk, bc).all(axis=(1, 3)) & blocks.all(axis=(1, 3))
        for qt in range(nq):
            tag, q, ns, lo, hi = next(lines).split()
            assert (tag, int(q)) == ("R", qt)
            ns, lo, hi = int(ns), int(lo), int(hi)
            assert 0 <= ns and (ns == 0 or ns < lo) and lo <= hi, (cfg, qt)
            listed = list(range(ns)) + list(range(lo, hi + 1))
            # exactly the key tiles holding a visible pair: nothing missed, nothing extra
            assert listed == list(np.nonzero(any_vis[qt])[0]), (cfg, qt)
        for kt in range(nk):
            tag, kk, lo, hi = next(lines).split()
            assert (tag, int(kk)) == ("C", kt)
            rows = np.nonzero(any_vis[:, kt])[0]
            if rows.size == 0:  # keys no query sees (they fall out of every window)
                assert int(lo) > int(hi), (cfg, kt)
                continue
            assert (int(lo), int(hi)) == (rows.min(), rows.max()), (cfg, kt)
            assert np.all(any_vis[rows.min():rows.max() + 1, kt]), (cfg, kt)
        vis = next(lines)
        assert vis[:2] == "V "
        got = np.frombuffer(vis[2:].encode(), dtype=np.uint8).reshape(Sq, Sk) == ord("1")
        assert np.array_equal(got, m), cfg
        classes = next(lines).split()[1] if nq * nk else ""
        want = np.where(~any_vis, "E", np.where(all_vis, "F", "P")).reshape(-1)
        assert classes == "".join(want), cfg
        checked += 1
    assert checked == len(cfgs)
