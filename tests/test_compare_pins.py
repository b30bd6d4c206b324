"""Pins for the parity metric itself (CPU only).

"From-scratch GPU LLM training", page summary ("Parity"): tensors are matched against a CPU
reference by relative L2 error. oracle.compare.rel_l2 reads that as ||x - ref||_2 / ||ref||_2 over
the whole tensor in float64 (||x - ref||_2 when ref is all zeros). Every GPU parity gate goes
through this one function, so it is pinned here by hand-computed values (no call to itself or to
a library norm) chosen so that each plausible slip -- a dropped square root, the wrong tensor in
the denominator, a max-abs or L1 norm, a per-row average, a zero reference returned as 0 --
changes at least one of them, and planted versions of those slips are shown to fail.
"""
import math

import numpy as np
import pytest

from oracle.compare import rel_l2

# (x, ref, exact value) -- each value worked out by hand:
CASES = [
    # diff (0.3, 0.4): norm 0.5; ref (3, 4): norm 5  ->  0.1
    ([3.3, 4.4], [3.0, 4.0], 0.1),
    # identical tensors -> 0
    ([1.5, -2.0, 7.25], [1.5, -2.0, 7.25], 0.0),
    # ||x|| = 2 differs from ||ref|| = 1: diff norm 1 / ||ref|| = 1  ->  1 (||x|| below would give 0.5)
    ([2.0, 0.0], [1.0, 0.0], 1.0),
    # four unit differences: L2 norm 2, max-abs 1, L1 4; ||ref|| = 2  ->  1
    ([3.0, 1.0, 1.0, 1.0], [2.0, 0.0, 0.0, 0.0], 1.0),
    # the whole tensor, not a mean over rows: rows with norms 1 and 100, only row 0 off by 1
    # -> 1 / sqrt(1 + 10000)   (a per-row mean would give 0.5)
    ([[2.0, 0.0], [0.0, 100.0]], [[1.0, 0.0], [0.0, 100.0]], 1.0 / math.sqrt(10001.0)),
    # signs: diff (-6, -8) norm 10, ref norm 5  ->  2
    ([-3.0, -4.0], [3.0, 4.0], 2.0),
    # zero reference: the absolute L2 norm of x, (3, 4) -> 5
    ([3.0, 4.0], [0.0, 0.0], 5.0),
]


def _check(fn):
    for x, ref, want in CASES:
        got = fn(np.array(x), np.array(ref))
        assert abs(got - want) <= 1e-14 * max(1.0, abs(want)), (x, ref, got, want)


def test_rel_l2_hand_values():
    _check(rel_l2)


def test_rel_l2_accumulates_in_float64():
    # float32 entries 1 + 2^-12 (exact in float32) against a zero reference: the result is
    # sqrt(3 (1 + 2^-12)^2) = sqrt(3) (1 + 2^-12), to float64 rounding. Squaring and summing in
    # float32 rounds 1 + 2^-11 + 2^-24 to 1 + 2^-11 and the square root to 24 bits: about
    # 2^-25 relative off, far outside the float64 bound below.
    x = np.full(3, 1.0 + 2.0 ** -12, dtype=np.float32)
    want = math.sqrt(3.0) * (1.0 + 2.0 ** -12)
    assert abs(rel_l2(x, np.zeros(3, dtype=np.float32)) - want) <= 4e-16 * want
    in_f32 = float(np.sqrt(np.sum(x * x, dtype=np.float32)))
    assert abs(in_f32 - want) > 1e-9 * want


# Plausible wrong versions of the metric; each must fail at least one hand value.
def _no_sqrt(x, ref):
    return float(np.sum((x - ref) ** 2) / np.sum(ref ** 2)) if np.any(ref) else float(np.sum((x - ref) ** 2))


def _x_denominator(x, ref):
    return float(np.linalg.norm(x - ref) / np.linalg.norm(x))


def _max_abs(x, ref):
    return float(np.max(np.abs(x - ref)) / np.max(np.abs(ref))) if np.any(ref) else float(np.max(np.abs(x)))


def _l1(x, ref):
    return float(np.sum(np.abs(x - ref)) / np.sum(np.abs(ref))) if np.any(ref) else float(np.sum(np.abs(x)))


def _row_mean(x, ref):
    x2, r2 = np.atleast_2d(x), np.atleast_2d(ref)
    vals = [np.linalg.norm(a - b) / np.linalg.norm(b) if np.any(b) else np.linalg.norm(a) for a, b in zip(x2, r2)]
    return float(np.mean(vals))


def _zero_ref_is_zero(x, ref):
    return float(np.linalg.norm(x - ref) / np.linalg.norm(ref)) if np.any(ref) else 0.0


MUTANTS = {"no_sqrt": _no_sqrt, "x_denominator": _x_denominator, "max_abs": _max_abs, "l1": _l1,
           "row_mean": _row_mean, "zero_ref_is_zero": _zero_ref_is_zero}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_metric_mistake_is_caught(name):
    with pytest.raises(AssertionError):
        _check(MUTANTS[name])
