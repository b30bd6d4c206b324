"""Comparison metric used by the parity gates (TEST INFRASTRUCTURE, see oracle/attention.py).

"From-scratch GPU LLM training", page summary ("Parity"): tensors are compared with a CPU
reference by relative L2 error. Reading: rel-L2(x, ref) = ||x - ref||_2 / ||ref||_2 over the
whole tensor, accumulated in float64, with ref the oracle's result.
"""
from __future__ import annotations

import numpy as np


def rel_l2(x, ref) -> float:
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    num = np.sqrt(np.sum((x - ref) ** 2))
    den = np.sqrt(np.sum(ref ** 2))
    if den == 0.0:
        return float(num)
    return float(num / den)
