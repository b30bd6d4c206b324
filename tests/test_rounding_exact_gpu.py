"""Bit-exact check of the output rounding (fp32 accumulation, then round-to-nearest-even to the
element type) on a case whose exact result is known.

Q = 0 makes every visible score 0, and a window of 2 lets row i see keys i-1 and i (row 0 only key
0). So every visible P is exactly 1/2 (1 for row 0) and, exactly:
    O_i   = (V_{i-1} + V_i) / 2                      (O_0 = V_0)
    dV_j  = sum over the group's heads of (P_jj dO_j + P_{j+1,j} dO_{j+1})   (bf16 path)
    dK    = 0                                        (dK = scale * sum dS Q and Q = 0)
    LSE_i = ln 2                                     (LSE_0 = 0)
V and dO are drawn from +-[1, 2) on the bf16 grid, so every fp32 sum above is exact and the only
rounding is the final conversion to the element type; half the sums fall between two bf16 values,
many on a tie, which exercises ties-to-even. The expected values are the oracle's fp64 results
rounded by torch's CPU conversion (an implementation independent of the HIP path).
"""
import math

import numpy as np
import pytest

import oracle
from gpu_util import run_hip, say

pytestmark = pytest.mark.gpu


def _grid_values(shape, seed):
    """Random +-(1 + k/128), k in 0..127: exactly representable in bf16 and in fp32."""
    rng = np.random.default_rng(seed)
    k = rng.integers(0, 128, size=shape)
    s = rng.choice(np.array([-1.0, 1.0]), size=shape)
    return (s * (1.0 + k / 128.0)).astype(np.float32)


def _to_elem_bits(x64: np.ndarray, dtype: str) -> np.ndarray:
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x64, dtype=np.float64))
    if dtype == "bf16":
        return t.to(torch.bfloat16).view(torch.int16).numpy()
    return t.to(torch.float32).view(torch.int32).numpy()


def _gpu_bits(x64: np.ndarray, dtype: str) -> np.ndarray:
    # the GPU values come back as float64 copies of element-type values: converting back is exact
    return _to_elem_bits(x64, dtype)


@pytest.mark.parametrize("dtype,S,D,Hq,Hkv", [
    ("bf16", 300, 128, 4, 2), ("bf16", 257, 64, 4, 4), ("bf16", 1100, 128, 8, 2), ("f32", 200, 64, 2, 1),
])
def test_window_two_zero_queries_round_exactly(dtype, S, D, Hq, Hkv):
    say(f"exact rounding {dtype} S={S} D={D} Hq={Hq} Hkv={Hkv}")
    q = np.zeros((1, Hq, S, D), np.float32)
    rng = np.random.default_rng(7)
    k = rng.standard_normal((1, Hkv, S, D)).astype(np.float32)
    k = _grid_values(k.shape, 8) if dtype == "bf16" else k
    v = _grid_values((1, Hkv, S, D), 9)
    do = _grid_values((1, Hq, S, D), 10)
    scale = 1.0 / math.sqrt(D)
    got = run_hip(q, k, v, do, dtype, True, 2, scale)
    ref = oracle.forward_backward(q, k, v, do, True, 2, scale)

    # the closed form holds in the oracle too (checks the case itself)
    G = Hq // Hkv
    o_closed = v[0, np.arange(Hq) // G].astype(np.float64)
    o_closed[:, 1:] = 0.5 * (o_closed[:, 1:] + o_closed[:, :-1])
    assert np.array_equal(ref["O"][0], o_closed)

    assert np.array_equal(_gpu_bits(got["O"], dtype), _to_elem_bits(ref["O"], dtype)), "O"
    if dtype == "bf16":
        # P = exp2(-LSE log2 e) is within an ulp of 1/2 and becomes exactly 1/2 as a bf16 operand
        assert np.array_equal(_gpu_bits(got["dV"], dtype), _to_elem_bits(ref["dV"], dtype)), "dV"
    else:
        # the fp32 path keeps P in fp32: within an ulp of 1/2, so dV matches to a few ulps
        assert np.allclose(got["dV"], ref["dV"], rtol=1e-6, atol=0), "dV"
    assert np.all(got["dK"] == 0.0), "dK"
    lse_want = np.full(S, math.log(2.0))
    lse_want[0] = 0.0
    for h in range(Hq):
        assert got["LSE"][0, h, 0] == 0.0
        # ln 2 to within one fp32 ulp (the kernel forms it as log2(l) * ln 2)
        assert np.all(np.abs(got["LSE"][0, h] - lse_want) <= np.spacing(np.float32(math.log(2.0))))
