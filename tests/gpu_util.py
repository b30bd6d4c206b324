"""Helpers shared by the GPU tests: upload seeded inputs, run the HIP path through the C ABI
binding, and apply the parity gates."""
from __future__ import annotations

import sys

import numpy as np

# rel-L2 gates: fp32 path 1e-5 for every tensor; bf16 path 1e-2 for O and LSE, 2e-2 for dQ/dK/dV.
GATES = {
    "f32": {"O": 1e-5, "LSE": 1e-5, "dQ": 1e-5, "dK": 1e-5, "dV": 1e-5},
    "bf16": {"O": 1e-2, "LSE": 1e-2, "dQ": 2e-2, "dK": 2e-2, "dV": 2e-2},
}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def tdtype(dtype: str):
    import torch
    return {"f32": torch.float32, "bf16": torch.bfloat16}[dtype]


def upload(x: np.ndarray, dtype: str):
    """x holds element-type-representable float32 values; the conversion is exact."""
    import torch
    return torch.from_numpy(np.ascontiguousarray(x)).to(tdtype(dtype)).cuda()


def download(t) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def run_hip(q, k, v, do, dtype, causal=True, window=0, scale=None, want_bwd=True, sink=0):
    """Run attn_fwd (+ attn_bwd) -- their _qk forms for S_q < S_k or sink keys -- on the GPU;
    returns numpy float64 arrays."""
    import torch
    import causal_attention_fa2_amd as fa
    tq, tk, tv = upload(q, dtype), upload(k, dtype), upload(v, dtype)
    o, lse = fa.forward(tq, tk, tv, causal, window, scale, sink=sink)
    out = {}
    if want_bwd:
        tdo = upload(do, dtype)
        dq, dk, dv = fa.backward(tq, tk, tv, o, lse, tdo, causal, window, scale, sink=sink)
        torch.cuda.synchronize()
        out.update(dQ=download(dq), dK=download(dk), dV=download(dv))
        del tdo, dq, dk, dv
    torch.cuda.synchronize()
    out.update(O=download(o), LSE=lse.double().cpu().numpy())
    del tq, tk, tv, o, lse
    return out


def assert_parity(got: dict, ref: dict, dtype: str, names=("O", "LSE", "dQ", "dK", "dV"), tag=""):
    from oracle import rel_l2
    errs = {}
    for n in names:
        if n not in got:
            continue
        g, r = np.asarray(got[n]), np.asarray(ref[n])
        assert g.shape == r.shape, (n, g.shape, r.shape)
        assert np.all(np.isfinite(g)), f"{tag} {n}: non-finite values"
        errs[n] = rel_l2(g, r)
    say(f"  parity {tag}: " + " ".join(f"{n}={e:.2e}" for n, e in errs.items()))
    for n, e in errs.items():
        assert e <= GATES[dtype][n], f"{tag} {n}: rel-L2 {e:.3e} > {GATES[dtype][n]}"
    return errs
