"""Build libattn.so (the C-ABI attention library) in-tree with hipcc for gfx950.

    python -m causal_attention_fa2_amd.build
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libattn.so")
# (source, extra flags). attn_dkdv.hip keeps MFMA results in VGPRs: its S / dP products feed VALU
# work directly, and without the flag the compiler parks them in AGPRs and copies them back.
SOURCES = [
    ("attn_api.cpp", []),
    ("attn_fwd.hip", []),
    ("attn_bwd.hip", []),
    ("attn_dkdv.hip", ["-mllvm", "-amdgpu-mfma-vgpr-form"]),
    ("attn_decode.hip", []),
    ("attn_noalloc.hip", []),
]

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # keep hipcc from forming packed fp32 instructions on its own
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    path = os.path.join(rocm, "bin", "hipcc")
    return path if os.path.exists(path) else "hipcc"


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"hipcc failed with status {r.returncode}")


def build(verbose: bool = False) -> str:
    """Compile every HIP source (each with its own flags) and link libattn.so next to this file;
    returns its path."""
    from concurrent.futures import ThreadPoolExecutor
    out_dir = os.path.join(ROOT, "_build")
    os.makedirs(out_dir, exist_ok=True)
    jobs = []
    for src, extra in SOURCES:
        obj = os.path.join(out_dir, os.path.splitext(src)[0] + ".o")
        jobs.append((obj, [hipcc(), *HIPCC_FLAGS, *extra, "-I", INCLUDE, "-I", CSRC, "-c",
                           os.path.join(CSRC, src), "-o", obj]))
    # the sources compile independently: one hipcc per source, in parallel
    workers = max(1, min(len(jobs), os.cpu_count() or 1))
    with ThreadPoolExecutor(max_workers=workers) as pool:
        for f in [pool.submit(_run, cmd, verbose) for _, cmd in jobs]:
            f.result()
    objs = [obj for obj, _ in jobs]
    tmp = LIB + ".tmp"
    _run([hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
