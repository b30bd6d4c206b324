"""Code-generation guard (CPU, needs hipcc): in the forward kernels every group of four
v_dot2c_f32_bf16 that sums one P fragment must read four different packed registers. An earlier
formulation (elements extracted from an assembled u32x4) was compiled into four reads of the same
register, which silently corrupts the softmax denominator."""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "causal_attention_fa2_amd", "csrc")


@pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                    reason="hipcc not available")
def test_forward_dot2_reads_distinct_words(tmp_path):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    out = tmp_path / "fwd.s"
    subprocess.run([hipcc, "--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang", "-target-feature",
                    "-Xclang", "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
                    "--cuda-device-only", "-S", os.path.join(CSRC, "attn_fwd.hip"), "-o", str(out)],
                   check=True, capture_output=True)
    asm = out.read_text()
    kernels = re.split(r"\n(?=_ZN2fa10fwd_kernel\w*:)", asm)
    checked = 0
    for k in kernels:
        if not k.startswith("_ZN2fa10fwd_kernelINS_4BF16"):
            continue
        srcs = re.findall(r"v_dot2c_f32_bf16_e32\s+v\d+,\s*\S+,\s*(v\d+)", k)
        assert srcs and len(srcs) % 4 == 0
        for i in range(0, len(srcs), 4):
            assert len(set(srcs[i:i + 4])) == 4, (k[:60], srcs[i:i + 4])
        checked += 1
    # bf16 D=64 and D=128: dense (8 waves), sliding window (4 waves), paged K/V, packed documents
    assert checked == 8
