"""Code-generation guard (CPU, needs hipcc): the forward and decode kernels form their softmax row
sums with plain fp32 adds, never v_dot2c_f32_bf16. On gfx950 that instruction runs about 2.5x
slower while another wave of the SIMD issues matrix products (and an earlier formulation of it was
miscompiled into four reads of one packed register), so it must not come back."""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "causal_attention_fa2_amd", "csrc")


def _asm(src, tmp_path):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    out = tmp_path / (os.path.basename(src) + ".s")
    subprocess.run([hipcc, "--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang", "-target-feature",
                    "-Xclang", "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
                    "--cuda-device-only", "-S", os.path.join(CSRC, src), "-o", str(out)],
                   check=True, capture_output=True)
    return out.read_text()


@pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                    reason="hipcc not available")
# bf16 and f32 forward kernels (dense 4 and 8 waves, the 8-wave one with one or two softmax updates per
# barrier, paged, packed documents), dense and paged decode
@pytest.mark.parametrize("src,pattern,count", [("attn_fwd.hip", "fwd_kernel", 16),
                                               ("attn_decode.hip", "decode_kernel", 4)])
def test_row_sums_use_no_dot2(src, pattern, count, tmp_path):
    asm = _asm(src, tmp_path)
    kernels = [k for k in re.split(r"\n(?=_ZN2fa\w*:)", asm) if re.match(rf"_ZN2fa\d+{pattern}", k)]
    assert len(kernels) == count, [k[:80] for k in kernels]
    for k in kernels:
        assert "v_dot2c_f32_bf16" not in k, k[:80]
        assert "v_exp_f32" in k, k[:80]
