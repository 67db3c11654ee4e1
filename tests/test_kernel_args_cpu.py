"""The compiled kernels keep their arguments preloaded into SGPRs: one
translation unit of the row kernels and one of the backward, compiled for
gfx950 with the library's own flags to AMD assembly (device code only, no GPU
needed), and the preload length read from each kernel descriptor.  A kernel
that took its arguments as one struct again would show a length of 0."""
import os
import re
import shutil
import subprocess

import pytest

from rmsnorm_row_normalisation_amd import build

HIPCC = build.HIPCC


def _descriptors(src: str, out: str) -> dict[str, dict[str, int]]:
    cmd = [HIPCC, *build.COMMON, "--cuda-device-only", "-S", src, "-o", out]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    text = open(out).read()
    kernels = {}
    for m in re.finditer(r"\.amdhsa_kernel (\S+)\n(.*?)\.end_amdhsa_kernel", text, re.S):
        fields = dict((k, int(v)) for k, v in re.findall(r"\.amdhsa_(\w+) (\d+)\n", m.group(2)))
        kernels[m.group(1)] = fields
    return kernels


@pytest.mark.skipif(not (HIPCC and os.path.exists(HIPCC)) and shutil.which("hipcc") is None,
                    reason="needs hipcc")
def test_row_and_backward_kernels_preload_their_arguments(tmp_path):
    rows = _descriptors(os.path.join(build.CSRC, "ks_vec_bf16_rms.hip"), str(tmp_path / "rms.s"))
    assert len(rows) > 100
    for name, f in rows.items():
        # y, x, res, w, rows, hidden, eps: 48 bytes in 12 SGPRs
        assert f["user_sgpr_kernarg_preload_length"] == 12, name
        assert f["private_segment_fixed_size"] == 0, name

    bwd = _descriptors(os.path.join(build.CSRC, "ks_bwd_bf16.hip"), str(tmp_path / "bwd.s"))
    row_kernels = [n for n in bwd if "rms_norm_backward_vec" in n]
    dw_kernels = [n for n in bwd if "rms_norm_backward_dw" in n]
    assert row_kernels and dw_kernels
    for name in row_kernels:
        # dx, dy, x, w, rows, hidden, eps and the partial-row pointer (14 SGPRs)
        assert bwd[name]["user_sgpr_kernarg_preload_length"] == 14, name
    for name in dw_kernels:
        assert bwd[name]["user_sgpr_kernarg_preload_length"] == 6, name
