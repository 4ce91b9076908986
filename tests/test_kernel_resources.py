"""Register use of the tiled grouped-GEMM kernels, from the compiler's resource
report (hipcc for gfx950 on the host, no GPU).

The tiled kernels read their MFMA fragments from LDS with inline-asm loads
whose completion they await explicitly; the compiler takes such an output
register as written when the load is issued.  A spill (or copy) of one of
those registers before its wait would store a stale value, so none of these
kernels may spill."""
import os
import re
import shutil
import subprocess

import pytest

from sparse_mixture_experts_03_amd import build as hip_build

SRC = os.path.join(hip_build.CSRC, "gemm_tiled.hip")


def resource_report(src, tmp_path):
    if not os.path.exists(hip_build.HIPCC) and shutil.which("hipcc") is None:
        pytest.skip("hipcc not available")
    out = os.path.join(str(tmp_path), "k.o")
    r = subprocess.run([hip_build.HIPCC, *hip_build.FLAGS, "-c", src, "-o", out,
                        "-Rpass-analysis=kernel-resource-usage"], capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-2000:]
    kernels = {}
    name = None
    for line in r.stderr.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            name = m.group(1)
            kernels[name] = {}
            continue
        m = re.search(r"remark:\s+([A-Za-z ]+?)(?: \[[^\]]*\])?: (\d+)", line)
        if m and name:
            kernels[name][m.group(1).strip()] = int(m.group(2))
    return kernels


def test_tiled_kernels_do_not_spill(tmp_path):
    kernels = resource_report(SRC, tmp_path)
    tiled = {k: v for k, v in kernels.items() if "gemm_tiled" in k and "kernel" in k}
    assert len(tiled) >= 8, sorted(kernels)  # bf16 and INT4, GEMM1 (three activations) and GEMM2
    for name, res in tiled.items():
        assert res.get("VGPRs Spill", 0) == 0, (name, res)
        assert res.get("SGPRs Spill", 0) == 0, (name, res)
