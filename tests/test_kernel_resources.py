"""Register and scratch use of the grouped-GEMM kernels, from the compiler's
resource report (hipcc for gfx950 on the host, no GPU), and the compiler the
kernels were validated with.

The tiled kernels read their MFMA fragments (and the INT4 kernel its codes and
scales) from LDS with inline-asm loads whose completion they await
explicitly; the compiler takes such an output register as written when the
load is issued.  A spill or copy of one of those registers before its wait
would store a stale value, so no tiled or streaming instantiation may spill a
register or use scratch memory at all (the streaming kernels are held to the
same rule: their pipelines are tuned on the assumption that nothing lives in
scratch).  The inline-asm reads were validated on the GPU with the compiler
named in build.VALIDATED_COMPILER; another compiler builds (with a warning),
but this test then fails, so that the parity tests are run again before its
binaries are trusted."""
import os
import re
import shutil
import subprocess

import pytest

from sparse_mixture_experts_03_amd import build as hip_build

SOURCES = ["gemm_tiled.hip", "gemm_stream.hip"]


def _hipcc():
    if not os.path.exists(hip_build.HIPCC) and shutil.which("hipcc") is None:
        pytest.skip("hipcc not available")
    return hip_build.HIPCC


def resource_report(src, tmp_path):
    out = os.path.join(str(tmp_path), os.path.basename(src) + ".o")
    r = subprocess.run([_hipcc(), *hip_build.FLAGS, "-c", src, "-o", out,
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


@pytest.mark.parametrize("src", SOURCES)
def test_gemm_kernels_do_not_spill_or_use_scratch(tmp_path, src):
    kernels = resource_report(os.path.join(hip_build.CSRC, src), tmp_path)
    gemm = {k: v for k, v in kernels.items() if "gemm_" in k and "kernel" in k}
    # tiled: GEMM1 with three activations and GEMM2, for INT4 and for bf16 weights; streaming: every
    # (weight type, GEMM, tile shape) instantiation the launcher can choose
    assert len(gemm) >= {"gemm_tiled.hip": 8, "gemm_stream.hip": 8}[src], sorted(kernels)
    for name, res in gemm.items():
        assert "ScratchSize" in res, (name, res)
        assert res.get("VGPRs Spill", 0) == 0, (name, res)
        assert res.get("SGPRs Spill", 0) == 0, (name, res)
        assert res["ScratchSize"] == 0, (name, res)


def test_compiler_is_the_validated_one():
    _hipcc()
    version = hip_build.compiler_version()
    assert hip_build.VALIDATED_COMPILER in version, version
