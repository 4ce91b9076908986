"""Build the HIP library (libmoe_mi355x.so) in-tree for gfx950 with hipcc.

Every .hip file under csrc/ is compiled to an object in _build/ and the objects
are linked into one shared library next to this file.  Packed fp32 VALU
instructions are disabled (-packed-fp32-ops) for all device code.

The tiled GEMM kernels read LDS through inline asm whose results the compiler
sees as written at issue; their schedules were validated on the GPU with the
compiler named in VALIDATED_COMPILER.  Another hipcc still builds, with a
warning, and the parity tests must then be run again before its binaries are
trusted.
"""
import concurrent.futures
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libmoe_mi355x.so")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
VALIDATED_COMPILER = "AMD clang version 22.0.0git (https://github.com/RadeonOpenCompute/llvm-project roc-7.2.0 26014"
FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-result",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _compile(src):
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                     if "packed-fp32-ops" not in l or "error" in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{msgs}")
    return obj, msgs


def compiler_version():
    r = subprocess.run([HIPCC, "--version"], capture_output=True, text=True)
    return r.stdout


def build(verbose=True, jobs=None):
    """Compile all sources and link the library; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    if VALIDATED_COMPILER not in compiler_version():
        print(f"warning: {HIPCC} is not the compiler the kernels were validated with "
              f"({VALIDATED_COMPILER}); run the GPU parity tests before using this build", file=sys.stderr)
    srcs = sources()
    jobs = jobs or min(len(srcs), max(1, min(8, os.cpu_count() or 1)))
    with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as ex:
        results = list(ex.map(_compile, srcs))
    for _, msgs in results:
        if msgs.strip() and verbose:
            print(msgs, file=sys.stderr)
    objs = [o for o, _ in results]
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}", file=sys.stderr)
    return LIB


if __name__ == "__main__":
    build()
