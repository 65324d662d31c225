"""Build libint4dq.so (HIP kernels + C ABI) for gfx950 with hipcc, in-tree.

Usage: ``python dequantizing_gemm_amd/build.py`` (or ``__graft_entry__.build()``). It
is run by path, not as ``-m``: importing the package loads the library, which
may be missing or older than the sources being built.
Object files go to ``_build/`` at the repository root; the shared library is
written next to this file, where the binding loads it.
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libint4dq.so")

HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
ARCH = "gfx950"

# -fhip-fp32-correctly-rounded-divide-sqrt: `a / b` on floats is the IEEE
#   division (the quantizer's scale and codes must match a CPU reference bit
#   for bit); no fast-math anywhere.
# -fno-gpu-flush-denormals-to-zero: keep fp32 subnormals.
# -packed-fp32-ops off: no packed fp32 instructions are generated.
HIPFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-fhip-fp32-correctly-rounded-divide-sqrt", "-fno-gpu-flush-denormals-to-zero",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]

SOURCES = ["api.cpp", "quantize.hip", "unpack.hip", "dequantize.hip", "matmul_generic.hip",
           "matmul_skinny.hip", "matmul_tiled.hip", "matmul_gemv.hip"]

# The tiled and gemv kernels read or rescale their MFMA accumulators with VALU
# ops; selecting the VGPR form of the MFMA instructions keeps the accumulators
# in VGPRs instead of AGPRs (no accvgpr read/write around them).
EXTRA = {"matmul_tiled.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=true"],
         "matmul_gemv.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=true"]}


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    lang = ["-x", "hip"]
    cmd = [HIPCC, *HIPFLAGS, *EXTRA.get(src, []), *lang, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
    # the host pass warns that it does not know the packed-fp32 feature: harmless
    noise = [ln for ln in r.stderr.splitlines() if "packed-fp32-ops" not in ln and ln.strip()]
    if noise:
        sys.stderr.write("\n".join(noise) + "\n")
    return obj


def build(verbose: bool = True) -> str:
    """Compile every HIP source for gfx950 and link the shared library. Always rebuilds."""
    os.makedirs(BUILD, exist_ok=True)
    jobs = min(len(SOURCES), int(os.environ.get("MAX_JOBS", os.cpu_count() or 4)), 16)
    with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp%d" % os.getpid()
    r = subprocess.run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build()
