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
import re
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

# The gemv kernels read their MFMA accumulators with VALU ops; selecting the
# VGPR form of the MFMA instructions keeps the accumulators in VGPRs instead of
# AGPRs (no accvgpr read/write around them). The tiled kernel never touches its
# accumulators inside the loop and keeps them in AGPRs, which leaves the VGPRs
# to the operands.
EXTRA = {"matmul_gemv.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=true"]}


# Every kernel's resource-usage remark is read back: a kernel that uses scratch
# memory (register spills, or a register array moved to the stack) fails the
# build, since on these kernels that means a several-fold slowdown.
RESOURCE_REMARKS = ["-Rpass-analysis=kernel-resource-usage"]


def _scratch_users(stderr: str) -> list[str]:
    out = []
    for block in re.split(r"remark: [^\n]*?Function Name: ", stderr)[1:]:
        name = block.split()[0]
        m = re.search(r"ScratchSize \[bytes/lane\]: (\d+)", block)
        if m and int(m.group(1)) > 0:
            out.append(f"{name} ({m.group(1)} B/lane)")
    return out


def _compile(src: str) -> str:
    path = src if os.path.isabs(src) else os.path.join(CSRC, src)
    obj = os.path.join(BUILD, os.path.splitext(os.path.basename(src))[0] + ".o")
    lang = ["-x", "hip"]
    cmd = [HIPCC, *HIPFLAGS, *EXTRA.get(src, []), *RESOURCE_REMARKS, *lang, "-c", path, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
    spills = _scratch_users(r.stderr)
    if spills:
        raise RuntimeError(f"kernels in {src} use scratch memory: " + "; ".join(spills))
    # the host pass warns that it does not know the packed-fp32 feature: harmless;
    # the resource remarks were read above
    noise = [ln for ln in r.stderr.splitlines()
             if "packed-fp32-ops" not in ln and "kernel-resource-usage" not in ln and ln.strip()
             and not ln.lstrip().startswith(("|", "^"))
             and not re.match(r"\s*\d+ \|", ln)]
    if noise:
        sys.stderr.write("\n".join(noise) + "\n")
    return obj


# The measurement probes (a plain streaming read and an MFMA-only loop, the
# ceilings the benchmark compares bandwidth- and matrix-core-bound kernels
# with) are their own small library: not part of the path, never loaded by
# the binding.
PROBE_SRCS = [os.path.join(PKG, "probe", "stream_read.hip"), os.path.join(PKG, "probe", "mfma_peak.hip")]
PROBE_LIB = os.path.join(PKG, "probe", "libint4dq_probe.so")


def _link(objs, out):
    tmp = out + ".tmp%d" % os.getpid()
    r = subprocess.run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, out)


def build(verbose: bool = True) -> str:
    """Compile every HIP source for gfx950 and link the shared library (and the
    measurement probe). Always rebuilds."""
    os.makedirs(BUILD, exist_ok=True)
    jobs = min(len(SOURCES) + 1, int(os.environ.get("MAX_JOBS", os.cpu_count() or 4)), 16)
    with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as ex:
        probes = [ex.submit(_compile, src) for src in PROBE_SRCS]
        objs = list(ex.map(_compile, SOURCES))
        probe_objs = [f.result() for f in probes]
    _link(objs, LIB)
    _link(probe_objs, PROBE_LIB)
    if verbose:
        print(f"built {LIB} and {PROBE_LIB}")
    return LIB


if __name__ == "__main__":
    build()
