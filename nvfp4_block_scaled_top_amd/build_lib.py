"""Build step for libmegamoe.so (gfx950) from csrc/: one hipcc invocation, in-tree output.

Run ``python -m nvfp4_block_scaled_top_amd.build_lib`` or call ``build()``.
"""
from __future__ import annotations

import os
import re
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
LIB_NAME = "libmegamoe.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)
ARCH = "gfx950"

SOURCES = ["router.hip", "route.hip", "quant.hip", "gemm.hip", "dense.hip", "combine.hip", "api.cpp"]

# Device code: gfx950 only, no fast-math (the quantizer relies on IEEE division, fma and rint),
# and packed fp32 instructions disabled.
HIP_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libmegamoe.so)")


# The compiler's per-kernel resource remarks (registers, LDS, scratch) are requested so that the
# build can refuse kernels that spill to scratch memory (a spill in a hot loop turns a kernel many
# times slower without changing its results, so no numerics test would notice).
RESOURCE_FLAG = "-Rpass-analysis=kernel-resource-usage"


def kernel_scratch(remarks: str) -> dict:
    """{kernel symbol: scratch bytes per lane} from the compiler's resource-usage remarks."""
    out, name = {}, None
    for line in remarks.splitlines():
        m = re.search(r"remark: Function Name: (\S+)", line)
        if m:
            name = m.group(1)
            continue
        m = re.search(r"remark:\s+ScratchSize \[bytes/lane\]: (\d+)", line)
        if m and name is not None:
            out[name] = int(m.group(1))
    return out


def build(verbose: bool = False) -> str:
    """Compile every source into LIB_PATH (always recompiles) and return the path.  Raises if the
    compile fails or if any kernel spills to scratch memory."""
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc(), *HIP_FLAGS, RESOURCE_FLAG, "-I", os.path.join(ROOT, "include"),
           *[os.path.join(CSRC, s) for s in SOURCES], "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature; that warning is expected.
    lines = [l for l in res.stderr.splitlines() if "packed-fp32-ops" not in l]
    errs = "\n".join(l for l in lines if "kernel-resource-usage" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{errs}")
    scratch = kernel_scratch("\n".join(lines))
    if not scratch:
        raise RuntimeError("hipcc printed no kernel resource usage; cannot check for spills")
    spills = {k: v for k, v in scratch.items() if v > 0}
    if spills:
        raise RuntimeError(f"kernels spill to scratch memory (bytes per lane): {spills}")
    if verbose and errs.strip():
        print(errs, file=sys.stderr)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


PROBE_SOURCE = "probe.hip"
PROBE_LIB_PATH = os.path.join(PKG_DIR, "libmegamoe_probe.so")


def build_probe(verbose: bool = False) -> str:
    """Compile the measurement kernels bench.py uses (csrc/probe.hip, not part of the layer) into
    PROBE_LIB_PATH and return the path."""
    tmp = PROBE_LIB_PATH + ".tmp"
    cmd = [hipcc(), *HIP_FLAGS, os.path.join(CSRC, PROBE_SOURCE), "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    errs = "\n".join(l for l in res.stderr.splitlines() if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{errs}")
    os.replace(tmp, PROBE_LIB_PATH)
    return PROBE_LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
    print(build_probe(verbose=True))
