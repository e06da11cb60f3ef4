"""Builds libmoe_mi355x.so: the HIP kernels plus the C ABI, compiled by hipcc for gfx950.

Usage: python -m mixture_experts_layer_deterministic_amd.build
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libmoe_mi355x.so")
SOURCES = ["api.cpp", "router.hip", "permute.hip", "gemm.hip", "wgrad.hip", "mx.hip",
           "elementwise.hip", "fused.hip"]
ARCH = "gfx950"

# Packed fp32 ops are disabled for the device code; the host pass warns that it does not know
# the feature, which is harmless.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall",
          "-Wno-unused-function", f"-I{os.path.join(ROOT, 'include')}"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _compile(src: str, obj: str) -> dict:
    """Compiles one source. Returns {kernel: scratch bytes per lane} from the compiler's
    resource-usage remarks."""
    lang = ["-x", "hip"] if src.endswith(".cpp") else []
    cmd = [hipcc(), *COMMON, *DEVICE_FLAGS, *lang, "-Rpass-analysis=kernel-resource-usage",
           "-fno-caret-diagnostics",
           "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    scratch, name, other = {}, None, []
    for line in r.stderr.splitlines():
        if "kernel-resource-usage" in line:
            if "Function Name:" in line:
                name = line.split("Function Name:")[1].split("[")[0].strip()
            elif "ScratchSize [bytes/lane]:" in line and name:
                scratch[name] = int(line.split("ScratchSize [bytes/lane]:")[1].split("[")[0])
        elif noise not in line and not line.startswith("In file included from"):
            other.append(line)
    err = "\n".join(other)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{err}")
    if err.strip():
        print(err)
    return scratch


def build(verbose: bool = True) -> str:
    """Compiles every source and links the shared library in-tree. Returns its path."""
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    objs = [os.path.join(objdir, os.path.splitext(s)[0] + ".o") for s in SOURCES]
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        usage = list(ex.map(lambda so: _compile(*so), zip(SOURCES, objs)))
    # Every kernel keeps its state in registers and LDS: a private (scratch) array or a spill
    # puts memory waits into its inner loop, so the build refuses one.
    scratch = {k: v for u in usage for k, v in u.items() if v}
    if scratch:
        raise RuntimeError(f"kernels using scratch memory (bytes per lane): {scratch}")
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build()
