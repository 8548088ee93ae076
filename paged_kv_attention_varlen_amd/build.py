"""Build libcb.so (host scheduler/planner + gfx950 kernels) in-tree with hipcc.

    python -m paged_kv_attention_varlen_amd.build      # or: python paged_kv_attention_varlen_amd/build.py

Always recompiles. The library lands next to this file, where the Python binding loads it from.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libcb.so")
ARCH = "gfx950"

# packed-fp32 VALU instructions are disabled for all device code. MFMA results are kept in ordinary VGPRs: the
# attention kernels read every score tile back with VALU instructions, and accumulation registers would cost a copy
# per element.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-mllvm", "-amdgpu-mfma-vgpr-form"]


def _hipcc():
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build the cb library)")


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l and "--hip-link" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"build step failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = False) -> str:
    hipcc = _hipcc()
    bdir = os.path.join(HERE, "_build")
    os.makedirs(bdir, exist_ok=True)
    common = ["-O3", "-std=c++17", "-fPIC", f"-I{INCLUDE}", "-Wall", "-Wno-unused-function"]
    dev_o = os.path.join(bdir, "cb_device.o")
    host_o = os.path.join(bdir, "cb_host.o")
    logs = []
    logs.append(_run([hipcc, f"--offload-arch={ARCH}", *DEVICE_FLAGS, *common, "-c",
                      os.path.join(CSRC, "cb_device.hip"), "-o", dev_o]))
    logs.append(_run([hipcc, "-x", "c++", *common, "-c", os.path.join(CSRC, "cb_host.cpp"), "-o", host_o]))
    prefix_o = os.path.join(bdir, "cb_prefix.o")
    logs.append(_run([hipcc, "-x", "c++", *common, "-c", os.path.join(CSRC, "cb_prefix.cpp"), "-o", prefix_o]))
    tmp = LIB + ".tmp"
    logs.append(_run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", dev_o, host_o, prefix_o, "-o", tmp]))
    os.replace(tmp, LIB)
    if verbose:
        print("\n".join(x for x in logs if x.strip()))
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
