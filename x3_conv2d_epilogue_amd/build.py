"""Build libx3conv.so (HIP, gfx950) in-tree.

hipcc cross-compiles for gfx950 without a GPU.  Packed-fp32 instructions are
disabled for the device code (hipcc's host pass warns that it does not know
the feature; that warning is harmless).  No fast-math.
"""
import os
import re
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRC = os.path.join(PKG, "csrc", "x3conv.hip")
LIB = os.path.join(PKG, "libx3conv.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    "-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC", "-shared",
    "-fvisibility=hidden",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def build(verbose: bool = False) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    cmd = [hipcc, *HIPCC_FLAGS, "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(PKG, "csrc"), SRC, "-o", LIB + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    cmd += ["-Rpass-analysis=kernel-resource-usage", "-fno-caret-diagnostics"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    # drop the host pass's harmless note about the device-only feature flag
    # and collect the per-kernel resource remarks
    noise = "'-packed-fp32-ops' is not a recognized feature"
    usage, other, name = {}, [], None
    for line in res.stderr.splitlines():
        if noise in line:
            continue
        m = re.search(r"remark: Function Name: (\S+)", line)
        if m:
            name = m.group(1)
            usage[name] = {}
            continue
        m = re.search(r"remark:\s+([A-Za-z][^:]*?)(?: \[[^]]*\])?: (\d+) \[-Rpass", line)
        if m and name:
            usage[name][m.group(1)] = int(m.group(2))
            continue
        if "kernel-resource-usage" not in line:
            other.append(line)
    if any(("warning" in l or "error" in l) for l in other):
        print("\n".join(other), file=sys.stderr)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode})")
    # A kernel that touches scratch memory has spilled registers or demoted
    # its accumulators to memory: that is a performance bug, refuse it.
    bad = [k for k, u in usage.items() if u.get("ScratchSize", 0) > 0]
    if bad:
        raise RuntimeError("kernels using scratch memory: " + ", ".join(bad))
    if verbose:
        for k, u in usage.items():
            print(f"  {k[:90]}: VGPRs={u.get('VGPRs')} AGPRs={u.get('AGPRs')} "
                  f"occupancy={u.get('Occupancy')} LDS={u.get('LDS Size')}")
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
