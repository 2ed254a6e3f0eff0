"""Build libx3conv.so (HIP, gfx950) in-tree.

Each translation unit under csrc/ (the C ABI, and one per epilogue, which
instantiates that epilogue's kernels) is compiled to an object in parallel,
then the objects are linked into the shared library.

hipcc cross-compiles for gfx950 without a GPU.  Packed-fp32 instructions are
disabled for the device code (hipcc's host pass warns that it does not know
the feature; that warning is harmless).  No fast-math.
"""
import os
import re
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
SOURCES = ["x3conv.hip", "epi_min_tanh2.hip", "epi_mul_lrelu_gelu.hip",
           "epi_mul_lrelu_gelu_tanh.hip", "epi_scale_min.hip", "epi_gn_pool.hip",
           "epi_split.hip", "epi_nhwc.hip", "epi_gn_poolk.hip", "epi_gn_poolk_nhwc.hip",
           "probe.hip"]
LIB = os.path.join(PKG, "libx3conv.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    "-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC",
    "-fvisibility=hidden",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]
NOISE = "'-packed-fp32-ops' is not a recognized feature"


def _parse(stderr):
    """Split hipcc's stderr into per-kernel resource remarks and the rest."""
    usage, other, name = {}, [], None
    for line in stderr.splitlines():
        if NOISE in line:
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
    return usage, other


def _compile(hipcc, src, obj, verbose):
    cmd = [hipcc, *HIPCC_FLAGS, "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    cmd += ["-Rpass-analysis=kernel-resource-usage", "-fno-caret-diagnostics"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    usage, other = _parse(res.stderr)
    return src, res.returncode, usage, other


def build(verbose: bool = False) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    jobs = max(1, min(len(SOURCES), int(os.environ.get("MAX_JOBS", "8"))))
    usage, failed = {}, []
    with tempfile.TemporaryDirectory(prefix="x3build_") as tmp:
        objs = [os.path.join(tmp, os.path.splitext(s)[0] + ".o") for s in SOURCES]
        with ThreadPoolExecutor(jobs) as ex:
            results = list(ex.map(lambda so: _compile(hipcc, so[0], so[1], verbose),
                                  zip(SOURCES, objs)))
        for src, rc, u, other in results:
            if any(("warning" in l or "error" in l) for l in other):
                print(f"--- {src}", file=sys.stderr)
                print("\n".join(other), file=sys.stderr)
            if rc != 0:
                failed.append(src)
            usage.update(u)
        if failed:
            raise RuntimeError("hipcc failed on " + ", ".join(failed))
        link = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs,
                "-o", LIB + ".tmp"]
        if verbose:
            print(" ".join(link), flush=True)
        res = subprocess.run(link, capture_output=True, text=True)
        if res.returncode != 0:
            print(res.stderr, file=sys.stderr)
            raise RuntimeError(f"link failed ({res.returncode})")

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
