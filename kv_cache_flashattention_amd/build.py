"""Build libkvfa.so (the HIP kernels and the C ABI) for gfx950, in-tree.

    python -m kv_cache_flashattention_amd.build      # or build() from Python

Every source under csrc/ is compiled by hipcc into _build/, then linked into
kv_cache_flashattention_amd/libkvfa.so.  Packed-FP32 instructions are turned
off for the device code (-target-feature -packed-fp32-ops); fast-math is never
used, so float division stays correctly rounded (the fp8 scale rule relies on
IEEE division).
"""
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libkvfa.so")
ARCH = "gfx950"


COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", INCLUDE, "-I", CSRC,
          "-Wall", "-Wno-unused-function"]
DEVICE = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-fno-fast-math", "-ffp-contract=fast"]


def _hipcc():
    for c in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def _compile(src):
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [_hipcc()] + COMMON + DEVICE + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    noise = "is not a recognized feature for this target"
    warn = "\n".join(l for l in r.stderr.splitlines() if noise not in l).strip()
    return obj, warn


def build(verbose=True):
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(f for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))
    with ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        results = list(ex.map(_compile, srcs))
    for (obj, warn), src in zip(results, srcs):
        if warn and verbose:
            print(f"[{src}]\n{warn}", file=sys.stderr)
    tmp = LIB + ".tmp"
    cmd = [_hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}"] + [o for o, _ in results] + \
          ["-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build()
