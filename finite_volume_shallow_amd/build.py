"""Build libswe.so (HIP for gfx950) in-tree with hipcc.

Every source is compiled to an object in parallel, then linked into
finite_volume_shallow_amd/libswe.so.  Packed fp32 instructions are disabled
for all device code.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libswe.so")
ARCH = os.environ.get("SWE_OFFLOAD_ARCH", "gfx950")

# (source, preprocessor symbol): kern_cart.hip is compiled twice, the second
# time for the streaming-mode kernels of the structured path only
SOURCES = [("swe_api.hip", None), ("mesh_host.cpp", None), ("kern_edge.hip", None), ("kern_cart.hip", None),
           ("kern_cart.hip", "SWE_CART_STREAM_TU"), ("kern_tri.hip", None)]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-result",
          "-I" + os.path.join(HERE, "..", "include")]
DEVICE = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang",
          "-packed-fp32-ops"]


def _compile(spec, verbose: bool) -> str:
    src, define = spec
    obj = os.path.join(BUILD, os.path.basename(src) + (f".{define}" if define else "") + ".o")
    path = os.path.join(CSRC, src)
    extra = [f"-D{define}"] if define else []
    if src.endswith(".hip"):
        cmd = [HIPCC, "-x", "hip", *DEVICE, *COMMON, *extra, "-c", path, "-o", obj]
    else:
        cmd = [HIPCC, *COMMON, *extra, "-c", path, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {src}\n{r.stdout}\n{r.stderr}")
    noisy = [ln for ln in r.stderr.splitlines() if "packed-fp32-ops" not in ln and ln.strip()]
    if verbose and noisy:
        print("\n".join(noisy), flush=True)
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + ".tmp"
    # -z defs: a symbol that no object defines fails the link, not the load
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-Wl,-z,defs", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
