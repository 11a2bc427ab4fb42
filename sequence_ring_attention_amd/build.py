"""Compile the HIP sources into the in-tree shared library ``libusp.so``.

hipcc cross-compiles for gfx950 without a GPU present.  Every source is
compiled on each call (no staleness check), in parallel, then linked.
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libusp.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["api.cpp", "noalloc.hip", "copy_kernels.hip", "merge_kernel.hip", "attn_fp32.hip", "attn_bf16.hip", "bwd_prep.hip",
           "attn_bwd_fp32.hip", "attn_bwd_bf16.hip"]

# Packed fp32 VALU ops are switched off: the kernels use scalar and vector
# float code only, and this keeps the compiler from fusing pairs of it.
COMMON = ["--offload-arch=gfx950", "-O3", "-fPIC", "-std=c++17", "-Wall",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-I", os.path.join(os.path.dirname(PKG), "include")]


def _compile(src):
    obj = os.path.join(BUILD, src + ".o")
    cmd = [HIPCC, *COMMON, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = [l for l in (r.stdout + r.stderr).splitlines()
            if "packed-fp32-ops" not in l]           # the host pass does not know the feature
    return src, r.returncode, "\n".join(msgs), obj


def build(verbose=False):
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 1)) as ex:
        results = list(ex.map(_compile, SOURCES))
    failed = [(s, m) for s, rc, m, _ in results if rc != 0]
    for s, rc, m, _ in results:
        if m.strip() and (verbose or rc != 0):
            print(f"--- {s}\n{m}", file=sys.stderr)
    if failed:
        raise RuntimeError("HIP compilation failed: " + ", ".join(s for s, _ in failed))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *[o for *_, o in results]]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
