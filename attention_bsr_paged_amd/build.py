"""Build libabp.so (HIP, gfx950) in-tree.

    python -m attention_bsr_paged_amd.build [--jobs N] [--debug]

Each source under csrc/ is compiled to an object with hipcc, in parallel, and
linked into attention_bsr_paged_amd/lib/libabp.so. Packed fp32 instructions
are disabled for all device code.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIBDIR = os.path.join(PKG, "lib")
LIB = os.path.join(LIBDIR, "libabp.so")
ARCH = "gfx950"

SOURCES = ["api.cpp", "plan.cpp", "merge.hip", "decode.hip", "append.hip", "append_rope.hip",
           "upload.hip", "page_append.hip", "decode_mfma.hip", "pod.hip", "static_ws.hip"]

COMMON = [
    "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
    "-I" + os.path.join(os.path.dirname(PKG), "include"),
]
DEVICE = [
    "--offload-arch=" + ARCH,
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # kernels never produce NaN on purpose: max/min need no NaN quieting
    # (infinities keep their meaning: masked scores are -inf)
    "-fno-honor-nans",
]
# per-source device flags: these kernels keep their matrix-product
# accumulators in VGPRs; in the default form the compiler moves them between
# AGPRs and VGPRs around the vector work (see the headers of append_rope.hip
# and decode_mfma.hip)
VGPR_FORM = ["-mllvm", "-amdgpu-mfma-vgpr-form"]
EXTRA = {"append_rope.hip": VGPR_FORM, "decode_mfma.hip": VGPR_FORM}


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build libabp)")


def compile_one(src: str, opt: list, verbose: bool) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), "-c", os.path.join(CSRC, src), "-o", obj] + COMMON + opt
    if src.endswith(".hip"):
        cmd += DEVICE + EXTRA.get(src, []) + ["-x", "hip"]
    else:
        # host-only translation units: no device code object
        cmd += ["--offload-arch=" + ARCH, "-x", "hip", "--cuda-host-only"]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    errs = "\n".join(line for line in (r.stderr or "").splitlines()
                     if "packed-fp32-ops" not in line)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{errs}")
    if errs.strip() and verbose:
        print(errs, file=sys.stderr)
    return obj


def build(jobs: int = 8, debug: bool = False, verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    os.makedirs(LIBDIR, exist_ok=True)
    opt = ["-O0", "-g"] if debug else ["-O3"]
    with cf.ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = list(ex.map(lambda s: compile_one(s, opt, verbose), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "-shared", "-o", tmp] + objs + ["--offload-arch=" + ARCH, "-fPIC"]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stderr)
    os.replace(tmp, LIB)
    return LIB


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--jobs", type=int, default=min(8, os.cpu_count() or 1))
    ap.add_argument("--debug", action="store_true")
    ap.add_argument("-v", "--verbose", action="store_true")
    a = ap.parse_args(argv)
    print(build(a.jobs, a.debug, a.verbose))
    return 0


if __name__ == "__main__":
    sys.exit(main())
