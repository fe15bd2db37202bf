"""Build libmxfa.so (HIP, gfx950) in-tree: ``python -m tiled_attention_amd.build``.

Each ``csrc/*.hip`` is compiled with hipcc for gfx950 (in parallel), then the
objects are linked into ``tiled_attention_amd/libmxfa.so``. Packed fp32 VALU
forms are disabled for the device code (``-packed-fp32-ops``); the host pass
warns that it does not know the feature, which is harmless.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libmxfa.so")
BUILD_DIR = os.path.join(ROOT, "_build")
ARCH = "gfx950"


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libmxfa.so)")


def compile_flags() -> list:
    return [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", INCLUDE, "-I", CSRC]


# Extra flags per source. The decode and bf16 forward kernels keep 128 fp32
# accumulators per lane live next to a Q^T operand held in AGPRs; left to its
# heuristics the compiler moves the accumulators between VGPRs and AGPRs
# around every tile, so their MFMAs are pinned to the VGPR form.
FILE_FLAGS = {
    "decode_mla.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
    "fwd_bf16.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}


def build(verbose: bool = False, jobs: int = 0) -> str:
    """Compile every HIP source and link libmxfa.so; returns the library path."""
    hipcc = _hipcc()
    os.makedirs(BUILD_DIR, exist_ok=True)
    sources = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    if not sources:
        raise RuntimeError("no HIP sources found")
    objs = [os.path.join(BUILD_DIR, os.path.basename(s)[:-4] + ".o") for s in sources]

    def compile_one(src_obj):
        src, obj = src_obj
        cmd = [hipcc, *compile_flags(), *FILE_FLAGS.get(os.path.basename(src), []), "-c", src, "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        out = r.stdout + r.stderr
        # the host pass does not know the device-only feature flag
        out = "\n".join(l for l in out.splitlines() if "packed-fp32-ops" not in l)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed for {os.path.basename(src)}:\n{out}")
        if verbose and out.strip():
            print(out, file=sys.stderr)
        return obj

    workers = jobs or min(len(sources), os.cpu_count() or 4, 8)
    with cf.ThreadPoolExecutor(max_workers=workers) as ex:
        list(ex.map(compile_one, zip(sources, objs)))
    tmp = LIB + ".tmp%d" % os.getpid()
    r = subprocess.run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link of libmxfa.so failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
