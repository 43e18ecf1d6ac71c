"""Builds libpkv.so, the HIP library behind include/pkv.h, for gfx950.

Run as ``python -m paged_kv_cache_189_amd.build``.  The library lands next to
this file and is what the Python binding loads.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libpkv.so")
ARCH = "gfx950"

HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # keep the compiler from emitting packed fp32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA accumulators in ordinary VGPRs: the online-softmax rescale works on
    # them with VALU ops, which cannot address AGPRs
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
]
CXX_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall"]


def _hipcc() -> str:
    for c in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def build(verbose: bool = False, extra_flags=(), out: str = LIB) -> str:
    """Compile libpkv.so.  extra_flags go to every hipcc compile (for example
    -DPKV_DEPTH_FP8=4 to change a tuning constant); out is the library path."""
    hipcc = _hipcc()
    with tempfile.TemporaryDirectory(prefix="pkv_build_") as tmp:
        objs = []

        def run(cmd):
            if verbose:
                print(" ".join(cmd), flush=True)
            subprocess.run(cmd, check=True)

        for name in ("kernels", "decode_merge", "cache_write", "prefill", "read_probe"):
            obj = os.path.join(tmp, name + ".o")
            run([hipcc, *HIP_FLAGS, *extra_flags, "-c", os.path.join(CSRC, name + ".hip"), "-o", obj])
            objs.append(obj)
        cobj = os.path.join(tmp, "capi.o")
        run([hipcc, "-x", "hip", *HIP_FLAGS, *extra_flags, "-c", os.path.join(CSRC, "capi.cpp"), "-o", cobj])
        objs.append(cobj)
        for name in ("block_manager", "sim"):
            obj = os.path.join(tmp, name + ".o")
            run(["g++", *CXX_FLAGS, "-c", os.path.join(CSRC, name + ".cpp"), "-o", obj])
            objs.append(obj)
        out_tmp = out + ".tmp"
        run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", out_tmp])
        os.replace(out_tmp, out)
    return out


if __name__ == "__main__":
    import argparse

    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("-v", "--verbose", action="store_true")
    ap.add_argument("--define", action="append", default=[], metavar="NAME=VALUE",
                    help="a preprocessor definition for every HIP compile (for example "
                         "PKV_DECODE_VALU_SCORES=1, the vector-unit q.K variant of decode)")
    ap.add_argument("--out", default=LIB, help="library path (default: next to this file)")
    args = ap.parse_args()
    print(build(verbose=args.verbose, extra_flags=[f"-D{d}" for d in args.define], out=args.out))
