"""Build libiqattn.so (the C-ABI library with its gfx950 kernels) in-tree.

Each translation unit under csrc/ is compiled by hipcc for gfx950 in
parallel, then linked into one shared library next to this file.
"""
from __future__ import annotations

import glob
import os
import subprocess
import tempfile
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libiqattn.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# Packed FP32 instructions are disabled for all device code (the kernels need
# none; this keeps the compiler from forming them).
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall", "-I", INCLUDE,
          "-I", CSRC]
# The specialised kernels keep their MFMA accumulators in VGPRs (the VALU works
# on them right away; AGPR copies would cost one instruction per logit).
PER_FILE = {"iqattn_fast.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


BUILD_DIR = os.path.join(ROOT, "_build")  # in-tree scratch for objects (not tracked)


def build(verbose: bool = False) -> str:
    srcs = sources()
    os.makedirs(BUILD_DIR, exist_ok=True)
    env = dict(os.environ, TMPDIR=BUILD_DIR)  # the compiler's own temporaries too
    with tempfile.TemporaryDirectory(prefix="iqattn_build_", dir=BUILD_DIR) as tmpd:
        objs = [os.path.join(tmpd, os.path.basename(s) + ".o") for s in srcs]

        def compile_one(args):
            src, obj = args
            extra = PER_FILE.get(os.path.basename(src), [])
            cmd = [HIPCC, *COMMON, *DEVICE_FLAGS, *extra, "-c", src, "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            subprocess.check_call(cmd, env=env)

        with ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
            list(ex.map(compile_one, zip(srcs, objs)))
        tmp = LIB + ".tmp"
        cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.check_call(cmd, env=env)
        os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
