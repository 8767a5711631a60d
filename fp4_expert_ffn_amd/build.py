"""Build the HIP library in-tree: ``fp4_expert_ffn_amd/libmoe_fp4.so`` for gfx950.

Run as ``python -m fp4_expert_ffn_amd.build`` (or through ``__graft_entry__.build()``).
Every call compiles from source; object files go to ``_build/`` next to the package.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_NAME = "libmoe_fp4.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)

SOURCES = ["api.cpp", "kernels_pack.hip", "kernels_route.hip", "kernels_ffn.hip",
           "kernels_batched.hip", "kernels_norm.hip", "kernels_probe.hip", "kernels_small_m.hip",
           "kernels_fp8.hip", "kernels_prefetch.hip"]

# Packed-fp32 VALU ops are switched off for the device code: the compiler otherwise forms
# them from ordinary float code, and this library does not rely on them.
HIP_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]

# Per-source extra flags. The matrix-core probe keeps its accumulators in ordinary VGPRs:
# in the accumulation-register form the compiler rotates independent accumulators through
# register moves every iteration, which chains the operations and understates the peak.
EXTRA_FLAGS = {"kernels_probe.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP library cannot be built")


def _compile(src: str, build_dir: str = BUILD_DIR, defines=(), csrc: str = CSRC) -> str:
    obj = os.path.join(build_dir, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *HIP_FLAGS, *EXTRA_FLAGS.get(src, []), "-I", csrc, *[f"-D{d}" for d in defines], "-c",
           os.path.join(csrc, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in res.stdout.splitlines() if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{out}")
    if out.strip():
        sys.stderr.write(out + "\n")
    return obj


def build(verbose: bool = True, lib_path: str = LIB_PATH, build_dir: str = BUILD_DIR,
          defines=(), csrc: str = CSRC) -> str:
    """Compile every source and link the shared library. `defines` (NAME=VALUE strings)
    override the compile-time launch-shape constants; `csrc` builds another source tree
    of the same file names."""
    os.makedirs(build_dir, exist_ok=True)
    jobs = min(len(SOURCES), max(1, (os.cpu_count() or 2)))
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda src: _compile(src, build_dir, defines, csrc), SOURCES))
    tmp = lib_path + ".tmp"
    cmd = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}")
    os.replace(tmp, lib_path)
    if verbose:
        print(f"built {lib_path}")
    return lib_path


if __name__ == "__main__":
    build()
