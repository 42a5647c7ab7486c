"""Build libpkv.so (the HIP kernels and their C ABI) for gfx950, in-tree.

Usage: ``python -m paged_kv_attention_out_amd.build`` or ``build()``.
Every call recompiles; objects go to ``_build/`` beside this file and the
shared library to ``libpkv.so`` beside this file.
"""

from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(HERE, "_build")
LIB_PATH = os.path.join(HERE, "libpkv.so")
ARCH = "gfx950"

# -packed-fp32-ops: no packed fp32 VALU instructions are emitted.
# -fno-honor-nans: the kernels mask with -inf and never read unowned slots, so
# fmaxf over MFMA results needs no NaN-quieting pass (one VALU op per score).
# -amdgpu-mfma-vgpr-form: MFMA accumulators stay in VGPRs; the softmax reads
# every score, and accumulators in AGPRs would cost a VALU move per read.
HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-fno-honor-nans",
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def _hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP toolchain is required to build libpkv.so")


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _compile(hipcc: str, src: str, extra) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [hipcc, *HIP_FLAGS, *extra, "-c", src, "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    return obj


def build(verbose: bool = False, extra_flags=()) -> str:
    """Compile every kernel source and link libpkv.so; returns its path."""
    hipcc = _hipcc()
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = sources()
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(hipcc, s, list(extra_flags)), srcs))
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB_PATH)
    if verbose:
        print(f"built {LIB_PATH}")
    return LIB_PATH


def code_objects():
    """Unbundle the gfx950 code object of every compiled source (for ISA
    checks of what the last compile produced); returns their paths."""
    llvm = "/opt/rocm/llvm/bin"
    paths = []
    for src in sources():
        obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
        fatbin = obj + ".fatbin"
        co = obj + f".{ARCH}.co"
        subprocess.run([f"{llvm}/llvm-objcopy", f"--dump-section=.hip_fatbin={fatbin}", obj],
                       check=True, capture_output=True)
        subprocess.run([f"{llvm}/clang-offload-bundler", "--type=o",
                        f"--targets=hipv4-amdgcn-amd-amdhsa--{ARCH}", f"--input={fatbin}",
                        f"--output={co}", "--unbundle"], check=True, capture_output=True)
        paths.append(co)
    return paths


if __name__ == "__main__":
    build(verbose=True, extra_flags=sys.argv[1:])
