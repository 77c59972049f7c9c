"""Compile the HIP sources into libgptq_mi355x.so (gfx950), in-tree.

    python -m post_weight_quantization_layer_amd.build

Each source is compiled separately (in parallel) into _build/, then linked.
Every HIP compile carries ``-Xclang -target-feature -Xclang -packed-fp32-ops``
so the compiler emits no packed-fp32 VALU instructions.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libgptq_mi355x.so")
SOURCES = ["abi.hip", "hessian.hip", "gemm.hip", "prepare.hip", "sweep.hip", "pack.hip",
           "w4a16.hip", "forward.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    p = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    return p


def compile_flags() -> list[str]:
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
        f"-I{INCLUDE}", f"-I{CSRC}",
    ]


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    cc = hipcc()

    def one(src):
        obj = os.path.join(BUILD, src.replace(".hip", ".o"))
        cmd = [cc, *compile_flags(), "-c", os.path.join(CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                        if "packed-fp32-ops" not in l)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{msg}")
        if verbose and msg.strip():
            print(msg)
        return obj

    with ThreadPoolExecutor(min(8, len(SOURCES))) as ex:
        objs = list(ex.map(one, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
