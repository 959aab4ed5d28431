"""Builds libfa.so (the HIP kernels and the C ABI of include/fa.h) for gfx950, in-tree.

    python -m tiled_attention_causal_amd.build        # or __graft_entry__.build()

Every call recompiles every source. Objects go to _build/ at the repository root; the
shared library lands next to this file, where the Python binding loads it.
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libfa.so")
SOURCES = ["fa_api.hip", "fa_bf16.hip", "fa_f32.hip"]
ARCH = "gfx950"

# Packed fp32 VALU ops are kept out of the generated code; hipcc's host pass warns that it
# does not know the feature, which is harmless.
CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA results in VGPRs: the softmax reads every score register, so AGPR accumulators
    # would cost a copy per element.
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    f"-I{os.path.join(ROOT, 'include')}",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP toolchain is needed to build libfa.so")


def _run(cmd):
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    lines = [ln for ln in p.stdout.splitlines() if "not a recognized feature" not in ln]
    if p.returncode != 0:
        raise RuntimeError("command failed: " + " ".join(cmd) + "\n" + "\n".join(lines))
    return "\n".join(lines)


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    cc = hipcc()
    objs = []
    jobs = []
    for src in SOURCES:
        obj = os.path.join(BUILD, src.replace(".hip", ".o"))
        objs.append(obj)
        jobs.append([cc, *CFLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(len(jobs), 8)) as ex:
        for out in ex.map(_run, jobs):
            if verbose and out:
                print(out)
    tmp = LIB + ".tmp"
    _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
