"""Build the HIP shared library libsv.so for gfx950, in-tree, with hipcc.

Usage:  python -m tree_verify_sparse_amd.build   (or call build()).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libsv.so")
SOURCES = ["api.cpp", "verify.hip", "topk.hip", "sparse.hip", "accept.hip", "build_tree.hip", "validate.hip", "noalloc.hip"]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build the HIP library)")


def flags() -> list[str]:
    return [
        "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
        # keep the compiler from emitting packed fp32 arithmetic
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        # MFMA accumulators in ordinary VGPRs: the attention loops rescale their
        # accumulators with vector ALU ops, and the AGPR form made the compiler
        # copy them between register files on every iteration
        "-mllvm", "-amdgpu-mfma-vgpr-form=true",
        "-I", INCLUDE, "-I", CSRC,
        "-Wall", "-Wno-unused-function", "-Wno-unused-result",
    ]


def build(verbose: bool = False, jobs: int = 4) -> str:
    """Compile every source to an object file (in parallel), then link libsv.so."""
    cc = hipcc()
    tmp = tempfile.mkdtemp(prefix="sv_build_")
    try:
        procs, objs = [], []
        for src in SOURCES:
            obj = os.path.join(tmp, src + ".o")
            objs.append(obj)
            lang = ["-x", "hip"] if src.endswith(".cpp") else []
            cmd = [cc] + flags() + lang + ["-c", os.path.join(CSRC, src), "-o", obj]
            procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)))
        failed = []
        for src, p in procs:
            out, _ = p.communicate()
            out = "\n".join(line for line in out.splitlines() if "packed-fp32-ops" not in line)
            if p.returncode != 0:
                failed.append((src, out))
            elif verbose and out.strip():
                print(out)
        if failed:
            raise RuntimeError("hipcc failed:\n" + "\n".join(f"--- {s}\n{o}" for s, o in failed))
        tmp_lib = LIB + ".tmp"
        link = [cc, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp_lib] + objs
        r = subprocess.run(link, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
        if r.returncode != 0:
            raise RuntimeError("link failed:\n" + r.stdout)
        os.replace(tmp_lib, LIB)
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
