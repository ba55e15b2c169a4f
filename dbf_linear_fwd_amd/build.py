"""Build libdbf.so in-tree with hipcc for gfx950.

Usage: python -m dbf_linear_fwd_amd.build   (or call build()).
Always recompiles every source; the objects go to dbf_linear_fwd_amd/_build/.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libdbf.so")

HIP_SOURCES = ["runtime.hip", "decode_mfma.hip", "decode_i8.hip", "prefill.hip", "grad.hip", "bqq.hip", "factor.hip"]
CXX_SOURCES = ["pack.cpp"]

ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-result",
    # keep fp32 arithmetic on plain (non-packed) VALU instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # denormals are ordinary values in this library: never flush them
    "-fno-gpu-flush-denormals-to-zero",
    # no implicit contraction: every product and sum rounds where the source
    # writes it (no fused multiply-add); the epilogues keep a product that
    # feeds an fp16 conversion in fp32 themselves (fp32_value), which the
    # backend would otherwise fuse into the conversion in some kernel forms
    "-ffp-contract=off",
    "-I", INCLUDE,
    "-I", CSRC,
]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the DBF library needs ROCm's hipcc to build")


def build(verbose: bool = False) -> str:
    hipcc = _hipcc()
    os.makedirs(BUILD, exist_ok=True)
    jobs = []
    objs = []
    for src in HIP_SOURCES:
        obj = os.path.join(BUILD, src.replace(".hip", ".o"))
        cmd = [hipcc, *HIPCC_FLAGS, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
        jobs.append((src, cmd))
        objs.append(obj)
    for src in CXX_SOURCES:
        obj = os.path.join(BUILD, src.replace(".cpp", ".o"))
        cmd = ["g++", "-O2", "-std=c++17", "-fPIC", "-Wall", "-I", INCLUDE, "-I", CSRC, "-c",
               os.path.join(CSRC, src), "-o", obj]
        jobs.append((src, cmd))
        objs.append(obj)
    procs = []
    for src, cmd in jobs:
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
    failed = []
    for src, cmd, p in procs:
        out, _ = p.communicate()
        text = out.decode(errors="replace")
        # hipcc's host pass does not know the packed-fp32 feature flag; harmless
        lines = [ln for ln in text.splitlines() if "packed-fp32-ops" not in ln and ln.strip()]
        if p.returncode != 0:
            failed.append(src)
            sys.stderr.write(f"--- {src} failed:\n{text}\n")
        elif lines and verbose:
            print("\n".join(lines))
    if failed:
        raise RuntimeError(f"compilation failed: {failed}")
    tmp = LIB + ".tmp"
    # rocBLAS: the plain fp32 GEMMs of the factorization
    link = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs, "-L/opt/rocm/lib", "-lrocblas",
            "-Wl,-rpath,/opt/rocm/lib"]
    if verbose:
        print(" ".join(link), flush=True)
    res = subprocess.run(link, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
    if res.returncode != 0:
        sys.stderr.write(res.stdout.decode(errors="replace"))
        raise RuntimeError("link failed")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
