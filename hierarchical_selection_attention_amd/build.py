"""Build liblighthouse.so (the gfx950 HIP kernels and the C ABI) in-tree with hipcc.

Usage: python hierarchical_selection_attention_amd/build.py [-v]
(run as a file: the package itself refuses to import until the library exists)
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build", "lighthouse")
LIB = os.path.join(PKG, "liblighthouse.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

COMMON = ["--offload-arch=gfx950", "-O3", "-fPIC", "-std=c++17", "-Wall",
          # packed fp32 arithmetic stays off: hipcc would otherwise form v_pk_* fp32 ops
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-I", os.path.join(ROOT, "include"), "-I", CSRC]

# per-file flags: the scoring pass must keep its stated fp32 operation order
SOURCES = {
    "lh_stream.hip": ["-ffp-contract=off"],
    "lh_topk.hip": [],
    # MFMA accumulators in ordinary VGPRs: the softmax rescale and the split of P
    # work on them with VALU ops, which cannot read AGPRs
    "lh_attn.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
    "lh_prep.hip": [],
    "lh_probe.hip": [],
    "lh_api.cpp": ["-x", "hip"],
    # the projections around the layer (hipBLASLt GEMMs)
    "lh_block.cpp": ["-x", "hip"],
}
ROCM_LIB = "/opt/rocm/lib"


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    procs, objs = [], []
    for src, extra in SOURCES.items():
        obj = os.path.join(BUILD, src + ".o")
        objs.append(obj)
        cmd = [HIPCC, *COMMON, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
    failed = []
    for src, p in procs:
        out, _ = p.communicate()
        text = out.decode(errors="replace")
        if p.returncode != 0:
            failed.append(src)
            sys.stderr.write(text)
        elif verbose and text.strip():
            sys.stderr.write(text)
    if failed:
        raise RuntimeError(f"hipcc failed for {failed}")
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs,
           "-L", ROCM_LIB, "-lhipblaslt", f"-Wl,-rpath,{ROCM_LIB}"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    # every symbol must resolve (a kernel whose host stub was not emitted only
    # shows up here, as an undefined __device_stub__)
    ctypes.CDLL(tmp, mode=os.RTLD_NOW)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
