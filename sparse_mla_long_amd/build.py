"""Compile the gfx950 HIP library (libmla_sparse.so) in-tree with hipcc."""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libmla_sparse.so")
SOURCES = ["api.hip", "indexer.hip", "topk.hip", "attention.hip", "attention_f8.hip", "merge.hip",
           "decode_ds656.hip"]
ARCH = "gfx950"

HIPCC_FLAGS = [
    "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
    # keep the compiler from forming packed-fp32 VALU ops
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]
# Per-source additions. The attention kernels run two waves per SIMD whose
# roles hold their large arrays in different code paths; with MFMA
# accumulators in VGPRs both paths share one 256-register allocation (in
# accumulation registers the output tiles of one path and the operands of the
# other would add up instead).
FILE_FLAGS = {"attention.hip": ["-mllvm", "--amdgpu-mfma-vgpr-form"],
              "attention_f8.hip": ["-mllvm", "--amdgpu-mfma-vgpr-form"]}
BUILD = os.path.join(PKG, "_build")


def compile_flags(source: str) -> list:
    """hipcc flags (without -c/-o) that compile one source of the library."""
    return [*HIPCC_FLAGS, *FILE_FLAGS.get(source, []), "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "packed-fp32-ops"   # the host pass does not know the feature; harmless
    msgs = [l for l in (res.stdout + res.stderr).splitlines() if l.strip() and noise not in l]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs), file=sys.stderr)


def build_library(verbose: bool = False) -> str:
    """Compile every source to an object (in parallel), then link the library."""
    from concurrent.futures import ThreadPoolExecutor
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    os.makedirs(BUILD, exist_ok=True)
    objs = [os.path.join(BUILD, s + ".%d.o" % os.getpid()) for s in SOURCES]
    jobs = [[hipcc, *compile_flags(s), "-c", os.path.join(CSRC, s), "-o", o] for s, o in zip(SOURCES, objs)]
    try:
        with ThreadPoolExecutor(max_workers=min(len(jobs), 8)) as ex:
            for f in [ex.submit(_run, j, verbose) for j in jobs]:
                f.result()
        tmp = LIB + ".tmp%d" % os.getpid()
        _run([hipcc, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp, *objs], verbose)
        os.replace(tmp, LIB)
    finally:
        for o in objs:
            if os.path.exists(o):
                os.remove(o)
    return LIB


if __name__ == "__main__":
    print(build_library(verbose=True))
