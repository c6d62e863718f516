"""Compile libfa16attn.so for gfx950 in-tree with hipcc.

Run `python -m fp16_attention_amd.build` (or call build()). The library is
written next to this file so it travels with the source tree.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libfa16attn.so")
SOURCES = ["abi.cpp", "attn_fwd.hip", "e4m3_bridge.hip", "noalloc.hip", "prefix_fp8.hip", "vsa_lists.hip",
           "vsa_select.hip"]
# The measurement aid (FP16 MFMA ceiling) is a library of its own, so that the
# attention library exports only the method's entry points.
MEASURE_CSRC = os.path.join(HERE, "measure_csrc")
MEASURE_SOURCES = ["mfma_ceiling.hip"]
MEASURE_LIB = os.path.join(HERE, "libfa16measure.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# -packed-fp32-ops: keep the compiler from forming packed FP32 VALU ops.
# -amdgpu-mfma-vgpr-form: MFMA accumulators in VGPRs, so the D=256 attention
# kernels can rescale their FP32 output accumulators without moving them
# between the AGPR and VGPR files every iteration (read-only operands go to
# AGPRs instead).
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-mllvm", "-amdgpu-mfma-vgpr-form",
         "-I", os.path.join(ROOT, "include")]


def _compile(sources, csrc, bdir, verbose):
    objs, procs = [], []
    for src in sources:
        obj = os.path.join(bdir, os.path.splitext(src)[0] + ".o")
        cmd = [HIPCC] + FLAGS + ["-x", "hip", "-c", os.path.join(csrc, src), "-o", obj]
        procs.append((cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
        objs.append(obj)
    failed = False
    for cmd, p in procs:
        out = p.communicate()[0].decode(errors="replace")
        out = "\n".join(l for l in out.splitlines() if "packed-fp32-ops" not in l)
        if p.returncode != 0:
            failed = True
            sys.stderr.write(" ".join(cmd) + "\n" + out + "\n")
        elif verbose and out.strip():
            sys.stderr.write(out + "\n")
    if failed:
        raise RuntimeError("hipcc failed")
    return objs


def _link(objs, lib):
    tmp = lib + ".tmp%d" % os.getpid()
    subprocess.check_call([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs)
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    """Compile every HIP source and link the attention library and the
    measurement library; returns the attention library's path."""
    bdir = os.path.join(ROOT, "_build")
    os.makedirs(bdir, exist_ok=True)
    _link(_compile(SOURCES, CSRC, bdir, verbose), LIB)
    mdir = os.path.join(bdir, "measure")
    os.makedirs(mdir, exist_ok=True)
    _link(_compile(MEASURE_SOURCES, MEASURE_CSRC, mdir, verbose), MEASURE_LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
