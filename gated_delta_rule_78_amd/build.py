"""Build ``libkda.so`` (the C-ABI library) in-tree with hipcc for gfx950.

Usage: python -m gated_delta_rule_78_amd.build   (or call ``build()``)
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libkda.so")
SOURCES = ["kda_abi.cpp", "kda_plan.cpp", "kda_decode.hip", "kda_chunk.hip", "kda_intra.hip", "kda_inter.hip", "kda_fused.hip", "kda_scan.hip", "kda_varlen.hip", "kda_bwd.hip", "kda_noalloc.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

COMMON = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
          # Packed fp32 arithmetic (v_pk_*_f32) stays off in all device code.
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          # MFMA results in architectural VGPRs: the state accumulators are also read by VALU
          # code every chunk, and the AGPR form costs a v_accvgpr move per such read.
          "-mllvm", "-amdgpu-mfma-vgpr-form",
          "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def _compile(src):
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC] + COMMON + ["-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd = [HIPCC] + COMMON + ["-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = "\n".join(line for line in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in line)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s" % (src, msgs))
    return obj, msgs


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        results = list(ex.map(_compile, SOURCES))
    for _, msgs in results:
        if verbose and msgs.strip():
            print(msgs)
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + [o for o, _ in results]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
