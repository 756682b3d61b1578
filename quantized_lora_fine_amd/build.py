"""Builds libnf4lora.so in-tree with hipcc for gfx950.

    python quantized_lora_fine_amd/build.py

(run by path: importing the package would load the library being rebuilt)

Every HIP source is compiled with packed fp32 vector ops disabled, without
fast-math (IEEE fp32 division, denormals kept), then linked with the host
C++ ABI layer into quantized_lora_fine_amd/libnf4lora.so.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libnf4lora.so")
ARCH = os.environ.get("NF4LORA_ARCH", "gfx950")

HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"

def _common(csrc):
    return ["-O3", "-fPIC", "-std=c++17", f"-I{INCLUDE}", f"-I{csrc}", "-Wall", "-Wno-unused-function"]


DEVICE = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
# per-source extra flags: the quantization kernels must round exactly as the
# format defines (one rounding per multiply, no fused multiply-add across
# statements)
EXTRA = {"quant.hip": ["-ffp-contract=off"],
         # dequantized weights (and the two-stage sum) must round like nf4_dequantize: no fused multiply-add
         "gemm.hip": ["-ffp-contract=off"],
         "merge.hip": ["-ffp-contract=off"]}

HIP_SOURCES = ["quant.hip", "gemm.hip", "skinny.hip", "merge.hip", "probe.hip", "scratch.hip"]
CPP_SOURCES = ["api.cpp", "nf4_table.cpp", "plan.cpp"]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"build step failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = False, csrc: str = CSRC, out: str = LIB, build_dir: str = BUILD) -> str:
    os.makedirs(build_dir, exist_ok=True)
    jobs = []
    for src in HIP_SOURCES:
        obj = os.path.join(build_dir, src + ".o")
        jobs.append([HIPCC, "-x", "hip", *_common(csrc), *DEVICE, *EXTRA.get(src, []), "-c",
                     os.path.join(csrc, src), "-o", obj])
    for src in CPP_SOURCES:
        obj = os.path.join(build_dir, src + ".o")
        jobs.append([HIPCC, *_common(csrc), "-D__HIP_PLATFORM_AMD__", "-c", os.path.join(csrc, src), "-o", obj])
    with ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        outs = list(ex.map(_run, jobs))
    if verbose:
        for o in outs:
            if o.strip():
                print(o)
    objs = [os.path.join(build_dir, s + ".o") for s in HIP_SOURCES + CPP_SOURCES]
    tmp = out + ".tmp"
    _run([HIPCC, "-shared", f"--offload-arch={ARCH}", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
