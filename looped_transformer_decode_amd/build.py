"""Builds the HIP libraries in-tree for gfx950.

  looped_transformer_decode_amd/liblla.so   the LLA C ABI (include/lla.h)
  synth/libllasynth.so                       the device-side synthetic filler

Each source is compiled with hipcc in parallel, then linked into a shared
library.  Always recompiles (the build check must exercise the compiler).
"""
from __future__ import annotations

import concurrent.futures
import os
import re
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "liblla.so")
SYNTH_SRC = os.path.join(ROOT, "synth", "fill.hip")
SYNTH_LIB = os.path.join(ROOT, "synth", "libllasynth.so")

ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
          # never emit packed-FP32 VALU instructions
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-I", INCLUDE, "-I", CSRC]
SOURCES = ["lla_api.cpp", "decode_valu.hip", "decode_mfma.hip", "encode_valu.hip",
           "encode_mfma.hip", "decode2d_mfma.hip", "kvcache.hip",
           "svd_init.hip", "decode_mq.hip"]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "is not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"build failed: {' '.join(cmd)}\n{out}")
    return out


# Kernels that count their own outstanding vector-memory operations
# (s_waitcnt vmcnt(n) after buffer loads into LDS): a register spill would
# add scratch loads/stores to that count, so they must compile without any.
NO_SPILL = {"decode_mfma.hip", "decode2d_mfma.hip"}


def _compile(src: str, obj: str):
    extra = []
    if os.path.basename(src) in NO_SPILL:
        extra = ["-Rpass-analysis=kernel-resource-usage"]
    out = _run([HIPCC, *COMMON, "-x", "hip", *extra, "-c", src, "-o", obj])
    if extra:
        spills = [l for l in out.splitlines()
                  if re.search(r"(VGPRs|SGPRs) Spill: [1-9]", l)]
        if spills:
            raise RuntimeError(f"{src}: register spills in a kernel that counts vmcnt itself:\n"
                               + "\n".join(spills))
        out = ""  # the resource remarks are not build output
    return out


def build(verbose: bool = False) -> list[str]:
    os.makedirs(BUILD, exist_ok=True)
    jobs = []
    for s in SOURCES:
        jobs.append((os.path.join(CSRC, s), os.path.join(BUILD, os.path.splitext(s)[0] + ".o")))
    jobs.append((SYNTH_SRC, os.path.join(BUILD, "synth_fill.o")))
    workers = min(len(jobs), max(1, min(8, os.cpu_count() or 1)))
    with concurrent.futures.ThreadPoolExecutor(workers) as ex:
        logs = list(ex.map(lambda j: _compile(*j), jobs))
    if verbose:
        for l in logs:
            if l.strip():
                print(l)
    objs = [o for _, o in jobs[:-1]]
    tmp = LIB + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, LIB)
    tmp = SYNTH_LIB + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, jobs[-1][1]])
    os.replace(tmp, SYNTH_LIB)
    return [LIB, SYNTH_LIB]


if __name__ == "__main__":
    for p in build(verbose=True):
        print("built", p)
