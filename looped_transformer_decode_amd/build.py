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
           "svd_init.hip", "decode_mq.hip", "decode_noalloc.hip", "encode_stream.hip"]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "is not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"build failed: {' '.join(cmd)}\n{out}")
    return out


# Kernels that count their own outstanding vector-memory operations
# (s_waitcnt vmcnt(n) after buffer loads into LDS): a register spill or any
# other scratch access would add loads/stores to that count, so they must
# compile without any.
NO_SPILL = {"decode_mfma.hip", "decode2d_mfma.hip", "decode_mq.hip", "encode_stream.hip"}


# Per-source code-generation options.  The multi-query decode feeds every
# MFMA result straight into vector arithmetic: with the VGPR form of the
# MFMA instructions its results need no accumulator-register copies.  The
# same holds for the per-head decode at the larger ranks, whose waves use
# more than 256 registers (measured: B = 32 call 78.0 -> 76.2 us, long
# recurrence 342.5 -> 336.8 us).
SOURCE_FLAGS = {"decode_mq.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
                "decode_mfma.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
                "encode_stream.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _compile(src: str, obj: str):
    extra = list(SOURCE_FLAGS.get(os.path.basename(src), []))
    if os.path.basename(src) in NO_SPILL:
        extra += ["-Rpass-analysis=kernel-resource-usage"]
    out = _run([HIPCC, *COMMON, "-x", "hip", *extra, "-c", src, "-o", obj])
    if extra:
        spills = [l for l in out.splitlines()
                  if re.search(r"(VGPRs|SGPRs) Spill: [1-9]|ScratchSize \[bytes/lane\]: [1-9]", l)]
        if spills:
            raise RuntimeError(f"{src}: register spills in a kernel that counts vmcnt itself:\n"
                               + "\n".join(spills))
        out = ""  # the resource remarks are not build output
    return out


def _check_defined(lib: str):
    """A kernel whose host pass could not instantiate it leaves its launch
    stub undefined while the compile still succeeds; refuse such a library."""
    r = subprocess.run(["nm", "-D", "--undefined-only", lib], stdout=subprocess.PIPE,
                       stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"nm failed on {lib}:\n{r.stdout}")
    missing = [l.split()[-1] for l in r.stdout.splitlines() if "_ZN3lla" in l]
    if missing:
        raise RuntimeError(f"{lib}: undefined library symbols:\n" + "\n".join(missing))


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
    _check_defined(tmp)
    os.replace(tmp, LIB)
    tmp = SYNTH_LIB + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, jobs[-1][1]])
    os.replace(tmp, SYNTH_LIB)
    return [LIB, SYNTH_LIB]


# Host-side sanitizer build of the C ABI: the two files that hold host
# arithmetic (argument validation, sizes, offsets, splits, the RoPE table,
# the scratch lookup) are compiled with AddressSanitizer and
# UndefinedBehaviorSanitizer on their host pass only (-Xarch_host; the device
# code is built as usual) and linked with the regular build's other objects
# into _build/liblla_san.so.  The sanitizer runtime is not linked in: load it
# first with LD_PRELOAD=sanitizer_runtime() and point the binding at the
# library with LLA_LIBRARY (tests/test_sanitized_abi.py does both).
SAN_SOURCES = ["lla_api.cpp", "decode_noalloc.hip"]
SAN_LIB = os.path.join(BUILD, "liblla_san.so")
SAN_FLAGS = ["-g", "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


def sanitizer_runtime() -> str:
    """The clang AddressSanitizer runtime (it carries the UBSan handlers)."""
    res = _run([HIPCC, "-print-resource-dir"]).strip().splitlines()[-1]
    path = os.path.join(res, "lib", "linux", "libclang_rt.asan-x86_64.so")
    if not os.path.exists(path):
        raise RuntimeError(f"sanitizer runtime not found at {path}")
    return path


def build_sanitized() -> str:
    build()
    objs = []
    for s in SOURCES:
        if s in SAN_SOURCES:
            o = os.path.join(BUILD, os.path.splitext(s)[0] + "_san.o")
            _run([HIPCC, *COMMON, *SAN_FLAGS, "-x", "hip", "-c", os.path.join(CSRC, s), "-o", o])
        else:
            o = os.path.join(BUILD, os.path.splitext(s)[0] + ".o")
        objs.append(o)
    tmp = SAN_LIB + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, SAN_LIB)
    return SAN_LIB


if __name__ == "__main__":
    import sys
    if sys.argv[1:] == ["--sanitize"]:
        print("built", build_sanitized())
        print("runtime", sanitizer_runtime())
    else:
        for p in build(verbose=True):
            print("built", p)
