"""Build libgdr.so (the HIP kernels and the C ABI) for gfx950 with hipcc, in-tree.

    python -m gated_delta_rule_73_amd.build      # or gated_delta_rule_73_amd.build.build()

Sources are compiled in parallel to objects under gated_delta_rule_73_amd/_build/ and linked
into gated_delta_rule_73_amd/libgdr.so.  The same sources built with -DGDR_LDS_POISON are linked
into libgdr_poison.so (objects under _build/poison/), the LDS-poisoning debug build the tests
compare with the release library.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libgdr.so")
POISON_LIB = os.path.join(PKG, "libgdr_poison.so")
POISON_BUILD = os.path.join(BUILD, "poison")
SOURCES = ["gdr.cpp", "fwd.hip", "bwd.hip", "gdn2.hip", "kda.hip", "seg.hip", "decode.hip"]
ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # packed float32 vector ops are kept out of the generated device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the library)")


def _compile(src: str, poison: bool = False) -> str:
    out_dir = POISON_BUILD if poison else BUILD
    obj = os.path.join(out_dir, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *FLAGS, *(["-DGDR_LDS_POISON"] if poison else []), "-x", "hip", "-c",
           os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def _link(objs, lib: str) -> None:
    tmp = lib + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)


def build(verbose: bool = False, poison: bool = True) -> str:
    """Build libgdr.so and (poison=True) the LDS-poisoning debug build libgdr_poison.so."""
    os.makedirs(BUILD, exist_ok=True)
    os.makedirs(POISON_BUILD, exist_ok=True)
    variants = [False, True] if poison else [False]
    jobs = min(len(SOURCES) * len(variants), max(1, int(os.environ.get("MAX_JOBS", os.cpu_count() or 1))))
    with ThreadPoolExecutor(jobs) as ex:
        futs = {v: [ex.submit(_compile, src, v) for src in SOURCES] for v in variants}
        objs = {v: [f.result() for f in fs] for v, fs in futs.items()}
    _link(objs[False], LIB)
    if verbose:
        print(f"built {LIB}")
    if poison:
        _link(objs[True], POISON_LIB)
        if verbose:
            print(f"built {POISON_LIB}")
    return LIB


def build_poisoned(verbose: bool = False) -> str:
    """libgdr_poison.so alone: the kernels built with -DGDR_LDS_POISON, which fill a kernel's LDS
    with 0xFF bytes (NaN in bfloat16 and float32) at entry, the scans' LDS between chunk steps and
    the chunk kernels' LDS regions where their contents die.  A read of LDS that was never written
    (or of dead contents) then shows up as NaN; otherwise the results are the release build's,
    bit for bit.  Slower (extra barriers and stores): for tests only."""
    os.makedirs(POISON_BUILD, exist_ok=True)
    jobs = min(len(SOURCES), max(1, int(os.environ.get("MAX_JOBS", os.cpu_count() or 1))))
    with ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda src: _compile(src, True), SOURCES))
    _link(objs, POISON_LIB)
    if verbose:
        print(f"built {POISON_LIB}")
    return POISON_LIB


SAN_LIB = os.path.join(PKG, "libgdr_san.so")
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=all"]


def build_sanitized(verbose: bool = False) -> str:
    """The library with its host code (the C ABI: argument checks, planning, workspace carving)
    built with AddressSanitizer and UndefinedBehaviorSanitizer, for the ABI tests on a host
    without a GPU; the kernels' objects are the regular ones.  Load it only in a process started
    with the ASan runtime preloaded, and never to launch kernels (device code is not instrumented)."""
    os.makedirs(BUILD, exist_ok=True)
    objs = []
    for src in SOURCES:
        if src == "gdr.cpp":
            obj = os.path.join(BUILD, "gdr_san.o")
            cmd = [hipcc(), *FLAGS, *SAN_FLAGS, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
            r = subprocess.run(cmd, capture_output=True, text=True)
            if r.returncode != 0:
                raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
            objs.append(obj)
        else:
            obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
            objs.append(obj if os.path.exists(obj) else _compile(src))
    clang = os.path.join(os.path.dirname(os.path.realpath(hipcc())), "..", "llvm", "bin", "clang++")
    if not os.path.exists(clang):
        clang = "/opt/rocm/llvm/bin/clang++"
    cmd = [clang, "-shared", "-fPIC", "-fsanitize=address,undefined", "-shared-libsan", "-o", SAN_LIB, *objs,
           "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    if verbose:
        print(f"built {SAN_LIB}")
    return SAN_LIB


def asan_runtime() -> str:
    """Path of the ASan runtime the sanitized library needs preloaded."""
    clang = "/opt/rocm/llvm/bin/clang++"
    r = subprocess.run([clang, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    return r.stdout.strip()


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
