"""Compile the HIP library libwave_index.so for gfx950, in-tree (kv_vector_index_amd/lib/)."""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIBDIR = os.path.join(HERE, "lib")
LIB = os.path.join(LIBDIR, "libwave_index.so")
SAN_LIB = os.path.join(LIBDIR, "libwave_index_san.so")
SOURCES = ["api.cpp", "build_kernels.hip", "decode_kernels.hip", "anns_kernels.hip"]
HEADERS = ["wave_common.h", "wave_kernels.h"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Wall", "-Wno-unused-function",
    # packed-fp32 VALU ops stay off (see the notes on correctness of the packed forms)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the wave-index library needs ROCm's hipcc")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                     if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{msgs}")
    if verbose and msgs.strip():
        print(msgs)


def build(verbose: bool = False) -> str:
    """Compile every source to an object (in parallel), then link the shared library."""
    objdir = os.path.join(LIBDIR, "obj")
    os.makedirs(objdir, exist_ok=True)
    compile_flags = [f for f in HIPCC_FLAGS if f != "-shared"]
    jobs = []
    for src in SOURCES:
        obj = os.path.join(objdir, os.path.splitext(src)[0] + ".o")
        jobs.append(([hipcc(), *compile_flags, "-c", os.path.join(CSRC, src), "-o", obj], obj))
    with ThreadPoolExecutor(max_workers=len(jobs)) as pool:
        for f in [pool.submit(_run, cmd, verbose) for cmd, _ in jobs]:
            f.result()
    tmp = LIB + ".tmp"
    _run([hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", *[o for _, o in jobs], "-o", tmp],
         verbose)
    os.replace(tmp, LIB)
    return LIB


def build_sanitized(verbose: bool = False) -> str:
    """The C ABI's host side alone (argument validation, workspace layout; kernel launchers
    replaced by host_stubs.cpp, which report that nothing can run), built by the host
    compiler with AddressSanitizer and UndefinedBehaviorSanitizer. Load it with the ASan
    runtime preloaded (`g++ -print-file-name=libasan.so`)."""
    os.makedirs(LIBDIR, exist_ok=True)
    cxx = shutil.which("g++")
    if not cxx:
        raise RuntimeError("g++ not found")
    tmp = SAN_LIB + ".tmp"
    cmd = [cxx, "-std=c++17", "-O1", "-g", "-fPIC", "-shared",
           "-fsanitize=address,undefined", "-fno-omit-frame-pointer", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", "/opt/rocm/include",
           os.path.join(CSRC, "api.cpp"), os.path.join(CSRC, "host_stubs.cpp"), "-o", tmp]
    _run(cmd, verbose)
    os.replace(tmp, SAN_LIB)
    return SAN_LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
