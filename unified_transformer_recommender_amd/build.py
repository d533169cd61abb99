"""Build libonetrans.so (HIP, gfx950) in-tree with hipcc.

Every translation unit is compiled to an object in parallel and linked into one shared
library next to this file. Packed fp32 VALU ops are disabled for all device code.
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
LIB = os.path.join(PKG, "libonetrans.so")
ARCH = os.environ.get("ONETRANS_ARCH", "gfx950")

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
    "-I", INCLUDE, "-I", CSRC,
]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [hipcc(), *FLAGS, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    if err.strip():
        sys.stderr.write(err + "\n")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    with ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stderr)
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-omit-frame-pointer"]


def asan_runtime() -> str:
    """The shared AddressSanitizer runtime a process must preload to load the sanitized library."""
    r = subprocess.run([hipcc(), "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    return r.stdout.strip()


def build_host_sanitized() -> str:
    """A copy of the library whose host code (the C ABI's validation and the planner in
    onetrans.hip) is built with AddressSanitizer and UndefinedBehaviorSanitizer; device code is
    not instrumented. Written to _build/asan/libonetrans.so; the other objects come from build()."""
    out_dir = os.path.join(BUILD, "asan")
    os.makedirs(out_dir, exist_ok=True)
    planner = os.path.join(CSRC, "onetrans.hip")
    others = [s for s in sources() if s != planner]
    objs = [os.path.join(BUILD, os.path.basename(s) + ".o") for s in others]
    if not all(os.path.exists(o) for o in objs):
        os.makedirs(BUILD, exist_ok=True)
        with ThreadPoolExecutor(max_workers=min(8, len(others))) as ex:
            objs = list(ex.map(_compile, others))
    obj = os.path.join(out_dir, "onetrans.hip.o")
    cmd = [hipcc(), *[f for f in FLAGS if f != "-O3"], "-O1", "-g", *SANITIZE, "-c", planner, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("sanitized compile failed:\n" + r.stderr)
    lib = os.path.join(out_dir, "libonetrans.so")
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *SANITIZE, "-Xarch_host", "-shared-libsan",
           "-o", lib, *objs, obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("sanitized link failed:\n" + r.stderr)
    return lib


if __name__ == "__main__":
    build(verbose=True)
