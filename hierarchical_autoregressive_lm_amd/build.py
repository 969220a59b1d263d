"""Compile the HIP sources into the in-tree shared library libphoton.so.

Every source is compiled for gfx950 with hipcc; the C ABI is declared in
include/photon.h.  Objects go to _build/ next to the package; the library is
written beside this file so that the binding loads it from the tree.
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "libphoton.so")
BUILD = os.path.join(ROOT, "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

SOURCES = ["gemm.hip", "attention.hip", "elementwise.hip", "sampling.hip", "photon.cpp"]
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
         # packed fp32 instructions stay off (see the build notes)
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wno-unused-result", "-I", os.path.join(ROOT, "include")]


# Host-sanitized variant for the CPU tests of the C ABI: AddressSanitizer and
# UndefinedBehaviorSanitizer on the host code only (each -fsanitize= behind
# -Xarch_host; the device code is built as usual).
SAN_BUILD = os.path.join(BUILD, "hostsan")
SAN_OUT = os.path.join(SAN_BUILD, "libphoton_hostsan.so")
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-omit-frame-pointer"]


def sanitizer_runtime():
    """The clang AddressSanitizer runtime the sanitized build links against
    (a process that loads the library preloads it)."""
    import glob
    hits = sorted(glob.glob(os.path.join(os.path.dirname(os.path.dirname(HIPCC)), "llvm", "lib", "clang", "*",
                                         "lib", "linux", "libclang_rt.asan-x86_64.so")))
    return hits[-1] if hits else None


def _compile(src, flags=FLAGS, build=BUILD):
    obj = os.path.join(build, os.path.basename(src) + ".o")
    cmd = [HIPCC, *flags, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def build(verbose=False):
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(4, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = OUT + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, OUT)
    if verbose:
        print(f"built {OUT}")
    return OUT


def build_hostsan(verbose=False):
    """The host-sanitized library (SAN_OUT), for CPU tests only."""
    os.makedirs(SAN_BUILD, exist_ok=True)
    flags = [f for f in FLAGS if f != "-O3"] + ["-O1", "-g", *SAN_FLAGS]
    with ThreadPoolExecutor(max_workers=min(4, len(SOURCES))) as ex:
        objs = list(ex.map(lambda src: _compile(src, flags, SAN_BUILD), SOURCES))
    tmp = SAN_OUT + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *SAN_FLAGS, "-shared-libsan", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, SAN_OUT)
    if verbose:
        print(f"built {SAN_OUT}")
    return SAN_OUT


if __name__ == "__main__":
    build(verbose="-q" not in sys.argv)
