"""Builds libdsa.so (the gfx950 HIP kernels + the C ABI of include/dsa.h) in-tree.

    python sparse_attention_16_amd/build.py               # in-tree libdsa.so
    python sparse_attention_16_amd/build.py --host-asan   # _build/asan/libdsa.so
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libdsa.so")
ARCH = os.environ.get("DSA_OFFLOAD_ARCH", "gfx950")

HIPCC_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "-shared",
    f"--offload-arch={ARCH}",
    # keep fp32 math out of the packed-fp32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # inputs are NaN-free by contract: no quieting of max/min operands
    "-fno-honor-nans",
    "-Wall", "-Wno-unused-function",
]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def build(verbose: bool = False) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc, *HIPCC_FLAGS, "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           *sources(), "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass warns that it does not know the packed-fp32 feature: harmless
    msgs = [ln for ln in (r.stdout + r.stderr).splitlines()
            if "packed-fp32-ops" not in ln and "--hip-link" not in ln]
    if r.returncode != 0:
        if os.path.exists(tmp):
            os.remove(tmp)
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs))
    os.replace(tmp, LIB)
    return LIB


def build_host_asan(out_dir: str) -> str:
    """Builds the library with AddressSanitizer on its host code only.

    The device code is compiled as usual (the sanitizer does not reach it);
    the host side (argument validation, workspace sizing, launch set-up) is
    instrumented.  Load it with the sanitizer runtime preloaded (clang's
    libclang_rt.asan) and select it with DSA_LIBRARY.  The sources are
    compiled in parallel, one process per file.
    """
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    os.makedirs(out_dir, exist_ok=True)
    flags = [f for f in HIPCC_FLAGS if f not in ("-O3", "-shared")]
    flags += ["-O1", "-g", "-Xarch_host", "-fsanitize=address",
              "-Xarch_host", "-fno-omit-frame-pointer"]
    procs, objs = [], []
    for src in sources():
        obj = os.path.join(out_dir, os.path.basename(src)[:-4] + ".o")
        objs.append(obj)
        procs.append(subprocess.Popen(
            [hipcc, "-c", *flags, "-I", os.path.join(ROOT, "include"), "-I", CSRC, src, "-o", obj],
            stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True))
    errs = []
    for p in procs:
        out, _ = p.communicate()
        if p.returncode != 0:
            errs.append(out)
    if errs:
        raise RuntimeError("hipcc failed:\n" + "\n".join(errs))
    lib = os.path.join(out_dir, "libdsa.so")
    r = subprocess.run([hipcc, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", lib],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc link failed:\n" + r.stdout + r.stderr)
    return lib


if __name__ == "__main__":
    if "--host-asan" in sys.argv:
        print(build_host_asan(os.path.join(ROOT, "_build", "asan")))
    else:
        print(build(verbose="-v" in sys.argv))
