"""Build libbfp8.so in-tree with hipcc for gfx950.

Usage: ``python -m blockwise_fp8_gemm_bfp8_amd.build`` (or call ``build()``).
The library is written next to this file so it travels with the source tree.
"""

import os
import shutil
import subprocess
import sys
import tempfile

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_PATH = os.path.join(PKG_DIR, "libbfp8.so")
SOURCES = ["api.cpp", "quantize.hip", "gemm.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP toolchain is required to build libbfp8")


def compile_flags():
    return [
        "-O3",
        "-std=c++17",
        "-fPIC",
        f"--offload-arch={ARCH}",
        "-I", INCLUDE,
        "-I", CSRC,
        # packed-fp32 VALU forms are disabled for all device code
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wno-unused-command-line-argument",
    ]


def build(verbose: bool = False) -> str:
    """Compile every HIP/C++ source and link libbfp8.so; returns its path."""
    cc = hipcc()
    with tempfile.TemporaryDirectory(prefix="bfp8_build_") as tmp:
        objs, cmds = [], []
        for src in SOURCES:
            obj = os.path.join(tmp, src.replace(".", "_") + ".o")
            lang = ["-x", "hip"]
            cmds.append([cc, *compile_flags(), *lang, "-c", os.path.join(CSRC, src), "-o", obj])
            objs.append(obj)
        # the sources compile independently: one hipcc process each, at once
        procs = []
        for cmd in cmds:
            if verbose:
                print(" ".join(cmd), flush=True)
            procs.append((cmd, subprocess.Popen(cmd)))
        failed = [cmd for cmd, pr in procs if pr.wait() != 0]
        if failed:
            raise subprocess.CalledProcessError(1, failed[0])
        tmp_lib = os.path.join(tmp, "libbfp8.so")
        cmd = [cc, "-shared", f"--offload-arch={ARCH}", "-fPIC", *objs, "-o", tmp_lib]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        shutil.copyfile(tmp_lib, LIB_PATH + ".tmp")
        os.replace(LIB_PATH + ".tmp", LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
