"""Build libspecverify.so (gfx950) in-tree with hipcc.

``python -m draft_block_verification_spec_amd.build`` compiles every HIP source
under ``csrc/`` and links the shared library next to this file.  No GPU is
needed: hipcc cross-compiles for gfx950.
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
LIB = os.path.join(PKG, "libspecverify.so")
PEAKS_LIB = os.path.join(PKG, "libsvpeaks.so")  # achievable-peak probes (measurement only)
PEAKS_SRC = os.path.join(CSRC, "probe", "peaks.hip")
ARCH = "gfx950"

SOURCES = ["spec_verify.hip", "gemm_stream.hip", "gemm_tiled.hip", "verify_kernels.hip", "commit.hip"]

# Packed fp32 instructions are left to no one: the compiler must not form them.
HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found: the HIP toolchain is required to build libspecverify")


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "is not a recognized feature for this target" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    cc = hipcc()
    objs = []
    cmds = []
    for s in SOURCES:
        o = os.path.join(BUILD, s.replace(".hip", ".o"))
        objs.append(o)
        cmds.append([cc, *HIPCC_FLAGS, "-c", os.path.join(CSRC, s), "-o", o])
    with ThreadPoolExecutor(len(cmds)) as ex:
        outs = list(ex.map(_run, cmds))
    tmp = LIB + ".tmp"
    outs.append(_run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]))
    os.replace(tmp, LIB)
    tmp = PEAKS_LIB + ".tmp"
    outs.append(_run([cc, *HIPCC_FLAGS, "-shared", PEAKS_SRC, "-o", tmp]))
    os.replace(tmp, PEAKS_LIB)
    if verbose:
        for o in outs:
            if o.strip():
                print(o)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))


# A build of the library whose host code carries AddressSanitizer and
# UndefinedBehaviorSanitizer (the device code is built as usual, without them), and the
# C++ program that runs the host-side ABI checks against it; the checks never reach the
# device, so no GPU is needed.  Every sanitizer flag applies to the host pass only.
SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer"]
HOST_CHECKS_SRC = os.path.join(ROOT, "tests", "abi_host_checks.cpp")


def build_host_checks(out_dir: str) -> str:
    """Build the host-sanitized library and the check program into out_dir; return the
    program's path."""
    os.makedirs(out_dir, exist_ok=True)
    cc = hipcc()
    base = [f"--offload-arch={ARCH}", "-O1", "-g", "-std=c++17", "-fPIC", "-fvisibility=hidden",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wno-unused-command-line-argument", f"-I{INCLUDE}", f"-I{CSRC}", *SANITIZE]
    objs, cmds = [], []
    for s in SOURCES:
        o = os.path.join(out_dir, s.replace(".hip", ".o"))
        objs.append(o)
        cmds.append([cc, *base, "-c", os.path.join(CSRC, s), "-o", o])
    with ThreadPoolExecutor(len(cmds)) as ex:
        list(ex.map(_run, cmds))
    lib = os.path.join(out_dir, "libspecverify.so")
    _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *SANITIZE, *objs, "-o", lib])
    exe = os.path.join(out_dir, "abi_host_checks")
    clangxx = os.path.join(os.path.dirname(os.path.realpath(cc)), "..", "lib", "llvm", "bin", "clang++")
    if not os.path.exists(clangxx):
        clangxx = "/opt/rocm/lib/llvm/bin/clang++"
    _run([clangxx, "-O1", "-g", "-std=c++17", *SANITIZE, f"-I{INCLUDE}", HOST_CHECKS_SRC, "-o", exe,
          f"-L{out_dir}", "-lspecverify", f"-Wl,-rpath,{out_dir}"])
    return exe

