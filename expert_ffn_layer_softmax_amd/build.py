"""Build the gfx950 HIP library ``libmoe_mi355x.so`` in-tree with hipcc.

Every source is compiled for gfx950 only.  Packed-fp32 VALU instructions are
disabled on the device side (``-target-feature -packed-fp32-ops``).

``--debug-checks`` builds ``libmoe_mi355x_dbg.so``: the same library with
-DMOE_DEBUG_CHECKS, whose kernels bounds-check every index they read from
memory (see moe_debug_check in include/moe.h).

``--sanitize`` builds ``libmoe_mi355x_san.so`` instead, whose host code (the
C ABI's validation, workspace plan and launch logic) carries AddressSanitizer
and UndefinedBehaviorSanitizer; device code is compiled as usual.  Load it
with the ASan runtime preloaded (``sanitizer_runtime()``) and
``MOE_MI355X_LIB`` pointing at it.
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libmoe_mi355x.so")
SAN_LIB = os.path.join(PKG, "libmoe_mi355x_san.so")
DBG_LIB = os.path.join(PKG, "libmoe_mi355x_dbg.so")

SOURCES = ["abi.cpp", "route.hip", "permute.hip", "gemv.hip", "combine.hip", "grouped_gemm.hip",
           "scratch.hip"]

ARCH = "gfx950"
# host-only sanitizers: each flag applies to the host compilation pass alone
SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer",
            "-Xarch_host", "-g"]
COMMON = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
    "-I", CSRC,
]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the MI355X library needs ROCm's hipcc")


_SAN_LINK = ["-fsanitize=address", "-fsanitize=undefined"]


def _clangxx() -> str:
    for cand in ("/opt/rocm/llvm/bin/clang++", shutil.which("clang++")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("clang++ not found")


def sanitizer_runtime() -> str:
    """Path of the shared ASan runtime of hipcc's clang (to LD_PRELOAD)."""
    for cand in ("/opt/rocm/llvm/bin/clang", shutil.which("clang")):
        if cand and os.path.exists(cand):
            r = subprocess.run([cand, "-print-file-name=libclang_rt.asan-x86_64.so"],
                               capture_output=True, text=True)
            path = r.stdout.strip()
            if r.returncode == 0 and os.path.isabs(path) and os.path.exists(path):
                return path
    raise RuntimeError("the clang ASan runtime was not found")


def _compile(src: str, hipcc: str, extra, build_dir: str) -> str:
    obj = os.path.join(build_dir, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc, *COMMON, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops" not in l and l.strip())
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{out}")
    if out:
        print(out, file=sys.stderr)
    return obj


def build(verbose: bool = False, extra=(), sanitize: bool = False, debug_checks: bool = False) -> str:
    """Compile every source and link the shared library; returns its path."""
    assert not (sanitize and debug_checks), "one variant at a time"
    build_dir = BUILD + ("_san" if sanitize else "_dbg" if debug_checks else "")
    lib = SAN_LIB if sanitize else DBG_LIB if debug_checks else LIB
    extra = list(extra) + (SANITIZE if sanitize else []) + (["-DMOE_DEBUG_CHECKS"] if debug_checks else [])
    os.makedirs(build_dir, exist_ok=True)
    hipcc = _hipcc()
    srcs = [s for s in SOURCES if os.path.exists(os.path.join(CSRC, s))]
    jobs = min(len(srcs), max(1, min(8, os.cpu_count() or 1)))
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, hipcc, extra, build_dir), srcs))
    tmp = lib + ".tmp"
    cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp,
           "-Wl,-rpath,/opt/rocm/lib"]
    if sanitize:
        # host-only link: clang++ with the shared sanitizer runtimes and the
        # HIP runtime the objects' host code calls
        cmd = [_clangxx(), "-shared", "-fPIC", *objs, "-o", tmp, "-L/opt/rocm/lib", "-lamdhip64",
               "-Wl,-rpath,/opt/rocm/lib", "-shared-libsan", *_SAN_LINK]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, lib)
    if verbose:
        print(f"built {lib}")
    return lib


if __name__ == "__main__":
    build(verbose=True, sanitize="--sanitize" in sys.argv[1:], debug_checks="--debug-checks" in sys.argv[1:])
