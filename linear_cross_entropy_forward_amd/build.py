"""Build libcce.so (HIP, gfx950) in-tree with hipcc.

Run as a script or call build().  The library is placed next to this file so
that it travels with the source tree.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libcce.so")
SOURCES = ["cce_kernels.hip", "cce_api.hip", "cce_noalloc.hip"]
ARCH = os.environ.get("CCE_OFFLOAD_ARCH", "gfx950")


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set HIPCC or install ROCm)")


def build(verbose: bool = False) -> str:
    """Compile every HIP source (one hipcc process per source, in parallel)
    and link them into libcce.so; returns its path."""
    flags = ["-O3", f"--offload-arch={ARCH}", "-std=c++20", "-fPIC",
             # keep the compiler from forming packed fp32 ALU ops (v_pk_*_f32)
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wno-unused-command-line-argument"]
    objs, procs = [], []
    for src in SOURCES:
        obj = os.path.join(CSRC, src + f".{os.getpid()}.o")
        cmd = [hipcc()] + flags + ["-c", "-o", obj, os.path.join(CSRC, src)]
        if verbose:
            print(" ".join(cmd), flush=True)
        objs.append(obj)
        procs.append(subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True))
    errs, failed = [], False
    for p in procs:
        out = p.communicate()[0]
        errs += [l for l in out.splitlines() if "packed-fp32-ops" not in l and l.strip()]
        failed |= p.returncode != 0
    tmp = LIB + ".tmp"
    try:
        if failed:
            raise RuntimeError("hipcc failed:\n" + "\n".join(errs))
        r = subprocess.run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs,
                           capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"link failed ({r.returncode}):\n{r.stdout}{r.stderr}")
    finally:
        for o in objs:
            if os.path.exists(o):
                os.remove(o)
    if verbose and errs:
        print("\n".join(errs))
    os.replace(tmp, LIB)
    return LIB


ROOT = os.path.dirname(HERE)
C_CHECK_SRC = os.path.join(ROOT, "tests", "c_abi", "cce_abi_check.c")
C_CHECK_BIN = os.path.join(ROOT, "tests", "c_abi", "cce_abi_check")


def build_c_check(out: str = C_CHECK_BIN) -> str:
    """Compile the plain-C caller of the ABI (tests/c_abi) against libcce.so
    with the host C compiler; returns the executable's path."""
    cc = os.environ.get("CC") or shutil.which("gcc") or shutil.which("cc")
    if not cc:
        raise RuntimeError("no C compiler for the C ABI check")
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    cmd = [cc, "-O2", "-std=c11", "-Wall", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(rocm, "include"), C_CHECK_SRC,
           "-L", HERE, "-lcce", "-L", os.path.join(rocm, "lib"), "-lamdhip64", "-lm",
           "-Wl,-rpath,$ORIGIN/../../linear_cross_entropy_forward_amd", f"-Wl,-rpath,{HERE}",
           f"-Wl,-rpath,{os.path.join(rocm, 'lib')}", "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"C ABI check failed to build ({r.returncode}):\n{r.stdout}{r.stderr}")
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
    print(build_c_check())
