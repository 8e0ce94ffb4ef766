"""Compile the library ``libfa_fwd.so``: the HIP sources (``csrc/fa_fwd.hip``, ``csrc/fa_bwd.hip``) for gfx950
with hipcc, and the host CPU variant (``csrc/fa_cpu.cpp``) with the system C++ compiler.

The library is built in-tree, next to this file, so it travels with the source
tree. ``build()`` always recompiles.
"""
import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRCS = [os.path.join(HERE, "csrc", "fa_fwd.hip"), os.path.join(HERE, "csrc", "fa_bwd.hip")]
CPU_SRC = os.path.join(HERE, "csrc", "fa_cpu.cpp")
CPU_OBJ = os.path.join(HERE, "fa_cpu.o")
# -fopenmp-simd: the loops' simd pragmas only (no OpenMP runtime); the AVX2 path is chosen at run time
CXX_FLAGS = ["-O3", "-std=c++17", "-fPIC", "-fopenmp-simd", "-fno-math-errno"]
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libfa_fwd.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-shared",
    "-fPIC",
    # packed fp32 VALU ops stay off: only scalar and float2 code that hipcc lowers to plain VALU
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{INCLUDE}",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP library cannot be built")


def cxx() -> str:
    for cand in (os.environ.get("CXX"), shutil.which("g++"), shutil.which("c++")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("no host C++ compiler found")


def _run(cmd, what, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    return subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True), what


def _wait(jobs):
    for proc, what in jobs:
        _, err = proc.communicate()
        if proc.returncode != 0:
            raise RuntimeError(f"{what} failed ({proc.returncode}):\n{err}")


def build(verbose: bool = False) -> str:
    """Always recompiles: each source to an object (in parallel), then one link."""
    objs = [os.path.join(HERE, os.path.basename(src) + ".o") for src in SRCS]
    jobs = [_run([hipcc(), *[f for f in HIPCC_FLAGS if f != "-shared"], "-c", src, "-o", obj],
                 f"hipcc -c {os.path.basename(src)}", verbose) for src, obj in zip(SRCS, objs)]
    jobs.append(_run([cxx(), *CXX_FLAGS, f"-I{INCLUDE}", "-c", CPU_SRC, "-o", CPU_OBJ],
                     "C++ compile of the CPU variant", verbose))
    _wait(jobs)
    tmp = LIB + ".tmp"
    _wait([_run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, CPU_OBJ, "-lpthread", "-o", tmp],
                "hipcc link", verbose)])
    os.replace(tmp, LIB)
    for obj in objs + [CPU_OBJ]:
        os.remove(obj)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
