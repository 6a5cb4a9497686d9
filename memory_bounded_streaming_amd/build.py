"""Build libcqsa.so (gfx950) in-tree from csrc/.

Host C++ (planner, engine, C ABI) is compiled with ROCm's clang++, the HIP kernels
with hipcc for gfx950, and everything is linked into
``memory_bounded_streaming_amd/libcqsa.so`` next to this file.

    python -m memory_bounded_streaming_amd.build
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "libcqsa.so")
OBJ = os.path.join(ROOT, "_build")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
ARCH = "gfx950"

HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 VALU forms are kept out of all device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]
HOST_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-D__HIP_PLATFORM_AMD__", f"-I{ROCM}/include", "-Wall", "-Wextra"]


def _run(cmd):
    proc = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(line for line in proc.stdout.splitlines() if "not a recognized feature" not in line)
    if proc.returncode != 0:
        raise RuntimeError(f"build step failed ({proc.returncode}): {' '.join(cmd)}\n{out}")
    return out


def _check_stubs(lib):
    """Every kernel launch stub the host code references must be defined in the library."""
    nm = subprocess.run(["nm", lib], stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True).stdout
    missing = [ln.split()[-1] for ln in nm.splitlines() if ln.split()[:1] == ["U"] and "__device_stub__" in ln]
    if missing:
        raise RuntimeError("kernel launch stubs missing from the host pass: " + ", ".join(missing))


def build(verbose: bool = False) -> str:
    """Compile every source and link libcqsa.so; returns its path."""
    os.makedirs(OBJ, exist_ok=True)
    hipcc = os.path.join(ROCM, "bin", "hipcc")
    cxx = os.path.join(ROCM, "llvm", "bin", "clang++")
    jobs = []
    for name in sorted(os.listdir(CSRC)):
        src = os.path.join(CSRC, name)
        obj = os.path.join(OBJ, name + ".o")
        if name.endswith(".hip"):
            jobs.append([hipcc, *HIP_FLAGS, "-c", src, "-o", obj])
        elif name.endswith(".cpp"):
            jobs.append([cxx, *HOST_FLAGS, "-c", src, "-o", obj])
    with ThreadPoolExecutor(max_workers=min(8, len(jobs))) as pool:
        logs = list(pool.map(_run, jobs))
    objs = [j[-1] for j in jobs]
    tmp = OUT + ".tmp"
    logs.append(_run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs,
                      f"-L{ROCM}/lib", "-lamdhip64", f"-Wl,-rpath,{ROCM}/lib"]))
    _check_stubs(tmp)
    os.replace(tmp, OUT)
    if verbose:
        for log in logs:
            if log.strip():
                print(log)
    return OUT


if __name__ == "__main__":
    path = build(verbose=True)
    print(path)
    sys.exit(0)
