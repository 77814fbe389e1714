"""Build libharp.so in-tree for gfx950 with hipcc.

    python rotated_bit_amd/build.py          # or  __graft_entry__.build()

(Run it as a file: importing the package loads the library.)

Every HIP source is compiled with packed-FP32 instructions disabled
(``-Xclang -target-feature -Xclang -packed-fp32-ops``).  The argument checks
(validate.cpp) and the offline mixed-radix block expansion
(mixed_expand.cpp) are plain C++ built with g++, so they carry no HIP
dependency.  The library is written next to this file.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libharp.so")
ARCH = os.environ.get("HARP_OFFLOAD_ARCH", "gfx950")

HIP_SOURCES = ["rotate.hip", "mixed.hip", "gemv.hip", "gemv_f4.hip", "gemv_mc.hip", "skinny.hip", "skinny_wide.hip", "gemm.hip",
               "dequant.hip", "prep.hip", "chain.hip", "harp_api.cpp"]
CXX_SOURCES = ["validate.cpp", "mixed_expand.cpp"]

# Code object v5: loadable by the HIP runtime that ships inside torch, which
# is the runtime the library shares with its caller (one runtime per process).
HIP_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-mcode-object-version=5",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
]
CXX_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libharp)")


def _run(cmd):
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in p.stdout.splitlines()
                    if "packed-fp32-ops" not in l)   # host pass does not know it
    if p.returncode != 0:
        raise RuntimeError(f"build step failed ({p.returncode}): {' '.join(cmd)}\n{out}")
    return out


def torch_lib_dir():
    """torch's lib directory (holds the HIP runtime torch uses), or None."""
    import importlib.util
    spec = importlib.util.find_spec("torch")
    if spec is None or not spec.origin:
        return None
    d = os.path.join(os.path.dirname(spec.origin), "lib")
    return d if os.path.exists(os.path.join(d, "libamdhip64.so")) else None


def build(verbose: bool = False, jobs: int = 8) -> str:
    """Compile every source and link libharp.so; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    cc = hipcc()
    cmds = []
    objs = []
    for src in HIP_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        objs.append(obj)
        cmds.append([cc, "-c", *HIP_FLAGS, "-o", obj, os.path.join(CSRC, src)])
    for src in CXX_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        objs.append(obj)
        cmds.append(["g++", "-c", *CXX_FLAGS, "-o", obj, os.path.join(CSRC, src)])
    with ThreadPoolExecutor(max_workers=max(1, min(jobs, len(cmds)))) as ex:
        outs = list(ex.map(_run, cmds))
    if verbose:
        for c, o in zip(cmds, outs):
            print(" ".join(c))
            if o.strip():
                print(o)
    tmp = LIB + ".tmp"
    link = [cc, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-mcode-object-version=5"]
    tl = torch_lib_dir()
    if tl:
        # Resolve libamdhip64.so.7 to torch's copy when loaded on its own;
        # when torch is already loaded the loader reuses its copy (same soname).
        link += [f"-L{tl}", f"-Wl,-rpath,{tl}"]
    _run(link + ["-o", tmp, *objs])
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
