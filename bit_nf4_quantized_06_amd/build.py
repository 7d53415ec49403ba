"""Build libqlora_nf4.so in-tree for gfx950.

Kernel translation units are compiled by hipcc; host-only units by g++.  The
library is linked against the HIP runtime that PyTorch ships (torch/lib), so
a process that has imported torch runs torch and this library on one HIP
runtime and torch's streams can be passed straight through the C ABI.
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
BUILD = os.path.join(PKG, "_build")
LIB_NAME = "libqlora_nf4.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)

HIP_SOURCES = ["quantize.hip", "lora.hip", "gemm.hip", "gemv.hip", "merge.hip", "adamw.hip",
               "dropout.hip", "noalloc.hip"]
HOST_SOURCES = ["abi.cpp", "validate.cpp"]
ARCH = "gfx950"


def _rocm_path() -> str:
    return os.environ.get("ROCM_PATH", "/opt/rocm")


def _torch_lib_dir() -> str:
    import importlib.util
    spec = importlib.util.find_spec("torch")
    if spec is None or spec.origin is None:
        raise RuntimeError("torch is required: the library links torch's HIP runtime")
    return os.path.join(os.path.dirname(spec.origin), "lib")


def hipcc_flags() -> list:
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
        "-ffp-contract=off",                        # every rounding is explicit
        "-mcode-object-version=5",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wno-unused-command-line-argument",
        f"-I{INCLUDE}", f"-I{CSRC}",
    ]


def host_flags() -> list:
    return ["-O2", "-std=c++17", "-fPIC", "-Wall", "-D__HIP_PLATFORM_AMD__",
            f"-I{_rocm_path()}/include", f"-I{INCLUDE}", f"-I{CSRC}"]


def _run(cmd: list, verbose: bool) -> None:
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout)
        raise RuntimeError(f"build step failed ({res.returncode}): {' '.join(cmd)}")
    elif verbose and res.stdout.strip():
        print(res.stdout)


def build(verbose: bool = False, jobs: int = 4) -> str:
    """Compile every source and link the shared library; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    hipcc = os.path.join(_rocm_path(), "bin", "hipcc")
    steps = []
    objs = []
    for src in HIP_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        steps.append([hipcc, *hipcc_flags(), "-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    for src in HOST_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        steps.append(["g++", *host_flags(), "-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        list(ex.map(lambda c: _run(c, verbose), steps))
    tlib = _torch_lib_dir()
    tmp = LIB_PATH + ".tmp"
    _run(["g++", "-shared", "-o", tmp, *objs, f"-L{tlib}", "-l:libamdhip64.so",
          f"-Wl,-rpath,{tlib}", "-Wl,--no-undefined"], verbose)
    shutil.move(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
