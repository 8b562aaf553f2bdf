"""Build tests/c_abi_check (a plain C program that drives libar.so through
include/ar.h with raw device pointers).  Test helper; built by build()."""
from __future__ import annotations

import pathlib
import subprocess

TESTS = pathlib.Path(__file__).resolve().parent
ROOT = TESTS.parent
SRC = TESTS / "c_abi_check.c"
EXE = TESTS / "c_abi_check"
ROCM = pathlib.Path("/opt/rocm")


def build(verbose: bool = False) -> pathlib.Path:
    lib_dir = ROOT / "allreduce_reduction_way_amd"
    cmd = ["gcc", "-std=c11", "-O2", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           f"-I{ROCM / 'include'}", f"-I{ROOT / 'include'}", str(SRC), "-o", str(EXE),
           f"-L{lib_dir}", "-lar", f"-L{ROCM / 'lib'}", "-lamdhip64",
           "-Wl,-rpath,$ORIGIN/../allreduce_reduction_way_amd", f"-Wl,-rpath,{ROCM / 'lib'}"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    return EXE


if __name__ == "__main__":
    print(build(verbose=True))
