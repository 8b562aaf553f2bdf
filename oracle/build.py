"""Compile the CPU oracle (oracle.c) into liboracle.so with gcc.

Test infrastructure: building the checker is not using it.  Flags keep IEEE
binary32 semantics: no -ffast-math, no floating-point contraction.
"""
import pathlib
import subprocess

HERE = pathlib.Path(__file__).resolve().parent
SRC = HERE / "oracle.c"
LIB = HERE / "liboracle.so"

CFLAGS = ["-O1", "-std=c11", "-Wall", "-Wextra", "-Werror", "-ffp-contract=off",
          "-fno-fast-math", "-fPIC", "-shared"]


def build(verbose: bool = False) -> pathlib.Path:
    tmp = LIB.with_suffix(".so.tmp")
    cmd = ["gcc", *CFLAGS, str(SRC), "-o", str(tmp)]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    tmp.replace(LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
