"""Build libar.so: the HIP sources under csrc/ compiled for gfx950 with hipcc.

Flags: -O3 for gfx950 only; packed-fp32 instructions disabled on the device
pass (the host pass warns that it does not know the feature, which is
harmless); no fast-math and no denormal flushing, so binary32 adds keep IEEE
semantics (round to nearest even, subnormals preserved).
"""
from __future__ import annotations

import pathlib
import subprocess

PKG = pathlib.Path(__file__).resolve().parent
ROOT = PKG.parent
CSRC = PKG / "csrc"
LIB = PKG / "libar.so"
RESOURCES = PKG / "libar.resources.txt"   # per-kernel register/scratch report of the last build
SOURCES = ["host.hip", "reduce.hip", "packet.hip", "probe.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Wall", "-Wextra",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fno-gpu-flush-denormals-to-zero",
]


def build(verbose: bool = False) -> pathlib.Path:
    tmp = LIB.with_suffix(".so.tmp")
    cmd = ["hipcc", *HIPCC_FLAGS, "-Rpass-analysis=kernel-resource-usage",
           f"-I{ROOT / 'include'}", f"-I{CSRC}", *[str(CSRC / s) for s in SOURCES], "-o", str(tmp)]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "'-packed-fp32-ops' is not a recognized feature for this target"
    lines = (res.stdout + res.stderr).splitlines()
    report = [l.split("remark: ", 1)[1].replace(" [-Rpass-analysis=kernel-resource-usage]", "")
              for l in lines if "remark: " in l and "kernel-resource-usage" in l]
    msgs = [l for l in lines if noise not in l and "kernel-resource-usage" not in l
            and not l.startswith(" ") and l.strip() != "|"]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs))
    tmp.replace(LIB)
    RESOURCES.write_text("\n".join(report) + "\n")
    return LIB


def build_c_program(src: pathlib.Path, exe: pathlib.Path, verbose: bool = False) -> pathlib.Path:
    """Compile a plain C program that calls libar.so through include/ar.h
    (gcc, C11, no HIP compiler): linked against libar.so and the HIP runtime,
    with an rpath to the library beside it in this package."""
    rocm = pathlib.Path("/opt/rocm")
    rel = pathlib.Path(*[".."] * len(exe.resolve().parent.relative_to(ROOT).parts)) / PKG.name
    cmd = ["gcc", "-std=c11", "-O2", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           f"-I{rocm / 'include'}", f"-I{ROOT / 'include'}", str(src), "-o", str(exe),
           f"-L{PKG}", "-lar", f"-L{rocm / 'lib'}", "-lamdhip64",
           f"-Wl,-rpath,$ORIGIN/{rel}", f"-Wl,-rpath,{rocm / 'lib'}"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    return exe


if __name__ == "__main__":
    print(build(verbose=True))
