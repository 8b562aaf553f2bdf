"""The C ABI driven from plain C (tests/c_abi_check.c): raw hipMalloc'd
device pointers, one stream, no PyTorch in the call path.  The program checks
that every entry point agrees with write mode (the no-alloc packet share
where it fits the library's static scratch, AR_ENOSPACE where it does not);
this test checks its result against the CPU oracle."""
from __future__ import annotations

import pathlib
import subprocess

import numpy as np
import pytest

from allreduce_reduction_way_amd import inputs as I
from gpu_util import announce
from oracle import oracle as O

pytestmark = pytest.mark.gpu

EXE = pathlib.Path(__file__).resolve().parent / "c_abi_check"


@pytest.mark.parametrize("P,n", [(8, 440 * 5120), (3, 1001), (2, 7)])
def test_plain_c_caller_matches_oracle(tmp_path, P, n):
    if not EXE.exists():
        raise FileNotFoundError(f"{EXE} is not built: run the package build")
    xs = I.make_inputs("uniform", P, n, seed=P + n)
    src, dst = tmp_path / "in.bin", tmp_path / "out.bin"
    np.concatenate(xs).astype("<u2").tofile(src)
    announce(f"c_abi_check P={P} n={n}")
    res = subprocess.run([str(EXE), str(P), str(n), str(src), str(dst)], capture_output=True,
                         text=True, timeout=60)
    assert res.returncode == 0, res.stderr
    got = np.fromfile(dst, dtype="<u2")
    assert np.array_equal(got, O.oneshot_sum(xs))
