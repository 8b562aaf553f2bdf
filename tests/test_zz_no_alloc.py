"""GPU tests of ar_packet_fused_noalloc, the fused packet share that keeps
its control block and scratch in the library's static device array: its
outputs equal those of ar_packet_fused_epoch (caller-allocated scratch) and
the oracle's, call after call, with the shape changing between calls."""
from __future__ import annotations

import numpy as np
import pytest
import torch

from allreduce_reduction_way_amd import ar, inputs
from gpu_util import DEV, announce, ctrl_block, ctrl_status, to_dev, to_host
from oracle import oracle as O

pytestmark = pytest.mark.gpu


def _max_n(P: int) -> int:
    """Largest n whose scratch fits the static array (host-side helper rule)."""
    def need(n):
        per = -(-ar.ar_packet_scratch_bytes(P, n) // 256) * 256
        return 256 + P * per
    lo, hi = 0, 1 << 24
    while lo < hi:
        mid = (lo + hi + 1) // 2
        if need(mid) <= ar.AR_NOALLOC_SCRATCH_BYTES:
            lo = mid
        else:
            hi = mid - 1
    return lo


def _status_word() -> torch.Tensor:
    return torch.full((1,), 12345, dtype=torch.int32, device=DEV)


def _epoch_reference(d_in, P, n):
    """The existing entry point on caller-allocated scratch and control block."""
    nb = ar.ar_packet_scratch_bytes(P, n)
    scratch = [torch.zeros(nb, dtype=torch.uint8, device=DEV) for _ in range(P)]
    ctrl = ctrl_block()
    outs = [torch.full((n,), 0x5A5A, dtype=torch.int16, device=DEV) for _ in range(P)]
    ar.ar_packet_fused_epoch(d_in, scratch, outs, ctrl)
    torch.cuda.synchronize()
    assert ctrl_status(ctrl) == 0
    return [to_host(o) for o in outs]


def _noalloc(d_in, P, n, max_spins=0):
    outs = [torch.full((n,), 0x5A5A, dtype=torch.int16, device=DEV) for _ in range(P)]
    st = _status_word()
    ar.ar_packet_fused_noalloc(d_in, outs, st, max_spins=max_spins)
    torch.cuda.synchronize()
    return [to_host(o) for o in outs], int(st.item())


def _check_call(P, n, seed):
    announce(f"noalloc P={P} n={n} seed={seed}")
    xs = inputs.make_inputs("uniform", P, n, seed)
    d_in = [to_dev(x) for x in xs]
    got, status = _noalloc(d_in, P, n)
    assert status == ar.AR_OK
    ref = _epoch_reference(d_in, P, n)
    y = O.oneshot_sum(xs)
    for r in range(P):
        assert np.array_equal(got[r], ref[r]), f"rank {r} differs from ar_packet_fused_epoch"
        assert np.array_equal(got[r], y), f"rank {r} differs from the oracle"


def test_two_calls_second_smaller():
    # several chunks plus a ragged tail, then a smaller call on the same array
    _check_call(8, 512 * 1024 + 37, seed=11)
    _check_call(8, 4096 + 5, seed=12)


def test_shape_changes_between_calls_and_maximum_size():
    P = 8
    nmax = _max_n(P)
    _check_call(P, nmax, seed=21)            # the largest call the array holds
    _check_call(3, 100_003, seed=22)         # other P, other layout over older packets
    _check_call(P, 1, seed=23)               # a single element
    _check_call(2, 128 * 2 * 3 + 1, seed=24)


def test_too_large_is_rejected_before_the_gpu():
    P = 8
    n = _max_n(P) + 1
    d = [torch.empty(n, dtype=torch.int16, device=DEV) for _ in range(P)]
    o = [torch.empty(n, dtype=torch.int16, device=DEV) for _ in range(P)]
    with pytest.raises(ar.ArError) as ei:
        ar.ar_packet_fused_noalloc(d, o, _status_word())
    assert ei.value.code == ar.AR_ENOSPACE


def test_timeout_is_reported_and_cleared_for_the_next_call():
    """A one-poll bound may make some wait run out (reported as AR_ETIMEDOUT,
    outputs undefined); the next call must start from a clear status and give
    the exact result."""
    P, n = 8, 64 * 1024 + 3
    xs = inputs.make_inputs("uniform", P, n, 31)
    d_in = [to_dev(x) for x in xs]
    announce(f"noalloc one-poll bound P={P} n={n}")
    _, status = _noalloc(d_in, P, n, max_spins=1)
    assert status in (ar.AR_OK, ar.AR_ETIMEDOUT)
    announce(f"noalloc after the one-poll call P={P} n={n}")
    got, status = _noalloc(d_in, P, n)
    assert status == ar.AR_OK
    y = O.oneshot_sum(xs)
    assert all(np.array_equal(g, y) for g in got)
