"""Every peer count P = 2..8 through every entry point: each P is its own
template instantiation of the kernels, so each gets a bit-exact comparison
with the CPU oracle on a ragged size that spans several chunks (and, for the
packet paths, the full scratch image after two calls with rotating flags)."""
from __future__ import annotations

import numpy as np
import pytest
import torch

from allreduce_reduction_way_amd import ar, inputs as I
from gpu_util import DEV, announce, ctrl_block, ctrl_status, to_dev, to_host
from oracle import oracle as O

pytestmark = pytest.mark.gpu

PS = [2, 3, 4, 5, 6, 7, 8]


def _n(P):
    # several 128-element slice units per rank, a ragged remainder, and more
    # than one 512-word chunk per packet slot
    return 128 * P * 9 + 8 * 1024 + 77 + P


@pytest.mark.parametrize("P", PS)
def test_reduce_entry_points_every_P(P):
    n = _n(P)
    xs = I.make_inputs("uniform", P, n, seed=300 + P)
    d_in = [to_dev(x) for x in xs]
    y = O.oneshot_sum(xs)

    announce(f"every-P oneshot P={P} n={n}")
    one = torch.zeros(n, dtype=torch.int16, device=DEV)
    ar.ar_oneshot_sum(d_in, one)
    torch.cuda.synchronize()
    assert np.array_equal(to_host(one), y)

    announce(f"every-P write_bcast P={P} n={n}")
    outs = [torch.zeros(n, dtype=torch.int16, device=DEV) for _ in range(P)]
    ar.ar_oneshot_write_bcast(d_in, outs)
    torch.cuda.synchronize()
    for t in outs:
        assert np.array_equal(to_host(t), y)

    announce(f"every-P twoshot P={P} n={n}, owners 0..P-1")
    two = [torch.full((n,), 0x0F0F, dtype=torch.int16, device=DEV) for _ in range(P)]
    prior = [np.full(n, 0x0F0F, np.uint16) for _ in range(P)]
    for r in range(P):
        ar.ar_twoshot_share(d_in, two, r)
        torch.cuda.synchronize()
        prior = O.twoshot_share(xs, r, prior)
        for t, w in zip(two, prior):
            assert np.array_equal(to_host(t), w), r

    rc = n // P
    announce(f"every-P reduce_scatter P={P} recvcount={rc}")
    blk = [x[: P * rc] for x in xs]
    for r in range(P):
        out = torch.zeros(rc, dtype=torch.int16, device=DEV)
        ar.ar_reduce_scatter_share(d_in, out, r, recvcount=rc)
        torch.cuda.synchronize()
        assert np.array_equal(to_host(out), O.reduce_scatter(blk, r)), r


@pytest.mark.parametrize("P", PS)
@pytest.mark.parametrize("path", ["fused", "three_op", "epoch"])
def test_packet_paths_every_P(P, path):
    n = _n(P)
    nb = O.packet_scratch_bytes(P, n)
    scratch = [torch.zeros(nb, dtype=torch.uint8, device=DEV) for _ in range(P)]
    images = [np.zeros(nb, np.uint8) for _ in range(P)]
    ctrl = ctrl_block()
    for call in range(2):
        f = call + 1
        xs = I.make_inputs("uniform", P, n, seed=400 + 10 * P + call)
        d_in = [to_dev(x) for x in xs]
        outs = [torch.zeros(n, dtype=torch.int16, device=DEV) for _ in range(P)]
        announce(f"every-P packet {path} P={P} n={n} call {call} (flag {f})")
        if path == "fused":
            ar.ar_packet_fused(d_in, scratch, outs, f, ctrl)
        elif path == "epoch":
            ar.ar_packet_fused_epoch(d_in, scratch, outs, ctrl)
        else:
            ar.ar_packet_send(d_in, scratch, f, n=n)
            ar.ar_packet_recv_reduce_send(scratch, n, f, ctrl)
            ar.ar_packet_recv(scratch, outs, f, ctrl, n=n)
        torch.cuda.synchronize()
        assert ctrl_status(ctrl) == 0
        want, images = O.packet_fused(xs, f, images)
        for r in range(P):
            assert np.array_equal(to_host(outs[r]), want[r]), (call, r)
        for r in range(P):
            assert np.array_equal(scratch[r].cpu().numpy(), images[r]), (call, r)
