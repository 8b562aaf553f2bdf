"""Every peer count P = 2..8 through every entry point (and IEEE special
values through every path): each P is its own
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


def _special_inputs(P, n, seed):
    """Arbitrary bit patterns with NaN, +-Inf, +-0, subnormals and extremes
    planted: the packet path reduces through its own word routine."""
    rng = np.random.default_rng(seed)
    xs = [rng.integers(0, 1 << 16, n, dtype=np.uint32).astype(np.uint16) for _ in range(P)]
    specials = np.array([0x0000, 0x8000, 0x7F80, 0xFF80, 0x7FC0, 0xFFC1, 0x0001, 0x8001, 0x007F,
                         0x7F7F, 0xFF7F, 0x3F80, 0xBF80], dtype=np.uint16)
    for x in xs:
        idx = rng.integers(0, n, max(1, n // 6))
        x[idx] = specials[rng.integers(0, specials.size, idx.size)]
    return xs


@pytest.mark.parametrize("P", [3, 8])
def test_special_values_through_every_path(P):
    n = _n(P)
    xs = _special_inputs(P, n, seed=900 + P)
    d_in = [to_dev(x) for x in xs]
    y = O.oneshot_sum(xs)

    announce(f"specials write_bcast P={P}")
    outs = [torch.zeros(n, dtype=torch.int16, device=DEV) for _ in range(P)]
    ar.ar_oneshot_write_bcast(d_in, outs)
    torch.cuda.synchronize()
    for t in outs:
        assert np.array_equal(to_host(t), y)

    announce(f"specials twoshot P={P}, every owner")
    two = [torch.zeros(n, dtype=torch.int16, device=DEV) for _ in range(P)]
    for r in range(P):
        ar.ar_twoshot_share(d_in, two, r)
    torch.cuda.synchronize()
    for t in two:
        assert np.array_equal(to_host(t), y)

    nb = O.packet_scratch_bytes(P, n)
    for path in ("fused", "three_op"):
        scratch = [torch.zeros(nb, dtype=torch.uint8, device=DEV) for _ in range(P)]
        ctrl = ctrl_block()
        outs = [torch.zeros(n, dtype=torch.int16, device=DEV) for _ in range(P)]
        announce(f"specials packet {path} P={P}")
        if path == "fused":
            ar.ar_packet_fused(d_in, scratch, outs, 1, ctrl)
        else:
            ar.ar_packet_send(d_in, scratch, 1, n=n)
            ar.ar_packet_recv_reduce_send(scratch, n, 1, ctrl)
            ar.ar_packet_recv(scratch, outs, 1, ctrl, n=n)
        torch.cuda.synchronize()
        assert ctrl_status(ctrl) == 0
        want, images = O.packet_fused(xs, 1, [np.zeros(nb, np.uint8) for _ in range(P)])
        for r in range(P):
            assert np.array_equal(to_host(outs[r]), want[r]), (path, r)
            assert np.array_equal(scratch[r].cpu().numpy(), images[r]), (path, r)


@pytest.mark.parametrize("P", [2, 8])
@pytest.mark.parametrize("n", [1, 2, 3, 5, 127, 128 * 8 - 1])
def test_tiny_sizes_every_path(P, n):
    """Degenerate sizes: fewer elements than one 128-element slice unit per
    rank (L = 0: the last rank owns everything), a single packet, and a
    partial last packet."""
    xs = I.make_inputs("uniform", P, n, seed=1200 + n + P)
    d_in = [to_dev(x) for x in xs]
    y = O.oneshot_sum(xs)
    announce(f"tiny n={n} P={P}: write_bcast, two-shot, packets")
    outs = [torch.zeros(n, dtype=torch.int16, device=DEV) for _ in range(P)]
    ar.ar_oneshot_write_bcast(d_in, outs)
    two = [torch.zeros(n, dtype=torch.int16, device=DEV) for _ in range(P)]
    for r in range(P):
        ar.ar_twoshot_share(d_in, two, r)
    torch.cuda.synchronize()
    for t in outs + two:
        assert np.array_equal(to_host(t), y)
    nb = O.packet_scratch_bytes(P, n)
    scratch = [torch.zeros(nb, dtype=torch.uint8, device=DEV) for _ in range(P)]
    ctrl = ctrl_block()
    pk_out = [torch.zeros(n, dtype=torch.int16, device=DEV) for _ in range(P)]
    ar.ar_packet_fused(d_in, scratch, pk_out, 1, ctrl)
    torch.cuda.synchronize()
    assert ctrl_status(ctrl) == 0
    want, images = O.packet_fused(xs, 1, [np.zeros(nb, np.uint8) for _ in range(P)])
    for r in range(P):
        assert np.array_equal(to_host(pk_out[r]), want[r])
        assert np.array_equal(scratch[r].cpu().numpy(), images[r])
