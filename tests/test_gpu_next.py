"""GPU parity of the widened rows: the one-shot reduce-scatter sibling, the
unfused three-operation packet decomposition, and the fused packet kernel
whose flag lives on the device (including HIP-graph capture and replay),
each bit-exact against the CPU oracle."""
from __future__ import annotations

import time

import numpy as np
import pytest
import torch

from allreduce_reduction_way_amd import ar, inputs as I
from gpu_util import DEV, Guarded, announce, ctrl_block, ctrl_status, to_dev, to_host
from oracle import oracle as O

pytestmark = pytest.mark.gpu


def _scratch(P, n):
    return [torch.zeros(O.packet_scratch_bytes(P, n), dtype=torch.uint8, device=DEV)
            for _ in range(P)]


def _zero_images(P, n):
    return [np.zeros(O.packet_scratch_bytes(P, n), np.uint8) for _ in range(P)]


def _check_images(scratch, images, tag):
    for r, t in enumerate(scratch):
        assert np.array_equal(t.cpu().numpy(), images[r]), (tag, r)


# ------------------------------------------------------------ reduce-scatter

@pytest.mark.parametrize("P", [2, 3, 4, 8])
@pytest.mark.parametrize("rc", [1, 7, 100, 4096 + 3, 281600])
def test_reduce_scatter_every_rank(P, rc):
    xs = I.make_inputs("uniform", P, P * rc, seed=rc % 11)
    d_in = [to_dev(x) for x in xs]
    for r in range(P):
        out = Guarded(rc)
        announce(f"reduce_scatter P={P} rc={rc} rank={r}")
        ar.ar_reduce_scatter_share(d_in, out.view, r)
        torch.cuda.synchronize()
        assert np.array_equal(out.host(), O.reduce_scatter(xs, r)), r
        assert out.guards_intact()


def test_reduce_scatter_in_place_and_misaligned():
    P, rc = 8, 5003
    xs = I.make_inputs("uniform", P, P * rc, seed=2)
    ins = [Guarded(P * rc, shift=3, init=x) for x in xs]
    r = 5
    want = O.reduce_scatter(xs, r)
    out = ins[r].view[r * rc:(r + 1) * rc]          # rank r's own block of its own input
    announce("reduce_scatter in place, misaligned")
    ar.ar_reduce_scatter_share([g.view for g in ins], out, r)
    torch.cuda.synchronize()
    assert np.array_equal(to_host(out), want)
    host = ins[r].host()
    assert np.array_equal(host[:r * rc], xs[r][:r * rc])
    assert np.array_equal(host[(r + 1) * rc:], xs[r][(r + 1) * rc:])
    assert ins[r].guards_intact()


# -------------------------------------------------- three-op decomposition

def _three_op(d_in, scratch, outs, f, ctrl, lo=0, hi=None, stream=None, n=None):
    n = d_in[0].numel() if n is None else n
    ar.ar_packet_send(d_in, scratch, f, rank_lo=lo, rank_hi=hi, n=n, stream=stream)
    ar.ar_packet_recv_reduce_send(scratch, n, f, ctrl, rank_lo=lo, rank_hi=hi, stream=stream)
    ar.ar_packet_recv(scratch, outs, f, ctrl, rank_lo=lo, rank_hi=hi, n=n, stream=stream)


@pytest.mark.parametrize("P,n", [(8, 1024 * 3 + 5), (8, 1000), (3, 777), (4, 4096 * 5 + 130),
                                 (8, 512 * 7168)])
def test_three_op_matches_oracle_over_three_calls(P, n):
    scratch = _scratch(P, n)
    images = _zero_images(P, n)
    ctrl = ctrl_block()
    for call in range(3):
        f = call + 1
        xs = I.make_inputs("uniform", P, n, seed=call)
        outs = [torch.full((n,), 0x1111, dtype=torch.int16, device=DEV) for _ in range(P)]
        announce(f"three-op P={P} n={n} flag={f}")
        _three_op([to_dev(x) for x in xs], scratch, outs, f, ctrl)
        torch.cuda.synchronize()
        assert ctrl_status(ctrl) == 0
        want, images = O.packet_fused(xs, f, images)
        for r in range(P):
            assert np.array_equal(to_host(outs[r]), want[r]), (call, r)
        _check_images(scratch, images, call)


def test_fused_and_three_op_interleave_bit_for_bit():
    P, n = 8, 8192 * 5 + 77
    scratch = _scratch(P, n)
    images = _zero_images(P, n)
    ctrl = ctrl_block()
    for call, how in enumerate(["fused", "three-op", "fused", "three-op"]):
        f = call + 1
        xs = I.make_inputs("uniform", P, n, seed=10 + call)
        d_in = [to_dev(x) for x in xs]
        outs = [torch.zeros(n, dtype=torch.int16, device=DEV) for _ in range(P)]
        announce(f"interleave call {call} {how}")
        if how == "fused":
            ar.ar_packet_fused(d_in, scratch, outs, f, ctrl)
        else:
            _three_op(d_in, scratch, outs, f, ctrl)
        torch.cuda.synchronize()
        assert ctrl_status(ctrl) == 0
        want, images = O.packet_fused(xs, f, images)
        for r in range(P):
            assert np.array_equal(to_host(outs[r]), want[r]), (call, r)
        _check_images(scratch, images, call)


def test_three_op_receiver_on_another_stream():
    """Producers (send, recv-reduce-send) are queued on stream A, the
    receiver on stream B right after.  Whether the runtime runs the two
    streams concurrently (the receiver then waits on flags) or one after the
    other, every wait is on work queued earlier, so the call completes."""
    P, n = 8, 8192 * 3 + 1
    xs = I.make_inputs("uniform", P, n, seed=31)
    d_in = [to_dev(x) for x in xs]
    scratch = _scratch(P, n)
    outs = [torch.zeros(n, dtype=torch.int16, device=DEV) for _ in range(P)]
    ctrl_a, ctrl_b = ctrl_block(), ctrl_block()
    s_a, s_b = torch.cuda.Stream(), torch.cuda.Stream()
    torch.cuda.synchronize()
    announce("three-op: producers on stream A, receiver on stream B")
    ar.ar_packet_send(d_in, scratch, 1, n=n, stream=s_a)
    ar.ar_packet_recv_reduce_send(scratch, n, 1, ctrl_a, stream=s_a)
    ar.ar_packet_recv(scratch, outs, 1, ctrl_b, n=n, stream=s_b)
    torch.cuda.synchronize()
    assert ctrl_status(ctrl_a) == 0 and ctrl_status(ctrl_b) == 0
    y = O.oneshot_sum(xs)
    for t in outs:
        assert np.array_equal(to_host(t), y)


# ------------------------------------------------------- device-resident flag

def _epoch(ctrl):
    w = ctrl.view(torch.int32).cpu().numpy()
    return int(w[1]), int(w[2])


@pytest.mark.parametrize("P,n", [(8, 4096 * 3 + 9), (4, 1000), (8, 512 * 7168)])
def test_epoch_flag_sequence_matches_oracle(P, n):
    scratch = _scratch(P, n)
    images = _zero_images(P, n)
    ctrl = ctrl_block()
    for call in range(3):
        xs = I.make_inputs("uniform", P, n, seed=40 + call)
        outs = [torch.zeros(n, dtype=torch.int16, device=DEV) for _ in range(P)]
        announce(f"epoch call {call} P={P} n={n}")
        ar.ar_packet_fused_epoch([to_dev(x) for x in xs], scratch, outs, ctrl)
        torch.cuda.synchronize()
        assert ctrl_status(ctrl) == 0
        assert _epoch(ctrl) == (call + 1, 0)
        want, images = O.packet_fused(xs, call + 1, images)
        for r in range(P):
            assert np.array_equal(to_host(outs[r]), want[r]), (call, r)
        _check_images(scratch, images, call)


def test_epoch_flag_graph_replay_with_changing_inputs():
    """One fused call captured into a HIP graph and replayed: the flag comes
    from the device, so each replay uses the next flag; the inputs are
    rewritten eagerly before each replay and every replay is checked."""
    P, n = 8, 8192 * 7 + 3
    d_in = [torch.zeros(n, dtype=torch.int16, device=DEV) for _ in range(P)]
    outs = [torch.zeros(n, dtype=torch.int16, device=DEV) for _ in range(P)]
    scratch = _scratch(P, n)
    ctrl = ctrl_block()
    images = _zero_images(P, n)

    xs = I.make_inputs("uniform", P, n, seed=50)
    for t, x in zip(d_in, xs):
        t.copy_(to_dev(x))
    announce("epoch graph: eager warm-up call (flag 1)")
    ar.ar_packet_fused_epoch(d_in, scratch, outs, ctrl)
    torch.cuda.synchronize()
    want, images = O.packet_fused(xs, 1, images)
    for r in range(P):
        assert np.array_equal(to_host(outs[r]), want[r])

    g = torch.cuda.CUDAGraph()
    announce("epoch graph: capture")
    with torch.cuda.graph(g):
        ar.ar_packet_fused_epoch(d_in, scratch, outs, ctrl)
    torch.cuda.synchronize()
    assert _epoch(ctrl) == (1, 0)     # capture launched nothing

    for rep in range(4):
        f = rep + 2
        xs = I.make_inputs("uniform", P, n, seed=60 + rep)
        for t, x in zip(d_in, xs):
            t.copy_(to_dev(x))
        for t in outs:
            t.fill_(0x2222)
        torch.cuda.synchronize()
        announce(f"epoch graph: replay {rep} (flag {f})")
        g.replay()
        torch.cuda.synchronize()
        assert ctrl_status(ctrl) == 0
        assert _epoch(ctrl) == (f, 0)
        want, images = O.packet_fused(xs, f, images)
        for r in range(P):
            assert np.array_equal(to_host(outs[r]), want[r]), (rep, r)
        _check_images(scratch, images, rep)


def test_three_op_two_byte_aligned_buffers():
    P, n = 4, 4096 * 5 + 3
    xs = I.make_inputs("uniform", P, n, seed=91)
    ins = [Guarded(n, shift=1, init=x) for x in xs]
    outs = [Guarded(n, shift=3) for _ in range(P)]
    scratch = _scratch(P, n)
    ctrl = ctrl_block()
    announce("three-op, 2-byte-aligned inputs and outputs")
    _three_op([g.view for g in ins], scratch, [o.view for o in outs], 1, ctrl, n=n)
    torch.cuda.synchronize()
    assert ctrl_status(ctrl) == 0
    want, img = O.packet_fused(xs, 1, _zero_images(P, n))
    for r in range(P):
        assert np.array_equal(outs[r].host(), want[r]) and outs[r].guards_intact()
    _check_images(scratch, img, 0)
