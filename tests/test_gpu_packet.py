"""GPU parity of the LL-packet codec and the fused packet share against the
CPU oracle: outputs bit-exact, and the scratch images (every packet word and
flag) byte-exact after each call of a flag-rotating sequence.  Waits that
must fail are forced from the host (a stale flag plus a small spin bound), so
every kernel still exits on its own."""
from __future__ import annotations

import time

import numpy as np
import pytest
import torch

from allreduce_reduction_way_amd import ar, inputs as I, workloads as W
from gpu_util import DEV, Guarded, announce, ctrl_block, ctrl_status, to_dev, to_host
from oracle import oracle as O

pytestmark = pytest.mark.gpu

SMALL_SPINS = 4096      # bound for waits that are meant to time out


def _scratch(P, n, images=None):
    nbytes = O.packet_scratch_bytes(P, n)
    if images is None:
        return [torch.zeros(nbytes, dtype=torch.uint8, device=DEV) for _ in range(P)]
    return [torch.from_numpy(np.ascontiguousarray(im)).to(DEV) for im in images]


def _images(scratch):
    return [t.cpu().numpy() for t in scratch]


# ------------------------------------------------------------------ codec

@pytest.mark.parametrize("n", [1, 2, 3, 4, 5, 7, 8, 63, 64, 65, 1000, 4096 * 9 + 3])
def test_ll_encode_bytes_match_oracle(n):
    rng = np.random.default_rng(n)
    y = rng.integers(0, 1 << 16, n, dtype=np.uint32).astype(np.uint16)
    f = 0x11223344 + n
    pk = torch.zeros(16 * O.ll_packets(n) + 64, dtype=torch.uint8, device=DEV)
    announce(f"ll_encode n={n}")
    ar.ar_ll_encode(to_dev(y), pk, f)
    torch.cuda.synchronize()
    got = pk.cpu().numpy()
    assert got[16 * O.ll_packets(n):].sum() == 0          # nothing past the last packet
    assert np.array_equal(got[: 16 * O.ll_packets(n)].view(np.uint32), O.ll_encode(y, f))


@pytest.mark.parametrize("n", [1, 3, 4, 5, 999, 4096 * 9 + 3])
@pytest.mark.parametrize("shift", [0, 1])
def test_ll_decode_of_oracle_packets(n, shift):
    rng = np.random.default_rng(n + 7)
    y = rng.integers(0, 1 << 16, n, dtype=np.uint32).astype(np.uint16)
    f = 9
    pk = to_dev(O.ll_encode(y, f).view(np.uint16))
    out = Guarded(n, shift=shift)
    ctrl = ctrl_block()
    announce(f"ll_decode n={n} shift={shift}")
    ar.ar_ll_decode(pk, out.view, f, ctrl)
    torch.cuda.synchronize()
    assert ctrl_status(ctrl) == 0
    assert np.array_equal(out.host(), y) and out.guards_intact()


def test_ll_round_trip_on_device_and_stale_flag_times_out():
    n = 50001
    y = I.uniform_bf16(n, 0, 0)
    pk = torch.zeros(16 * O.ll_packets(n), dtype=torch.uint8, device=DEV)
    out = Guarded(n)
    ctrl = ctrl_block()
    announce("ll round trip flag 5")
    ar.ar_ll_encode(to_dev(y), pk, 5)
    ar.ar_ll_decode(pk, out.view, 5, ctrl)
    torch.cuda.synchronize()
    assert ctrl_status(ctrl) == 0 and np.array_equal(out.host(), y)
    announce("ll decode of stale packets (flag 5, waiting for 6), small spin bound")
    ar.ar_ll_decode(pk, out.view, 6, ctrl, max_spins=SMALL_SPINS)
    torch.cuda.synchronize()
    assert ctrl_status(ctrl) == ar.AR_ETIMEDOUT


def test_ll_decode_without_control_block():
    """ctrl = NULL: a decode of arrived packets works as usual, and one that
    can never complete still ends after its bounded polls (nothing to report
    the time-out to)."""
    n = 4096 * 3 + 1
    y = I.uniform_bf16(n, 2, 0)
    pk = to_dev(O.ll_encode(y, 9).view(np.uint16))
    out = Guarded(n)
    announce("ll decode, no control block")
    ar.ar_ll_decode(pk, out.view, 9, None)
    torch.cuda.synchronize()
    assert np.array_equal(out.host(), y) and out.guards_intact()
    announce("ll decode, no control block, stale flag, small spin bound")
    stale = Guarded(n)
    ar.ar_ll_decode(pk, stale.view, 10, None, max_spins=1024)
    torch.cuda.synchronize()                     # returns: every wait is bounded
    assert stale.guards_intact()


def test_ll_decode_half_stale_packet_times_out():
    # one packet whose second flag word is stale: the packet is not arrived
    n = 4096
    y = I.uniform_bf16(n, 1, 0)
    words = O.ll_encode(y, 3)
    words[4 * 100 + 3] = 2
    out = Guarded(n)
    ctrl = ctrl_block()
    announce("ll decode with one half-stale packet")
    ar.ar_ll_decode(to_dev(words.view(np.uint16)), out.view, 3, ctrl, max_spins=SMALL_SPINS)
    torch.cuda.synchronize()
    assert ctrl_status(ctrl) == ar.AR_ETIMEDOUT


# ---------------------------------------------------------- fused packet path

@pytest.mark.parametrize("P,n", [(8, 1024 * 3 + 5), (8, 1000), (8, 4096), (2, 513), (3, 777),
                                 (4, 4096 * 5 + 130), (8, 8192 * 9 + 1)])
def test_packet_fused_three_calls_match_oracle(P, n):
    scratch = _scratch(P, n)
    images = [np.zeros(O.packet_scratch_bytes(P, n), np.uint8) for _ in range(P)]
    ctrl = ctrl_block()
    for call in range(3):
        f = call + 1
        xs = I.make_inputs("uniform", P, n, seed=call)
        outs = [Guarded(n) for _ in range(P)]
        announce(f"packet_fused P={P} n={n} call={call} flag={f}")
        ar.ar_packet_fused([to_dev(x) for x in xs], scratch, [o.view for o in outs], f, ctrl)
        torch.cuda.synchronize()
        assert ctrl_status(ctrl) == 0
        want_outs, images = O.packet_fused(xs, f, images)
        for r in range(P):
            assert np.array_equal(outs[r].host(), want_outs[r]), (call, r)
            assert outs[r].guards_intact()
        got = _images(scratch)
        for r in range(P):
            assert np.array_equal(got[r], images[r]), (call, r)


def test_packet_fused_512x7168_p8_workload():
    w = W.PACKET_512x7168
    P, n = w.P, w.n
    scratch = _scratch(P, n)
    images = [np.zeros(O.packet_scratch_bytes(P, n), np.uint8) for _ in range(P)]
    ctrl = ctrl_block()
    d_out = [torch.zeros(n, dtype=torch.int16, device=DEV) for _ in range(P)]
    for call in range(w.calls):
        f = call + 1
        xs = I.make_inputs(w.dist, P, n, seed=call)
        announce(f"{w.name} call={call} flag={f}")
        ar.ar_packet_fused([to_dev(x) for x in xs], scratch, d_out, f, ctrl)
        torch.cuda.synchronize()
        assert ctrl_status(ctrl) == 0
        want_outs, images = O.packet_fused(xs, f, images)
        for r in range(P):
            assert np.array_equal(to_host(d_out[r]), want_outs[r]), (call, r)
        got = _images(scratch)
        for r in range(P):
            assert np.array_equal(got[r], images[r]), (call, r)


def _without_rank(images, P, n, rank):
    """The oracle's images with every packet that `rank` writes zeroed: its
    slot in every inbox and every resbox."""
    S = O.packet_slot_packets(P, n)
    out = []
    for im in images:
        im = im.copy()
        words = im.view(np.uint32).reshape(2 * P, 4 * S)
        words[rank] = 0
        words[P + rank] = 0
        out.append(im)
    return out


@pytest.mark.parametrize("P,n,rank", [(8, 4096 * 3 + 11, 3), (8, 512 * 7168, 3), (4, 777, 0)])
def test_packet_single_rank_with_staged_peers(P, n, rank):
    xs = I.make_inputs("uniform", P, n, seed=5)
    zero = [np.zeros(O.packet_scratch_bytes(P, n), np.uint8) for _ in range(P)]
    want_outs, full = O.packet_fused(xs, 1, zero)
    scratch = _scratch(P, n, _without_rank(full, P, n, rank))
    outs = [Guarded(n) for _ in range(P)]
    ctrl = ctrl_block()
    announce(f"packet single rank {rank} of P={P} n={n}")
    ar.ar_packet_fused([to_dev(x) for x in xs], scratch, [o.view for o in outs], 1, ctrl,
                       rank_lo=rank, rank_hi=rank + 1)
    torch.cuda.synchronize()
    assert ctrl_status(ctrl) == 0
    assert np.array_equal(outs[rank].host(), want_outs[rank])
    for r in range(P):
        if r != rank:
            assert (outs[r].host() == 0x5A5A).all()      # other ranks' outputs untouched
        assert outs[r].guards_intact()
    got = _images(scratch)
    for r in range(P):
        assert np.array_equal(got[r], full[r])


def test_packet_single_rank_stale_peers_time_out():
    # peers staged for flag 1; the call waits for flag 2 -> bounded wait ends
    P, n, rank = 8, 4096 * 2 + 3, 3
    xs = I.make_inputs("uniform", P, n, seed=6)
    zero = [np.zeros(O.packet_scratch_bytes(P, n), np.uint8) for _ in range(P)]
    _, full = O.packet_fused(xs, 1, zero)
    scratch = _scratch(P, n, full)
    ctrl = ctrl_block()
    outs = [torch.zeros(n, dtype=torch.int16, device=DEV) for _ in range(P)]
    announce("packet single rank, stale peer packets, small spin bound")
    ar.ar_packet_fused([to_dev(x) for x in xs], scratch, outs, 2, ctrl, rank_lo=rank,
                       rank_hi=rank + 1, max_spins=SMALL_SPINS)
    torch.cuda.synchronize()
    assert ctrl_status(ctrl) == ar.AR_ETIMEDOUT


def test_packet_zeroed_scratch_single_rank_times_out():
    P, n = 4, 2048
    xs = I.make_inputs("uniform", P, n, seed=8)
    scratch = _scratch(P, n)
    ctrl = ctrl_block()
    outs = [torch.zeros(n, dtype=torch.int16, device=DEV) for _ in range(P)]
    announce("packet single rank, no peers at all, small spin bound")
    ar.ar_packet_fused([to_dev(x) for x in xs], scratch, outs, 1, ctrl, rank_lo=1, rank_hi=2,
                       max_spins=SMALL_SPINS)
    torch.cuda.synchronize()
    assert ctrl_status(ctrl) == ar.AR_ETIMEDOUT


def test_packet_split_launch_on_one_stream_with_staged_second_half():
    """Ranks 0..3 run in one launch against ranks 4..7's packets staged from
    the oracle's image, then ranks 4..7 run in a second launch on the same
    stream: both halves complete and together give the full result (two
    launches that wait on each other would need two concurrently running
    streams, which HIP does not guarantee)."""
    P, n = 8, 8192 * 5 + 9
    xs = I.make_inputs("uniform", P, n, seed=12)
    zero = [np.zeros(O.packet_scratch_bytes(P, n), np.uint8) for _ in range(P)]
    want, full = O.packet_fused(xs, 1, zero)
    staged = zero
    for r in range(4, 8):   # keep only ranks 4..7's packets
        staged = [np.where(_rank_mask(P, n, r), f_, s_) for f_, s_ in zip(full, staged)]
    scratch = _scratch(P, n, staged)
    outs = [torch.zeros(n, dtype=torch.int16, device=DEV) for _ in range(P)]
    ctrl = ctrl_block()
    d_in = [to_dev(x) for x in xs]
    announce("packet split launch: ranks 0..3 against staged 4..7, then 4..7")
    ar.ar_packet_fused(d_in, scratch, outs, 1, ctrl, rank_lo=0, rank_hi=4)
    ar.ar_packet_fused(d_in, scratch, outs, 1, ctrl, rank_lo=4, rank_hi=8)
    torch.cuda.synchronize()
    assert ctrl_status(ctrl) == 0
    for r in range(P):
        assert np.array_equal(to_host(outs[r]), want[r])
    got = _images(scratch)
    for r in range(P):
        assert np.array_equal(got[r], full[r])


def _rank_mask(P, n, rank):
    """Byte mask of the packets `rank` writes: its slot in every inbox and
    every resbox."""
    S = O.packet_slot_packets(P, n)
    m = np.zeros((2 * P, 16 * S), bool)
    m[rank] = True
    m[P + rank] = True
    return m.reshape(-1)


@pytest.mark.parametrize("schedule", [0, 1])
@pytest.mark.parametrize("per_rank,wpl", [(1, 1), (3, 2), (7, 1), (0, 1), (0, 2), (64, 2)])
@pytest.mark.parametrize("P,n", [(8, 8192 * 9 + 1), (3, 4096 * 7 + 5)])
def test_packet_fused_every_launch_shape(per_rank, wpl, P, n, schedule):
    """Pipeline depth (chunks per workgroup) and chunk width change the
    schedule, never the result: outputs and scratch images stay bit-exact."""
    xs = I.make_inputs("uniform", P, n, seed=per_rank + wpl)
    scratch = _scratch(P, n)
    outs = [torch.zeros(n, dtype=torch.int16, device=DEV) for _ in range(P)]
    ctrl = ctrl_block()
    ar.ar_set_packet_tuning(per_rank, wpl, schedule)
    try:
        announce(f"packet launch shape per_rank={per_rank} wpl={wpl} schedule={schedule} "
                 f"P={P} n={n}")
        for f in (1, 2):
            ar.ar_packet_fused([to_dev(x) for x in xs], scratch, outs, f, ctrl)
        torch.cuda.synchronize()
    finally:
        ar.ar_set_packet_tuning(0, 0, 0)
    assert ctrl_status(ctrl) == 0
    zero = [np.zeros(O.packet_scratch_bytes(P, n), np.uint8) for _ in range(P)]
    _, img1 = O.packet_fused(xs, 1, zero)
    want, img2 = O.packet_fused(xs, 2, img1)
    for r in range(P):
        assert np.array_equal(to_host(outs[r]), want[r])
    got = _images(scratch)
    for r in range(P):
        assert np.array_equal(got[r], img2[r])


def test_packet_fused_fifty_calls_rotating_flags():
    """Fifty consecutive calls on one scratch set, inputs changing every call:
    each call's outputs are checked, and the full scratch image on a few."""
    P, n = 8, 8192 * 9 + 1
    scratch = _scratch(P, n)
    images = [np.zeros(O.packet_scratch_bytes(P, n), np.uint8) for _ in range(P)]
    ctrl = ctrl_block()
    outs = [torch.zeros(n, dtype=torch.int16, device=DEV) for _ in range(P)]
    announce("packet fused: 50 calls, flags 1..50")
    for call in range(50):
        f = call + 1
        xs = I.make_inputs("uniform", P, n, seed=100 + call)
        ar.ar_packet_fused([to_dev(x) for x in xs], scratch, outs, f, ctrl)
        torch.cuda.synchronize()
        assert ctrl_status(ctrl) == 0, call
        want, images = O.packet_fused(xs, f, images)
        for r in range(P):
            assert np.array_equal(to_host(outs[r]), want[r]), (call, r)
        if call in (0, 17, 49):
            got = _images(scratch)
            for r in range(P):
                assert np.array_equal(got[r], images[r]), (call, r)


@pytest.mark.parametrize("in_shift,out_shift", [(1, 0), (0, 1), (1, 1), (3, 2)])
def test_packet_fused_two_byte_aligned_buffers(in_shift, out_shift):
    """Inputs or outputs that are only 2-byte aligned take the element-wise
    path for the bf16 pairs; results and images stay bit-exact."""
    P, n = 8, 8192 * 3 + 7
    xs = I.make_inputs("uniform", P, n, seed=70 + in_shift)
    ins = [Guarded(n, shift=in_shift, init=x) for x in xs]
    outs = [Guarded(n, shift=out_shift) for _ in range(P)]
    scratch = _scratch(P, n)
    ctrl = ctrl_block()
    announce(f"packet fused, element shifts in={in_shift} out={out_shift}")
    ar.ar_packet_fused([g.view for g in ins], scratch, [o.view for o in outs], 1, ctrl)
    torch.cuda.synchronize()
    assert ctrl_status(ctrl) == 0
    want, img = O.packet_fused(xs, 1, [np.zeros(O.packet_scratch_bytes(P, n), np.uint8)
                                       for _ in range(P)])
    for r in range(P):
        assert np.array_equal(outs[r].host(), want[r]) and outs[r].guards_intact()
    got = _images(scratch)
    for r in range(P):
        assert np.array_equal(got[r], img[r])


@pytest.mark.parametrize("n", [1, 2, 5, 4096 * 3 + 3])
@pytest.mark.parametrize("shift", [1, 2])
def test_ll_encode_from_two_or_four_byte_aligned_source(n, shift):
    """shift 1: a 2-byte-aligned source (one word per lane throughout);
    shift 2: 4-byte but not 8-byte aligned (the bulk path)."""
    rng = np.random.default_rng(n + 99)
    y = rng.integers(0, 1 << 16, n, dtype=np.uint32).astype(np.uint16)
    src = Guarded(n, shift=shift, init=y)
    pk = torch.zeros(16 * O.ll_packets(n) + 64, dtype=torch.uint8, device=DEV)
    announce(f"ll_encode from a source at element offset {shift} n={n}")
    ar.ar_ll_encode(src.view, pk, 77)
    torch.cuda.synchronize()
    got = pk.cpu().numpy()
    assert got[16 * O.ll_packets(n):].sum() == 0          # nothing past the last packet
    assert np.array_equal(got[: 16 * O.ll_packets(n)].view(np.uint32), O.ll_encode(y, 77))
    assert src.guards_intact()


@pytest.mark.parametrize("in_shift,out_shift", [(0, 0), (2, 0), (0, 2), (1, 3), (2, 2)])
def test_packet_every_path_and_alignment(in_shift, out_shift):
    """The fused kernel, its epoch variant and the three-launch decomposition
    with buffers 8-, 4- and 2-byte aligned (element accesses fall back from
    pairs to single elements): outputs and scratch images bit-exact, call
    after call, the paths interleaved on one scratch set."""
    P, n = 8, 8192 * 5 + 13
    scratch = _scratch(P, n)
    images = [np.zeros(O.packet_scratch_bytes(P, n), np.uint8) for _ in range(P)]
    ctrl = ctrl_block()
    for f, path in ((1, "fused"), (2, "three-op"), (3, "fused")):
        xs = I.make_inputs("uniform", P, n, seed=90 + f + in_shift)
        ins = [Guarded(n, shift=in_shift, init=x) for x in xs]
        outs = [Guarded(n, shift=out_shift) for _ in range(P)]
        announce(f"packet {path} flag={f} shifts in={in_shift} out={out_shift}")
        iv, ov = [g.view for g in ins], [o.view for o in outs]
        if path == "fused":
            ar.ar_packet_fused(iv, scratch, ov, f, ctrl)
        else:
            ar.ar_packet_send(iv, scratch, f)
            ar.ar_packet_recv_reduce_send(scratch, n, f, ctrl)
            ar.ar_packet_recv(scratch, ov, f, ctrl)
        torch.cuda.synchronize()
        assert ctrl_status(ctrl) == 0
        want, images = O.packet_fused(xs, f, images)
        for r in range(P):
            assert np.array_equal(outs[r].host(), want[r]), (f, r)
            assert outs[r].guards_intact()
        got = _images(scratch)
        for r in range(P):
            assert np.array_equal(got[r], images[r]), (f, r)
    # the device-epoch variant on a fresh scratch set (flag 1, then 2)
    scratch = _scratch(P, n)
    images = [np.zeros(O.packet_scratch_bytes(P, n), np.uint8) for _ in range(P)]
    ectrl = ctrl_block()
    for f in (1, 2):
        xs = I.make_inputs("uniform", P, n, seed=95 + f)
        outs = [Guarded(n, shift=out_shift) for _ in range(P)]
        ins = [Guarded(n, shift=in_shift, init=x) for x in xs]
        announce(f"packet epoch call {f} shifts in={in_shift} out={out_shift}")
        ar.ar_packet_fused_epoch([g.view for g in ins], scratch, [o.view for o in outs], ectrl)
        torch.cuda.synchronize()
        assert ctrl_status(ectrl) == 0
        want, images = O.packet_fused(xs, f, images)
        for r in range(P):
            assert np.array_equal(outs[r].host(), want[r]), (f, r)
        got = _images(scratch)
        for r in range(P):
            assert np.array_equal(got[r], images[r]), (f, r)
