"""HIP-graph capture and replay of the reduce entry points and the LL codec:
one graph holds several calls (one-shot, write mode, a two-shot owner, a
reduce-scatter block, encode then decode); the inputs are rewritten eagerly
before every replay and every replay's outputs are compared with the CPU
oracle.  The library records only kernel launches (no memset or copy nodes),
so each replay must redo the whole computation on the new inputs."""
from __future__ import annotations

import numpy as np
import pytest
import torch

from allreduce_reduction_way_amd import ar, inputs as I
from gpu_util import DEV, announce, ctrl_block, ctrl_status, to_dev, to_host
from oracle import oracle as O

pytestmark = pytest.mark.gpu


def test_reduce_and_codec_graph_replays():
    P, n = 8, 440 * 512 + 5
    rc = n // P
    d_in = [torch.zeros(n, dtype=torch.int16, device=DEV) for _ in range(P)]
    one = torch.zeros(n, dtype=torch.int16, device=DEV)
    bcast = [torch.zeros(n, dtype=torch.int16, device=DEV) for _ in range(P)]
    two = [torch.zeros(n, dtype=torch.int16, device=DEV) for _ in range(P)]
    rs = torch.zeros(rc, dtype=torch.int16, device=DEV)
    pk = torch.zeros(16 * O.ll_packets(n), dtype=torch.uint8, device=DEV)
    dec = torch.zeros(n, dtype=torch.int16, device=DEV)
    ctrl = ctrl_block()
    flag = 0x5151

    def calls():
        ar.ar_oneshot_sum(d_in, one)
        ar.ar_oneshot_write_bcast(d_in, bcast)
        ar.ar_twoshot_share(d_in, two, 5)
        ar.ar_reduce_scatter_share(d_in, rs, 2)
        ar.ar_ll_encode(one, pk, flag)
        ar.ar_ll_decode(pk, dec, flag, ctrl)

    announce("graph: eager warm-up of the six calls")
    calls()                                          # library set-up happens outside capture
    torch.cuda.synchronize()
    assert ctrl_status(ctrl) == 0
    one.fill_(0x2468)
    torch.cuda.synchronize()

    side = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    announce("graph: capture of one-shot, write mode, two-shot, reduce-scatter, encode, decode")
    with torch.cuda.graph(g, stream=side):
        calls()
    torch.cuda.synchronize()
    assert bool((one == 0x2468).all())               # capture launched nothing

    for rep in range(4):
        xs = I.make_inputs("uniform", P, n, seed=700 + rep)
        for t, x in zip(d_in, xs):
            t.copy_(to_dev(x))
        for t in [one, dec, rs, *bcast, *two]:
            t.fill_(0x1357)
        pk.zero_()
        torch.cuda.synchronize()
        announce(f"graph: replay {rep}")
        g.replay()
        torch.cuda.synchronize()
        y = O.oneshot_sum(xs)
        assert np.array_equal(to_host(one), y), rep
        for t in bcast:
            assert np.array_equal(to_host(t), y), rep
        prior = [np.full(n, 0x1357, np.uint16) for _ in range(P)]
        want2 = O.twoshot_share(xs, 5, prior)
        for t, w in zip(two, want2):
            assert np.array_equal(to_host(t), w), rep
        assert np.array_equal(to_host(rs), O.reduce_scatter([x[:P * rc] for x in xs], 2)), rep
        assert np.array_equal(pk.cpu().numpy().view(np.uint32), O.ll_encode(y, flag)), rep
        assert ctrl_status(ctrl) == 0
        assert np.array_equal(to_host(dec), y), rep
