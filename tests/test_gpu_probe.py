"""GPU checks of the measurement kernels behind the same-size ceilings
(ar_probe_traffic): they touch exactly the bytes they claim to.  The copy
kernel copies every input into its output, the read-only kernel changes
nothing, the write-only kernel writes every element of all 2P buffers and
nothing outside them (guard bands)."""
from __future__ import annotations

import numpy as np
import pytest
import torch

from allreduce_reduction_way_amd import ar, inputs as I
from gpu_util import Guarded, announce

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("policy", [0, 1])
@pytest.mark.parametrize("P", [4, 8])
@pytest.mark.parametrize("threads,unroll,blocks", [(64, 1, 0), (256, 2, 0), (64, 4, 0), (128, 1, 3)])
@pytest.mark.parametrize("n", [8, 8 * 64 * 4 * 3 + 8, 100_000])
def test_probe_kernels_touch_exactly_their_buffers(P, threads, unroll, blocks, n, policy):
    xs = I.make_inputs("uniform", P, n, seed=n % 31)
    ins = [Guarded(n, init=x) for x in xs]
    outs = [Guarded(n, fill=0x1111) for _ in range(P)]
    iv, ov = [g.view for g in ins], [o.view for o in outs]
    if unroll <= 2:
        announce(f"probe read P={P} n={n} {threads}x{unroll} blocks={blocks}")
        ar.ar_probe_traffic(0, iv, ov, threads, unroll, blocks, policy)
        torch.cuda.synchronize()
        assert all(np.array_equal(g.host(), x) for g, x in zip(ins, xs))
        assert all((o.host() == 0x1111).all() for o in outs)
    announce(f"probe copy P={P} n={n} {threads}x{unroll} blocks={blocks}")
    ar.ar_probe_traffic(2, iv, ov, threads, unroll, blocks, policy)
    torch.cuda.synchronize()
    for g, o, x in zip(ins, outs, xs):
        assert np.array_equal(o.host(), x) and o.guards_intact()
        assert np.array_equal(g.host(), x)
    announce(f"probe write P={P} n={n} {threads}x{unroll} blocks={blocks}")
    ar.ar_probe_traffic(1, iv, ov, threads, unroll, blocks, policy)
    torch.cuda.synchronize()
    v = np.arange(n // 8, dtype=np.uint32)
    want = np.stack([v, np.full_like(v, 0x3F803F80), v, np.full_like(v, 0x3F803F80)], 1)
    want = want.reshape(-1).view(np.uint16)
    for g in ins + outs:
        assert np.array_equal(g.host(), want) and g.guards_intact()
