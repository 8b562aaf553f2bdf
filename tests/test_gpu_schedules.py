"""GPU parity of the reduce entry points under every launch schedule the
library can take (grid-stride batches, the pipelined kernel with 2, 4 or 8
stages of 1 or 2 vectors per lane, and the phased one-pass kernel with 1 to 8
vectors per lane, 7 and 8 taken as 6 at P >= 7, for 64/128/256-lane
workgroups), forced
through the benchmark tuning hook.  Results must not depend on the schedule:
bit-exact against the oracle, guard bands intact, in place included.  Sizes
leave ragged last workgroups, partial stages and scalar heads and tails."""
from __future__ import annotations

import numpy as np
import pytest
import torch

from allreduce_reduction_way_amd import ar, inputs as I
from gpu_util import Guarded, announce, to_dev, to_host
from oracle import oracle as O

pytestmark = pytest.mark.gpu

# (unroll, threads, max_blocks, schedule)
SHAPES = [(1, 64, 0, 1), (2, 256, 7, 1), (4, 128, 0, 1),
          (1, 64, 0, 2), (2, 64, 0, 2), (1, 256, 0, 2), (2, 128, 0, 2),
          (1, 64, 0, 4), (2, 64, 0, 4), (1, 128, 0, 4), (2, 256, 0, 4),
          (1, 64, 0, 8), (2, 64, 0, 8), (1, 256, 0, 8),
          (1, 64, 0, 16), (2, 64, 0, 16), (3, 64, 0, 16), (4, 64, 0, 16), (5, 64, 0, 16),
          (6, 64, 0, 16), (7, 64, 0, 16), (8, 64, 0, 16), (2, 128, 0, 16), (4, 256, 0, 16),
          (5, 256, 0, 16)]
# vectors per workgroup-stage for 64 lanes = 64; 2 x 64 x 8 x 5 + 3 leaves a ragged stage
SIZES = [1, 9, 8 * 64 * 3 + 5, 8 * 2 * 64 * 8 * 5 + 3 * 8 + 5, 100_003]


@pytest.fixture
def tuning():
    def set_shape(shape):
        ar.ar_set_reduce_tuning(*shape)
    yield set_shape
    ar.ar_set_reduce_tuning(0, 0, 0, 0)


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "u{}_t{}_b{}_s{}".format(*s))
@pytest.mark.parametrize("P", [3, 8])
def test_write_bcast_and_oneshot_every_schedule(tuning, shape, P):
    tuning(shape)
    for n in SIZES:
        for shift in (0, 3):
            xs = I.make_inputs("uniform", P, n, seed=n % 101 + P)
            y = O.oneshot_sum(xs)
            ins = [Guarded(n, shift=shift, init=x) for x in xs]
            outs = [Guarded(n, shift=shift) for _ in range(P)]
            announce(f"schedule {shape} write_bcast P={P} n={n} shift={shift}")
            ar.ar_oneshot_write_bcast([g.view for g in ins], [o.view for o in outs])
            one = Guarded(n, shift=shift)
            ar.ar_oneshot_sum([g.view for g in ins], one.view)
            torch.cuda.synchronize()
            for o in outs:
                assert np.array_equal(o.host(), y)
                assert o.guards_intact()
            assert np.array_equal(one.host(), y) and one.guards_intact()


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "u{}_t{}_b{}_s{}".format(*s))
def test_in_place_every_schedule(tuning, shape):
    tuning(shape)
    P, n = 8, 8 * 2 * 64 * 8 * 5 + 29
    xs = I.make_inputs("uniform", P, n, seed=77)
    d_in = [to_dev(x) for x in xs]
    announce(f"schedule {shape} write_bcast in place n={n}")
    # output k is input k: every element is read before the same lane writes it
    ar.ar_oneshot_write_bcast(d_in, d_in)
    torch.cuda.synchronize()
    y = O.oneshot_sum(xs)
    assert all(np.array_equal(to_host(t), y) for t in d_in)


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "u{}_t{}_b{}_s{}".format(*s))
def test_twoshot_and_reduce_scatter_every_schedule(tuning, shape):
    tuning(shape)
    P, n = 8, 680 * 5120
    xs = I.make_inputs("uniform", P, n, seed=5)
    d_in = [to_dev(x) for x in xs]
    prior = [np.full(n, 0x5A5A, np.uint16) for _ in range(P)]
    outs = [to_dev(p) for p in prior]
    announce(f"schedule {shape} twoshot rank 3 n={n}")
    ar.ar_twoshot_share(d_in, outs, 3)
    rc = 2252800 // P
    rs_in = [to_dev(x) for x in I.make_inputs("uniform", P, P * rc, seed=6)]
    rs_out = Guarded(rc)
    announce(f"schedule {shape} reduce-scatter rank 3 recvcount={rc}")
    ar.ar_reduce_scatter_share(rs_in, rs_out.view, 3)
    torch.cuda.synchronize()
    want = O.twoshot_share(xs, 3, prior)
    for t, w in zip(outs, want):
        assert np.array_equal(to_host(t), w)
    rs_host = [to_host(t) for t in rs_in]
    assert np.array_equal(rs_out.host(), O.reduce_scatter(rs_host, 3))
    assert rs_out.guards_intact()


# The automatic rule switches shape at 256, 768 and 2560 bulk vectors per CU
# (256 CUs: 524,288, 1,572,864 and 5,242,880 elements); sizes on both sides.
@pytest.mark.parametrize("P,n", [(8, 524_288 - 8), (8, 524_288 + 9), (4, 524_288 + 9),
                                 (8, 1_572_864 - 3), (5, 1_572_864 - 3), (3, 1_000_003),
                                 (8, 1_572_864 + 11), (2, 1_572_864 + 11),
                                 (8, 5_242_880 - 7), (8, 5_242_880 + 5), (3, 5_242_880 + 5),
                                 (6, 5_242_880 - 7), (7, 2_252_800 + 1)])
def test_automatic_shape_classes(P, n):
    ar.ar_set_reduce_tuning(0, 0, 0, 0)
    for shift in (0, 5):
        xs = I.make_inputs("uniform", P, n, seed=P * 7 + shift)
        y = O.oneshot_sum(xs)
        ins = [Guarded(n, shift=shift, init=x) for x in xs]
        outs = [Guarded(n, shift=shift) for _ in range(P)]
        announce(f"automatic shape write_bcast P={P} n={n} shift={shift}")
        ar.ar_oneshot_write_bcast([g.view for g in ins], [o.view for o in outs])
        torch.cuda.synchronize()
        for o in outs:
            assert np.array_equal(o.host(), y)
            assert o.guards_intact()


# With one output (one-shot sum, reduce-scatter) the rule takes the phased
# kernel with two vectors per lane beyond 2560 bulk vectors per CU; sizes on
# both sides of every switch, aligned and misaligned.
@pytest.mark.parametrize("P,n", [(8, 524_288 + 9), (4, 1_572_864 + 11), (8, 5_242_880 - 7),
                                 (8, 5_242_880 + 5), (2, 5_242_880 + 5), (4, 8_388_608 + 3)])
def test_automatic_shape_classes_one_output(P, n):
    ar.ar_set_reduce_tuning(0, 0, 0, 0)
    for shift in (0, 5):
        xs = I.make_inputs("uniform", P, n, seed=P * 11 + shift)
        y = O.oneshot_sum(xs)
        ins = [Guarded(n, shift=shift, init=x) for x in xs]
        out = Guarded(n, shift=shift)
        announce(f"automatic shape oneshot_sum P={P} n={n} shift={shift}")
        ar.ar_oneshot_sum([g.view for g in ins], out.view)
        torch.cuda.synchronize()
        assert np.array_equal(out.host(), y)
        assert out.guards_intact()


def test_automatic_reduce_scatter_past_2560_vectors_per_cu():
    P, rc = 2, 5_242_880 + 13
    xs = I.make_inputs("uniform", P, P * rc, seed=17)
    rs_in = [to_dev(x) for x in xs]
    ar.ar_set_reduce_tuning(0, 0, 0, 0)
    for rank in (0, 1):
        out = Guarded(rc)
        announce(f"automatic shape reduce-scatter P={P} recvcount={rc} rank={rank}")
        ar.ar_reduce_scatter_share(rs_in, out.view, rank)
        torch.cuda.synchronize()
        assert np.array_equal(out.host(), O.reduce_scatter(xs, rank))
        assert out.guards_intact()
