"""Pins of the CPU oracle against facts that do not come from the oracle.

Each test checks the oracle against something the mathematics or the pages
fix: closed forms, hand-derived IEEE 754 corner cases, an exact-rational model
of binary32/bf16 rounding built from the standard's definitions, a library
cast on inputs whose sum is exact, library binary32 adds and bf16 cast on
arbitrary bit patterns, hand-derived packet and slice tables, and
invariants of the fused packet path.  A dropped term, a wrong rank or element
index, a swapped operand or a wrong rounding rule fails at least one of them.
"""
from __future__ import annotations

import pathlib

import numpy as np
import pytest
import torch

import exact_ref as E
from allreduce_reduction_way_amd import inputs as I
from oracle import oracle as O

GOLDEN = pathlib.Path(__file__).resolve().parent / "golden"


def _lines(name):
    for raw in (GOLDEN / name).read_text().splitlines():
        line = raw.split("#", 1)[0].strip()
        if line:
            yield line


# ---------------------------------------------------------------- closed forms

@pytest.mark.parametrize("P", range(2, 9))
def test_all_ones_sum_to_P(P):
    # Every input 1.0 -> the sum is exactly P (small integers are exact in bf16).
    n = 1000
    y = O.oneshot_sum([np.full(n, 0x3F80, np.uint16)] * P)
    expected = {2: 0x4000, 3: 0x4040, 4: 0x4080, 5: 0x40A0, 6: 0x40C0, 7: 0x40E0, 8: 0x4100}[P]
    assert (y == expected).all()


@pytest.mark.parametrize("P", range(2, 9))
def test_rank_constant_sums_to_triangle(P):
    # x_r == r -> sum 0 + 1 + ... + (P-1) = P(P-1)/2, exact.
    n = 777
    bf16_of = {0: 0x0000, 1: 0x3F80, 2: 0x4000, 3: 0x4040, 4: 0x4080, 5: 0x40A0, 6: 0x40C0,
               7: 0x40E0}
    xs = [np.full(n, bf16_of[r], np.uint16) for r in range(P)]
    expected = {2: 0x3F80, 3: 0x4040, 4: 0x40C0, 5: 0x4120, 6: 0x4170, 7: 0x41A8, 8: 0x41E0}[P]
    assert (O.oneshot_sum(xs) == expected).all()


def test_single_input_is_identity_for_every_bf16():
    # P = 1: widening to binary32 and rounding back is exact for every bf16;
    # every NaN pattern comes back as the canonical 7FC0.
    x = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    y = O.oneshot_sum([x])
    is_nan = ((x & 0x7F80) == 0x7F80) & ((x & 0x007F) != 0)
    assert (y[~is_nan] == x[~is_nan]).all()
    assert (y[is_nan] == 0x7FC0).all()


# ---------------------------------------------------------- IEEE corner cases

def _corner_cases():
    for line in _lines("rne_corners.txt"):
        lhs, rhs = line.split("->")
        yield [int(t, 16) for t in lhs.split()], int(rhs.split()[0], 16)


@pytest.mark.parametrize("values,expected", list(_corner_cases()))
def test_rne_corner_table(values, expected):
    xs = [np.array([v], np.uint16) for v in values]
    assert int(O.oneshot_sum(xs)[0]) == expected
    # and the independent exact-rational model agrees with the hand derivation
    assert E.reduce_element(values) == expected


# ------------------------------------------------ exact-rational brute force

def _random_bf16(rng, n, mode):
    if mode == "any_finite":
        v = rng.integers(0, 1 << 16, n, dtype=np.uint32).astype(np.uint16)
        bad = (v & 0x7F80) == 0x7F80
        v[bad] &= 0xBFFF  # clear the top exponent bit: finite
        return v
    if mode == "narrow":
        # exponents within a few binades and random mantissas: lots of ties
        sign = rng.integers(0, 2, n, dtype=np.uint32) << 15
        exp = rng.integers(124, 130, n, dtype=np.uint32) << 7
        man = rng.integers(0, 128, n, dtype=np.uint32)
        return (sign | exp | man).astype(np.uint16)
    if mode == "tiny":
        # subnormals and the smallest normals
        sign = rng.integers(0, 2, n, dtype=np.uint32) << 15
        mag = rng.integers(0, 0x0200, n, dtype=np.uint32)
        return (sign | mag).astype(np.uint16)
    if mode == "uniform":
        return I.uniform_bf16(n, int(rng.integers(0, 1 << 20)), 0)
    raise ValueError(mode)


@pytest.mark.parametrize("P", range(2, 9))
@pytest.mark.parametrize("mode", ["any_finite", "narrow", "tiny", "uniform"])
def test_brute_force_against_exact_rational_model(P, mode):
    rng = np.random.default_rng(1234 + P * 17 + len(mode))
    n = 64
    xs = [_random_bf16(rng, n, mode) for _ in range(P)]
    y = O.oneshot_sum(xs)
    for i in range(n):
        assert int(y[i]) == E.reduce_element([int(x[i]) for x in xs]), (P, mode, i)


def test_many_pairs_against_exact_rational_model():
    rng = np.random.default_rng(99)
    n = 4000
    a = _random_bf16(rng, n, "any_finite")
    b = _random_bf16(rng, n, "narrow")
    y = O.oneshot_sum([a, b])
    for i in range(n):
        assert int(y[i]) == E.reduce_element([int(a[i]), int(b[i])]), i


# ----------------------------------------- exact sums reduce to a library cast

@pytest.mark.parametrize("P", [2, 4, 8])
def test_position_fill_equals_library_cast_of_exact_sum(P):
    # Every position-fill value is k/128 with |k| <= 125; the binary32 sum of
    # up to eight of them is exact, so the result is the library's bf16 cast
    # of the exact (integer) sum, whatever the order.
    n = 5000
    xs = I.make_inputs("position", P, n)
    k_sum = np.zeros(n, dtype=np.int64)
    for r in range(P):
        i = np.arange(n, dtype=np.int64)
        k_sum += (i * 131 + r * 17) % 251 - 125
    exact = torch.from_numpy(k_sum.astype(np.float64) / 128.0)
    expected = exact.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert (O.oneshot_sum(xs) == expected).all()
    assert (O.oneshot_sum(xs[::-1]) == expected).all()


# ------------------------------ library binary32 adds and library bf16 cast

@pytest.mark.parametrize("P", [2, 3, 8])
def test_library_adds_and_cast_on_arbitrary_bit_patterns(P):
    # numpy's elementwise binary32 additions are IEEE round-to-nearest-even
    # with subnormals kept; torch's binary32 -> bf16 conversion rounds to
    # nearest even.  Summing in rank order with the one and converting with
    # the other gives the definition independently of the oracle's code, on
    # 200,000 arbitrary bit patterns per input (NaN, Inf, zeros and
    # subnormals included).  NaN results are compared by NaN-ness only (the
    # library keeps a payload; the definition stores 0x7FC0).
    rng = np.random.default_rng(2024 + P)
    n = 200_000
    xs = [rng.integers(0, 1 << 16, n, dtype=np.uint32).astype(np.uint16) for _ in range(P)]
    widened = [(x.astype(np.uint32) << 16).view(np.float32) for x in xs]
    acc = widened[0].copy()
    with np.errstate(invalid="ignore", over="ignore"):
        for w in widened[1:]:
            acc = acc + w
    expected = torch.from_numpy(acc).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = O.oneshot_sum(xs)
    nan = np.isnan(acc)
    assert nan.any() and (~nan).sum() > n // 2
    assert np.array_equal(got[~nan], expected[~nan])
    assert (got[nan] == 0x7FC0).all()


# --------------------------------------------------------------- write mode

def test_write_bcast_outputs_identical_and_equal_oneshot():
    xs = I.make_inputs("uniform", 8, 3001, seed=5)
    y = O.oneshot_sum(xs)
    outs = O.write_bcast(xs)
    assert len(outs) == 8
    for o in outs:
        assert (o == y).all()


# ------------------------------------------------------------------ slices

def _slice_rows():
    for line in _lines("slices.txt"):
        yield tuple(int(t) for t in line.split())


@pytest.mark.parametrize("P,n,r,b,e", list(_slice_rows()))
def test_slice_table(P, n, r, b, e):
    assert O.slice_range(P, n, r) == (b, e)


@pytest.mark.parametrize("P", [2, 3, 4, 8])
@pytest.mark.parametrize("n", [0, 1, 127, 128, 1023, 1024, 1025, 5000, 128 * 8 * 7 - 1,
                               128 * 8 * 7, 128 * 8 * 7 + 1])
def test_slices_partition_and_align(P, n):
    prev_end = 0
    for r in range(P):
        b, e = O.slice_range(P, n, r)
        assert b == prev_end and b <= e
        assert b % 128 == 0
        if r < P - 1:
            assert (e - b) % 128 == 0 and (e - b) == O.slice_range(P, n, 0)[1]
        prev_end = e
    assert prev_end == n


def test_twoshot_union_is_oneshot_and_rest_untouched():
    P, n = 8, 1024 * 3 + 77
    xs = I.make_inputs("uniform", P, n, seed=3)
    y = O.oneshot_sum(xs)
    sentinel = [np.full(n, 0xA5A5, np.uint16) for _ in range(P)]
    outs = sentinel
    for r in range(P):
        b, e = O.slice_range(P, n, r)
        new = O.twoshot_share(xs, r, outs)
        for j in range(P):
            assert (new[j][b:e] == y[b:e]).all()
            mask = np.ones(n, bool)
            mask[b:e] = False
            assert (new[j][mask] == outs[j][mask]).all()
        outs = new
    for o in outs:
        assert (o == y).all()


# ---------------------------------------------------------------- LL codec

def _packet_rows():
    for line in _lines("ll_packets.txt"):
        flag, elems, image = (t.strip() for t in line.split("|"))
        yield int(flag, 16), [int(t, 16) for t in elems.split()], bytes(int(t, 16) for t in image.split())


@pytest.mark.parametrize("flag,elems,image", list(_packet_rows()))
def test_ll_encode_golden_bytes(flag, elems, image):
    pk = O.ll_encode(np.array(elems, np.uint16), flag)
    assert pk.tobytes() == image
    assert (O.ll_decode(pk, len(elems), flag) == np.array(elems, np.uint16)).all()


@pytest.mark.parametrize("n", [0, 1, 2, 3, 4, 5, 6, 7, 8, 63, 64, 65, 1001])
def test_ll_round_trip_and_flag_positions(n):
    rng = np.random.default_rng(n)
    y = rng.integers(0, 1 << 16, n, dtype=np.uint32).astype(np.uint16)
    f = 0x01020304 + n
    pk = O.ll_encode(y, f)
    assert pk.size == 4 * ((n + 3) // 4)
    words = pk.reshape(-1, 4)
    assert (words[:, 1] == f).all() and (words[:, 3] == f).all()
    assert (O.ll_decode(pk, n, f) == y).all()
    # padding elements of a ragged last packet are zero
    flat = pk.reshape(-1, 4)[:, [0, 2]].reshape(-1).view(np.uint16)
    assert (flat[n:] == 0).all()


def test_ll_decode_rejects_wrong_flag():
    y = np.arange(10, dtype=np.uint16)
    pk = O.ll_encode(y, 5)
    with pytest.raises(O.OracleError):
        O.ll_decode(pk, 10, 4)
    pk2 = pk.copy()
    pk2[4 * 2 + 3] = 4  # second flag word of the last packet is stale
    with pytest.raises(O.OracleError):
        O.ll_decode(pk2, 10, 5)


# ------------------------------------------------------ fused packet path

def _decode_np(words: np.ndarray, n: int, flag: int):
    """Independent numpy decoder used to read the oracle's scratch image."""
    p = (n + 3) // 4
    w = words[: 4 * p].reshape(p, 4)
    assert (w[:, 1] == flag).all() and (w[:, 3] == flag).all()
    return w[:, [0, 2]].reshape(-1).view(np.uint16)[:n]


@pytest.mark.parametrize("P,n", [(8, 1024 * 3 + 5), (8, 1000), (4, 4096 + 130), (2, 513), (3, 777)])
def test_packet_fused_three_calls(P, n):
    S = O.packet_slot_packets(P, n)
    nbytes = O.packet_scratch_bytes(P, n)
    assert nbytes == 2 * P * S * 16
    imgs = [np.zeros(nbytes, np.uint8) for _ in range(P)]
    slices = [O.slice_range(P, n, j) for j in range(P)]
    for call in range(3):
        f = call + 1
        xs = I.make_inputs("uniform", P, n, seed=call)
        prev = [im.copy() for im in imgs]
        outs, imgs = O.packet_fused(xs, f, imgs)
        y = O.oneshot_sum(xs)
        for o in outs:
            assert (o == y).all()
        for j in range(P):
            words = imgs[j].view(np.uint32).reshape(2 * P, S * 4)
            prev_words = prev[j].view(np.uint32).reshape(2 * P, S * 4)
            b, e = slices[j]
            for s in range(P):
                # inbox_j[slot s] holds rank s's piece of slice j
                assert (_decode_np(words[s], e - b, f) == xs[s][b:e]).all()
                # resbox_j[slot s] holds the reduced slice s
                bs, es = slices[s]
                assert (_decode_np(words[P + s], es - bs, f) == y[bs:es]).all()
                # packets past a slice's end keep their previous contents
                used_in = 4 * ((e - b + 3) // 4)
                used_res = 4 * ((es - bs + 3) // 4)
                assert (words[s][used_in:] == prev_words[s][used_in:]).all()
                assert (words[P + s][used_res:] == prev_words[P + s][used_res:]).all()


def test_packet_fused_rejects_flag_zero():
    xs = I.make_inputs("uniform", 2, 256)
    imgs = [np.zeros(O.packet_scratch_bytes(2, 256), np.uint8) for _ in range(2)]
    with pytest.raises(O.OracleError):
        O.packet_fused(xs, 0, imgs)


def test_packet_scratch_size_for_512x7168():
    # 512x7168 elements over 8 ranks: slices of 458752 elements (exact),
    # 114688 packets per slot, 2 boxes x 8 slots x 114688 x 16 B per rank.
    assert O.packet_slot_packets(8, 512 * 7168) == 114688
    assert O.packet_scratch_bytes(8, 512 * 7168) == 29360128


# ------------------------------------------------------------ reduce-scatter

@pytest.mark.parametrize("P", [2, 3, 8])
def test_reduce_scatter_closed_form(P):
    rc = 100
    xs = [np.full(P * rc, 0x3F80, np.uint16)] * P
    expected = {2: 0x4000, 3: 0x4040, 8: 0x4100}[P]
    for r in range(P):
        assert (O.reduce_scatter(xs, r) == expected).all()


@pytest.mark.parametrize("P", [2, 4, 8])
def test_reduce_scatter_against_exact_rational_model(P):
    rng = np.random.default_rng(77 + P)
    rc = 16
    xs = [_random_bf16(rng, P * rc, "narrow") for _ in range(P)]
    for r in range(P):
        y = O.reduce_scatter(xs, r)
        for i in range(rc):
            assert int(y[i]) == E.reduce_element([int(x[r * rc + i]) for x in xs]), (r, i)


def test_reduce_scatter_blocks_tile_the_oneshot_sum():
    P, rc = 8, 1000
    xs = I.make_inputs("uniform", P, P * rc, seed=9)
    y = O.oneshot_sum(xs)
    blocks = [O.reduce_scatter(xs, r) for r in range(P)]
    assert np.array_equal(np.concatenate(blocks), y)
