"""GPU parity at the largest index ranges: buffers of more than 2**31
elements (byte offsets past 4 GiB; packet word indices past 2**31 for the
codec), where a 32-bit index anywhere in a kernel or its launch would wrap.

Inputs are the position fill x_r[i] = ((131 i + 17 r) mod 251 - 125) / 128,
which depends on i only through i mod 251.  A block of BLOCK elements (a
multiple of 251) is generated on the host and tiled on the device, so the
full inputs are exactly the position fill of length n; every result of the
path is elementwise, hence periodic with the same block, and each device
chunk is compared in full with the oracle's result on the host block.  A
wrapped index reads a different residue mod 251 and fails the comparison.

Memory: at most 48 GiB of device memory per test, released after each."""
from __future__ import annotations

import numpy as np
import pytest
import torch

from allreduce_reduction_way_amd import ar, inputs as I
from gpu_util import DEV, announce, ctrl_block, ctrl_status, to_dev
from oracle import oracle as O

pytestmark = pytest.mark.gpu

BLOCK = 251 * (1 << 17)                  # 32,899,072 elements: the fill's period divides it
BIG = (1 << 31) + (1 << 20) + 13         # past the int32 element range, ragged tail


@pytest.fixture(autouse=True)
def _release_memory():
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _tiled(block: np.ndarray, n: int, shift: int = 0) -> torch.Tensor:
    """A device view of n elements (at element offset `shift` in its
    allocation) holding `block` repeated."""
    assert block.size % 251 == 0
    base = torch.empty(n + shift, dtype=torch.int16, device=DEV)
    t = base[shift:]
    b = to_dev(block)
    for off in range(0, n, block.size):
        m = min(block.size, n - off)
        t[off: off + m].copy_(b[:m])
    return t


def _equal_tiled(t: torch.Tensor, block: np.ndarray, lo: int = 0, hi: int | None = None,
                 outside: int | None = None) -> bool:
    """t[i] == block[i mod BLOCK] for lo <= i < hi, and t[i] == outside for
    the other i (when `outside` is given)."""
    n = t.numel()
    hi = n if hi is None else hi
    b = to_dev(block)
    for off in range(0, n, block.size):
        m = min(block.size, n - off)
        seg = t[off: off + m]
        a, e = max(lo, off) - off, min(hi, off + m) - off
        if a < e and not torch.equal(seg[a:e], b[a:e]):
            return False
        if outside is not None:
            fill = outside - (1 << 16) if outside >= 1 << 15 else outside   # as int16
            if a > 0 and not bool((seg[: min(a, m)] == fill).all()):
                return False
            if e < m and not bool((seg[max(e, 0):] == fill).all()):
                return False
    return True


def _blocks(P):
    return [I.position_fill_bf16(BLOCK, r) for r in range(P)]


@pytest.mark.parametrize("shift", [0, 3])
def test_oneshot_past_2_31_elements(shift):
    P, n = 2, BIG
    blk = _blocks(P)
    announce(f"large oneshot P={P} n={n} shift={shift} (filling)")
    ins = [_tiled(b, n, shift) for b in blk]
    out = _tiled(np.zeros(BLOCK, np.uint16), n, shift)
    announce(f"large oneshot P={P} n={n} shift={shift} (kernel)")
    ar.ar_oneshot_sum(ins, out)
    torch.cuda.synchronize()
    assert _equal_tiled(out, O.oneshot_sum(blk))


def test_misaligned_inputs_past_2_31_elements():
    """Inputs at element shifts 3 and 6 against aligned outputs: the scalar
    path over the whole 32-bit-overflowing range."""
    P, n = 2, BIG
    blk = _blocks(P)
    announce(f"large misaligned write_bcast P={P} n={n} (filling)")
    ins = [_tiled(b, n, shift) for b, shift in zip(blk, (3, 6))]
    outs = [torch.empty(n, dtype=torch.int16, device=DEV) for _ in range(P)]
    announce(f"large misaligned write_bcast P={P} n={n} (kernel)")
    ar.ar_oneshot_write_bcast(ins, outs)
    torch.cuda.synchronize()
    y = O.oneshot_sum(blk)
    for o in outs:
        assert _equal_tiled(o, y)


def test_write_bcast_past_2_31_elements():
    P, n = 3, BIG
    blk = _blocks(P)
    announce(f"large write_bcast P={P} n={n} (filling)")
    ins = [_tiled(b, n) for b in blk]
    outs = [torch.empty(n, dtype=torch.int16, device=DEV) for _ in range(P)]
    announce(f"large write_bcast P={P} n={n} (kernel)")
    ar.ar_oneshot_write_bcast(ins, outs)
    torch.cuda.synchronize()
    y = O.oneshot_sum(blk)
    for o in outs:
        assert _equal_tiled(o, y)


def test_twoshot_last_owner_past_2_31_elements():
    """The last owner's slice starts past byte 2**31 of every buffer, runs
    past element 2**31 and absorbs the remainder; every output outside the
    slice keeps its prior contents."""
    P, n, rank = 4, BIG, 3
    blk = _blocks(P)
    b, e = O.slice_range(P, n, rank)
    assert 2 * b > (1 << 31) and e == n > (1 << 31)
    announce(f"large twoshot P={P} n={n} rank={rank} slice=[{b},{e}) (filling)")
    ins = [_tiled(x, n) for x in blk]
    outs = [torch.full((n,), 0xA5A5 - (1 << 16), dtype=torch.int16, device=DEV)
            for _ in range(P)]
    announce(f"large twoshot P={P} n={n} rank={rank} (kernel)")
    ar.ar_twoshot_share(ins, outs, rank)
    torch.cuda.synchronize()
    y = O.oneshot_sum(blk)
    for o in outs:
        assert _equal_tiled(o, y, b, e, outside=0xA5A5)


def test_packet_fused_past_2_31_elements():
    P, n = 2, BIG
    blk = _blocks(P)
    nb = ar.ar_packet_scratch_bytes(P, n)
    announce(f"large packet_fused P={P} n={n} scratch={nb} B per rank (filling)")
    ins = [_tiled(x, n) for x in blk]
    outs = [torch.empty(n, dtype=torch.int16, device=DEV) for _ in range(P)]
    scratch = [torch.zeros(nb, dtype=torch.uint8, device=DEV) for _ in range(P)]
    ctrl = ctrl_block()
    announce(f"large packet_fused P={P} n={n} (kernel)")
    ar.ar_packet_fused(ins, scratch, outs, 0x9E3779B9, ctrl)
    torch.cuda.synchronize()
    assert ctrl_status(ctrl) == 0
    y = O.oneshot_sum(blk)
    for o in outs:
        assert _equal_tiled(o, y)


def test_ll_codec_past_2_31_words():
    """n = 2**32 + 6 elements: 2**31 + 4 packet words, so word indices pass
    the int32 range.  Packets are compared chunk by chunk with the oracle's
    encoding of the block (the last chunk: of its own prefix), and the
    decode restores the input."""
    n, flag = (1 << 32) + 6, 0xC0FFEE01
    blk = I.position_fill_bf16(BLOCK, 5)
    announce(f"large ll codec n={n} (filling)")
    src = _tiled(blk, n)
    npk = ar.ar_ll_packets(n)
    pk = torch.zeros(16 * npk, dtype=torch.uint8, device=DEV)
    announce(f"large ll codec n={n} packets={npk} (encode)")
    ar.ar_ll_encode(src, pk, flag)
    torch.cuda.synchronize()
    want = to_dev(O.ll_encode(blk, flag).view(np.uint16)).view(torch.uint8)
    per = 16 * (BLOCK // 4)
    for off in range(0, n, BLOCK):
        m = min(BLOCK, n - off)
        seg = pk[off * 4: off * 4 + 16 * O.ll_packets(m)]
        ref = want[:per] if m == BLOCK else \
            to_dev(O.ll_encode(blk[:m], flag).view(np.uint16)).view(torch.uint8)
        assert torch.equal(seg, ref), off
    del want
    dst = torch.empty(n, dtype=torch.int16, device=DEV)
    ctrl = ctrl_block()
    announce(f"large ll codec n={n} (decode)")
    ar.ar_ll_decode(pk, dst, flag, ctrl)
    torch.cuda.synchronize()
    assert ctrl_status(ctrl) == 0
    assert torch.equal(dst, src)
