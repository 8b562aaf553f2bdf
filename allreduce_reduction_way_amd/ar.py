"""Thin ctypes binding of libar.so (declared in include/ar.h).

Argument marshalling only: every step of the computation runs in the HIP
kernels of libar.so.  The functions carry the C names.  Buffer arguments may
be torch CUDA tensors (bf16 / int16 / uint16 elements, uint8 for scratch and
control blocks) or raw device addresses as ints; ``stream`` may be None (the
current torch stream), a ``torch.cuda.Stream`` or a raw hipStream_t int.
A non-zero status raises :class:`ArError`.  The library is loaded on first
use; if it is not built, that first call raises: there is no fallback.
"""
from __future__ import annotations

import ctypes
import pathlib
from typing import Sequence

LIB_PATH = pathlib.Path(__file__).resolve().with_name("libar.so")

AR_MAX_P = 8
AR_OK, AR_EINVAL, AR_EALIAS, AR_ELAUNCH, AR_ETIMEDOUT, AR_ENOSPACE = 0, -1, -2, -3, -4, -5
AR_CTRL_BYTES = 64
AR_NOALLOC_SCRATCH_BYTES = 64 << 20
AR_DEFAULT_MAX_SPINS = 1 << 22

_NAMES = {AR_OK: "AR_OK", AR_EINVAL: "AR_EINVAL", AR_EALIAS: "AR_EALIAS",
          AR_ELAUNCH: "AR_ELAUNCH", AR_ETIMEDOUT: "AR_ETIMEDOUT", AR_ENOSPACE: "AR_ENOSPACE"}


class ArError(RuntimeError):
    def __init__(self, code: int, what: str):
        super().__init__(f"{what}: {_NAMES.get(code, code)} ({code})")
        self.code = code


class ar_ptrs(ctypes.Structure):
    _fields_ = [("p", ctypes.c_void_p * AR_MAX_P)]


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libar.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not LIB_PATH.exists():
            raise ImportError(f"{LIB_PATH} is not built: run "
                              "`python -c 'import __graft_entry__ as g; g.build()'`")
        L = ctypes.CDLL(str(LIB_PATH))
        i32, i64, u32, u64, vp = (ctypes.c_int, ctypes.c_int64, ctypes.c_uint32,
                                  ctypes.c_uint64, ctypes.c_void_p)
        sig = {
            "ar_oneshot_sum": (i32, [ar_ptrs, vp, i32, i64, vp]),
            "ar_oneshot_write_bcast": (i32, [ar_ptrs, ar_ptrs, i32, i64, vp]),
            "ar_twoshot_share": (i32, [ar_ptrs, ar_ptrs, i32, i32, i64, vp]),
            "ar_ll_packets": (i64, [i64]),
            "ar_ll_encode": (i32, [vp, vp, i64, u32, vp]),
            "ar_ll_decode": (i32, [vp, vp, i64, u32, vp, u64, vp]),
            "ar_packet_fused": (i32, [ar_ptrs, ar_ptrs, ar_ptrs, i32, i32, i32, i64, u32, vp,
                                      u64, vp]),
            "ar_reduce_scatter_share": (i32, [ar_ptrs, vp, i32, i32, i64, vp]),
            "ar_packet_fused_epoch": (i32, [ar_ptrs, ar_ptrs, ar_ptrs, i32, i32, i32, i64, vp, u64,
                                            vp]),
            "ar_packet_fused_noalloc": (i32, [ar_ptrs, ar_ptrs, i32, i64, vp, u64, vp]),
            "ar_packet_send": (i32, [ar_ptrs, ar_ptrs, i32, i32, i32, i64, u32, vp]),
            "ar_packet_recv_reduce_send": (i32, [ar_ptrs, i32, i32, i32, i64, u32, vp, u64, vp]),
            "ar_packet_recv": (i32, [ar_ptrs, ar_ptrs, i32, i32, i32, i64, u32, vp, u64, vp]),
            "ar_slice_range": (i32, [i32, i32, i64, ctypes.POINTER(i64), ctypes.POINTER(i64)]),
            "ar_packet_slot_packets": (i64, [i32, i64]),
            "ar_packet_scratch_bytes": (i64, [i32, i64]),
            "ar_strerror": (ctypes.c_char_p, [i32]),
            "ar_noop": (i32, [vp]),
            "ar_probe_traffic": (i32, [i32, ar_ptrs, ar_ptrs, i32, i64, i32, i32, i32, i32, vp]),
            "ar_set_reduce_tuning": (i32, [i32, i32, i32, i32]),
            "ar_set_packet_tuning": (i32, [i32, i32, i32]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype, fn.argtypes = res, args
        _lib = L
    return _lib


# ---------------------------------------------------------------- marshalling
#
# A torch tensor is checked before its address goes to the C library: it must
# be contiguous, hold elements of the right width (2-byte bf16 / int16 /
# uint16 for data, any type for byte buffers such as scratch, packets and
# control blocks) and span at least the bytes the call touches.  The C side
# cannot see sizes, so without this a short, strided or expanded tensor would
# be read or written out of bounds.  An int is a raw device address that the
# caller vouches for, passed as is.

_ELEM_BYTES = 2
_ELEM_DTYPES = ("torch.bfloat16", "torch.int16", "torch.uint16")


def _addr(buf) -> int:
    """Device address of a torch CUDA tensor, or an int taken as an address."""
    if isinstance(buf, int):
        return buf
    if getattr(buf, "is_cuda", False):
        return int(buf.data_ptr())
    raise TypeError(f"expected a CUDA tensor or a device address, got {type(buf).__name__}")


def _numel(buf) -> int:
    return int(buf.numel())


def _require(buf, nbytes: int, what: str, elems: bool = False, word: int = 0) -> None:
    """Raises ValueError unless the tensor `buf` is contiguous, has the element
    type the argument takes and spans at least `nbytes` bytes.  `elems`: a bf16
    data buffer; `word`: the exact element width (4 for a status word); else a
    byte buffer of any element type."""
    if isinstance(buf, int) or buf is None:
        return
    if not hasattr(buf, "element_size"):
        raise TypeError(f"{what}: expected a CUDA tensor or a device address, "
                        f"got {type(buf).__name__}")
    if elems and str(buf.dtype) not in _ELEM_DTYPES:
        raise ValueError(f"{what}: bf16 elements expected (bfloat16, int16 or uint16), "
                         f"got {buf.dtype}")
    if word and buf.element_size() != word:
        raise ValueError(f"{what}: {word}-byte elements expected, got {buf.dtype}")
    if not buf.is_contiguous():
        raise ValueError(f"{what}: the tensor must be contiguous")
    have = int(buf.numel()) * int(buf.element_size())
    if have < nbytes:
        raise ValueError(f"{what}: {have} bytes, the call touches {nbytes}")


def _require_all(bufs: Sequence, nbytes: int, what: str, elems: bool = False) -> None:
    for k, b in enumerate(bufs):
        _require(b, nbytes, f"{what}[{k}]", elems=elems)


def _stream(stream) -> int:
    if stream is None:
        import torch
        return int(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, int):
        return stream
    return int(stream.cuda_stream)


def _ptrs(bufs: Sequence) -> ar_ptrs:
    if len(bufs) > AR_MAX_P:
        raise ValueError(f"at most {AR_MAX_P} buffers")
    p = ar_ptrs()
    for k, b in enumerate(bufs):
        p.p[k] = _addr(b)
    return p


def _n(n, bufs) -> int:
    if n is not None:
        return int(n)
    b = bufs[0]
    if isinstance(b, int):
        raise ValueError("n is required when buffers are raw addresses")
    return _numel(b)


def _scratch_bytes(P: int, n: int) -> int:
    """Bytes of one rank's packet scratch, or 0 where the C call will reject
    P or n itself."""
    v = int(lib().ar_packet_scratch_bytes(P, n)) if n >= 0 else -1
    return max(v, 0)


def _check(rc: int, what: str) -> None:
    if rc != AR_OK:
        raise ArError(rc, what)


# ------------------------------------------------------------------ entry points

def ar_oneshot_sum(inputs: Sequence, out, n: int | None = None, stream=None) -> None:
    n = _n(n, inputs)
    _require_all(inputs, _ELEM_BYTES * n, "inputs", elems=True)
    _require(out, _ELEM_BYTES * n, "out", elems=True)
    _check(lib().ar_oneshot_sum(_ptrs(inputs), _addr(out), len(inputs), n, _stream(stream)),
           "ar_oneshot_sum")


def ar_oneshot_write_bcast(inputs: Sequence, outputs: Sequence, n: int | None = None,
                           stream=None) -> None:
    if len(outputs) != len(inputs):
        raise ValueError("write mode needs one output per input")
    n = _n(n, inputs)
    _require_all(inputs, _ELEM_BYTES * n, "inputs", elems=True)
    _require_all(outputs, _ELEM_BYTES * n, "outputs", elems=True)
    _check(lib().ar_oneshot_write_bcast(_ptrs(inputs), _ptrs(outputs), len(inputs), n,
                                        _stream(stream)), "ar_oneshot_write_bcast")


def ar_twoshot_share(inputs: Sequence, outputs: Sequence, rank: int, n: int | None = None,
                     stream=None) -> None:
    if len(outputs) != len(inputs):
        raise ValueError("the two-shot share needs one output per input")
    n = _n(n, inputs)
    _require_all(inputs, _ELEM_BYTES * n, "inputs", elems=True)
    _require_all(outputs, _ELEM_BYTES * n, "outputs", elems=True)
    _check(lib().ar_twoshot_share(_ptrs(inputs), _ptrs(outputs), len(inputs), rank, n,
                                  _stream(stream)), "ar_twoshot_share")


def ar_ll_packets(n: int) -> int:
    return int(lib().ar_ll_packets(n))


def ar_ll_encode(src, dst_pkts, flag: int, n: int | None = None, stream=None) -> None:
    n = _n(n, [src])
    _require(src, _ELEM_BYTES * n, "src", elems=True)
    _require(dst_pkts, 16 * ar_ll_packets(n), "dst_pkts")
    _check(lib().ar_ll_encode(_addr(src), _addr(dst_pkts), n, flag, _stream(stream)),
           "ar_ll_encode")


def ar_ll_decode(src_pkts, dst, flag: int, ctrl, n: int | None = None, max_spins: int = 0,
                 stream=None) -> None:
    n = _n(n, [dst])
    _require(src_pkts, 16 * ar_ll_packets(n), "src_pkts")
    _require(dst, _ELEM_BYTES * n, "dst", elems=True)
    _require(ctrl, AR_CTRL_BYTES, "ctrl")
    _check(lib().ar_ll_decode(_addr(src_pkts), _addr(dst), n, flag,
                              0 if ctrl is None else _addr(ctrl),
                              max_spins, _stream(stream)), "ar_ll_decode")


def _packet_buffers(P, n, inputs=None, scratch=None, outputs=None, ctrl=None):
    """Size, type and layout checks of a packet-path call's buffers."""
    if inputs is not None:
        _require_all(inputs, _ELEM_BYTES * n, "inputs", elems=True)
    if scratch is not None:
        _require_all(scratch, _scratch_bytes(P, n), "scratch")
    if outputs is not None:
        _require_all(outputs, _ELEM_BYTES * n, "outputs", elems=True)
    if ctrl is not None:
        _require(ctrl, AR_CTRL_BYTES, "ctrl")


def ar_packet_fused(inputs: Sequence, scratch: Sequence, outputs: Sequence, flag: int, ctrl,
                    rank_lo: int = 0, rank_hi: int | None = None, n: int | None = None,
                    max_spins: int = 0, stream=None) -> None:
    P = len(inputs)
    if len(scratch) != P or len(outputs) != P:
        raise ValueError("the packet path needs P inputs, P scratch buffers and P outputs")
    hi = P if rank_hi is None else rank_hi
    n = _n(n, inputs)
    _packet_buffers(P, n, inputs, scratch, outputs, ctrl)
    _check(lib().ar_packet_fused(_ptrs(inputs), _ptrs(scratch), _ptrs(outputs), P, rank_lo, hi,
                                 n, flag, _addr(ctrl), max_spins, _stream(stream)),
           "ar_packet_fused")


def ar_reduce_scatter_share(inputs: Sequence, out, rank: int, recvcount: int | None = None,
                            stream=None) -> None:
    P = len(inputs)
    if recvcount is None and isinstance(out, int):
        raise ValueError("recvcount is required when the output is a raw address")
    rc = _numel(out) if recvcount is None else int(recvcount)
    _require_all(inputs, _ELEM_BYTES * P * rc, "inputs", elems=True)
    _require(out, _ELEM_BYTES * rc, "out", elems=True)
    _check(lib().ar_reduce_scatter_share(_ptrs(inputs), _addr(out), P, rank, rc, _stream(stream)),
           "ar_reduce_scatter_share")


def ar_packet_fused_epoch(inputs: Sequence, scratch: Sequence, outputs: Sequence, ctrl,
                          rank_lo: int = 0, rank_hi: int | None = None, n: int | None = None,
                          max_spins: int = 0, stream=None) -> None:
    P = len(inputs)
    if len(scratch) != P or len(outputs) != P:
        raise ValueError("the packet path needs P inputs, P scratch buffers and P outputs")
    hi = P if rank_hi is None else rank_hi
    n = _n(n, inputs)
    _packet_buffers(P, n, inputs, scratch, outputs, ctrl)
    _check(lib().ar_packet_fused_epoch(_ptrs(inputs), _ptrs(scratch), _ptrs(outputs), P, rank_lo,
                                       hi, n, _addr(ctrl), max_spins, _stream(stream)),
           "ar_packet_fused_epoch")


def ar_packet_fused_noalloc(inputs: Sequence, outputs: Sequence, status=None,
                            n: int | None = None, max_spins: int = 0, stream=None) -> None:
    """The fused packet share of all P ranks with the library's static scratch
    (nothing is allocated).  `status`: None, or a device int32 that receives
    AR_OK or AR_ETIMEDOUT when the call completes."""
    P = len(inputs)
    if len(outputs) != P:
        raise ValueError("the packet path needs P inputs and P outputs")
    n = _n(n, inputs)
    _packet_buffers(P, n, inputs, None, outputs)
    _require(status, 4, "status", word=4)
    _check(lib().ar_packet_fused_noalloc(_ptrs(inputs), _ptrs(outputs), P, n,
                                         0 if status is None else _addr(status), max_spins,
                                         _stream(stream)), "ar_packet_fused_noalloc")


def ar_packet_send(inputs: Sequence, scratch: Sequence, flag: int, rank_lo: int = 0,
                   rank_hi: int | None = None, n: int | None = None, stream=None) -> None:
    P = len(inputs)
    if len(scratch) != P:
        raise ValueError("need P scratch buffers")
    hi = P if rank_hi is None else rank_hi
    n = _n(n, inputs)
    _packet_buffers(P, n, inputs, scratch)
    _check(lib().ar_packet_send(_ptrs(inputs), _ptrs(scratch), P, rank_lo, hi, n, flag,
                                _stream(stream)), "ar_packet_send")


def ar_packet_recv_reduce_send(scratch: Sequence, n: int, flag: int, ctrl, rank_lo: int = 0,
                               rank_hi: int | None = None, max_spins: int = 0,
                               stream=None) -> None:
    P = len(scratch)
    hi = P if rank_hi is None else rank_hi
    n = int(n)
    _packet_buffers(P, n, None, scratch, None, ctrl)
    _check(lib().ar_packet_recv_reduce_send(_ptrs(scratch), P, rank_lo, hi, n, flag,
                                            _addr(ctrl), max_spins, _stream(stream)),
           "ar_packet_recv_reduce_send")


def ar_packet_recv(scratch: Sequence, outputs: Sequence, flag: int, ctrl, rank_lo: int = 0,
                   rank_hi: int | None = None, n: int | None = None, max_spins: int = 0,
                   stream=None) -> None:
    P = len(scratch)
    if len(outputs) != P:
        raise ValueError("need P outputs")
    hi = P if rank_hi is None else rank_hi
    n = _n(n, outputs)
    _packet_buffers(P, n, None, scratch, outputs, ctrl)
    _check(lib().ar_packet_recv(_ptrs(scratch), _ptrs(outputs), P, rank_lo, hi, n, flag,
                                _addr(ctrl), max_spins, _stream(stream)), "ar_packet_recv")


def ar_slice_range(P: int, rank: int, n: int) -> tuple:
    b, e = ctypes.c_int64(), ctypes.c_int64()
    _check(lib().ar_slice_range(P, rank, n, ctypes.byref(b), ctypes.byref(e)), "ar_slice_range")
    return b.value, e.value


def ar_packet_slot_packets(P: int, n: int) -> int:
    v = int(lib().ar_packet_slot_packets(P, n))
    _check(min(v, 0), "ar_packet_slot_packets")
    return v


def ar_packet_scratch_bytes(P: int, n: int) -> int:
    v = int(lib().ar_packet_scratch_bytes(P, n))
    _check(min(v, 0), "ar_packet_scratch_bytes")
    return v


def ar_strerror(code: int) -> str:
    return lib().ar_strerror(code).decode()


def ar_noop(stream=None) -> None:
    _check(lib().ar_noop(_stream(stream)), "ar_noop")


def ar_probe_traffic(kind: int, inputs: Sequence, outputs: Sequence, threads: int = 64,
                     unroll: int = 1, blocks: int = 0, policy: int = 0, n: int | None = None,
                     stream=None) -> None:
    """Measurement helper: read (kind 0), write (1) or copy (2) the 2P
    buffers of a write-mode call with the reduce kernels' accesses."""
    if len(outputs) != len(inputs):
        raise ValueError("one output per input")
    n = _n(n, inputs)
    _require_all(inputs, _ELEM_BYTES * n, "inputs", elems=True)
    _require_all(outputs, _ELEM_BYTES * n, "outputs", elems=True)
    _check(lib().ar_probe_traffic(kind, _ptrs(inputs), _ptrs(outputs), len(inputs), n, threads,
                                  unroll, blocks, policy, _stream(stream)), "ar_probe_traffic")


def ar_set_reduce_tuning(unroll: int = 0, threads: int = 0, max_blocks: int = 0,
                         schedule: int = 0) -> None:
    _check(lib().ar_set_reduce_tuning(unroll, threads, max_blocks, schedule),
           "ar_set_reduce_tuning")


def ar_set_packet_tuning(per_rank: int = 0, words_per_lane: int = 0, schedule: int = 0) -> None:
    _check(lib().ar_set_packet_tuning(per_rank, words_per_lane, schedule), "ar_set_packet_tuning")
