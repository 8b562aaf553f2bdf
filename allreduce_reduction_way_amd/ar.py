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
AR_OK, AR_EINVAL, AR_EALIAS, AR_ELAUNCH, AR_ETIMEDOUT = 0, -1, -2, -3, -4
AR_CTRL_BYTES = 64
AR_DEFAULT_MAX_SPINS = 1 << 22

_NAMES = {AR_OK: "AR_OK", AR_EINVAL: "AR_EINVAL", AR_EALIAS: "AR_EALIAS",
          AR_ELAUNCH: "AR_ELAUNCH", AR_ETIMEDOUT: "AR_ETIMEDOUT"}


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
            "ar_packet_send": (i32, [ar_ptrs, ar_ptrs, i32, i32, i32, i64, u32, vp]),
            "ar_packet_recv_reduce_send": (i32, [ar_ptrs, i32, i32, i32, i64, u32, vp, u64, vp]),
            "ar_packet_recv": (i32, [ar_ptrs, ar_ptrs, i32, i32, i32, i64, u32, vp, u64, vp]),
            "ar_slice_range": (i32, [i32, i32, i64, ctypes.POINTER(i64), ctypes.POINTER(i64)]),
            "ar_packet_slot_packets": (i64, [i32, i64]),
            "ar_packet_scratch_bytes": (i64, [i32, i64]),
            "ar_strerror": (ctypes.c_char_p, [i32]),
            "ar_noop": (i32, [vp]),
            "ar_set_reduce_tuning": (i32, [i32, i32, i32]),
            "ar_set_packet_tuning": (i32, [i32, i32, i32]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype, fn.argtypes = res, args
        _lib = L
    return _lib


# ---------------------------------------------------------------- marshalling

def _addr(buf) -> int:
    """Device address of a torch CUDA tensor, or an int taken as an address."""
    if isinstance(buf, int):
        return buf
    if getattr(buf, "is_cuda", False):
        return int(buf.data_ptr())
    raise TypeError(f"expected a CUDA tensor or a device address, got {type(buf).__name__}")


def _numel(buf) -> int:
    return int(buf.numel())


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
    return _numel(bufs[0]) if n is None else int(n)


def _check(rc: int, what: str) -> None:
    if rc != AR_OK:
        raise ArError(rc, what)


# ------------------------------------------------------------------ entry points

def ar_oneshot_sum(inputs: Sequence, out, n: int | None = None, stream=None) -> None:
    _check(lib().ar_oneshot_sum(_ptrs(inputs), _addr(out), len(inputs), _n(n, inputs),
                                _stream(stream)), "ar_oneshot_sum")


def ar_oneshot_write_bcast(inputs: Sequence, outputs: Sequence, n: int | None = None,
                           stream=None) -> None:
    if len(outputs) != len(inputs):
        raise ValueError("write mode needs one output per input")
    _check(lib().ar_oneshot_write_bcast(_ptrs(inputs), _ptrs(outputs), len(inputs),
                                        _n(n, inputs), _stream(stream)), "ar_oneshot_write_bcast")


def ar_twoshot_share(inputs: Sequence, outputs: Sequence, rank: int, n: int | None = None,
                     stream=None) -> None:
    if len(outputs) != len(inputs):
        raise ValueError("the two-shot share needs one output per input")
    _check(lib().ar_twoshot_share(_ptrs(inputs), _ptrs(outputs), len(inputs), rank,
                                  _n(n, inputs), _stream(stream)), "ar_twoshot_share")


def ar_ll_packets(n: int) -> int:
    return int(lib().ar_ll_packets(n))


def ar_ll_encode(src, dst_pkts, flag: int, n: int | None = None, stream=None) -> None:
    _check(lib().ar_ll_encode(_addr(src), _addr(dst_pkts), _n(n, [src]), flag, _stream(stream)),
           "ar_ll_encode")


def ar_ll_decode(src_pkts, dst, flag: int, ctrl, n: int | None = None, max_spins: int = 0,
                 stream=None) -> None:
    _check(lib().ar_ll_decode(_addr(src_pkts), _addr(dst), _n(n, [dst]), flag,
                              0 if ctrl is None else _addr(ctrl),
                              max_spins, _stream(stream)), "ar_ll_decode")


def ar_packet_fused(inputs: Sequence, scratch: Sequence, outputs: Sequence, flag: int, ctrl,
                    rank_lo: int = 0, rank_hi: int | None = None, n: int | None = None,
                    max_spins: int = 0, stream=None) -> None:
    P = len(inputs)
    if len(scratch) != P or len(outputs) != P:
        raise ValueError("the packet path needs P inputs, P scratch buffers and P outputs")
    hi = P if rank_hi is None else rank_hi
    _check(lib().ar_packet_fused(_ptrs(inputs), _ptrs(scratch), _ptrs(outputs), P, rank_lo, hi,
                                 _n(n, inputs), flag, _addr(ctrl), max_spins, _stream(stream)),
           "ar_packet_fused")


def ar_reduce_scatter_share(inputs: Sequence, out, rank: int, recvcount: int | None = None,
                            stream=None) -> None:
    P = len(inputs)
    rc = _numel(out) if recvcount is None else int(recvcount)
    _check(lib().ar_reduce_scatter_share(_ptrs(inputs), _addr(out), P, rank, rc, _stream(stream)),
           "ar_reduce_scatter_share")


def ar_packet_fused_epoch(inputs: Sequence, scratch: Sequence, outputs: Sequence, ctrl,
                          rank_lo: int = 0, rank_hi: int | None = None, n: int | None = None,
                          max_spins: int = 0, stream=None) -> None:
    P = len(inputs)
    if len(scratch) != P or len(outputs) != P:
        raise ValueError("the packet path needs P inputs, P scratch buffers and P outputs")
    hi = P if rank_hi is None else rank_hi
    _check(lib().ar_packet_fused_epoch(_ptrs(inputs), _ptrs(scratch), _ptrs(outputs), P, rank_lo,
                                       hi, _n(n, inputs), _addr(ctrl), max_spins, _stream(stream)),
           "ar_packet_fused_epoch")


def ar_packet_send(inputs: Sequence, scratch: Sequence, flag: int, rank_lo: int = 0,
                   rank_hi: int | None = None, n: int | None = None, stream=None) -> None:
    P = len(inputs)
    if len(scratch) != P:
        raise ValueError("need P scratch buffers")
    hi = P if rank_hi is None else rank_hi
    _check(lib().ar_packet_send(_ptrs(inputs), _ptrs(scratch), P, rank_lo, hi, _n(n, inputs),
                                flag, _stream(stream)), "ar_packet_send")


def ar_packet_recv_reduce_send(scratch: Sequence, n: int, flag: int, ctrl, rank_lo: int = 0,
                               rank_hi: int | None = None, max_spins: int = 0,
                               stream=None) -> None:
    P = len(scratch)
    hi = P if rank_hi is None else rank_hi
    _check(lib().ar_packet_recv_reduce_send(_ptrs(scratch), P, rank_lo, hi, int(n), flag,
                                            _addr(ctrl), max_spins, _stream(stream)),
           "ar_packet_recv_reduce_send")


def ar_packet_recv(scratch: Sequence, outputs: Sequence, flag: int, ctrl, rank_lo: int = 0,
                   rank_hi: int | None = None, n: int | None = None, max_spins: int = 0,
                   stream=None) -> None:
    P = len(scratch)
    if len(outputs) != P:
        raise ValueError("need P outputs")
    hi = P if rank_hi is None else rank_hi
    _check(lib().ar_packet_recv(_ptrs(scratch), _ptrs(outputs), P, rank_lo, hi, _n(n, outputs),
                                flag, _addr(ctrl), max_spins, _stream(stream)), "ar_packet_recv")


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


def ar_set_reduce_tuning(unroll: int = 0, threads: int = 0, max_blocks: int = 0) -> None:
    _check(lib().ar_set_reduce_tuning(unroll, threads, max_blocks), "ar_set_reduce_tuning")


def ar_set_packet_tuning(per_rank: int = 0, words_per_lane: int = 0, schedule: int = 0) -> None:
    _check(lib().ar_set_packet_tuning(per_rank, words_per_lane, schedule), "ar_set_packet_tuning")
