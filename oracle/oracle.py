"""ctypes wrapper around liboracle.so (see oracle.c for the definitions).

Test infrastructure only: the tests, the smoke check and the benchmark's CPU
baseline call this; the library's product path never does.

All buffers are numpy ``uint16`` arrays holding bf16 bit patterns; packet
buffers are ``uint32`` arrays, four words per 16-byte packet.
"""
from __future__ import annotations

import ctypes
import pathlib

import numpy as np

_LIB_PATH = pathlib.Path(__file__).resolve().with_name("liboracle.so")
_lib = None

ORC_OK, ORC_EINVAL, ORC_EFLAG, ORC_ENOMEM, ORC_EFPENV = 0, -1, -2, -3, -5


class OracleError(RuntimeError):
    pass


def _load():
    global _lib
    if _lib is None:
        if not _LIB_PATH.exists():
            raise OracleError(f"{_LIB_PATH} is not built; run oracle/build.py")
        lib = ctypes.CDLL(str(_LIB_PATH))
        P16 = ctypes.POINTER(ctypes.c_void_p)
        i64, i32, u32, vp = ctypes.c_int64, ctypes.c_int, ctypes.c_uint32, ctypes.c_void_p
        sig = {
            "orc_oneshot_sum": (i32, [P16, i32, i64, vp]),
            "orc_write_bcast": (i32, [P16, i32, i64, P16]),
            "orc_slice": (i32, [i32, i64, i32, ctypes.POINTER(i64), ctypes.POINTER(i64)]),
            "orc_twoshot_share": (i32, [P16, i32, i64, i32, P16]),
            "orc_reduce_scatter": (i32, [P16, i32, i64, i32, vp]),
            "orc_ll_packets": (i64, [i64]),
            "orc_ll_encode": (i32, [vp, i64, u32, vp]),
            "orc_ll_decode": (i32, [vp, i64, u32, vp]),
            "orc_packet_slot_packets": (i64, [i32, i64]),
            "orc_packet_scratch_bytes": (i64, [i32, i64]),
            "orc_packet_fused": (i32, [P16, i32, i64, u32, P16, P16]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(lib, name)
            fn.restype, fn.argtypes = res, args
        _lib = lib
    return _lib


def _check(rc: int, what: str):
    if rc != ORC_OK:
        raise OracleError(f"{what} failed with code {rc}")


def _ptrs(arrays):
    arr = (ctypes.c_void_p * len(arrays))(*[a.ctypes.data for a in arrays])
    return ctypes.cast(arr, ctypes.POINTER(ctypes.c_void_p)), arr


def _as_inputs(xs):
    xs = [np.ascontiguousarray(x, dtype=np.uint16) for x in xs]
    n = xs[0].size
    if any(x.size != n for x in xs):
        raise ValueError("all inputs must have the same length")
    return xs, n


def oneshot_sum(xs) -> np.ndarray:
    """y[i] = bf16_rne(x_0[i] + x_1[i] + ... + x_{P-1}[i]) in binary32, rank order."""
    xs, n = _as_inputs(xs)
    y = np.empty(n, dtype=np.uint16)
    p, keep = _ptrs(xs)
    _check(_load().orc_oneshot_sum(p, len(xs), n, y.ctypes.data), "orc_oneshot_sum")
    return y


def write_bcast(xs) -> list:
    """P identical outputs, each equal to oneshot_sum(xs)."""
    xs, n = _as_inputs(xs)
    outs = [np.empty(n, dtype=np.uint16) for _ in xs]
    p, k1 = _ptrs(xs)
    q, k2 = _ptrs(outs)
    _check(_load().orc_write_bcast(p, len(xs), n, q), "orc_write_bcast")
    return outs


def slice_range(P: int, n: int, r: int) -> tuple:
    b, e = ctypes.c_int64(), ctypes.c_int64()
    _check(_load().orc_slice(P, n, r, ctypes.byref(b), ctypes.byref(e)), "orc_slice")
    return b.value, e.value


def twoshot_share(xs, r: int, prior_outs) -> list:
    """Copies of prior_outs with rank r's reduced slice written into each."""
    xs, n = _as_inputs(xs)
    outs = [np.array(o, dtype=np.uint16, copy=True) for o in prior_outs]
    if len(outs) != len(xs) or any(o.size != n for o in outs):
        raise ValueError("need P outputs of length n")
    p, k1 = _ptrs(xs)
    q, k2 = _ptrs(outs)
    _check(_load().orc_twoshot_share(p, len(xs), n, r, q), "orc_twoshot_share")
    return outs


def reduce_scatter(xs, r: int) -> np.ndarray:
    """Rank r's block of the sum: each input holds P blocks of n / P elements."""
    xs, n = _as_inputs(xs)
    P = len(xs)
    if n % P:
        raise ValueError("reduce-scatter inputs hold P equal blocks")
    rc = n // P
    y = np.empty(rc, dtype=np.uint16)
    p, keep = _ptrs(xs)
    _check(_load().orc_reduce_scatter(p, P, rc, r, y.ctypes.data), "orc_reduce_scatter")
    return y


def ll_packets(n: int) -> int:
    return int(_load().orc_ll_packets(n))


def ll_encode(y, flag: int) -> np.ndarray:
    y = np.ascontiguousarray(y, dtype=np.uint16)
    pk = np.zeros(4 * ll_packets(y.size), dtype=np.uint32)
    _check(_load().orc_ll_encode(y.ctypes.data, y.size, flag, pk.ctypes.data), "orc_ll_encode")
    return pk


def ll_decode(pk, n: int, flag: int) -> np.ndarray:
    pk = np.ascontiguousarray(pk, dtype=np.uint32)
    if pk.size < 4 * ll_packets(n):
        raise ValueError("packet buffer too short")
    y = np.empty(n, dtype=np.uint16)
    _check(_load().orc_ll_decode(pk.ctypes.data, n, flag, y.ctypes.data), "orc_ll_decode")
    return y


def packet_slot_packets(P: int, n: int) -> int:
    return int(_load().orc_packet_slot_packets(P, n))


def packet_scratch_bytes(P: int, n: int) -> int:
    return int(_load().orc_packet_scratch_bytes(P, n))


def packet_fused(xs, flag: int, scratch_images) -> tuple:
    """One fused call for all P ranks.

    Returns (outs, new_scratch_images); the images are copies of the given
    per-rank scratch images (uint8 arrays of packet_scratch_bytes bytes) with
    this call's packets written in.
    """
    xs, n = _as_inputs(xs)
    P = len(xs)
    nbytes = packet_scratch_bytes(P, n)
    imgs = [np.array(s, dtype=np.uint8, copy=True) for s in scratch_images]
    if len(imgs) != P or any(s.size != nbytes for s in imgs):
        raise ValueError(f"need P scratch images of {nbytes} bytes")
    outs = [np.zeros(n, dtype=np.uint16) for _ in range(P)]
    p, k1 = _ptrs(xs)
    s, k2 = _ptrs(imgs)
    q, k3 = _ptrs(outs)
    _check(_load().orc_packet_fused(p, P, n, flag, s, q), "orc_packet_fused")
    return outs, imgs
