"""Helpers for the GPU tests: host <-> device copies of bf16 bit patterns and
guard-banded device buffers (a sentinel before and after every output, so an
out-of-bounds write shows up as a changed guard)."""
from __future__ import annotations

import numpy as np
import torch

DEV = torch.device("cuda:0")
GUARD = 256          # elements of guard band on each side (512 bytes: keeps 256-B alignment)
SENTINEL = 0x5A5A


def to_dev(x: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.uint16).view(np.int16)).to(DEV)


def to_host(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy().view(np.uint16)


class Guarded:
    """A device buffer of n elements at element offset `shift` inside a
    guard-banded allocation filled with SENTINEL."""

    def __init__(self, n: int, shift: int = 0, fill: int = SENTINEL, init: np.ndarray | None = None):
        self.n, self.shift = n, shift
        total = GUARD + shift + n + GUARD
        host = np.full(total, fill, dtype=np.uint16)
        if init is not None:
            host[GUARD + shift: GUARD + shift + n] = init
        self.base = to_dev(host)
        self.view = self.base[GUARD + shift: GUARD + shift + n]
        self._fill = fill

    def host(self) -> np.ndarray:
        return to_host(self.view)

    def guards_intact(self) -> bool:
        h = to_host(self.base)
        lo = h[: GUARD + self.shift]
        hi = h[GUARD + self.shift + self.n:]
        return bool((lo == self._fill).all() and (hi == self._fill).all())


def ctrl_block() -> torch.Tensor:
    return torch.zeros(64, dtype=torch.uint8, device=DEV)


def ctrl_status(ctrl: torch.Tensor) -> int:
    return int(ctrl.view(torch.int32)[0].item())


def announce(msg: str) -> None:
    print(f"[gpu case] {msg}", flush=True)
