"""Helpers shared by the GPU parity tests (test code, not the product).

The simulated all-to-all here is a test stand-in for the collective that a
multi-GPU run would perform; the library itself never exchanges data.
"""

from __future__ import annotations

import sys

import numpy as np
import torch

DEV = "cuda"
CANARY_BITS = 0x5A5A  # 16-bit pattern written past the end of every output


def log(msg: str):
    """Name the case before each GPU step (flushed, so a fault shows it)."""
    print(f"[gpu-case] {msg}", file=sys.stderr, flush=True)


def f64(t: torch.Tensor) -> np.ndarray:
    """Exact float64 image of a bf16 / fp32 tensor."""
    return t.detach().float().cpu().numpy().astype(np.float64)


def bits(t: torch.Tensor) -> np.ndarray:
    """Raw bit patterns (for bit-exact comparisons)."""
    t = t.detach().contiguous().cpu()
    if t.element_size() == 2:
        return t.view(torch.int16).numpy()
    return t.view(torch.int32).numpy()


class Guarded:
    """A device tensor followed by a canary band, to catch writes past the end."""

    def __init__(self, shape, dtype, pad_elems: int = 4096, fill_bits: int | None = None):
        n = int(np.prod(shape)) if len(shape) else 1
        self.n = n
        self.pad = pad_elems
        self.raw = torch.empty(n + pad_elems, dtype=dtype, device=DEV)
        ibits = torch.int16 if self.raw.element_size() == 2 else torch.int32
        canary = CANARY_BITS if ibits == torch.int16 else (CANARY_BITS << 16) | CANARY_BITS
        self.raw.view(ibits).fill_(canary)
        if fill_bits is not None:
            self.raw[:n].view(ibits).fill_(fill_bits)
        self.t = self.raw[:n].view(*shape)
        self._ibits = ibits
        self._canary = canary

    def canary_ok(self) -> bool:
        tail = self.raw[self.n:].view(self._ibits)
        return bool((tail == self._canary).all().item())


def simulate_all_to_all(sends):
    """recv_r[p] = send_p[r] for a list of per-rank send buffers [U, ...]."""
    U = len(sends)
    return [torch.stack([sends[p][r] for p in range(U)]).contiguous() for r in range(U)]


def max_abs(a: np.ndarray, b: np.ndarray) -> float:
    if a.size == 0:
        return 0.0
    return float(np.max(np.abs(a - b)))


def bf16_half_spacing(x: np.ndarray) -> np.ndarray:
    """Half the distance between adjacent bf16 values around |x| (8
    significand bits): for |x| in [2^(E-1), 2^E) the spacing is 2^(E-8)."""
    _, e = np.frexp(np.abs(x))
    return np.where(x == 0, 0.0, np.ldexp(1.0, e - 9))
