"""Helpers shared by the GPU parity tests (device transfer and comparisons)."""

from __future__ import annotations

import numpy as np
import pytest


def require_gpu():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bit_block_scaled_bf16_amd as nv

    nv.load()  # raises when the library is missing: no silent fallback
    return torch


def to_device(x: np.ndarray, dtype: str):
    """float32 numpy (bf16-representable for dtype 'bf16') -> device tensor."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    if dtype == "bf16":
        t = t.to(torch.bfloat16)
    return t.cuda()


def host(t) -> np.ndarray:
    import torch

    torch.cuda.synchronize()
    return t.detach().cpu().numpy()


def e2m1_step_distance(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """Distance in E2M1 grid steps between two code arrays (signed line)."""
    def line(c):
        c = c.astype(np.int64)
        mag = c & 7
        return np.where((c & 8) != 0, -mag, mag)

    return np.abs(line(a) - line(b))


def announce(msg: str) -> None:
    print(msg, flush=True)
