"""Moving seeded workloads to the GPU for the parity tests (no arithmetic)."""

from __future__ import annotations

import numpy as np
import torch

from parity import sample_rows  # noqa: F401  (re-exported for the GPU tests)


def to_gpu(a: np.ndarray, device="cuda") -> torch.Tensor:
    """uint16 arrays are BF16 bit patterns; float32 stays float32."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(a).to(device)


def to_host(t: torch.Tensor) -> np.ndarray:
    """GPU tensor -> float64 numpy (exact for bf16 and float32)."""
    return t.detach().float().cpu().numpy().astype(np.float64)


def upload(layer, device="cuda"):
    return {n: to_gpu(getattr(layer, n), device) for n in ("q", "k", "v", "pair", "weight")}
