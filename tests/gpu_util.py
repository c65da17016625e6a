"""Moving seeded workloads to the GPU for the parity tests (no arithmetic)."""

from __future__ import annotations

import numpy as np
import torch

# Query positions checked at full size: tile and bias-cell edges, the
# variant rows, the end, plus a few seeded random positions.
def sample_rows(S, seed=0, extra=12):
    base = [0, 1, 15, 16, 31, 32, 63, 64, 65, S // 2 - 1, S // 2, S - 65, S - 64, S - 17,
            S - 16, S - 1]
    if S > 4101:
        base += list(range(4090, 4102))
    rng = np.random.Generator(np.random.PCG64(seed + S))
    base += rng.integers(0, S, size=extra).tolist()
    return np.array(sorted(set(int(r) for r in base if 0 <= r < S)))


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
