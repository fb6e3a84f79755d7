"""Seeded synthetic inputs shared by the tests, the benchmark and the oracle side.

This module holds no arithmetic of the method: it only draws random tensors.
Values are drawn in fp32 and cast to the working dtype with round-to-nearest-
even, so the GPU path and the oracle receive bit-identical arrays (the oracle
upcasts them exactly to fp64).

Seed recipe, one independent stream per tensor:
    seed = 1_000_000 * workload + 10_000 * block + 100 * step + tensor_id
with tensor ids Q=0, K=1, V=2, S=3, lengths=4.  On ``device="cpu"`` the stream is
torch's CPU generator; on a GPU device it is torch's device generator (a
different, equally deterministic stream, used only where the host copy would be
too large to draw quickly).
"""
from __future__ import annotations

import torch

TENSOR_Q, TENSOR_K, TENSOR_V, TENSOR_S, TENSOR_LEN = 0, 1, 2, 3, 4


def seed_of(workload: int, block: int = 0, step: int = 0, tensor: int = 0) -> int:
    return 1_000_000 * workload + 10_000 * block + 100 * step + tensor


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def normal(shape, seed: int, std: float = 1.0, dtype=torch.bfloat16, device="cpu") -> torch.Tensor:
    """N(0, std^2) drawn in fp32, then rounded (RNE) to ``dtype``."""
    x = torch.randn(tuple(shape), generator=_gen(seed, device), dtype=torch.float32, device=device)
    if std != 1.0:
        x.mul_(std)
    return x.to(dtype)


def uniform_int(n: int, lo: int, hi: int, seed: int) -> torch.Tensor:
    """n integers uniform on [lo, hi] inclusive (int64, CPU)."""
    return torch.randint(lo, hi + 1, (n,), generator=_gen(seed, "cpu"), dtype=torch.int64)


def cu_from_lengths(lengths) -> torch.Tensor:
    """Packed-sequence offsets [n+1] (int64, CPU) from per-request lengths."""
    lengths = torch.as_tensor(lengths, dtype=torch.int64)
    cu = torch.zeros(lengths.numel() + 1, dtype=torch.int64)
    cu[1:] = torch.cumsum(lengths, 0)
    return cu
