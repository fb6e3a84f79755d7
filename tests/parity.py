"""Shared helpers of the GPU-vs-oracle parity tests.

Tolerance rule: for the fp32 worked example max |O_gpu - O_ref| <= 1e-5 (an
absolute bound at that example's own scale, |O| of order 1-10).  Other fp32
cases scale the same bound with the output: max |err| <= 1e-5 * max(1,
max |O_ref|); fp32 accumulation of the ~d + B terms of one output carries a
few units of 2^-24 relative to the largest partial sum, far inside it.  For
bf16 inputs with fp32 accumulation max |O_gpu - O_ref| <= 2e-2 * max |O_ref|,
the max taken over the whole output of the call (or over every sampled unit
when a full-size output is checked by sampling).  The same rule applies to
states.  O_ref is the oracle's unrounded fp64 result on the identical input
values.
"""
from __future__ import annotations

import numpy as np
import torch

BF16_REL = 2e-2
F32_ABS = 1e-5


def to64(t) -> np.ndarray:
    if isinstance(t, torch.Tensor):
        return t.detach().float().cpu().double().numpy()
    return np.asarray(t, dtype=np.float64)


def state_to_oracle(state: torch.Tensor) -> np.ndarray:
    """The library stores each d x d block transposed (row = value dim);
    the oracle uses S[f][c] (row = feature).  Pure layout change."""
    return to64(state).transpose(0, 1, 3, 2).copy()


def state_from_oracle(S: np.ndarray, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(S.transpose(0, 1, 3, 2))).float().to(device)


def max_err(gpu, ref) -> tuple[float, float]:
    g, r = to64(gpu), np.asarray(ref, dtype=np.float64)
    assert g.shape == r.shape, (g.shape, r.shape)
    return float(np.abs(g - r).max(initial=0.0)), float(np.abs(r).max(initial=0.0))


def assert_parity(gpu, ref, dtype, what="", f32_absolute=False) -> float:
    """Applies the tolerance rule; returns the achieved error ratio.
    ``f32_absolute`` selects the plain 1e-5 bound (the worked example)."""
    err, mag = max_err(gpu, ref)
    if dtype == torch.float32:
        bound = F32_ABS if f32_absolute else F32_ABS * max(1.0, mag)
        assert err <= bound, f"{what}: max abs err {err:.3e} > {bound:.3e} (max |ref| {mag:.3e})"
        return err
    bound = BF16_REL * mag
    assert err <= bound, f"{what}: max abs err {err:.3e} > {BF16_REL} * {mag:.3e}"
    return err / mag if mag > 0 else 0.0


def rows_mask(blk_lens, n_req, blk) -> np.ndarray:
    """[n_req, blk] True where row i < B_r."""
    lens = np.full(n_req, blk) if blk_lens is None else to64(blk_lens).astype(np.int64)
    return np.arange(blk)[None, :] < np.minimum(lens, blk)[:, None]
