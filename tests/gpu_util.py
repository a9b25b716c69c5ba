"""Shared helpers for the GPU parity tests: tolerances and comparisons.

Tolerances (written here, used by every parity test):
* O: max |gpu - oracle| <= 2e-3 for fp16 outputs, <= 1.6e-2 for bf16 outputs,
  over every compared element; any NaN or Inf fails.
* lse: |gpu - oracle| <= 1e-4 * max(1, |oracle|) (relative, with an absolute
  floor of 1e-4 near zero where a pure relative bound is ill-posed).
"""

from __future__ import annotations

import numpy as np
import torch

O_TOL = {torch.float16: 2e-3, torch.bfloat16: 1.6e-2}
LSE_REL = 1e-4


def to64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def check_o(gpu: torch.Tensor, ref: np.ndarray, dtype, what: str = "O"):
    g = to64(gpu)
    assert g.shape == ref.shape, (what, g.shape, ref.shape)
    assert np.isfinite(g).all(), f"{what}: non-finite values in GPU output"
    err = np.abs(g - ref)
    worst = np.unravel_index(np.argmax(err), err.shape)
    tol = O_TOL[dtype]
    assert err.max() <= tol, (f"{what}: max |err| {err.max():.3e} > {tol} at {worst} "
                              f"(gpu {g[worst]:.6f}, oracle {ref[worst]:.6f})")
    return float(err.max())


def check_lse(gpu: torch.Tensor, ref: np.ndarray, what: str = "lse"):
    g = to64(gpu)
    assert g.shape == ref.shape, (what, g.shape, ref.shape)
    assert np.isfinite(g).all(), f"{what}: non-finite values"
    bound = LSE_REL * np.maximum(1.0, np.abs(ref))
    err = np.abs(g - ref)
    ratio = err / bound
    worst = np.unravel_index(np.argmax(ratio), ratio.shape)
    assert (err <= bound).all(), f"{what}: |err| {err[worst]:.3e} > {bound[worst]:.3e} at {worst}"
    return float(ratio.max())


WAVE_ROWS = 32  # query rows one prefill wave owns


def sample_rows(N: int, causal: bool, rng: np.random.Generator, count: int = 24) -> np.ndarray:
    """Query rows to compare at full size: both ends, tile edges, random rows,
    and one random row in every 32-row slice, so that every wave of every
    query block of the launch is compared element by element."""
    fixed = [0, 1, 31, 32, 63, 64, 127, 128, 129, N // 2, N - 129, N - 128, N - 65, N - 64, N - 2, N - 1]
    rnd = rng.integers(0, N, size=max(0, count - len(fixed)))
    starts = np.arange(0, N, WAVE_ROWS)
    per_slice = starts + rng.integers(0, WAVE_ROWS, size=starts.size)
    rows = np.unique(np.clip(np.concatenate([fixed, rnd, per_slice]), 0, N - 1))
    assert set((rows // WAVE_ROWS).tolist()) == set(range((N + WAVE_ROWS - 1) // WAVE_ROWS))
    return rows
