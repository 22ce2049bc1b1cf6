"""Host <-> device plumbing for the GPU parity tests (no attention arithmetic)."""
from __future__ import annotations

import numpy as np
import torch

DEV = "cuda:0"

# Tolerances: bf16 and fp32 outputs within |gpu - oracle| <= ATOL + RTOL*|oracle|,
# natural-log LSE within LSE_TOL (absolute).
ATOL = 1e-2
RTOL = 1e-2
LSE_TOL = 1e-3


def to_dev(a: np.ndarray) -> torch.Tensor:
    """numpy -> cuda tensor; uint16 arrays are raw bf16 bits."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(DEV).view(torch.bfloat16)
    return torch.from_numpy(a).to(DEV)


def bits(t: torch.Tensor) -> np.ndarray:
    """Raw storage of a cuda tensor as numpy (bf16 -> uint16 bits)."""
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def check_close(got: np.ndarray, ref: np.ndarray, what: str, atol=ATOL, rtol=RTOL):
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite values in the GPU output"
    err = np.abs(got - ref)
    bound = atol + rtol * np.abs(ref)
    bad = err > bound
    if bad.any():
        i = np.unravel_index(np.argmax(err - bound), err.shape)
        raise AssertionError(f"{what}: {bad.sum()} of {bad.size} elements out of tolerance; "
                             f"worst at {i}: gpu {got[i]} oracle {ref[i]}")
    return float(err.max()) if err.size else 0.0


def check_lse(got: np.ndarray, ref: np.ndarray, what: str, tol=LSE_TOL):
    assert got.shape == ref.shape
    fin = np.isfinite(ref)
    assert np.array_equal(np.isfinite(got), fin), f"{what}: -inf pattern differs"
    assert np.array_equal(got[~fin], ref[~fin])
    if fin.any():
        e = np.abs(got[fin] - ref[fin]).max()
        assert e <= tol, f"{what}: lse error {e}"
        return float(e)
    return 0.0


def say(msg: str):
    """Print and flush a line naming the GPU case about to run."""
    print(msg, flush=True)
