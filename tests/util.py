"""Shared helpers for the GPU parity tests (comparison only; no arithmetic of
the method lives here)."""
import sys

import numpy as np
import torch


def log(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu", torch.float64).numpy()


def assert_bitexact(got: torch.Tensor, ref: np.ndarray, what: str = ""):
    g = f64(got)
    ref = np.asarray(ref, np.float64)
    assert g.shape == ref.shape, (what, g.shape, ref.shape)
    bad = np.flatnonzero(g != ref)
    assert bad.size == 0, f"{what}: {bad.size} mismatches, first at {np.unravel_index(bad[0], g.shape)}: " \
                          f"{g.flat[bad[0]]} vs {ref.flat[bad[0]]}"


def normwise_err(got, ref) -> float:
    g = f64(got) if isinstance(got, torch.Tensor) else np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    return float(np.max(np.abs(g - ref)) / max(np.max(np.abs(ref)), 1e-300))


def assert_normwise(got, ref, tol: float = 1e-2, what: str = ""):
    """The acceptance criterion for bf16 work: max|y - r| / max|r| <= tol
    against the float64 oracle."""
    e = normwise_err(got, ref)
    log(f"  {what}: normwise max rel err {e:.3e} (tol {tol:g})")
    assert e <= tol, f"{what}: normwise error {e:.3e} > {tol}"
    return e


def assert_within(got, ref, bound, what: str = ""):
    """Elementwise |y - r| <= bound (bound derived from the arithmetic)."""
    g = f64(got) if isinstance(got, torch.Tensor) else np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    bound = np.broadcast_to(np.asarray(bound, np.float64), ref.shape)
    err = np.abs(g - ref)
    bad = np.flatnonzero(err > bound)
    assert bad.size == 0, (f"{what}: {bad.size} of {ref.size} outside the bound; worst ratio "
                           f"{np.max(err / np.maximum(bound, 1e-300)):.3g} at {np.unravel_index(bad[0], ref.shape)}")


# Elementwise bounds derived from the arithmetic (fp32 accumulation of exact
# bf16 x bf16 products; RNE rounding to bf16 on store).
U32 = 2.0 ** -24      # unit roundoff of float32
U16 = 2.0 ** -8       # unit roundoff of bfloat16


def gemm_bound(x: np.ndarray, w: np.ndarray, ref: np.ndarray, out_bf16: bool) -> np.ndarray:
    K = x.shape[1]
    acc = 1.01 * K * U32 * (np.abs(x) @ np.abs(w).T)
    if out_bf16:
        return U16 * (np.abs(ref) + acc) + acc
    return acc
