"""Parity bounds and the elementwise checker shared by the oracle and GPU tests.

Bounds (elementwise, on y and on the last state):
  * float32 inputs/outputs:                 |x - x_ref| <= 1e-4 * (1 + |x_ref|)
  * bfloat16 inputs/outputs, fp32 state:    |x - x_ref| <= 2e-2 * (1 + |x_ref|)
"""
import numpy as np

TOL = {"f32": 1e-4, "bf16": 2e-2}


def normalised_error(x, ref) -> np.ndarray:
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return np.abs(x - ref) / (1.0 + np.abs(ref))


def max_normalised_error(x, ref) -> float:
    e = normalised_error(x, ref)
    if e.size == 0:
        return 0.0
    # NaN anywhere (in x but not ref, or vice versa) is a failure
    nan_mismatch = np.isnan(np.asarray(x, dtype=np.float64)) != np.isnan(np.asarray(ref, dtype=np.float64))
    if nan_mismatch.any():
        return float("inf")
    return float(np.nanmax(e))


def within(x, ref, tol) -> bool:
    return max_normalised_error(x, ref) <= tol


def assert_within(x, ref, tol, what=""):
    err = max_normalised_error(x, ref)
    assert err <= tol, f"{what}: max normalised error {err:.3e} exceeds {tol:.1e}"
    return err


def scan_only_relative_error(y, y_ref, direct_ref) -> float:
    """||y - y_ref||_2 / ||y_ref - direct_ref||_2 where direct_ref is D*u*silu(z) (the non-scan part)."""
    y = np.asarray(y, dtype=np.float64)
    y_ref = np.asarray(y_ref, dtype=np.float64)
    den = np.linalg.norm(y_ref - np.asarray(direct_ref, dtype=np.float64))
    return float(np.linalg.norm(y - y_ref) / max(den, 1e-300))
