"""Parity measures for fp32 outputs.

Element-wise relative error is undefined near zero outputs under any change
of summation order, so the tolerance reads the relative error against
max(|oracle element|, rms(oracle)): e = max over elements of
|gpu - oracle| / max(|oracle|, rms(oracle)).  The tolerance is 1e-5.
"""
import numpy as np

TOL = 1e-5


def normalized_max_error(gpu: np.ndarray, ref: np.ndarray) -> float:
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    if ref.size == 0:
        return 0.0
    rms = float(np.sqrt(np.mean(ref * ref)))
    denom = np.maximum(np.abs(ref), rms)
    denom[denom == 0] = 1.0
    return float((np.abs(gpu - ref) / denom).max())


def report(gpu: np.ndarray, ref: np.ndarray) -> dict:
    g = np.asarray(gpu, np.float32)
    r = np.asarray(ref, np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        elem = np.abs(g.astype(np.float64) - r) / np.abs(r.astype(np.float64))
    elem = elem[np.isfinite(elem)]
    return {
        "normalized_max_error": normalized_max_error(g, r),
        "elementwise_max_rel": float(elem.max()) if elem.size else 0.0,
        "count_over_tol_elementwise": int((elem > TOL).sum()),
        "bit_identical_fraction": float((g.view(np.uint32) == r.view(np.uint32)).mean()) if g.size else 1.0,
    }
