"""Storage-to-float64 conversion and the log-normaliser, written for the oracle alone."""

import numpy as np


def as_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact upcast of stored values: bf16 bits (uint16) or float32 -> float64."""
    if dtype == "bf16":
        assert a.dtype == np.uint16
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    if dtype == "f32":
        return np.asarray(a, dtype=np.float32).astype(np.float64)
    raise ValueError(dtype)


def logsumexp(l: np.ndarray, axis: int = -1) -> np.ndarray:
    """log sum exp along an axis, shifted by the maximum (entries may be -inf)."""
    m = np.max(l, axis=axis, keepdims=True)
    m_safe = np.where(np.isfinite(m), m, 0.0)
    s = np.sum(np.exp(l - m_safe), axis=axis, keepdims=True)
    return np.squeeze(m_safe + np.log(s), axis=axis)
