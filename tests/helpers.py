"""Shared test helpers: tolerances and error metrics (no block arithmetic)."""
import numpy as np

# Tolerances for floating point parity, from the arithmetic:
#   fp32 path: true fp32 products with fp32 accumulation -> 1e-5;
#   bf16 path: bf16 storage of z, H and outputs with fp32 accumulation -> 2e-2.
TOL = {"f32": 1e-5, "bf16": 2e-2}


def scaled_max_err(got, ref):
    """max_j |g_j - r_j| / max(|r_j|, rms(r)).

    A relative error that stays meaningful where the reference is near zero:
    each denominator is at least the tensor's RMS and at most max|r|, so the
    value is never looser than the normwise max|g - r| / max|r|.
    """
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    if ref.size == 0:
        return 0.0
    rms = float(np.sqrt(np.mean(ref * ref)))
    den = np.maximum(np.abs(ref), rms)
    den = np.where(den == 0.0, 1.0, den)
    return float(np.max(np.abs(got - ref) / den))


def normwise_err(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if ref.size == 0:
        return 0.0
    m = float(np.max(np.abs(ref)))
    return float(np.max(np.abs(got - ref))) / (m if m else 1.0)
