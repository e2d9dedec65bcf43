"""The acceptance rule for floating-point results and the bit-level helpers the tests share.

A computed element passes when |d - d_ref| <= 1e-2 * |d_ref| + 1e-3 * rms(D_ref), rms taken
over the elements the method computes (valid rows only). The 1e-2 relative term covers the
bf16 rounding of D (relative 2^-9) with margin, and the rms term covers cancellation.
"""
import numpy as np

REL = 1e-2
RMS = 1e-3


def rms(x: np.ndarray) -> float:
    x = np.asarray(x, dtype=np.float64)
    return float(np.sqrt(np.mean(x * x))) if x.size else 0.0


def tol_violations(d: np.ndarray, ref: np.ndarray, rel: float = REL,
                   rms_frac: float = RMS) -> np.ndarray:
    """Boolean mask of elements outside the tolerance (NaN anywhere counts as a violation).
    The same rule holds for the bf16 outputs and for the FP32 output of the K-grouped form;
    for the latter every element of D[G, M, N] is computed, so the rms is over all of it."""
    d = np.asarray(d, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    bound = rel * np.abs(ref) + rms_frac * rms(ref)
    err = np.abs(d - ref)
    return ~(err <= bound)


def within_tol(d, ref) -> bool:
    return not tol_violations(d, ref).any()


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64, exact."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def f64_to_bf16_rne(x: np.ndarray) -> np.ndarray:
    """Round float64 to bf16 bit patterns (nearest-even), via an exact float32 step when the
    value is representable, else through the float64 value's own bits."""
    x = np.asarray(x, dtype=np.float64)
    # round to bf16 directly from float64: bf16 has 8 significant bits
    m, e = np.frexp(x)                      # x = m * 2^e, 0.5 <= |m| < 1
    q = np.round(m * 256.0) / 256.0         # numpy rounds half to even
    y = np.ldexp(q, e).astype(np.float32)
    return (y.view(np.uint32) >> 16).astype(np.uint16)
