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


# ---------------------------------------------------------------------------------------------
# Codes of the fused activation step (first MoE GEMM, then SwiGLU and the 1x128 FP8 cast on its
# FP32 result).  The codes are integers decided from floating point that the kernel and the
# oracle compute differently, so a code must equal the oracle's where an error bound on the
# kernel's y = h / scale cannot move y across a rounding boundary, and may be either neighbour
# elsewhere.  The bound is derived from the formats:
#  * GEMM result: a 128-term MFMA block sum rounds at most once per addition (2^-24 of the sum
#    of the magnitudes of its products), and its promotion (scale product, multiply, add) and
#    the K/128 additions of promoted blocks add a few FP32 roundings each, so
#    |dD1| <= 2^-24 (128 + KB + 3) * sum_kb |sa sb| * sum_k |a b|, the last sum bounded by the
#    product of the block's Euclidean norms (Cauchy-Schwarz).
#  * SwiGLU: first order in the errors of gate and up, plus the kernel's own FP32 steps
#    (hardware exp and reciprocal: 2^-19 + |gate| 2^-21 relative, as the activation step).
#  * Cast: the segment maximum moves by at most the largest error of its elements; y also
#    carries the rounding of 448 / amax and of the product (2^-22 relative).
SWIGLU_REL = 2.0 ** -19
SWIGLU_GATE_REL = 2.0 ** -21


def gemm_error_bound(a_bits, sfa_rows, b_bits, sfb, groups, table):
    """Upper bound on |D1_kernel - D1_exact| per element for the contiguous rows given:
    a_bits [R, K] (their A rows), sfa_rows [R, K/128] (their scales, row-major), groups [R]
    (each row's group), b_bits [G, N, K], sfb [G, ceil(N/128), K/128]."""
    r, k = a_bits.shape
    g_n, n, _ = b_bits.shape
    kb = k // 128
    na = np.empty((r, kb))
    for r0 in range(0, r, 2048):                      # decoded in chunks of rows (memory)
        blk = table[a_bits[r0:r0 + 2048]].reshape(-1, kb, 128)
        na[r0:r0 + 2048] = np.sqrt((blk ** 2).sum(axis=2))
    na *= np.abs(np.asarray(sfa_rows, np.float64))
    out = np.zeros((r, n))
    for g in np.unique(groups):
        rows = np.nonzero(groups == g)[0]
        nb = np.sqrt((table[b_bits[g]].reshape(n, kb, 128) ** 2).sum(axis=2))
        nb = nb * np.repeat(np.abs(sfb[g].astype(np.float64)), 128, axis=0)[:n]
        out[rows] = na[rows] @ nb.T
    return 2.0 ** -24 * (128 + kb + 3) * out


def fused_cast_violations(q, sf, d1, d1_err, h, scale, table, nearest):
    """(bad scale mask [R, I/128], bad code mask [R, I], count of ambiguous codes) for the
    kernel's codes q [R, I] and scales sf [R, I/128] of rows whose exact GEMM result is d1
    [R, 2I] with error bound d1_err [R, 2I], and whose exact activation is h [R, I] with scales
    `scale` [R, I/128] (the oracle's)."""
    r, n2 = d1.shape
    i = n2 // 2
    g, u = d1[:, :i], d1[:, i:]
    eg, eu = d1_err[:, :i], d1_err[:, i:]
    with np.errstate(over="ignore"):       # exp(-g) = inf for a very negative gate: sig -> 0
        sig = 1.0 / (1.0 + np.exp(-g))
    dh_dg = np.abs(u * (sig + g * sig * (1.0 - sig)))
    dh_du = np.abs(g * sig)
    dh = dh_dg * eg + dh_du * eu + (np.abs(u) + 1.0) * eg * (eg + eu) \
        + np.abs(h) * (SWIGLU_REL + np.abs(g) * SWIGLU_GATE_REL)
    floor = scale * 448.0
    damax = dh.reshape(r, i // 128, 128).max(axis=2)
    bad_s = ~(np.abs(sf - scale) <= (damax + floor * 2.0 ** -22) / 448.0 + scale * 2.0 ** -23)
    y = h / np.repeat(scale, 128, axis=1)
    rel = np.repeat(damax / floor, 128, axis=1) + 2.0 ** -22
    dy = dh * 448.0 / np.repeat(floor, 128, axis=1) + np.abs(y) * rel
    lo = nearest(np.clip(y - dy, -448.0, 448.0))
    hi = nearest(np.clip(y + dy, -448.0, 448.0))
    vq, vlo, vhi = table[q], table[lo], table[hi]
    unique = lo == hi
    bad_q = np.where(unique, q != lo,
                     ~((vq >= np.minimum(vlo, vhi)) & (vq <= np.maximum(vlo, vhi))))
    return bad_s, bad_q, int((~unique).sum())
