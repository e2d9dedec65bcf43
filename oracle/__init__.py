"""Python face of the CPU oracle (``dg_oracle.c``): plain float64 reference results.

TEST INFRASTRUCTURE ONLY. Only the test-suite, ``__graft_entry__.smoke()`` and the
benchmark's CPU-baseline leg may import this package. It imports nothing from the HIP
library package and the library imports nothing from here.

Every function takes numpy arrays in the layouts of ``workloads`` (e4m3 as uint8 bits,
FP32 scales with the A scales MN-major) and returns float64 results; rows the method does
not compute are NaN in the returned array.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "dg_oracle.c")
_LIB = os.path.join(_HERE, "libdg_oracle.so")
_lib = None


def build() -> str:
    """Compile the oracle with gcc (OpenMP, -O2, no fast-math: IEEE float64 as written)."""
    tmp = _LIB + ".tmp"
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-ffp-contract=off",
           "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        build()
    lib = ctypes.CDLL(_LIB)
    p, i64 = ctypes.c_void_p, ctypes.c_int64
    lib.dgo_e4m3_table.argtypes = [p]
    lib.dgo_num_threads.restype = ctypes.c_int
    lib.dgo_set_num_threads.argtypes = [ctypes.c_int]
    lib.dgo_block_partials.argtypes = [p, p, p, i64, i64, i64]
    lib.dgo_fp8_gemm_nt.argtypes = [p, p, i64, p, p, p, p, i64, i64, i64]
    lib.dgo_fp8_gemm_nt.restype = ctypes.c_int
    lib.dgo_m_grouped_fp8_gemm_nt_contiguous.argtypes = [p, p, i64, p, p, p, p, i64, i64, i64, i64]
    lib.dgo_m_grouped_fp8_gemm_nt_contiguous.restype = ctypes.c_int
    lib.dgo_m_grouped_fp8_gemm_nt_masked.argtypes = [p, p, i64, p, p, p, p, i64, i64, i64, i64]
    lib.dgo_m_grouped_fp8_gemm_nt_masked.restype = ctypes.c_int
    _lib = lib
    return lib


def _ptr(x: Optional[np.ndarray]):
    return None if x is None else x.ctypes.data


def _c(x, dtype):
    return np.ascontiguousarray(x, dtype=dtype)


def num_threads() -> int:
    return int(_load().dgo_num_threads())


def set_num_threads(n: int) -> None:
    """Threads of the oracle's OpenMP loops (timing only; results do not depend on it)."""
    _load().dgo_set_num_threads(int(n))


def e4m3_table() -> np.ndarray:
    """The 256 e4m3 (OCP E4M3FN) values indexed by bit pattern, as float64."""
    out = np.empty(256, dtype=np.float64)
    _load().dgo_e4m3_table(out.ctypes.data)
    return out


def block_partials(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """P[m, n, kb] = sum over the 128-deep block kb of dec(A[m,k]) * dec(B[n,k]) (no scales)."""
    a, b = _c(a, np.uint8), _c(b, np.uint8)
    m, k = a.shape
    n = b.shape[0]
    out = np.empty((m, n, k // 128), dtype=np.float64)
    _load().dgo_block_partials(a.ctypes.data, b.ctypes.data, out.ctypes.data, m, n, k)
    return out


def fp8_gemm_nt(a, sfa, b, sfb, c=None) -> np.ndarray:
    """D = C + A @ B.T with 1x128 A scales (MN-major ``sfa`` [K/128, ld]) and 128x128 B scales."""
    a, sfa, b, sfb = _c(a, np.uint8), _c(sfa, np.float32), _c(b, np.uint8), _c(sfb, np.float32)
    m, k = a.shape
    n = b.shape[0]
    c = None if c is None else _c(c, np.float32)
    d = np.full((m, n), np.nan, dtype=np.float64)
    rc = _load().dgo_fp8_gemm_nt(_ptr(a), _ptr(sfa), sfa.shape[1], _ptr(b), _ptr(sfb), _ptr(c),
                                 _ptr(d), m, n, k)
    if rc != 0:
        raise ValueError("oracle: unsupported dense shape")
    return d


def m_grouped_contiguous(a, sfa, b, sfb, m_indices) -> np.ndarray:
    a, sfa, b, sfb = _c(a, np.uint8), _c(sfa, np.float32), _c(b, np.uint8), _c(sfb, np.float32)
    m_indices = _c(m_indices, np.int32)
    m_total, k = a.shape
    g, n, _ = b.shape
    d = np.full((m_total, n), np.nan, dtype=np.float64)
    rc = _load().dgo_m_grouped_fp8_gemm_nt_contiguous(_ptr(a), _ptr(sfa), sfa.shape[1], _ptr(b),
                                                      _ptr(sfb), _ptr(d), _ptr(m_indices),
                                                      m_total, n, k, g)
    if rc != 0:
        raise ValueError("oracle: unsupported contiguous shape")
    return d


def m_grouped_masked(a, sfa, b, sfb, masked_m) -> np.ndarray:
    a, sfa, b, sfb = _c(a, np.uint8), _c(sfa, np.float32), _c(b, np.uint8), _c(sfb, np.float32)
    masked_m = _c(masked_m, np.int32)
    g, m_max, k = a.shape
    n = b.shape[1]
    d = np.full((g, m_max, n), np.nan, dtype=np.float64)
    rc = _load().dgo_m_grouped_fp8_gemm_nt_masked(_ptr(a), _ptr(sfa), sfa.shape[2], _ptr(b),
                                                  _ptr(sfb), _ptr(d), _ptr(masked_m), g, m_max,
                                                  n, k)
    if rc != 0:
        raise ValueError("oracle: unsupported masked shape")
    return d


# ---------------------------------------------------------------------------------------------
# UE8M0 scales: the packed power-of-two format of the method's newer hardware generation
# (pt.news.hada.io, "Interface GEMM e restrições de layout": four UE8M0 values packed into one
# 32-bit integer).  The reading taken: the four are consecutive K blocks of one row (or one
# 128-row B block), least significant byte first, in the same layouts as the FP32 scales
# with the K-block axis shortened to ceil(K/512); a byte e means 2^(e-127), and 0xFF is NaN.
# The result is then the plain definition above with those scales.

def ue8m0_decode(packed, axis: int, num_kblocks: int) -> np.ndarray:
    """Packed UE8M0 int32 array -> float32 scales with ``num_kblocks`` entries along
    ``axis``: entry 4q + j is byte j (least significant first) of packed entry q."""
    p = np.moveaxis(np.asarray(packed), axis, -1).astype(np.int64) & 0xFFFFFFFF
    kq = p.shape[-1]
    shifts = 8 * np.arange(4, dtype=np.int64)
    e = (p[..., :, None] >> shifts) & 0xFF                      # [..., kq, 4]
    e = e.reshape(p.shape[:-1] + (kq * 4,))[..., :num_kblocks]
    out = np.ldexp(np.float64(1.0), (e - 127).astype(np.int64))
    out[e == 255] = np.nan
    return np.moveaxis(out.astype(np.float32), -1, axis)       # every 2^e is exact in float32


def fp8_gemm_nt_ue8m0(a, sfa, b, sfb, c=None) -> np.ndarray:
    """``fp8_gemm_nt`` with packed UE8M0 scales (``sfa`` int32 [ceil(K/512), ld],
    ``sfb`` int32 [ceil(N/128), ceil(K/512)])."""
    kb = np.asarray(a).shape[1] // 128
    return fp8_gemm_nt(a, ue8m0_decode(sfa, 0, kb), b, ue8m0_decode(sfb, 1, kb), c)


def m_grouped_contiguous_ue8m0(a, sfa, b, sfb, m_indices) -> np.ndarray:
    kb = np.asarray(a).shape[1] // 128
    return m_grouped_contiguous(a, ue8m0_decode(sfa, 0, kb), b, ue8m0_decode(sfb, 2, kb),
                                m_indices)


def m_grouped_masked_ue8m0(a, sfa, b, sfb, masked_m) -> np.ndarray:
    kb = np.asarray(a).shape[2] // 128
    return m_grouped_masked(a, ue8m0_decode(sfa, 1, kb), b, ue8m0_decode(sfb, 2, kb),
                            masked_m)


# ---------------------------------------------------------------------------------------------
# K-grouped TN form (MoE weight gradient; pt.news.hada.io, "GEMM denso e grouped": grouping on
# the K axis with M and N fixed; "Interface GEMM e restrições de layout": D = C + A @ B, with
# the TN memory layout).  A is stored [K_total, M] and B [K_total, N] (both K-major in the
# mathematical sense of "transposed" A and "not transposed" B), the groups are consecutive runs
# of K of lengths ks[g] (multiples of 128), and both scale sets are one FP32 value per 128-deep
# K block per column: sfa [K_total/128, M], sfb [K_total/128, N].  The plain definition:
#   D[g, m, n] = C[g, m, n] + sum over the K blocks kb of group g of
#                sfa[kb, m] * sfb[kb, n] * sum_{k in kb} dec(A[k, m]) * dec(B[k, n])
# Each block sum is a matrix product of decoded values; every e4m3 value is an integer times
# 2^-9 below 2^18 in magnitude, so the 128-term sums are exact in float64 in any order, and a
# library product serves for them.  Then the scaled terms are added in float64, blocks in
# ascending order, and C last.

def k_grouped_tn(a, sfa, b, sfb, ks, c=None) -> np.ndarray:
    """float64 D [G, M, N] of the K-grouped TN GEMM (``a`` uint8 [K_total, M], ``b`` uint8
    [K_total, N], ``sfa`` [K_total/128, M], ``sfb`` [K_total/128, N], ``ks`` [G])."""
    a, b = _c(a, np.uint8), _c(b, np.uint8)
    sfa, sfb = _c(sfa, np.float32), _c(sfb, np.float32)
    ks = np.asarray(ks, dtype=np.int64)
    k_total, m = a.shape
    n = b.shape[1]
    if np.any(ks < 0) or np.any(ks % 128) or ks.sum() > k_total:
        raise ValueError("oracle: group extents must be non-negative multiples of 128")
    tab = e4m3_table()
    d = np.zeros((len(ks), m, n), dtype=np.float64)
    k0 = 0
    for g, kg in enumerate(ks):
        for kb in range(k0 // 128, (k0 + int(kg)) // 128):
            rows = slice(kb * 128, (kb + 1) * 128)
            part = tab[a[rows]].T @ tab[b[rows]]                     # exact block sums
            d[g] += (sfa[kb].astype(np.float64)[:, None] * sfb[kb].astype(np.float64)[None, :]) * part
        k0 += int(kg)
    if c is not None:
        d += _c(c, np.float32).astype(np.float64)
    return d


# ---------------------------------------------------------------------------------------------
# The other dense memory layouts (pt.news.hada.io, "Interface GEMM e restrições de layout": the
# NT, TN, NN and TT layouts of D = C + A @ B; "GEMM denso e grouped": fp8_gemm_{nt, nn, tn, tt}).
# The first letter is A's storage, the second B's: "n" for A is [M, K] and "t" is [K, M]; "t"
# for B is [N, K] (B given transposed, as in NT) and "n" is [K, N].  The scales keep the NT
# layouts (sfa [K/128, ld] one per 1x128 segment of a row of A, sfb [ceil(N/128), K/128] one
# per 128x128 block of B): only where the bytes sit changes, so the result is the NT
# definition of the same mathematical A [M, K] and B^T [N, K].

def fp8_gemm_layout(layout: str, a, sfa, b, sfb, c=None) -> np.ndarray:
    """D = C + A @ B for ``layout`` in {"nt", "nn", "tn", "tt"} (storage as described above)."""
    if layout not in ("nt", "nn", "tn", "tt"):
        raise ValueError(f"oracle: unknown layout {layout!r}")
    a_mk = np.asarray(a) if layout[0] == "n" else np.asarray(a).T
    b_nk = np.asarray(b) if layout[1] == "t" else np.asarray(b).T
    return fp8_gemm_nt(np.ascontiguousarray(a_mk), sfa, np.ascontiguousarray(b_nk), sfb, c)


# ---------------------------------------------------------------------------------------------
# The activation step between an expert's two GEMMs (the work the pages leave to the caller:
# pt.news.hada.io, "Interface GEMM e restrições de layout", casting to FP8 is the user's job;
# the feifmx.com release article's fine-grained scaling fixes the 1x128 granularity of the
# next GEMM's A).  Input: the first GEMM's bf16 output X [M, 2I], gate X[:, :I] and up
# X[:, I:].  SwiGLU: h = silu(gate) * up = gate * up / (1 + exp(-gate)).  Quantisation of h
# for the second GEMM: per 1x128 segment of a row, scale = max(amax, 1e-4) / 448 and
# code = the e4m3 value nearest to h / scale (ties to the even code), never past +-448; the
# scales go out MN-major, [I/128, ld] with ld = ceil(M/4)*4, the layout of the NT GEMM's sfa.

def bf16_decode(bits) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64, exact."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def swiglu(x_bits) -> np.ndarray:
    """float64 h [M, I] of a bf16 [M, 2I] input (gate first, then up)."""
    return swiglu_values(bf16_decode(x_bits))


def swiglu_values(x) -> np.ndarray:
    """float64 h [M, I] of float64 first-GEMM results x [M, 2I] (gate first, then up)."""
    x = np.asarray(x, dtype=np.float64)
    i = x.shape[1] // 2
    g, u = x[:, :i], x[:, i:]
    with np.errstate(over="ignore"):       # exp(-g) = inf for a very negative gate: h -> 0
        return g * u / (1.0 + np.exp(-g))


def e4m3_nearest(y) -> np.ndarray:
    """uint8 e4m3 codes nearest to float64 y (|y| <= 448), ties to the even code.  The format
    is sign-magnitude and its non-negative finite codes 0x00 .. 0x7E increase with their
    value, so the magnitude code is the lower or the upper end of the interval of the decode
    table that holds |y|: the nearer one, or on a tie the even one.  A negative y (or -0) sets
    the sign bit."""
    tab = e4m3_table()
    vals = tab[:0x7F]                                        # 0 .. 448, increasing
    y = np.asarray(y, dtype=np.float64)
    a = np.abs(y)
    lo = np.clip(np.searchsorted(vals, a, side="right") - 1, 0, 0x7E)
    hi = np.minimum(lo + 1, 0x7E)
    d_lo = a - vals[lo]
    d_hi = vals[hi] - a
    code = np.where(d_lo < d_hi, lo, np.where(d_hi < d_lo, hi, np.where(lo % 2 == 0, lo, hi)))
    return (code | np.where(np.signbit(y), 0x80, 0)).astype(np.uint8)


def swiglu_quant(x_bits, ld: Optional[int] = None):
    """(h float64 [M, I], scales float64 [I/128, ld], codes uint8 [M, I]) by the definition."""
    return quant_1x128(swiglu(x_bits), ld)


def quant_1x128(h, ld: Optional[int] = None):
    """The 1x128 FP8 cast of float64 h [M, I]: (h, scales [I/128, ld], codes [M, I])."""
    h = np.asarray(h, dtype=np.float64)
    m, i = h.shape
    if i % 128:
        raise ValueError("oracle: I must be a multiple of 128")
    ld = (m + 3) // 4 * 4 if ld is None else ld
    seg = h.reshape(m, i // 128, 128)
    scale = np.maximum(np.abs(seg).max(axis=2), 1e-4) / 448.0    # [M, I/128]
    y = np.clip(seg / scale[:, :, None], -448.0, 448.0).reshape(m, i)
    sf = np.zeros((i // 128, ld), dtype=np.float64)
    sf[:, :m] = scale.T
    return h, sf, e4m3_nearest(y)


# ---------------------------------------------------------------------------------------------
# The first GEMM of an expert with the activation step fused behind it (the single-GPU part of
# the MoE block that pt.news.hada.io's "Mega MoE" section describes as linear 1 -> SwiGLU ->
# linear 2 in one pass; "Interface GEMM e restrições de layout" leaves the FP8 cast of the next
# GEMM's input to the caller).  Reading taken: the activation applies to the first GEMM's
# unrounded result (no bf16 rounding in between): for every computed row m of the contiguous
# layout, D1[m] = the plain definition above (float64), gate = D1[m, :I], up = D1[m, I:],
# h = gate * up / (1 + exp(-gate)), and the 1x128 cast of h as in quant_1x128.

def m_grouped_contiguous_swiglu(a, sfa, b, sfb, m_indices, ld: Optional[int] = None):
    """(d1 [M, 2I], h [M, I], scales [I/128, ld], codes [M, I]) for the contiguous layout; rows
    the method does not compute (index outside [0, G)) are NaN in d1 and h, 0 in the scales and
    the codes."""
    d1 = m_grouped_contiguous(a, sfa, b, sfb, m_indices)
    m, n2 = d1.shape
    if n2 % 256:
        raise ValueError("oracle: N = 2I with I a multiple of 128")
    valid = ~np.isnan(d1).any(axis=1)
    ld = (m + 3) // 4 * 4 if ld is None else ld
    h = np.full((m, n2 // 2), np.nan)
    sf = np.zeros((n2 // 256, ld))
    q = np.zeros((m, n2 // 2), dtype=np.uint8)
    if valid.any():
        hv, sfv, qv = quant_1x128(swiglu_values(d1[valid]))
        h[valid] = hv
        sf[:, np.nonzero(valid)[0]] = sfv[:, :int(valid.sum())]
        q[valid] = qv
    return d1, h, sf, q
