"""Python binding of libdg.so: the fine-grained-scaled FP8 GEMM for MI355X (gfx950).

Thin marshalling over the C ABI declared in ``include/dg.h``: it checks that the tensors'
shapes agree with each other (so the kernels' index ranges match the memory handed over),
passes raw device pointers and the current HIP stream, and turns a non-zero status into an
exception.  Every step of the computation runs in the HIP kernels; there is no fallback.

Operation (DeepGEMM pages, pt.news.hada.io, "Interface GEMM e restrições de layout"):
D = C + A @ B.T, A e4m3 [M, K] with FP32 scales per 1x128 row segment stored MN-major as
``sfa`` [K/128, ld], B e4m3 [N, K] with FP32 scales per 128x128 block ``sfb``
[ceil(N/128), K/128], D bf16, C optional FP32.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np
import torch

__all__ = [
    "DGError", "fp8_gemm_nt", "fp8_gemm_nt_noalloc", "m_grouped_fp8_gemm_nt_contiguous", "m_grouped_fp8_gemm_nt_masked",
    "m_grouped_fp8_gemm_nt_contiguous_swiglu",
    "fp8_gemm_nn", "fp8_gemm_tn", "fp8_gemm_tt", "swiglu_fp8_quant",
    "fp8_gemm_nt_ue8m0", "m_grouped_fp8_gemm_nt_contiguous_ue8m0",
    "m_grouped_fp8_gemm_nt_masked_ue8m0", "k_grouped_fp8_gemm_tn_contiguous",
    "get_mk_alignment_for_contiguous_layout", "get_sf_aligned_m", "set_num_cus", "get_num_cus",
    "library_path",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libdg.so")
_lib = None

_FP8_DTYPES = (torch.uint8, torch.float8_e4m3fn)


class DGError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"dg error {code}: {message}")
        self.code = code


def library_path() -> str:
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(f"{_LIB_PATH} is not built; run __graft_entry__.build() or "
                           "python -m moe_grouped_gemm_fp8_amd.build")
    lib = ctypes.CDLL(_LIB_PATH)
    vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    lib.dg_fp8_gemm_nt.argtypes = [vp, vp, i64, vp, vp, vp, vp, i32, i32, i32, vp]
    lib.dg_fp8_gemm_nt.restype = i32
    lib.dg_m_grouped_fp8_gemm_nt_contiguous.argtypes = [vp, vp, i64, vp, vp, vp, vp, i32, i32,
                                                        i32, i32, vp]
    lib.dg_m_grouped_fp8_gemm_nt_contiguous.restype = i32
    lib.dg_m_grouped_fp8_gemm_nt_masked.argtypes = [vp, vp, i64, vp, vp, vp, vp, i32, i32, i32,
                                                    i32, i32, vp]
    lib.dg_m_grouped_fp8_gemm_nt_masked.restype = i32
    lib.dg_m_grouped_fp8_gemm_nt_contiguous_swiglu.argtypes = [vp, vp, i64, vp, vp, vp, vp, i64,
                                                               vp, i32, i32, i32, i32, vp]
    lib.dg_m_grouped_fp8_gemm_nt_contiguous_swiglu.restype = i32
    for name in ("dg_fp8_gemm_nn", "dg_fp8_gemm_tn", "dg_fp8_gemm_tt", "dg_fp8_gemm_nt_noalloc"):
        getattr(lib, name).argtypes = lib.dg_fp8_gemm_nt.argtypes
        getattr(lib, name).restype = i32
    for name in ("dg_fp8_gemm_nt", "dg_m_grouped_fp8_gemm_nt_contiguous",
                 "dg_m_grouped_fp8_gemm_nt_masked"):
        fn = getattr(lib, name + "_ue8m0")
        fn.argtypes = getattr(lib, name).argtypes
        fn.restype = i32
    lib.dg_k_grouped_fp8_gemm_tn_contiguous.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32,
                                                         i32, i32, vp]
    lib.dg_k_grouped_fp8_gemm_tn_contiguous.restype = i32
    lib.dg_swiglu_fp8_quant.argtypes = [vp, vp, vp, i64, i32, i32, vp]
    lib.dg_swiglu_fp8_quant.restype = i32
    lib.dg_get_mk_alignment_for_contiguous_layout.restype = i32
    lib.dg_get_sf_aligned_m.argtypes = [i64]
    lib.dg_get_sf_aligned_m.restype = i64
    lib.dg_set_num_cus.argtypes = [i32]
    lib.dg_set_num_cus.restype = i32
    lib.dg_get_num_cus.restype = i32
    lib.dg_last_error.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _check(rc: int):
    if rc != 0:
        raise DGError(rc, _load().dg_last_error().decode(errors="replace"))


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _need(cond: bool, msg: str):
    if not cond:
        raise ValueError(msg)


def _dev(t: torch.Tensor, name: str, dtypes, ndim: int):
    _need(isinstance(t, torch.Tensor), f"{name} must be a tensor")
    _need(t.is_cuda, f"{name} must be a device tensor")
    _need(t.dtype in (dtypes if isinstance(dtypes, tuple) else (dtypes,)),
          f"{name} has dtype {t.dtype}")
    _need(t.dim() == ndim, f"{name} must have {ndim} dims, has shape {tuple(t.shape)}")
    _need(t.is_contiguous(), f"{name} must be contiguous")
    return t.data_ptr()


def _scale_spec(k: int, ue8m0: bool):
    """dtype and K-axis length of the scale tensors: one FP32 per 128-wide K block, or one
    int32 per four K blocks holding their UE8M0 exponents (least significant byte first)."""
    kb = k // 128
    return (torch.int32, (kb + 3) // 4, "ceil(K/512)") if ue8m0 else (torch.float32, kb, "K/128")


def _fp8_gemm_nt(a, sfa, b, sfb, d, c, stream, ue8m0, layout="nt"):
    pa = _dev(a, "a", _FP8_DTYPES, 2)
    m, k = a.shape if layout[0] == "n" else (a.shape[1], a.shape[0])
    pb = _dev(b, "b", _FP8_DTYPES, 2)
    n, kb_ = b.shape if layout[1] == "t" else (b.shape[1], b.shape[0])
    _need(kb_ == k, "a and b disagree on K")
    _need(k % 128 == 0, "K must be a multiple of 128")
    sdt, ks, kname = _scale_spec(k, ue8m0)
    psfa = _dev(sfa, "sfa", sdt, 2)
    _need(sfa.shape[0] == ks, f"sfa must be [{kname}, ld]")
    psfb = _dev(sfb, "sfb", sdt, 2)
    _need(tuple(sfb.shape) == ((n + 127) // 128, ks), f"sfb must be [ceil(N/128), {kname}]")
    pd = _dev(d, "d", torch.bfloat16, 2)
    _need(tuple(d.shape) == (m, n), "d must be [M, N]")
    pc = None
    if c is not None:
        pc = _dev(c, "c", torch.float32, 2)
        _need(tuple(c.shape) == (m, n), "c must be [M, N]")
    lib = _load()
    fn = lib.dg_fp8_gemm_nt_ue8m0 if ue8m0 else getattr(lib, "dg_fp8_gemm_" + layout)
    _check(fn(pa, psfa, sfa.shape[1], pb, psfb, pc, pd, m, n, k, _stream(stream)))
    return d


def fp8_gemm_nt(a, sfa, b, sfb, d, c: Optional[torch.Tensor] = None, stream=None):
    """D = C + A @ B.T.  a [M,K] e4m3, sfa [K/128, ld>=M] f32, b [N,K] e4m3,
    sfb [ceil(N/128), K/128] f32, d [M,N] bf16 (written), c [M,N] f32 or None."""
    return _fp8_gemm_nt(a, sfa, b, sfb, d, c, stream, False)


def fp8_gemm_nt_noalloc(a, sfa, b, sfb, d, c: Optional[torch.Tensor] = None, stream=None):
    """fp8_gemm_nt through the entry point that allocates nothing (split-K partials in the
    library's static per-device scratch; overlapping calls on one device race)."""
    return _fp8_gemm_nt(a, sfa, b, sfb, d, c, stream, False, "nt_noalloc")


def fp8_gemm_nn(a, sfa, b, sfb, d, c: Optional[torch.Tensor] = None, stream=None):
    """D = C + A @ B with A [M, K] and B stored [K, N]; scales, C and D as in fp8_gemm_nt."""
    return _fp8_gemm_nt(a, sfa, b, sfb, d, c, stream, False, "nn")


def fp8_gemm_tn(a, sfa, b, sfb, d, c: Optional[torch.Tensor] = None, stream=None):
    """D = C + A @ B with A stored [K, M] and B stored [K, N]; as fp8_gemm_nt otherwise."""
    return _fp8_gemm_nt(a, sfa, b, sfb, d, c, stream, False, "tn")


def fp8_gemm_tt(a, sfa, b, sfb, d, c: Optional[torch.Tensor] = None, stream=None):
    """D = C + A @ B.T with A stored [K, M] and B [N, K]; as fp8_gemm_nt otherwise."""
    return _fp8_gemm_nt(a, sfa, b, sfb, d, c, stream, False, "tt")


def fp8_gemm_nt_ue8m0(a, sfa, b, sfb, d, c: Optional[torch.Tensor] = None, stream=None):
    """fp8_gemm_nt with packed UE8M0 scales: sfa int32 [ceil(K/512), ld>=M],
    sfb int32 [ceil(N/128), ceil(K/512)]; byte j of word q is the exponent of K block 4q+j."""
    return _fp8_gemm_nt(a, sfa, b, sfb, d, c, stream, True)


def _contiguous(a, sfa, b, sfb, d, m_indices, stream, ue8m0):
    pa = _dev(a, "a", _FP8_DTYPES, 2)
    m_total, k = a.shape
    pb = _dev(b, "b", _FP8_DTYPES, 3)
    g, n, kb_ = b.shape
    _need(kb_ == k, "a and b disagree on K")
    _need(k % 128 == 0, "K must be a multiple of 128")
    sdt, ks, kname = _scale_spec(k, ue8m0)
    psfa = _dev(sfa, "sfa", sdt, 2)
    _need(sfa.shape[0] == ks, f"sfa must be [{kname}, ld]")
    psfb = _dev(sfb, "sfb", sdt, 3)
    _need(tuple(sfb.shape) == (g, (n + 127) // 128, ks), f"sfb must be [G, ceil(N/128), {kname}]")
    pd = _dev(d, "d", torch.bfloat16, 2)
    _need(tuple(d.shape) == (m_total, n), "d must be [M_total, N]")
    pi = _dev(m_indices, "m_indices", torch.int32, 1)
    _need(m_indices.shape[0] == m_total, "m_indices must be [M_total]")
    lib = _load()
    fn = (lib.dg_m_grouped_fp8_gemm_nt_contiguous_ue8m0 if ue8m0
          else lib.dg_m_grouped_fp8_gemm_nt_contiguous)
    _check(fn(pa, psfa, sfa.shape[1], pb, psfb, pd, pi, m_total, n, k, g, _stream(stream)))
    return d


def m_grouped_fp8_gemm_nt_contiguous(a, sfa, b, sfb, d, m_indices, stream=None):
    """Contiguous M-grouped GEMM.  a [M_total,K], sfa [K/128, ld>=M_total], b [G,N,K],
    sfb [G, ceil(N/128), K/128], d [M_total,N] bf16, m_indices int32 [M_total] (-1 = padding)."""
    return _contiguous(a, sfa, b, sfb, d, m_indices, stream, False)


def m_grouped_fp8_gemm_nt_contiguous_ue8m0(a, sfa, b, sfb, d, m_indices, stream=None):
    """m_grouped_fp8_gemm_nt_contiguous with packed UE8M0 scales: sfa int32
    [ceil(K/512), ld>=M_total], sfb int32 [G, ceil(N/128), ceil(K/512)]."""
    return _contiguous(a, sfa, b, sfb, d, m_indices, stream, True)


def m_grouped_fp8_gemm_nt_contiguous_swiglu(a, sfa, b, sfb, q, sfq, m_indices, stream=None):
    """The contiguous GEMM with SwiGLU and the 1x128 FP8 cast fused into its epilogue.
    a [M_total, K], sfa [K/128, ld>=M_total], b [G, 2I, K] (gate rows first),
    sfb [G, 2I/128, K/128], m_indices int32 [M_total]; writes q [M_total, I] (uint8 or
    float8_e4m3fn) and sfq float32 [I/128, ld>=M_total] (MN-major) for the valid rows."""
    pa = _dev(a, "a", _FP8_DTYPES, 2)
    m_total, k = a.shape
    pb = _dev(b, "b", _FP8_DTYPES, 3)
    g, n, kb_ = b.shape
    _need(kb_ == k, "a and b disagree on K")
    _need(k % 128 == 0 and n % 256 == 0, "K must be a multiple of 128 and 2I of 256")
    psfa = _dev(sfa, "sfa", torch.float32, 2)
    _need(sfa.shape[0] == k // 128, "sfa must be [K/128, ld]")
    psfb = _dev(sfb, "sfb", torch.float32, 3)
    _need(tuple(sfb.shape) == (g, n // 128, k // 128), "sfb must be [G, 2I/128, K/128]")
    pq = _dev(q, "q", _FP8_DTYPES, 2)
    _need(tuple(q.shape) == (m_total, n // 2), "q must be [M_total, I]")
    psq = _dev(sfq, "sfq", torch.float32, 2)
    _need(sfq.shape[0] == n // 256, "sfq must be [I/128, ld]")
    pi = _dev(m_indices, "m_indices", torch.int32, 1)
    _need(m_indices.shape[0] == m_total, "m_indices must be [M_total]")
    _check(_load().dg_m_grouped_fp8_gemm_nt_contiguous_swiglu(
        pa, psfa, sfa.shape[1], pb, psfb, pq, psq, sfq.shape[1], pi, m_total, n, k, g,
        _stream(stream)))
    return q, sfq


def _masked(a, sfa, b, sfb, d, masked_m, expected_m, stream, ue8m0):
    pa = _dev(a, "a", _FP8_DTYPES, 3)
    g, m_max, k = a.shape
    pb = _dev(b, "b", _FP8_DTYPES, 3)
    _need(b.shape[0] == g and b.shape[2] == k, "a and b disagree on G or K")
    _need(k % 128 == 0, "K must be a multiple of 128")
    n = b.shape[1]
    sdt, ks, kname = _scale_spec(k, ue8m0)
    psfa = _dev(sfa, "sfa", sdt, 3)
    _need(sfa.shape[0] == g and sfa.shape[1] == ks, f"sfa must be [G, {kname}, ld]")
    psfb = _dev(sfb, "sfb", sdt, 3)
    _need(tuple(sfb.shape) == (g, (n + 127) // 128, ks), f"sfb must be [G, ceil(N/128), {kname}]")
    pd = _dev(d, "d", torch.bfloat16, 3)
    _need(tuple(d.shape) == (g, m_max, n), "d must be [G, M_max, N]")
    pm = _dev(masked_m, "masked_m", torch.int32, 1)
    _need(masked_m.shape[0] == g, "masked_m must be [G]")
    lib = _load()
    fn = (lib.dg_m_grouped_fp8_gemm_nt_masked_ue8m0 if ue8m0
          else lib.dg_m_grouped_fp8_gemm_nt_masked)
    _check(fn(pa, psfa, sfa.shape[2], pb, psfb, pd, pm, g, m_max, n, k, int(expected_m),
              _stream(stream)))
    return d


def m_grouped_fp8_gemm_nt_masked(a, sfa, b, sfb, d, masked_m, expected_m: int = 0, stream=None):
    """Masked M-grouped GEMM.  a [G,M_max,K], sfa [G, K/128, ld>=M_max], b [G,N,K],
    sfb [G, ceil(N/128), K/128], d [G,M_max,N] bf16, masked_m int32 [G] on the device."""
    return _masked(a, sfa, b, sfb, d, masked_m, expected_m, stream, False)


def m_grouped_fp8_gemm_nt_masked_ue8m0(a, sfa, b, sfb, d, masked_m, expected_m: int = 0,
                                       stream=None):
    """m_grouped_fp8_gemm_nt_masked with packed UE8M0 scales: sfa int32
    [G, ceil(K/512), ld>=M_max], sfb int32 [G, ceil(N/128), ceil(K/512)]."""
    return _masked(a, sfa, b, sfb, d, masked_m, expected_m, stream, True)


def k_grouped_fp8_gemm_tn_contiguous(a, sfa, b, sfb, d, ks, c: Optional[torch.Tensor] = None,
                                     stream=None):
    """K-grouped TN GEMM (MoE weight gradient): a [K_total, M] e4m3, sfa [K_total/128, M] f32,
    b [K_total, N] e4m3, sfb [K_total/128, N] f32, d [G, M, N] f32 (written), ks: G host ints
    (multiples of 128 summing to K_total), c [G, M, N] f32, None, or d itself."""
    pa = _dev(a, "a", _FP8_DTYPES, 2)
    k_total, m = a.shape
    pb = _dev(b, "b", _FP8_DTYPES, 2)
    _need(b.shape[0] == k_total, "a and b disagree on K_total")
    n = b.shape[1]
    _need(k_total % 128 == 0, "K_total must be a multiple of 128")
    psfa = _dev(sfa, "sfa", torch.float32, 2)
    _need(tuple(sfa.shape) == (k_total // 128, m), "sfa must be [K_total/128, M]")
    psfb = _dev(sfb, "sfb", torch.float32, 2)
    _need(tuple(sfb.shape) == (k_total // 128, n), "sfb must be [K_total/128, N]")
    ks_host = np.ascontiguousarray(np.asarray(ks, dtype=np.int32).reshape(-1))
    g = int(ks_host.shape[0])
    pd = _dev(d, "d", torch.float32, 3)
    _need(tuple(d.shape) == (g, m, n), "d must be [G, M, N]")
    pc = None
    if c is not None:
        pc = _dev(c, "c", torch.float32, 3)
        _need(tuple(c.shape) == (g, m, n), "c must be [G, M, N]")
    _check(_load().dg_k_grouped_fp8_gemm_tn_contiguous(
        pa, psfa, pb, psfb, pc, pd, ks_host.ctypes.data, g, m, n, k_total, _stream(stream)))
    return d


def swiglu_fp8_quant(x, q, sfa, stream=None):
    """SwiGLU of x (bf16 [M, 2I], gate then up) cast per 1x128 segment to e4m3: q [M, I] (uint8
    or float8_e4m3fn) and sfa float32 [I/128, ld >= M] (MN-major), both written."""
    px = _dev(x, "x", (torch.bfloat16, torch.int16, torch.uint16), 2)
    m, i2 = x.shape
    _need(i2 % 256 == 0, "x must be [M, 2I] with I a multiple of 128")
    i = i2 // 2
    pq = _dev(q, "q", _FP8_DTYPES, 2)
    _need(tuple(q.shape) == (m, i), "q must be [M, I]")
    psf = _dev(sfa, "sfa", torch.float32, 2)
    _need(sfa.shape[0] == i // 128 and sfa.shape[1] >= m, "sfa must be [I/128, ld >= M]")
    _check(_load().dg_swiglu_fp8_quant(px, pq, psf, sfa.shape[1], m, i, _stream(stream)))
    return q, sfa


def get_mk_alignment_for_contiguous_layout() -> int:
    return int(_load().dg_get_mk_alignment_for_contiguous_layout())


def get_sf_aligned_m(m: int) -> int:
    return int(_load().dg_get_sf_aligned_m(int(m)))


def set_num_cus(n: int) -> int:
    return int(_load().dg_set_num_cus(int(n)))


def get_num_cus() -> int:
    v = int(_load().dg_get_num_cus())
    if v < 0:
        _check(v)
    return v
