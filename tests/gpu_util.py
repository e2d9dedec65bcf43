"""Helpers shared by the GPU parity tests: moving generator outputs to the device, running the
library through its C ABI binding, and comparing against the oracle."""
import numpy as np
import torch

import moe_grouped_gemm_fp8_amd as dg
import oracle
import workloads as W
from tolerance import bf16_bits_to_f64, tol_violations

DEV = "cuda:0"


def dev(x, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(x))
    if dtype is not None:
        t = t.to(dtype)
    return t.to(DEV)


def sentinel_like(shape):
    """A bf16 tensor filled with the sentinel NaN pattern (marks elements never written)."""
    return torch.full(shape, W.BF16_SENTINEL, dtype=torch.int16, device=DEV).view(torch.bfloat16)


def bits(d: torch.Tensor) -> np.ndarray:
    return d.view(torch.int16).cpu().numpy().view(np.uint16)


def _ue8m0(p) -> bool:
    """Generator outputs carry packed UE8M0 scales as int32, FP32 scales as float32."""
    return p.sfa.dtype == np.int32


def run_dense(p: W.Dense, stream=None):
    d = sentinel_like((p.m, p.n))
    fn = dg.fp8_gemm_nt_ue8m0 if _ue8m0(p) else dg.fp8_gemm_nt
    fn(dev(p.a), dev(p.sfa), dev(p.b), dev(p.sfb), d, None if p.c is None else dev(p.c),
       stream=stream)
    torch.cuda.synchronize()
    return bits(d)


def run_contiguous(p: W.Contiguous):
    d = sentinel_like((p.m_total, p.n))
    fn = (dg.m_grouped_fp8_gemm_nt_contiguous_ue8m0 if _ue8m0(p)
          else dg.m_grouped_fp8_gemm_nt_contiguous)
    fn(dev(p.a), dev(p.sfa), dev(p.b), dev(p.sfb), d, dev(p.m_indices))
    torch.cuda.synchronize()
    return bits(d)


def run_masked(p: W.Masked, masked_m=None):
    d = sentinel_like((p.num_groups, p.m_max, p.n))
    mm = p.masked_m if masked_m is None else masked_m
    fn = dg.m_grouped_fp8_gemm_nt_masked_ue8m0 if _ue8m0(p) else dg.m_grouped_fp8_gemm_nt_masked
    fn(dev(p.a), dev(p.sfa), dev(p.b), dev(p.sfb), d, dev(np.asarray(mm, np.int32)))
    torch.cuda.synchronize()
    return bits(d)


def assert_parity(d_bits: np.ndarray, ref: np.ndarray, what: str = ""):
    """Rows where ref is NaN (not computed by the method) must still hold the sentinel bit for
    bit; every other element must be within the tolerance (rms over the computed rows)."""
    ref = np.asarray(ref, dtype=np.float64)
    untouched = np.isnan(ref)
    if untouched.any():
        bad = d_bits[untouched] != W.BF16_SENTINEL
        assert not bad.any(), f"{what}: {int(bad.sum())} untouched elements were written"
    comp = ~untouched
    got = bf16_bits_to_f64(d_bits[comp])
    viol = tol_violations(got, ref[comp])
    if viol.any():
        idx = np.argwhere(comp)[np.nonzero(viol)[0][:5]]
        raise AssertionError(f"{what}: {int(viol.sum())}/{viol.size} elements outside the "
                             f"tolerance; first at {idx.tolist()}: got "
                             f"{got[viol][:5].tolist()} want {ref[comp][viol][:5].tolist()}")


def fp32_scales(p):
    """(sfa, sfb) as FP32 arrays in the FP32 layouts: packed UE8M0 scales decoded by the
    oracle, FP32 ones as they are."""
    if not _ue8m0(p):
        return p.sfa, p.sfb
    kb = p.k // 128
    ka = p.sfa.ndim - 2                                           # K axis: 0 flat, 1 per group
    return oracle.ue8m0_decode(p.sfa, ka, kb), oracle.ue8m0_decode(p.sfb, p.sfb.ndim - 1, kb)


_REF_CACHE = {}


def cached_ref(key, compute):
    """The oracle's result for a full-size workload, computed once per test session (several
    tests and variants run the same seeded inputs)."""
    if key not in _REF_CACHE:
        _REF_CACHE[key] = compute()
    return _REF_CACHE[key]


def dense_rows_ref(p: W.Dense, rows):
    rows = np.asarray(rows)
    sfa, sfb = fp32_scales(p)
    sub = W.mn_major(sfa[:, rows].T)
    return oracle.fp8_gemm_nt(p.a[rows], sub, p.b, sfb, None if p.c is None else p.c[rows])
