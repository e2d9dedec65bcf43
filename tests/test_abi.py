"""The C ABI without a GPU: libdg.so loads, exports every function include/dg.h declares,
and rejects bad arguments on the host before any HIP call.  Only arguments that fail the
host checks are passed here, so no kernel is ever launched from these tests."""
import ctypes
import os
import re

import pytest

import moe_grouped_gemm_fp8_amd as dg

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dg.h")

DG_OK, DG_ERR_INVALID_ARG, DG_ERR_UNSUPPORTED, DG_ERR_MISALIGNED, DG_ERR_HIP = 0, -1, -2, -3, -4
P = 0x10000          # a 16-byte aligned stand-in address; never dereferenced by these calls


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dg_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(dg.library_path()):
        import importlib
        importlib.import_module("moe_grouped_gemm_fp8_amd.build").build()
    return dg._load()


def test_header_declares_the_three_gemm_calls():
    names = declared_functions()
    for f in ("dg_fp8_gemm_nt", "dg_m_grouped_fp8_gemm_nt_contiguous",
              "dg_m_grouped_fp8_gemm_nt_masked"):
        assert f in names
        assert f + "_ue8m0" in names


def test_library_exports_every_declared_function(lib):
    raw = ctypes.CDLL(dg.library_path())
    missing = [f for f in declared_functions() if not hasattr(raw, f)]
    assert not missing, missing


def test_host_helpers(lib):
    assert lib.dg_get_mk_alignment_for_contiguous_layout() == 128
    assert [lib.dg_get_sf_aligned_m(m) for m in (1, 4, 5, 4096, 4097)] == [4, 4, 8, 4096, 4100]
    prev = lib.dg_set_num_cus(77)
    assert lib.dg_set_num_cus(prev) == 77
    n = lib.dg_get_num_cus()
    assert n > 0 or n == DG_ERR_HIP


def dense(lib, a=P, sfa=P, ld=128, b=P, sfb=P, c=None, d=P, m=128, n=256, k=512):
    return lib.dg_fp8_gemm_nt(a, sfa, ld, b, sfb, c, d, m, n, k, None)


@pytest.mark.parametrize("kw,code", [
    (dict(a=None), DG_ERR_INVALID_ARG),
    (dict(sfa=None), DG_ERR_INVALID_ARG),
    (dict(b=None), DG_ERR_INVALID_ARG),
    (dict(sfb=None), DG_ERR_INVALID_ARG),
    (dict(d=None), DG_ERR_INVALID_ARG),
    (dict(m=-1), DG_ERR_INVALID_ARG),
    (dict(n=-16), DG_ERR_INVALID_ARG),
    (dict(k=0), DG_ERR_INVALID_ARG),
    (dict(k=500), DG_ERR_UNSUPPORTED),
    (dict(n=250), DG_ERR_UNSUPPORTED),
    (dict(ld=120), DG_ERR_INVALID_ARG),
    (dict(ld=130), DG_ERR_MISALIGNED),
    (dict(a=P + 8), DG_ERR_MISALIGNED),
    (dict(b=P + 4), DG_ERR_MISALIGNED),
    (dict(d=P + 2), DG_ERR_MISALIGNED),
    (dict(sfa=P + 2), DG_ERR_MISALIGNED),
    (dict(sfa=P + 4), DG_ERR_MISALIGNED),
    (dict(sfa=P + 8), DG_ERR_MISALIGNED),
    (dict(sfb=P + 2), DG_ERR_MISALIGNED),
    (dict(c=P + 8), DG_ERR_MISALIGNED),
    (dict(c=P, d=P), DG_ERR_INVALID_ARG),
])
def test_dense_rejects_bad_arguments_on_host(lib, kw, code):
    assert dense(lib, **kw) == code
    assert lib.dg_last_error().decode()


def dense_ue8m0(lib, a=P, sfa=P, ld=128, b=P, sfb=P, c=None, d=P, m=128, n=256, k=512):
    return lib.dg_fp8_gemm_nt_ue8m0(a, sfa, ld, b, sfb, c, d, m, n, k, None)


@pytest.mark.parametrize("kw,code", [
    (dict(sfa=None), DG_ERR_INVALID_ARG),
    (dict(k=500), DG_ERR_UNSUPPORTED),
    (dict(ld=130), DG_ERR_MISALIGNED),
    (dict(sfb=P + 2), DG_ERR_MISALIGNED),
    (dict(c=P, d=P), DG_ERR_INVALID_ARG),
])
def test_ue8m0_calls_share_the_host_checks(lib, kw, code):
    assert dense_ue8m0(lib, **kw) == code
    args = dict(a=P, sfa=P, ld=256, b=P, sfb=P, d=P, idx=P, m=256, n=256, k=512, g=4)
    args.update({k: v for k, v in kw.items() if k in args})
    if "ld" in kw:
        args["ld"] = kw["ld"] + 128      # same misalignment, at least M_total rows
    if "c" not in kw:
        assert lib.dg_m_grouped_fp8_gemm_nt_contiguous_ue8m0(
            args["a"], args["sfa"], args["ld"], args["b"], args["sfb"], args["d"], args["idx"],
            args["m"], args["n"], args["k"], args["g"], None) == code


def contig(lib, a=P, sfa=P, ld=256, b=P, sfb=P, d=P, idx=P, m=256, n=256, k=512, g=4):
    return lib.dg_m_grouped_fp8_gemm_nt_contiguous(a, sfa, ld, b, sfb, d, idx, m, n, k, g, None)


@pytest.mark.parametrize("kw,code", [
    (dict(idx=None), DG_ERR_INVALID_ARG),
    (dict(g=0), DG_ERR_INVALID_ARG),
    (dict(m=200, ld=200), DG_ERR_UNSUPPORTED),
    (dict(k=384 + 64), DG_ERR_UNSUPPORTED),
    (dict(idx=P + 2), DG_ERR_MISALIGNED),
    (dict(ld=128), DG_ERR_INVALID_ARG),
])
def test_contiguous_rejects_bad_arguments_on_host(lib, kw, code):
    assert contig(lib, **kw) == code


def masked(lib, a=P, sfa=P, ld=256, b=P, sfb=P, d=P, mm=P, g=4, m_max=256, n=256, k=512):
    return lib.dg_m_grouped_fp8_gemm_nt_masked(a, sfa, ld, b, sfb, d, mm, g, m_max, n, k, 0, None)


@pytest.mark.parametrize("kw,code", [
    (dict(mm=None), DG_ERR_INVALID_ARG),
    (dict(g=-1), DG_ERR_INVALID_ARG),
    (dict(m_max=-5), DG_ERR_INVALID_ARG),
    (dict(n=8), DG_ERR_UNSUPPORTED),
    (dict(mm=P + 1), DG_ERR_MISALIGNED),
    (dict(ld=252), DG_ERR_INVALID_ARG),
])
def test_masked_rejects_bad_arguments_on_host(lib, kw, code):
    assert masked(lib, **kw) == code


def test_binding_rejects_host_tensors_before_the_library():
    import torch
    a = torch.zeros(128, 512, dtype=torch.uint8)
    with pytest.raises(ValueError):
        dg.fp8_gemm_nt(a, torch.zeros(4, 128), torch.zeros(256, 512, dtype=torch.uint8),
                       torch.zeros(2, 4), torch.zeros(128, 256, dtype=torch.bfloat16))
    with pytest.raises(ValueError):
        dg.fp8_gemm_nt_ue8m0(a, torch.zeros(1, 128, dtype=torch.int32),
                             torch.zeros(256, 512, dtype=torch.uint8),
                             torch.zeros(2, 1, dtype=torch.int32),
                             torch.zeros(128, 256, dtype=torch.bfloat16))


def kgrouped(lib, a=P, sfa=P, b=P, sfb=P, c=None, d=P, ks=(128, 256), m=128, n=256, k=384):
    arr = (ctypes.c_int32 * len(ks))(*ks) if ks is not None else None
    return lib.dg_k_grouped_fp8_gemm_tn_contiguous(a, sfa, b, sfb, c, d, arr, len(ks or ()), m,
                                                   n, k, None)


@pytest.mark.parametrize("kw,code", [
    (dict(ks=None), DG_ERR_INVALID_ARG),
    (dict(ks=()), DG_ERR_UNSUPPORTED),
    (dict(ks=(128,) * 257, k=128 * 257), DG_ERR_UNSUPPORTED),
    (dict(m=120), DG_ERR_UNSUPPORTED),
    (dict(n=0), DG_ERR_INVALID_ARG),
    (dict(k=400), DG_ERR_UNSUPPORTED),
    (dict(ks=(128, 100), k=228 + 28), DG_ERR_UNSUPPORTED),
    (dict(ks=(128, 128)), DG_ERR_INVALID_ARG),
    (dict(d=None), DG_ERR_INVALID_ARG),
    (dict(a=P + 8), DG_ERR_MISALIGNED),
    (dict(sfb=P + 4), DG_ERR_MISALIGNED),
    (dict(c=P + 16), DG_ERR_INVALID_ARG),
    (dict(m=65536, n=65536, k=32768, ks=(32768,)), DG_ERR_UNSUPPORTED),
])
def test_k_grouped_rejects_bad_arguments_on_host(lib, kw, code):
    assert kgrouped(lib, **kw) == code
    assert lib.dg_last_error().decode()
