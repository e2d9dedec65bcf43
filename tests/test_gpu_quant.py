"""Parity of the fused activation step (SwiGLU + 1x128 FP8 cast) on the GPU with the CPU
oracle, on the same seeded inputs.  The codes are integers decided from floating point the
two sides compute differently (the kernel in FP32 with the hardware exponential, the oracle in
float64), so the comparison is exact wherever that difference cannot change the decision: a
code must equal the oracle's unless h / scale lies within the kernel's error bound of a
rounding boundary, where either neighbour is accepted; the scales must agree within that
bound.  Then the cast feeds the NT GEMM, whose parity is checked on the GPU's own codes."""
import sys

import numpy as np
import pytest
import torch

import moe_grouped_gemm_fp8_amd as dg
import oracle
import workloads as W
from gpu_util import DEV, assert_parity, bits, dev, sentinel_like

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"[quant] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(autouse=True)
def _announce(request):
    _say(f"start {request.node.name}")
    yield


def run(x_bits, ld=None):
    m, i2 = x_bits.shape
    i = i2 // 2
    ld = (m + 3) // 4 * 4 if ld is None else ld
    x = dev(x_bits.view(np.int16))
    q = torch.full((m, i), 0x7F, dtype=torch.uint8, device=DEV)
    sf = torch.full((i // 128, ld), float("nan"), dtype=torch.float32, device=DEV)
    dg.swiglu_fp8_quant(x, q, sf)
    torch.cuda.synchronize()
    return q.cpu().numpy(), sf.cpu().numpy()


def rel_bound(x_bits):
    """Per-element bound on the kernel's relative error in h: a few FP32 roundings, plus the
    exponential's argument rounding, which grows with |gate|."""
    g = oracle.bf16_decode(x_bits[:, :x_bits.shape[1] // 2])
    return 2.0 ** -19 + np.abs(g) * 2.0 ** -21


def check(x_bits, q, sf, what):
    h, sf_ref, q_ref = oracle.swiglu_quant(x_bits)
    m, i = h.shape
    eps = rel_bound(x_bits)
    seg_eps = eps.reshape(m, i // 128, 128).max(axis=2).T            # [I/128, M]
    s_ref = sf_ref[:, :m]
    s_gpu = sf[:, :m].astype(np.float64)
    bad_s = ~(np.abs(s_gpu - s_ref) <= (seg_eps + 2.0 ** -22) * s_ref)
    assert not bad_s.any(), f"{what}: {int(bad_s.sum())} scales off, first {np.argwhere(bad_s)[:3].tolist()}"
    # the codes, against the kernel's own scale
    s_el = np.repeat(s_gpu.T, 128, axis=1)                             # [M, I]
    y = h / s_el
    lo = oracle.e4m3_nearest(np.clip(y * (1 - eps * np.sign(y)), -448, 448))
    hi = oracle.e4m3_nearest(np.clip(y * (1 + eps * np.sign(y)), -448, 448))
    tab = oracle.e4m3_table()
    unique = lo == hi
    bad_u = unique & (q != lo)
    assert not bad_u.any(), (f"{what}: {int(bad_u.sum())} codes differ where the decision is "
                             f"unique, first {np.argwhere(bad_u)[:3].tolist()}")
    vlo, vhi, vq = tab[lo], tab[hi], tab[q]
    bad_n = ~unique & ~((vq >= np.minimum(vlo, vhi)) & (vq <= np.maximum(vlo, vhi)))
    assert not bad_n.any(), f"{what}: {int(bad_n.sum())} codes outside the rounding interval"
    return int((~unique).sum())


@pytest.mark.parametrize("m,i", [(37, 512), (5, 384), (64, 128), (1, 2048)])
def test_small_with_outliers_and_partial_tasks(m, i):
    x = W.make_swiglu_input(m, i, seed=100 + i)
    q, sf = run(x)
    near = check(x, q, sf, f"{m}x{i}")
    _say(f"{near} of {m * i} codes within the error bound of a boundary")


def test_scale_columns_past_m_are_not_written():
    x = W.make_swiglu_input(6, 256, seed=7)
    q, sf = run(x, ld=16)
    assert np.isnan(sf[:, 6:]).all()
    check(x, q, sf, "ld=16")


def test_workload_full():
    x = W.make_config("moe_swiglu_quant", seed=0)                 # 32768 x 2048
    q, sf = run(x)
    near = check(x, q, sf, "moe_swiglu_quant")
    _say(f"{near} of {q.size} codes within the error bound of a boundary")


def test_cast_feeds_the_nt_gemm():
    # the GPU's own codes and scales as A of the second GEMM: the layouts agree end to end
    m, i, n = 200, 512, 384
    x = W.make_swiglu_input(m, i, seed=8)
    q, sf = run(x)
    b = W.make_dense(16, n, i, seed=9)
    d = sentinel_like((m, n))
    dg.fp8_gemm_nt(dev(q), dev(sf), dev(b.b), dev(b.sfb), d)
    torch.cuda.synchronize()
    assert_parity(bits(d), oracle.fp8_gemm_nt(q, sf, b.b, b.sfb), "swiglu -> nt")


def test_host_checks():
    x = dev(W.make_swiglu_input(4, 256, seed=1).view(np.int16))
    q = torch.zeros((4, 256), dtype=torch.uint8, device=DEV)
    sf = torch.zeros((2, 3), dtype=torch.float32, device=DEV)
    with pytest.raises(ValueError):                                # the binding's own check
        dg.swiglu_fp8_quant(x, q, sf)
    lib = dg._load()
    assert lib.dg_swiglu_fp8_quant(x.data_ptr(), q.data_ptr(), sf.data_ptr(), 3, 4, 256,
                                   None) == -1                     # ld < m, the library's
    assert lib.dg_swiglu_fp8_quant(None, None, None, 0, 0, 256, None) == 0     # m == 0
    assert lib.dg_swiglu_fp8_quant(x.data_ptr(), q.data_ptr(), None, 4, 4, 200, None) == -2
