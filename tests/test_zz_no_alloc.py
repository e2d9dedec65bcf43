"""The NT GEMM entry point that allocates nothing (dg_fp8_gemm_nt_noalloc) against the
allocating one (dg_fp8_gemm_nt), through the C ABI: two calls in a row on skinny shapes that
split K (so the static scratch holds the partial tiles), the second smaller than the first,
each equal bit for bit to the allocating call and within the tolerance of the oracle; a shape
that does not split K; and the host's refusal of a shape whose partials exceed the scratch."""
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
    print(f"[no_alloc] {msg}", flush=True)
    sys.stdout.flush()


def _both(p):
    args = [dev(x) for x in (p.a, p.sfa, p.b, p.sfb)]
    c = None if p.c is None else dev(p.c)
    d_ref = sentinel_like((p.m, p.n))
    d_new = sentinel_like((p.m, p.n))
    dg.fp8_gemm_nt(*args, d_ref, c)
    dg.fp8_gemm_nt_noalloc(*args, d_new, c)
    torch.cuda.synchronize()
    return bits(d_ref), bits(d_new)


def test_two_calls_in_a_row_the_second_smaller(monkeypatch):
    monkeypatch.setenv("DG_PRINT_CONFIGS", "1")
    for shape, seed, with_c in (((64, 2112, 7168), 0, False), ((40, 1024, 2048), 1, True)):
        m, n, k = shape
        _say(f"start {m}x{n}x{k}")
        p = W.make_dense(m, n, k, seed=300 + seed, with_c=with_c)
        ref_bits, new_bits = _both(p)
        assert np.array_equal(new_bits, ref_bits), f"{shape}: differs from the allocating call"
        assert_parity(new_bits, oracle.fp8_gemm_nt(p.a, p.sfa, p.b, p.sfb, p.c), f"{shape}")


def test_a_shape_without_split_k():
    p = W.make_dense(256, 448, 512, seed=302, with_c=True)
    ref_bits, new_bits = _both(p)
    assert np.array_equal(new_bits, ref_bits)
    assert_parity(new_bits, oracle.fp8_gemm_nt(p.a, p.sfa, p.b, p.sfb, p.c), "no split")


def test_partials_beyond_the_scratch_are_refused():
    # 64 x 8256 x 8192: 129 tiles of 64 x 64 and 8 splits of 8 K blocks need 16.9 MB of
    # partial tiles, more than the 16 MiB scratch; the host refuses before any launch
    m, n, k = 64, 8256, 8192
    a = torch.zeros((m, k), dtype=torch.uint8, device=DEV)
    sfa = torch.ones((k // 128, m), dtype=torch.float32, device=DEV)
    b = torch.zeros((n, k), dtype=torch.uint8, device=DEV)
    sfb = torch.ones(((n + 127) // 128, k // 128), dtype=torch.float32, device=DEV)
    d = sentinel_like((m, n))
    with pytest.raises(dg.DGError) as e:
        dg.fp8_gemm_nt_noalloc(a, sfa, b, sfb, d)
    assert e.value.code == -2 and "static scratch" in str(e.value)
    torch.cuda.synchronize()
    assert np.all(bits(d) == W.BF16_SENTINEL)
