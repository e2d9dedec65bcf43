"""Parity of the K-grouped TN GEMM (MoE weight gradient) on the GPU with the CPU oracle, on the
same seeded inputs: ragged M and N tails, groups of every extent from zero blocks up, C added,
accumulated in place and absent, a single group, the full group table, and the full-size
workload compared in full.  D is FP32, compared under the same rule as the bf16 outputs:
|d - d_ref| <= 1e-2 |d_ref| + 1e-3 rms(D_ref), rms over all of D."""
import sys

import numpy as np
import pytest
import torch

import moe_grouped_gemm_fp8_amd as dg
import oracle
import workloads as W
from gpu_util import DEV, dev
from tolerance import tol_violations

pytestmark = pytest.mark.gpu

def _say(msg):
    print(f"[kgrouped] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(autouse=True)
def _announce(request):
    _say(f"start {request.node.name}")
    yield


def run(p, c_mode="given"):
    """c_mode: "given" (C as a separate tensor), "inplace" (D starts as C), "none"."""
    a, sfa, b, sfb = dev(p.a), dev(p.sfa), dev(p.b), dev(p.sfb)
    shape = (p.num_groups, p.m, p.n)
    if c_mode == "inplace":
        d = dev(p.c)
        dg.k_grouped_fp8_gemm_tn_contiguous(a, sfa, b, sfb, d, p.ks, c=d)
    else:
        d = torch.full(shape, float("nan"), dtype=torch.float32, device=DEV)
        c = dev(p.c) if (c_mode == "given" and p.c is not None) else None
        dg.k_grouped_fp8_gemm_tn_contiguous(a, sfa, b, sfb, d, p.ks, c=c)
    torch.cuda.synchronize()
    return d.cpu().numpy()


def check(got, ref, what):
    assert not np.isnan(got).any(), f"{what}: elements left unwritten"
    bad = tol_violations(got, ref)
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError(f"{what}: {int(bad.sum())}/{bad.size} outside the tolerance, "
                             f"first at {idx.tolist()}: got {got[bad][:5]} want {ref[bad][:5]}")


@pytest.mark.parametrize("c_mode", ["given", "inplace", "none"])
def test_small_groups_with_empty_and_ragged_tiles(c_mode):
    # M and N leave partial 128-wide tiles; extents 0, 1, 2 and 5 blocks
    p = W.make_k_grouped(5, 900, 208, 336, seed=81, counts=[0, 100, 250, 550, 0],
                         with_c=c_mode != "none")
    ref = oracle.k_grouped_tn(p.a, p.sfa, p.b, p.sfb, p.ks, p.c if c_mode != "none" else None)
    check(run(p, c_mode), ref, c_mode)


def test_stress_scales_and_one_group():
    p = W.make_k_grouped(1, 1200, 128, 256, seed=82, stress=True, with_c=True)
    check(run(p), oracle.k_grouped_tn(p.a, p.sfa, p.b, p.sfb, p.ks, p.c), "stress")


@pytest.mark.parametrize("blocks", [1, 2, 3, 4, 7])
def test_block_counts_around_the_pipeline_depth(blocks):
    p = W.make_k_grouped(2, 128 * blocks + 64, 256, 128, seed=83 + blocks,
                         counts=[128 * blocks, 64], with_c=True)
    check(run(p), oracle.k_grouped_tn(p.a, p.sfa, p.b, p.sfb, p.ks, p.c), f"{blocks} blocks")


@pytest.mark.parametrize("blocks", [1, 3, 4])
def test_narrow_tiles(blocks, monkeypatch):
    # the 128 x 128 tile (four slots, two B register sets), which DG_KG_TILE_N=128 selects
    monkeypatch.setenv("DG_KG_TILE_N", "128")
    p = W.make_k_grouped(3, 128 * blocks + 200, 208, 336, seed=90 + blocks,
                         counts=[128 * blocks, 0, 200], stress=True, with_c=True)
    check(run(p), oracle.k_grouped_tn(p.a, p.sfa, p.b, p.sfb, p.ks, p.c), f"narrow {blocks}")


def test_all_groups_empty_writes_c_or_zero():
    p = W.make_k_grouped(3, 0, 64, 48, seed=85, counts=[0, 0, 0], with_c=True)
    assert p.k_total == 0
    got = run(p)
    assert np.array_equal(got, p.c)
    q = W.make_k_grouped(3, 0, 64, 48, seed=85, counts=[0, 0, 0])
    assert not run(q, "none").any()


def test_full_group_table():
    counts = np.zeros(256, np.int64)
    counts[::37] = 129                                             # 7 groups of 2 blocks
    p = W.make_k_grouped(256, int(counts.sum()), 32, 64, seed=86, counts=counts)
    check(run(p, "none"), oracle.k_grouped_tn(p.a, p.sfa, p.b, p.sfb, p.ks), "256 groups")


def test_host_rejects_bad_extents():
    p = W.make_k_grouped(2, 256, 64, 64, seed=87, counts=[128, 128])
    a, sfa, b, sfb = dev(p.a), dev(p.sfa), dev(p.b), dev(p.sfb)
    d = torch.zeros(2, 64, 64, dtype=torch.float32, device=DEV)
    for ks, code in (([100, 156], -2), ([128, 0], -1), ([-128, 384], -2)):
        with pytest.raises(dg.DGError) as e:
            dg.k_grouped_fp8_gemm_tn_contiguous(a, sfa, b, sfb, d, ks)
        assert e.value.code == code, ks


def _k_grouped_ref_by_column_chunks(p, chunk=256):
    """The oracle on every column of A, in chunks of columns run on a thread pool: each output
    row m depends on column m of A and its scales only, so the chunks give exactly the whole
    result (numpy's products and element-wise passes run outside the interpreter lock)."""
    from concurrent.futures import ThreadPoolExecutor
    out = np.empty((p.num_groups, p.m, p.n), dtype=np.float64)

    def one(m0):
        cols = slice(m0, min(p.m, m0 + chunk))
        out[:, cols] = oracle.k_grouped_tn(np.ascontiguousarray(p.a[:, cols]),
                                           np.ascontiguousarray(p.sfa[:, cols]), p.b, p.sfb, p.ks)

    with ThreadPoolExecutor(max_workers=8) as ex:
        list(ex.map(one, range(0, p.m, chunk)))
    return out


def test_wgrad_workload_full():
    p = W.make_config("moe_wgrad", seed=0)                     # 8 experts, 4096 x 7168
    got = run(p, "none")
    assert not np.isnan(got).any(), "some outputs were never written"
    check(got, _k_grouped_ref_by_column_chunks(p), "moe_wgrad")
