"""Parity of the contiguous GEMM with the activation step fused into its epilogue
(dg_m_grouped_fp8_gemm_nt_contiguous_swiglu) with the oracle's fused reading, on the same
seeded inputs: the codes under the rule derived from the formats (exact wherever the kernel's
error bound cannot move a code across a rounding boundary, either neighbour elsewhere), the
scales within that bound, padding rows untouched; then the MoE block chained through the second
GEMM on the kernel's own codes; small cases over several tiles, persistent workgroups walking
many tiles, stress scales, and the full-size block."""
import sys

import numpy as np
import pytest
import torch

import moe_grouped_gemm_fp8_amd as dg
import oracle
import workloads as W
from gpu_util import DEV, assert_parity, bits, cached_ref, dev, sentinel_like
from tolerance import fused_cast_violations, gemm_error_bound

pytestmark = pytest.mark.gpu

Q_SENTINEL = 0x7F      # the e4m3 NaN code: never produced by the cast (codes stay within +-448)


def _say(msg):
    print(f"[fused] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(autouse=True)
def _announce(request):
    _say(f"start {request.node.name}")
    yield


def run_fused(p):
    i = p.n // 2
    ld = W.sf_aligned(p.m_total)
    q = torch.full((p.m_total, i), Q_SENTINEL, dtype=torch.uint8, device=DEV)
    sfq = torch.full((i // 128, ld), float("nan"), dtype=torch.float32, device=DEV)
    dg.m_grouped_fp8_gemm_nt_contiguous_swiglu(dev(p.a), dev(p.sfa), dev(p.b), dev(p.sfb), q, sfq,
                                               dev(p.m_indices))
    torch.cuda.synchronize()
    return q, sfq


def check_fused(p, q_dev, sfq_dev, d1=None, what=""):
    """Codes and scales of the valid rows against the oracle; padding rows untouched."""
    q = q_dev.cpu().numpy()
    sfq = sfq_dev.cpu().numpy()
    pad = p.m_indices < 0
    assert np.all(q[pad] == Q_SENTINEL), f"{what}: padding rows of q written"
    assert np.isnan(sfq[:, :p.m_total][:, pad]).all(), f"{what}: padding rows of sfq written"
    rows = np.nonzero(~pad)[0]
    assert not np.any(q[rows] == Q_SENTINEL), f"{what}: valid codes left unwritten"
    if d1 is None:
        d1 = oracle.m_grouped_contiguous(p.a, p.sfa, p.b, p.sfb, p.m_indices)
    tab = oracle.e4m3_table()
    amb_total, n_codes = 0, 0
    for r0 in range(0, rows.size, 4096):                # in chunks of rows (memory)
        rr = rows[r0:r0 + 4096]
        d1r = d1[rr]
        h, s_ref, _ = oracle.quant_1x128(oracle.swiglu_values(d1r))
        s_ref = s_ref[:, :rr.size].T
        err = gemm_error_bound(p.a[rr], p.sfa[:, rr].T, p.b, p.sfb, p.m_indices[rr], tab)
        bad_s, bad_q, amb = fused_cast_violations(q[rr], sfq[:, rr].T.astype(np.float64), d1r,
                                                  err, h, s_ref, tab, oracle.e4m3_nearest)
        if bad_s.any():
            idx = np.argwhere(bad_s)[:3]
            raise AssertionError(f"{what}: {int(bad_s.sum())} scales outside the bound, first "
                                 f"(row, segment) {[(int(rr[a]), int(b)) for a, b in idx]}")
        if bad_q.any():
            idx = np.argwhere(bad_q)[:3]
            raise AssertionError(f"{what}: {int(bad_q.sum())} codes outside the rule, first "
                                 f"(row, col) {[(int(rr[a]), int(b)) for a, b in idx]}")
        amb_total += amb
        n_codes += q[rr].size
    _say(f"{what}: {amb_total} of {n_codes} codes within the error bound of a boundary")
    return q, sfq


# 128 x 256 persistent tiles, and 256 x 256 tiles (scales in registers), whose tiles can hold
# two groups: [0,130,41,300,129] -> 128-row blocks 1 1 | 2 3 | 3 3 | 4 4 (one straddle),
# [41,0,300,1,130] -> 0 2 | 2 2 | 3 4 | 4 - (two, the last tile half past m_total); the second
# group of a straddle on a workgroup of its own, or (DG_STRADDLE_ROWS=0) in the tile's own
@pytest.mark.parametrize("cfg,served", [(None, None), ("128x256w8", None), ("256x256w8", None),
                                        ("256x256w8", "0")])
@pytest.mark.parametrize("i,k,counts", [(128, 128, [0, 130, 41, 300, 129]),
                                        (256, 640, [0, 130, 41, 300, 129]),
                                        (384, 384, [200, 0, 0, 57, 300]),
                                        (128, 256, [41, 0, 300, 1, 130])])
def test_small_with_padding_and_empty_groups(cfg, served, i, k, counts, monkeypatch):
    if cfg:
        monkeypatch.setenv("DG_FORCE_CONFIG", cfg)
    if served is not None:
        monkeypatch.setenv("DG_STRADDLE_ROWS", served)
    p = W.make_contiguous(5, sum(counts), 2 * i, k, seed=200 + i, counts=counts, pad_nan=True,
                          stress=True)
    check_fused(p, *run_fused(p), what=f"{cfg} i={i} k={k}")


# The tail: the tiles of the last-dispatched 256 x 256 workgroups run as 128 x 256 tiles at the
# end of the same launch (DG_TAIL_TILES forces how many; 9 is more than there are, so all but
# one), straddles and a tile half past m_total among them, and with few tail workgroups (each
# then walks several tiles)
@pytest.mark.parametrize("tail,wgs", [("1", None), ("3", None), ("9", None), ("5", "2")])
@pytest.mark.parametrize("served", [None, "1"])
@pytest.mark.parametrize("counts", [[0, 130, 41, 300, 129], [41, 0, 300, 1, 130]])
def test_tail_in_128_row_tiles(tail, wgs, served, counts, monkeypatch):
    monkeypatch.setenv("DG_FORCE_CONFIG", "256x256w8")
    monkeypatch.setenv("DG_TAIL_TILES", tail)
    if wgs is not None:
        monkeypatch.setenv("DG_PERSIST_WGS", wgs)
    if served is not None:
        monkeypatch.setenv("DG_STRADDLE_ROWS", served)
    p = W.make_contiguous(5, sum(counts), 512, 640, seed=213, counts=counts, pad_nan=True,
                          stress=True)
    check_fused(p, *run_fused(p), what=f"tail {tail} wgs={wgs} served={served} {counts}")


@pytest.mark.parametrize("wgs", ["3", "10"])
@pytest.mark.parametrize("k", [256, 1280])
def test_persistent_workgroups_walk_many_tiles(wgs, k, monkeypatch):
    # few workgroups: each walks a run of tiles, prefetching the next tile's first blocks (long
    # K) or restarting its pipeline per tile (short K); the segment maxima's LDS area is reused
    monkeypatch.setenv("DG_FORCE_CONFIG", "128x256w8")
    monkeypatch.setenv("DG_PERSIST_WGS", wgs)
    p = W.make_contiguous(4, 900, 768, k, seed=210, counts=[300, 41, 0, 559], pad_nan=True)
    check_fused(p, *run_fused(p), what=f"wgs={wgs} k={k}")


@pytest.mark.parametrize("cfg", ["128x256w8", "256x256w8"])
def test_stress_scales(cfg, monkeypatch):
    monkeypatch.setenv("DG_FORCE_CONFIG", cfg)
    p = W.make_contiguous(4, 700, 512, 512, seed=211, stress=True, pad_nan=True)
    check_fused(p, *run_fused(p), what=f"stress {cfg}")


def test_host_checks():
    p = W.make_contiguous(2, 256, 384, 256, seed=212, counts=[128, 128])
    q = torch.zeros((256, 192), dtype=torch.uint8, device=DEV)
    sfq = torch.zeros((1, 256), dtype=torch.float32, device=DEV)
    lib = dg._load()
    rc = lib.dg_m_grouped_fp8_gemm_nt_contiguous_swiglu(
        dev(p.a).data_ptr(), dev(p.sfa).data_ptr(), p.sfa.shape[1], dev(p.b).data_ptr(),
        dev(p.sfb).data_ptr(), q.data_ptr(), sfq.data_ptr(), 256, dev(p.m_indices).data_ptr(),
        256, 384, 256, 2, None)
    assert rc == -2                                   # n = 384: halves not multiples of 128


def _chain(blk, q, sfq):
    """The second GEMM of the block on the kernel's own codes and scales."""
    p = blk.up
    d2 = sentinel_like((p.m_total, blk.n2))
    dg.m_grouped_fp8_gemm_nt_contiguous(q, sfq, dev(blk.b2), dev(blk.sfb2), d2,
                                        dev(p.m_indices))
    torch.cuda.synchronize()
    return bits(d2)


def test_block_chained_through_the_second_gemm():
    blk = W.make_moe_block(5, 900, 512, 640, 384, seed=213, counts=[300, 41, 0, 430, 129])
    p = blk.up
    q, sfq = run_fused(p)
    qh, sh = check_fused(p, q, sfq, what="block linear 1")
    d2 = _chain(blk, q, sfq)
    ref = oracle.m_grouped_contiguous(qh, sh, blk.b2, blk.sfb2, p.m_indices)
    assert_parity(d2, ref, "block linear 2")


def test_block_workload_full():
    blk = W.make_config("moe_block", seed=0)       # the experts of moe_contiguous's routing
    p = blk.up
    q, sfq = run_fused(p)
    d1 = cached_ref("moe_contiguous", lambda: oracle.m_grouped_contiguous(
        p.a, p.sfa, p.b, p.sfb, p.m_indices))
    qh, sh = check_fused(p, q, sfq, d1=d1, what="moe_block linear 1")
    d2 = _chain(blk, q, sfq)
    ref = oracle.m_grouped_contiguous(qh, sh, blk.b2, blk.sfb2, p.m_indices)
    assert_parity(d2, ref, "moe_block linear 2")
