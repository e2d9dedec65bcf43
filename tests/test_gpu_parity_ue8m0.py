"""Parity of the UE8M0-scaled calls (packed power-of-two scales, four K blocks per int32,
applied by the block-scaled MFMA) with the CPU oracle on the same seeded inputs: every
pipelined tile configuration on ragged shapes, K-block counts that leave the last packed
word partly used, persistent workgroups looping over tiles, NaN scales, the grouped forms
with their padding and clamps, and the full-size workloads compared in full."""
import sys

import numpy as np
import pytest

import moe_grouped_gemm_fp8_amd as dg

import oracle
import workloads as W
from gpu_util import (assert_parity, fp32_scales, run_contiguous, run_dense,
                      run_masked)
from tolerance import bf16_bits_to_f64

pytestmark = pytest.mark.gpu

PIPELINED = ["256x224w8", "128x256w4", "128x128w4", "64x32w4", "256x128w8", "256x128w8p",
             "128x128w4d4", "128x128w8d4", "128x256w8", "256x256w8"]


def _say(msg):
    print(f"[parity-ue8m0] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(autouse=True)
def _announce(request):
    _say(f"start {request.node.name}")
    yield


def dense_ref(p):
    return oracle.fp8_gemm_nt_ue8m0(p.a, p.sfa, p.b, p.sfb, p.c)


# ------------------------------------------------------------------------------ dense

def test_dense_small_workload_full():
    p = W.make_config("dense_small", seed=0, ue8m0=True)
    assert_parity(run_dense(p), dense_ref(p), "dense_small ue8m0")


# Without C the MFMAs accumulate directly; with C (added to the accumulators inside the K
# loop) they produce per-block partials that the vector unit adds: both kernel variants.
@pytest.mark.parametrize("with_c", [False, True])
@pytest.mark.parametrize("cfg", PIPELINED)
def test_dense_ragged_every_tile_config(cfg, with_c, monkeypatch):
    monkeypatch.setenv("DG_FORCE_CONFIG", cfg)
    p = W.make_dense(200, 336, 640, seed=51, with_c=with_c, ue8m0=True)  # 5 K blocks: 2 words
    assert_parity(run_dense(p), dense_ref(p), f"{cfg} c={with_c}")


@pytest.mark.parametrize("with_c", [False, True])
@pytest.mark.parametrize("splits", [1, 2, 3, 7])
def test_streaming_split_k_with_ragged_tiles(splits, with_c, monkeypatch):
    # 9 K blocks in 3 packed words: splits start inside a word (kb0 = 5, 3, 2, ...)
    monkeypatch.setenv("DG_FORCE_CONFIG", "stream64")
    monkeypatch.setenv("DG_FORCE_SPLITS", str(splits))
    p = W.make_dense(100, 208, 1152, seed=52, with_c=with_c, ue8m0=True)
    assert_parity(run_dense(p), dense_ref(p), f"stream64 splits={splits} c={with_c}")


def test_dense_skinny_workload_full_and_deterministic():
    p = W.make_config("dense_skinny", seed=0, ue8m0=True)      # 64 x 2112 x 7168, split-K
    d1 = run_dense(p)
    assert_parity(d1, dense_ref(p), "dense_skinny ue8m0")
    assert np.array_equal(d1, run_dense(p)), "split-K reduction is not deterministic"


@pytest.mark.parametrize("k", [128, 256, 384, 512, 1152, 2048])
@pytest.mark.parametrize("cfg", ["256x224w8", "128x256w8"])
@pytest.mark.parametrize("with_c", [False, True])
def test_dense_k_blocks_across_packed_words(cfg, k, with_c, monkeypatch):
    # every position of the last K block inside its packed word (with C: added in the loop)
    monkeypatch.setenv("DG_FORCE_CONFIG", cfg)
    p = W.make_dense(256, 448, k, seed=53, with_c=with_c, c_std=2.0, ue8m0=True)
    assert_parity(run_dense(p), dense_ref(p), f"{cfg} k={k}")


PERSISTENT = ["128x256w8", "128x128w4", "64x32w4", "256x128w8p", "128x128w8d4"]


@pytest.mark.parametrize("cfg", PERSISTENT)
@pytest.mark.parametrize("wgs,with_c", [("3", True), ("10", False)])
def test_persistent_workgroups_loop_over_tiles(cfg, wgs, with_c, monkeypatch):
    monkeypatch.setenv("DG_FORCE_CONFIG", cfg)
    monkeypatch.setenv("DG_PERSIST_WGS", wgs)
    p = W.make_dense(300, 528, 1280, seed=54, with_c=with_c, ue8m0=True)
    assert_parity(run_dense(p), dense_ref(p), f"{cfg} wgs={wgs}")


def test_dense_stress_scales():
    # power-of-two multipliers 2^-8 .. 2^8 per segment and block: exponents 112..142 apart
    p = W.make_dense(256, 384, 1024, seed=55, stress=True, ue8m0=True)
    assert_parity(run_dense(p), dense_ref(p), "ue8m0 stress")


def test_dense_small_shapes():
    for m, n, k in [(1, 128, 128), (16, 2112, 1024), (64, 256, 7168)]:
        p = W.make_dense(m, n, k, seed=56 + m, ue8m0=True)
        assert_parity(run_dense(p), dense_ref(p), f"{m}x{n}x{k}")


def test_dense_nan_scale_poisons_its_row_or_block():
    p = W.make_dense(128, 256, 512, seed=57, ue8m0=True)
    sfa, sfb = p.sfa.copy(), p.sfb.copy()
    sfa[0, 5] = (sfa[0, 5] & ~0xFF0000) | (0xFF << 16)          # row 5, K block 2
    sfb[1, 0] = (sfb[1, 0] & ~0xFF) | 0xFF                      # columns 128..255, K block 0
    p.sfa, p.sfb = sfa, sfb
    ref = dense_ref(p)
    assert np.isnan(ref[5]).all() and np.isnan(ref[:, 128:]).all()
    got_bits = run_dense(p)
    got = bf16_bits_to_f64(got_bits)
    assert np.isnan(got[5]).all() and np.isnan(got[:, 128:]).all()
    keep = np.arange(128) != 5
    assert_parity(got_bits[keep][:, :128], ref[keep][:, :128], "finite part")


def test_dense_prefill_workload_full():
    p = W.make_config("dense_prefill", seed=0, ue8m0=True)      # 4096 x 7168 x 2048 with C
    got = run_dense(p)
    assert not np.any(got == W.BF16_SENTINEL), "some outputs were never written"
    assert_parity(got, oracle.fp8_gemm_nt_ue8m0(p.a, p.sfa, p.b, p.sfb, p.c), "dense_prefill ue8m0")


# ------------------------------------------------------------------------------ contiguous

@pytest.mark.parametrize("cfg", [None, "128x128w4", "64x32w4", "128x128w8d4", "128x256w8",
                                 "256x224w8", "256x128w8", "256x256w8"])
def test_contiguous_small_with_empty_group_and_nan_padding(cfg, monkeypatch):
    if cfg:
        monkeypatch.setenv("DG_FORCE_CONFIG", cfg)
    p = W.make_contiguous(5, 600, 256, 640, seed=61, counts=[0, 130, 41, 300, 129],
                          pad_nan=True, ue8m0=True)
    ref = oracle.m_grouped_contiguous_ue8m0(p.a, p.sfa, p.b, p.sfb, p.m_indices)
    assert_parity(run_contiguous(p), ref, f"contiguous ue8m0 {cfg}")


@pytest.mark.parametrize("counts", [[0, 130, 41, 300, 129], [41, 0, 300, 1, 130]])
def test_contiguous_256_row_tiles_across_group_boundaries(counts, monkeypatch):
    # 128-row blocks 1 1 | 2 3 | 3 3 | 4 4, and 0 2 | 2 2 | 3 4 | 4 - (last tile past m_total)
    monkeypatch.setenv("DG_FORCE_CONFIG", "256x224w8")
    p = W.make_contiguous(5, sum(counts), 448, 640, seed=62, counts=counts, stress=True,
                          pad_nan=True, ue8m0=True)
    ref = oracle.m_grouped_contiguous_ue8m0(p.a, p.sfa, p.b, p.sfb, p.m_indices)
    got = run_contiguous(p)
    assert_parity(got, ref, f"contiguous ue8m0 256-row {counts}")
    assert not np.any(got[p.m_indices >= 0] == W.BF16_SENTINEL), "valid rows left unwritten"


@pytest.mark.parametrize("tail", ["2", "7"])
@pytest.mark.parametrize("counts", [[0, 130, 41, 300, 129], [41, 0, 300, 1, 130]])
def test_contiguous_tail_launch(tail, counts, monkeypatch):
    # the tiles of the last-dispatched workgroups of the 256 x 256 launch as 128 x 128 tiles in
    # the same launch, straddles and a tile half past m_total among them
    monkeypatch.setenv("DG_FORCE_CONFIG", "256x256w8")
    monkeypatch.setenv("DG_TAIL_TILES", tail)
    p = W.make_contiguous(5, sum(counts), 400, 640, seed=62, counts=counts, stress=True,
                          pad_nan=True, ue8m0=True)
    ref = oracle.m_grouped_contiguous_ue8m0(p.a, p.sfa, p.b, p.sfb, p.m_indices)
    got = run_contiguous(p)
    assert_parity(got, ref, f"contiguous ue8m0 tail {tail} {counts}")
    assert not np.any(got[p.m_indices >= 0] == W.BF16_SENTINEL), "valid rows left unwritten"


def test_contiguous_workload_full():
    p = W.make_config("moe_contiguous", seed=0, ue8m0=True)    # 8 experts, 32768 x 4096 x 7168
    got = run_contiguous(p)
    pad = p.m_indices < 0
    assert np.all(got[pad] == W.BF16_SENTINEL), "padding rows were written"
    assert not np.any(got[~pad] == W.BF16_SENTINEL), "valid rows were left unwritten"
    ref = oracle.m_grouped_contiguous_ue8m0(p.a, p.sfa, p.b, p.sfb, p.m_indices)
    assert_parity(got, ref, "moe_contiguous ue8m0")


# ------------------------------------------------------------------------------ masked

@pytest.mark.parametrize("cfg", [None, "128x128w4", "64x32w4", "256x128w8", "256x128w8p",
                                 "256x224w8", "256x256w8"])
def test_masked_small_with_clamps_and_nan_tails(cfg, monkeypatch):
    if cfg:
        monkeypatch.setenv("DG_FORCE_CONFIG", cfg)
    mm = [0, 1, 255, 256, 130, 999, -3]
    p = W.make_masked(7, 256, 384, 640, seed=71, masked_m=mm, tail_nan=True, ue8m0=True)
    ref = oracle.m_grouped_masked_ue8m0(p.a, p.sfa, p.b, p.sfb, p.masked_m)
    assert_parity(run_masked(p), ref, f"masked ue8m0 {cfg}")


def test_masked_workload_full():
    p = W.make_config("moe_masked", seed=0, ue8m0=True)        # 16 x 256 x 7168 x 2048
    got = run_masked(p)
    for g in range(p.num_groups):
        valid = int(p.masked_m[g])
        assert np.all(got[g, valid:] == W.BF16_SENTINEL), f"group {g}: tail written"
        assert not np.any(got[g, :valid] == W.BF16_SENTINEL), f"group {g}: rows unwritten"
    ref = oracle.m_grouped_masked_ue8m0(p.a, p.sfa, p.b, p.sfb, p.masked_m)
    assert_parity(got, ref, "moe_masked ue8m0")


def test_masked_graph_replays_follow_device_masked_m():
    import torch
    from gpu_util import bits, dev, sentinel_like
    g_, m_max, n, k = 6, 256, 448, 640
    p = W.make_masked(g_, m_max, n, k, seed=73, ue8m0=True)
    a, sfa, b, sfb = dev(p.a), dev(p.sfa), dev(p.b), dev(p.sfb)
    mm_dev = dev(p.masked_m)
    d = sentinel_like((g_, m_max, n))
    call = lambda: dg.m_grouped_fp8_gemm_nt_masked_ue8m0(a, sfa, b, sfb, d, mm_dev)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    for r in range(4):
        mm = W.masked_counts(g_, m_max, seed=73, replay=r)
        d.view(torch.int16).fill_(W.BF16_SENTINEL)
        mm_dev.copy_(torch.from_numpy(mm))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        ref = oracle.m_grouped_masked_ue8m0(p.a, p.sfa, p.b, p.sfb, mm)
        assert_parity(bits(d), ref, f"ue8m0 graph replay {r}")
