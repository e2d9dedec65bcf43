"""Parity of the dense NN, TN and TT layouts (operands stored MN-major on one or both sides) on
the GPU with the CPU oracle, on the same seeded inputs: ragged M and N tiles, K-block counts
around the pipeline depth, extreme scales, N with a partial last B scale block, the full-size
prefill shape on sampled rows, and the host checks particular to the layouts."""
import sys

import numpy as np
import pytest

import moe_grouped_gemm_fp8_amd as dg
import oracle
import workloads as W
from gpu_util import assert_parity, dev, sentinel_like, bits
import torch

pytestmark = pytest.mark.gpu

LAYOUTS = ["nn", "tn", "tt"]


def _say(msg):
    print(f"[layouts] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(autouse=True)
def _announce(request):
    _say(f"start {request.node.name}")
    yield


def run(layout, p):
    d = sentinel_like((p.m, p.n))
    getattr(dg, "fp8_gemm_" + layout)(dev(p.a), dev(p.sfa), dev(p.b), dev(p.sfb), d,
                                      None if p.c is None else dev(p.c))
    torch.cuda.synchronize()
    return bits(d)


def ref(layout, p):
    return oracle.fp8_gemm_layout(layout, p.a, p.sfa, p.b, p.sfb, p.c)


# "transposed": MN-major operands transposed into the workspace, then the NT kernels (the
# default); "native": the layout kernel reads them directly (the path under graph capture
# before the workspace exists)
PATHS = ["transposed", "native"]


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("with_c", [False, True])
def test_ragged_tiles(layout, with_c, path, monkeypatch):
    monkeypatch.setenv("DG_LAYOUT_NATIVE", "1" if path == "native" else "0")
    p = W.stored_layout(W.make_dense(208, 336, 640, seed=91, with_c=with_c), layout)
    assert_parity(run(layout, p), ref(layout, p), f"{layout} c={with_c} {path}")


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("k", [128, 256, 384, 1152])
def test_k_blocks(layout, k, path, monkeypatch):
    monkeypatch.setenv("DG_LAYOUT_NATIVE", "1" if path == "native" else "0")
    p = W.stored_layout(W.make_dense(128, 256, k, seed=92, with_c=True, c_std=2.0), layout)
    assert_parity(run(layout, p), ref(layout, p), f"{layout} k={k} {path}")


@pytest.mark.parametrize("layout", LAYOUTS)
def test_graph_replays_of_the_transposed_path(layout):
    p = W.stored_layout(W.make_dense(256, 512, 512, seed=95, with_c=True), layout)
    a, sfa, b, sfb, c = dev(p.a), dev(p.sfa), dev(p.b), dev(p.sfb), dev(p.c)
    fn = getattr(dg, "fp8_gemm_" + layout)
    d = sentinel_like((p.m, p.n))
    fn(a, sfa, b, sfb, d, c)                                         # workspace in place
    torch.cuda.synchronize()
    eager = bits(d)
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g):
            fn(a, sfa, b, sfb, d, c)
    torch.cuda.current_stream().wait_stream(side)
    for r in range(3):
        d.view(torch.int16).fill_(W.BF16_SENTINEL)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(bits(d), eager), f"replay {r}"
    assert_parity(eager, ref(layout, p), f"{layout} graph")


@pytest.mark.parametrize("layout", LAYOUTS)
def test_stress_scales_and_partial_b_block(layout):
    p = W.stored_layout(W.make_dense(64, 2112, 1024, seed=93, stress=True), layout)
    assert_parity(run(layout, p), ref(layout, p), f"{layout} stress")


@pytest.mark.parametrize("layout", LAYOUTS)
def test_prefill_shape_sampled_rows(layout):
    q = W.make_config("dense_prefill", seed=0)                   # 4096 x 7168 x 2048 with C
    p = W.stored_layout(q, layout)
    got = run(layout, p)
    assert not np.any(got == W.BF16_SENTINEL), "some outputs were never written"
    rng = np.random.default_rng(130)
    rows = np.unique(np.concatenate([np.arange(4), np.arange(q.m - 4, q.m),
                                     rng.choice(q.m, 24, replace=False)]))
    want = oracle.fp8_gemm_nt(q.a[rows], W.mn_major(q.sfa[:, rows].T), q.b, q.sfb, q.c[rows])
    assert_parity(got[rows], want, f"{layout} prefill")


def test_host_checks_of_the_layouts():
    p = W.stored_layout(W.make_dense(200, 256, 256, seed=94), "tn")
    d = sentinel_like((200, 256))
    with pytest.raises(dg.DGError) as e:
        dg.fp8_gemm_tn(dev(p.a), dev(p.sfa), dev(p.b), dev(p.sfb), d)
    assert e.value.code == -2                                     # m % 16 with A stored [K, M]
    q = W.stored_layout(W.make_dense(200, 256, 256, seed=94), "nn")
    assert_parity(run("nn", q), ref("nn", q), "nn m=200")          # fine with A stored [M, K]


def test_graph_captured_before_the_workspace_grows_still_replays():
    # a graph records the workspace's address; a later, larger call replaces the workspace
    # with a bigger one, and the old graph must still find its buffer
    small = W.stored_layout(W.make_dense(128, 256, 256, seed=96, with_c=True), "tn")
    a, sfa, b, sfb, c = (dev(x) for x in (small.a, small.sfa, small.b, small.sfb, small.c))
    d = sentinel_like((small.m, small.n))
    dg.fp8_gemm_tn(a, sfa, b, sfb, d, c)
    torch.cuda.synchronize()
    eager = bits(d)
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g):
            dg.fp8_gemm_tn(a, sfa, b, sfb, d, c)
    torch.cuda.current_stream().wait_stream(side)
    # 8192 x 2048 bytes of A and of B to transpose (33.6 MB): more than any earlier call in
    # the suite needs (at most 23 MB, in 32 MB units), so the workspace is replaced
    big = W.stored_layout(W.make_dense(8192, 8192, 2048, seed=97), "tn")
    db = sentinel_like((big.m, big.n))
    dg.fp8_gemm_tn(dev(big.a), dev(big.sfa), dev(big.b), dev(big.sfb), db)
    torch.cuda.synchronize()
    d.view(torch.int16).fill_(W.BF16_SENTINEL)
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    assert np.array_equal(bits(d), eager)
    assert_parity(eager, ref("tn", small), "tn graph before growth")
