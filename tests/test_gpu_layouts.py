"""Parity of the dense NN, TN and TT layouts (operands stored MN-major on one or both sides) on
the GPU with the CPU oracle, on the same seeded inputs: ragged M and N tiles, K-block counts
around the pipeline depth, extreme scales, N with a partial last B scale block, the full-size
prefill shape compared in full, and the host checks particular to the layouts."""
import sys

import numpy as np
import pytest

import moe_grouped_gemm_fp8_amd as dg
import oracle
import workloads as W
from gpu_util import assert_parity, bits, cached_ref, dev, sentinel_like
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
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn(a, sfa, b, sfb, d, c)                                     # the stream's workspace
    torch.cuda.synchronize()
    eager = bits(d)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):                           # captured on that stream
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
def test_prefill_shape_full(layout):
    q = W.make_config("dense_prefill", seed=0)                   # 4096 x 7168 x 2048 with C
    p = W.stored_layout(q, layout)
    got = run(layout, p)
    assert not np.any(got == W.BF16_SENTINEL), "some outputs were never written"
    # the three layouts store the same mathematical problem: one oracle result serves all
    want = cached_ref("dense_prefill", lambda: oracle.fp8_gemm_nt(q.a, q.sfa, q.b, q.sfb, q.c))
    assert_parity(got, want, f"{layout} prefill")


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
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        dg.fp8_gemm_tn(a, sfa, b, sfb, d, c)                         # the stream's workspace
    torch.cuda.synchronize()
    eager = bits(d)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        dg.fp8_gemm_tn(a, sfa, b, sfb, d, c)
    torch.cuda.current_stream().wait_stream(side)
    # 8192 x 2048 bytes of A and of B to transpose (33.6 MB) on the same stream: more than the
    # small call's workspace holds, so it is replaced
    big = W.stored_layout(W.make_dense(8192, 8192, 2048, seed=97), "tn")
    db = sentinel_like((big.m, big.n))
    with torch.cuda.stream(side):
        dg.fp8_gemm_tn(dev(big.a), dev(big.sfa), dev(big.b), dev(big.sfb), db)
    torch.cuda.synchronize()
    d.view(torch.int16).fill_(W.BF16_SENTINEL)
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    assert np.array_equal(bits(d), eager)
    assert_parity(eager, ref("tn", small), "tn graph before growth")


def test_two_streams_at_once_use_their_own_workspaces():
    # NN calls on two streams, launched back to back with no synchronization between them:
    # each stream's transposes go to its own workspace, so neither result is disturbed
    ps = [W.stored_layout(W.make_dense(512, 1024, 1024, seed=98 + i, with_c=True), "nn")
          for i in range(2)]
    ins = [[dev(x) for x in (p.a, p.sfa, p.b, p.sfb, p.c)] for p in ps]
    outs = [sentinel_like((512, 1024)) for _ in ps]
    streams = [torch.cuda.Stream() for _ in ps]
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())
    for _ in range(10):
        for s, (a, sfa, b, sfb, c), d in zip(streams, ins, outs):
            with torch.cuda.stream(s):
                dg.fp8_gemm_nn(a, sfa, b, sfb, d, c)
    torch.cuda.synchronize()
    for p, d in zip(ps, outs):
        assert_parity(bits(d), ref("nn", p), "nn two streams")
