"""The XCD-aware tile mapping (``dg_tiles.h``, used by the GEMM kernels) checked on the host:
every tile id is assigned to exactly one workgroup, for persistent grids (fewer workgroups
than tiles), one workgroup per tile (up to 75008 tiles, where 32-bit products of the tile
count and the grid would wrap), and with straddle-serving workgroups ahead of the tiles; with
one workgroup per tile, the inverse (``xcd_tile_owner``, which the contiguous tail uses
to find the tiles of the workgroups dispatched last) names the workgroup of every tile.
CPU only: the header is plain C++ and is compiled here with g++."""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "moe_grouped_gemm_fp8_amd", "csrc")
SRC = os.path.join(ROOT, "tests", "native", "tile_cover.cpp")


@pytest.fixture(scope="module")
def tile_cover(tmp_path_factory):
    exe = str(tmp_path_factory.mktemp("tiles") / "tile_cover")
    subprocess.run(["g++", "-O2", "-std=c++17", "-Wall", "-Werror", "-I", CSRC, SRC, "-o", exe],
                   check=True)
    return exe


def _run(exe, cases):
    args = [str(v) for case in cases for v in case]
    out = subprocess.run([exe, *args], capture_output=True, text=True)
    assert out.returncode == 0, out.stdout + out.stderr
    assert out.stdout.count("ok ") == len(cases)


@pytest.mark.parametrize("lead", [0, 8, 24])
def test_one_workgroup_per_tile(tile_cover, lead):
    # G == total: 46341 is the first count whose total * G passes 2^31, 65536 the first whose
    # product passes 2^32, 75008 the 256x224 tile count of a 65536 x 65536 output
    _run(tile_cover, [(g, g, lead) for g in list(range(1, 41)) + [2080, 3640, 46341, 65536, 75008]])


@pytest.mark.parametrize("lead", [0, 16])
def test_persistent_workgroups(tile_cover, lead):
    cases = [(t, g, lead) for g in range(1, 10) for t in (g, g + 1, 1000, 46341, 65536, 75008)]
    cases += [(t, g, lead) for g in (255, 256, 46341, 65536)
              for t in (g, g + 7, 3 * g + 5, 1 << 21)]
    _run(tile_cover, cases)


@pytest.mark.parametrize("lead", [0, 8])
def test_more_workgroups_than_tiles(tile_cover, lead):
    # a persistent grid sized for more tiles than a launch finds (the contiguous tail
    # sizes its grid for the most tiles it may get): the spare workgroups get no tile
    _run(tile_cover, [(t, g, lead) for g in (2, 8, 9, 256, 1000) for t in (1, 3, g - 1, g // 2 + 1)
                      if 0 < t < g])


def test_tail_rule(tile_cover):
    # the contiguous forms leave the busy workgroups of a last partial wave to 128-row tiles
    # when they fill between an eighth and a quarter of the CUs; worked cases and the rule's
    # properties over every CU count to 320 (the kernel and the host both use tail_count)
    out = subprocess.run([tile_cover, "tail"], capture_output=True, text=True)
    assert out.returncode == 0 and "ok tail" in out.stdout, out.stdout + out.stderr
