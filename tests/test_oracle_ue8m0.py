"""Pins for the oracle's UE8M0 path (packed power-of-two scales): the format's closed form,
the byte order of the packing (a hand-worked fixture), exact rational arithmetic on tiny
problems (exponents read with plain integer operations, not the oracle's decode), and the
grouped forms against per-group dense calls.  CPU only."""
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_decode_every_exponent_matches_closed_form():
    # each byte value e in its own word position: 2^(e-127) exactly, 0xFF is NaN
    for j in range(4):
        e = np.arange(256, dtype=np.int64)
        packed = ((np.full(256, 0x7F7F7F7F, np.int64) & ~(0xFF << (8 * j))) | (e << (8 * j)))
        packed = packed.astype(np.uint32).view(np.int32).reshape(256, 1)
        got = oracle.ue8m0_decode(packed, 1, 4)
        for v in range(256):
            if v == 255:
                assert np.isnan(got[v, j])
            else:
                assert Fraction(float(got[v, j])) == Fraction(2) ** (v - 127), (j, v)
            for other in range(4):
                if other != j:
                    assert got[v, other] == 1.0


def test_byte_order_hand_worked_fixture():
    rows = []
    with open(os.path.join(GOLDEN, "ue8m0_packing.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                rows.append(line.split())
    assert len(rows) == 8
    for word, kb, byte, scale in rows:
        packed = np.array([[np.uint32(int(word, 16))]], np.uint32).view(np.int32)
        got = oracle.ue8m0_decode(packed, 1, 4)[0, int(kb)]
        if scale == "nan":
            assert np.isnan(got)
        else:
            assert Fraction(float(got)) == Fraction(2) ** int(scale.split("^")[1])


def test_decode_truncates_to_the_k_block_count_along_the_given_axis():
    packed = np.array([[0x7f80fe01, 0x00ff7e81]], np.uint32).view(np.int32)   # 8 K blocks
    got = oracle.ue8m0_decode(packed.T, 0, 6)                                 # axis 0
    assert got.shape == (6, 1)
    assert got[4, 0] == 4.0 and got[5, 0] == 0.5


def _exp(packed, q, j):
    return (int(np.uint32(packed[q])) >> (8 * j)) & 0xFF


def _fraction_gemm_ue8m0(a, sfa, b, sfb, c):
    """Exact D by rational arithmetic, scales read straight from the packed words."""
    tab = [None if np.isnan(x) else Fraction(float(x)) for x in oracle.e4m3_table()]
    m, k = a.shape
    n = b.shape[0]
    out = np.empty((m, n), dtype=object)
    for i in range(m):
        for jn in range(n):
            tot = Fraction(0)
            for kb in range(k // 128):
                blk = sum(tab[a[i, t]] * tab[b[jn, t]] for t in range(kb * 128, (kb + 1) * 128))
                ea = _exp(sfa[:, i], kb // 4, kb % 4)
                eb = _exp(sfb[jn // 128], kb // 4, kb % 4)
                tot += Fraction(2) ** (ea - 127) * Fraction(2) ** (eb - 127) * blk
            if c is not None:
                tot += Fraction(float(c[i, jn]))
            out[i, jn] = tot
    return out


@pytest.mark.parametrize("seed", [6, 7])
def test_ue8m0_gemm_matches_rational_brute_force(seed):
    # 5 K blocks: two packed words, the second partly padding; ragged N (2 B block rows)
    p = W.make_dense(3, 130, 640, seed=seed, with_c=True, stress=True, ue8m0=True)
    assert p.sfa.dtype == np.int32 and p.sfa.shape[0] == 2 and p.sfb.shape == (2, 2)
    d = oracle.fp8_gemm_nt_ue8m0(p.a, p.sfa, p.b, p.sfb, p.c)
    exact = _fraction_gemm_ue8m0(p.a, p.sfa, p.b, p.sfb, p.c)
    for i in range(p.m):
        for j in range(p.n):
            e = exact[i, j]
            err = abs(Fraction(float(d[i, j])) - e)
            assert err <= abs(e) * Fraction(1, 10 ** 14) + Fraction(1, 10 ** 300), (i, j)


def test_generator_scales_are_powers_of_two_that_do_not_saturate():
    p = W.make_dense(64, 256, 1024, seed=8, ue8m0=True)
    sa = oracle.ue8m0_decode(p.sfa, 0, 8)[:, :64]
    vals = oracle.e4m3_table()[p.a].reshape(64, 8, 128)
    assert np.all(np.abs(vals).max(axis=2) <= 448)
    m, e = np.frexp(sa.astype(np.float64))
    assert np.all(m == 0.5)


def test_grouped_ue8m0_equal_per_group_dense():
    q = W.make_contiguous(3, 300, 128, 512, seed=9, counts=[100, 0, 200], ue8m0=True)
    d = oracle.m_grouped_contiguous_ue8m0(q.a, q.sfa, q.b, q.sfb, q.m_indices)
    for g in range(3):
        rows = np.nonzero(q.m_indices == g)[0]
        if rows.size == 0:
            continue
        ref = oracle.fp8_gemm_nt_ue8m0(q.a[rows], q.sfa[:, rows], q.b[g], q.sfb[g])
        assert np.array_equal(d[rows], ref)
    assert np.all(np.isnan(d[q.m_indices < 0]))
    r = W.make_masked(3, 96, 128, 512, seed=10, masked_m=[96, 0, 37], ue8m0=True)
    d = oracle.m_grouped_masked_ue8m0(r.a, r.sfa, r.b, r.sfb, r.masked_m)
    for g in range(3):
        mm = int(r.masked_m[g])
        ref = oracle.fp8_gemm_nt_ue8m0(r.a[g, :mm], r.sfa[g][:, :mm], r.b[g], r.sfb[g])
        assert np.array_equal(d[g, :mm], ref)
        assert np.all(np.isnan(d[g, mm:]))
