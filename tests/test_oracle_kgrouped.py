"""Pins for the oracle's K-grouped TN form (MoE weight gradient): exact rational arithmetic
on tiny problems (decoded by torch's float8_e4m3fn, a library routine), the special case that
reduces to the NT oracle bit for bit, closed forms (one-hot operands, empty groups), the
generator's layout, and planted faults that the FP32-output tolerance must reject.  CPU only."""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tolerance import tol_violations


def _decode(bits):
    t = torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint8)).view(torch.float8_e4m3fn)
    return t.to(torch.float64).numpy()


def _fraction_k_grouped(a, sfa, b, sfb, ks, c):
    da, db = _decode(a), _decode(b)
    m, n = a.shape[1], b.shape[1]
    out = np.empty((len(ks), m, n), dtype=object)
    k0 = 0
    for g, kg in enumerate(ks):
        for i in range(m):
            for j in range(n):
                tot = Fraction(0)
                for kb in range(k0 // 128, (k0 + kg) // 128):
                    blk = sum(Fraction(float(da[t, i])) * Fraction(float(db[t, j]))
                              for t in range(kb * 128, (kb + 1) * 128))
                    tot += Fraction(float(sfa[kb, i])) * Fraction(float(sfb[kb, j])) * blk
                if c is not None:
                    tot += Fraction(float(c[g, i, j]))
                out[g, i, j] = tot
        k0 += kg
    return out


@pytest.mark.parametrize("seed", [0, 1])
def test_matches_rational_brute_force(seed):
    p = W.make_k_grouped(3, 300, 4, 3, seed=seed, counts=[130, 0, 170],
                         with_c=True, stress=True)
    d = oracle.k_grouped_tn(p.a, p.sfa, p.b, p.sfb, p.ks, p.c)
    exact = _fraction_k_grouped(p.a, p.sfa, p.b, p.sfb, [int(x) for x in p.ks], p.c)
    for idx in np.ndindex(d.shape):
        e = exact[idx]
        assert abs(Fraction(float(d[idx])) - e) <= abs(e) * Fraction(1, 10 ** 14) + Fraction(1, 10 ** 300), idx


def test_reduces_to_the_nt_oracle_when_b_scales_are_blockwise():
    # with sfb constant over each 128-column block, group g is the NT GEMM of its K run with
    # A and B transposed to K-major rows; both oracles then do the same float64 operations
    p = W.make_k_grouped(2, 500, 96, 256, seed=3, counts=[300, 200], with_c=True)
    kb_total = p.k_total // 128
    blk = np.random.default_rng(9).uniform(0.01, 2.0, size=(2, kb_total)).astype(np.float32)
    sfb_tn = np.repeat(blk.T, 128, axis=1)[:, :256].copy()      # [K_total/128, N]
    d = oracle.k_grouped_tn(p.a, p.sfa, p.b, sfb_tn, p.ks, p.c)
    k0 = 0
    for g, kg in enumerate(p.ks):
        kbs = slice(k0 // 128, (k0 + kg) // 128)
        a_nt = p.a[k0:k0 + kg].T.copy()                            # [M, K_g]
        b_nt = p.b[k0:k0 + kg].T.copy()                            # [N, K_g]
        sfa_nt = p.sfa[kbs].copy()                                 # [K_g/128, M] MN-major
        sfb_nt = blk[:, kbs].copy()                                # [N/128, K_g/128]
        ref = oracle.fp8_gemm_nt(a_nt, sfa_nt, b_nt, sfb_nt, p.c[g])
        assert np.array_equal(d[g], ref), g
        k0 += kg


def test_empty_groups_give_c_or_zero():
    p = W.make_k_grouped(4, 256, 32, 48, seed=4, counts=[0, 256, 0, 0], with_c=True)
    d = oracle.k_grouped_tn(p.a, p.sfa, p.b, p.sfb, p.ks, p.c)
    for g in (0, 2, 3):
        assert np.array_equal(d[g], p.c[g].astype(np.float64))
    d0 = oracle.k_grouped_tn(p.a, p.sfa, p.b, p.sfb, p.ks)
    for g in (0, 2, 3):
        assert not d0[g].any()


def test_one_hot_operands():
    # a single nonzero A[k0, m0]: row m0 of its group is sfa * sfb * dec(a) * dec(B[k0, :]),
    # every other row (and every other group) is zero
    ks = np.array([128, 256], dtype=np.int32)
    a = np.zeros((384, 16), np.uint8)
    b = np.random.default_rng(5).integers(0, 0x7E, size=(384, 32)).astype(np.uint8)
    k0, m0 = 200, 7
    a[k0, m0] = 0x44                                               # 2^(8-7) * (1 + 4/8) = 3
    sfa = np.full((3, 16), 0.5, np.float32)
    sfb = np.random.default_rng(6).uniform(0.1, 1, size=(3, 32)).astype(np.float32)
    d = oracle.k_grouped_tn(a, sfa, b, sfb, ks)
    want = np.zeros((2, 16, 32))
    want[1, m0] = 0.5 * sfb[k0 // 128].astype(np.float64) * 3.0 * _decode(b[k0])
    assert np.array_equal(d, want)


def test_generator_layout():
    p = W.make_k_grouped(3, 400, 64, 32, seed=7, counts=[100, 0, 300])
    assert list(p.ks) == [128, 0, 384] and p.k_total == 512
    assert p.a.shape == (512, 64) and p.b.shape == (512, 32)
    assert p.sfa.shape == (4, 64) and p.sfb.shape == (4, 32)
    # padding tokens are zero and every block's largest code reaches the cast's maximum
    assert not p.a[100:128].any() and not p.b[100:128].any() and not p.a[128 + 300:].any()
    dec = np.abs(_decode(p.a).reshape(4, 128, 64)).max(axis=1)
    assert np.all(dec == 448.0)


def test_planted_faults_fail_the_tolerance():
    p = W.make_k_grouped(3, 700, 64, 64, seed=8, counts=[300, 150, 250], with_c=True,
                         stress=True)
    ref = oracle.k_grouped_tn(p.a, p.sfa, p.b, p.sfb, p.ks, p.c)
    faults = {
        "sfb_kb_plus_1": dict(sfb=np.roll(p.sfb, -1, axis=0)),
        "sfa_kb_minus_1": dict(sfa=np.roll(p.sfa, 1, axis=0)),
        "sfa_sfb_swapped": dict(sfa=p.sfb, sfb=p.sfa),
        "boundary_moved": dict(ks=p.ks + np.array([128, -128, 0], np.int32)),
        "operands_swapped": dict(a=p.b, b=p.a),
    }
    for name, kw in faults.items():
        args = dict(a=p.a, sfa=p.sfa, b=p.b, sfb=p.sfb, ks=p.ks, c=p.c)
        args.update(kw)
        bad = oracle.k_grouped_tn(**args)
        assert tol_violations(bad.astype(np.float32), ref).any(), name
    q = W.make_k_grouped(2, 300, 32, 32, seed=9, counts=[140, 160], with_c=True, c_std=30.0)
    refc = oracle.k_grouped_tn(q.a, q.sfa, q.b, q.sfb, q.ks, q.c)
    bad = oracle.k_grouped_tn(q.a, q.sfa, q.b, q.sfb, q.ks)
    assert tol_violations(bad.astype(np.float32), refc).any(), "c_dropped"


def test_tolerance_accepts_fp32_rounding_of_the_exact_result():
    p = W.make_k_grouped(3, 700, 64, 64, seed=10, counts=[300, 150, 250], with_c=True)
    ref = oracle.k_grouped_tn(p.a, p.sfa, p.b, p.sfb, p.ks, p.c)
    assert not tol_violations(ref.astype(np.float32), ref).any()


def test_rejects_bad_group_extents():
    p = W.make_k_grouped(2, 256, 16, 16, seed=11, counts=[128, 128])
    for ks in ([100, 156], [-128, 384], [256, 128]):
        with pytest.raises(ValueError):
            oracle.k_grouped_tn(p.a, p.sfa, p.b, p.sfb, np.array(ks))
