"""Pins for the CPU oracle: each check ties it to something other than itself — the format's
closed-form values, a library decode, exact integer and rational arithmetic, closed forms,
and a library matmul in the special case with unit scales.  CPU only."""
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tolerance import within_tol, tol_violations, bf16_bits_to_f64

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_rows(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line.split())
    return rows


def torch_decode(bits: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint8)).view(torch.float8_e4m3fn)
    return t.to(torch.float64).numpy()


# ---------------------------------------------------------------- decode table

def test_decode_spot_values_from_format_definition():
    tab = oracle.e4m3_table()
    for hx, val in _read_rows("e4m3_spot_values.txt"):
        got = tab[int(hx, 16)]
        if val == "nan":
            assert np.isnan(got), hx
        else:
            assert got == float(val) and np.signbit(got) == val.startswith("-"), hx


def test_decode_table_equals_torch_float8_e4m3fn():
    tab = oracle.e4m3_table()
    ref = torch_decode(np.arange(256, dtype=np.uint8))
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(tab), nan)
    assert np.array_equal(tab[~nan], ref[~nan])
    assert np.array_equal(np.signbit(tab[~nan]), np.signbit(ref[~nan]))


# ---------------------------------------------------------------- block partials are exact

def _int_codes(bits):
    v = torch_decode(bits) * 512.0            # every finite e4m3 value is an integer times 2^-9
    assert np.all(v == np.round(v))
    return v.astype(np.int64)


def test_block_partials_equal_exact_integer_sums_dense_small():
    p = W.make_config("dense_small", seed=0)
    part = oracle.block_partials(p.a, p.b)
    ia, ib = _int_codes(p.a), _int_codes(p.b)
    kb = p.k // 128
    for j in range(kb):
        exact = ia[:, j * 128:(j + 1) * 128] @ ib[:, j * 128:(j + 1) * 128].T   # int64, exact
        assert np.abs(exact).max() < 2 ** 43
        assert np.array_equal(part[:, :, j], exact.astype(np.float64) * 2.0 ** -18)


@pytest.mark.parametrize("seed", [1, 2])
def test_block_partials_exact_on_extreme_codes(seed):
    # values at the format's extremes (max normal, subnormals, signed zeros) stress the exactness
    rng = np.random.default_rng(seed)
    pool = np.array([0x7E, 0xFE, 0x01, 0x81, 0x00, 0x80, 0x77, 0x08], dtype=np.uint8)
    a = rng.choice(pool, size=(5, 256)).astype(np.uint8)
    b = rng.choice(pool, size=(7, 256)).astype(np.uint8)
    part = oracle.block_partials(a, b)
    ia, ib = _int_codes(a), _int_codes(b)
    for j in range(2):
        exact = ia[:, j * 128:(j + 1) * 128] @ ib[:, j * 128:(j + 1) * 128].T
        assert np.array_equal(part[:, :, j], exact.astype(np.float64) * 2.0 ** -18)


# ---------------------------------------------------------------- whole result, exact arithmetic

def _fraction_gemm(a, sfa, b, sfb, c):
    """Exact D in rational arithmetic (inputs are dyadic rationals: e4m3, FP32 scales, FP32 C)."""
    da, db = torch_decode(a), torch_decode(b)
    m, k = a.shape
    n = b.shape[0]
    out = np.empty((m, n), dtype=object)
    for i in range(m):
        for j in range(n):
            tot = Fraction(0)
            for kb in range(k // 128):
                blk = sum(Fraction(float(da[i, t])) * Fraction(float(db[j, t]))
                          for t in range(kb * 128, (kb + 1) * 128))
                tot += Fraction(float(sfa[kb, i])) * Fraction(float(sfb[j // 128, kb])) * blk
            if c is not None:
                tot += Fraction(float(c[i, j]))
            out[i, j] = tot
    return out


def test_worked_example_by_hand():
    a = np.zeros((2, 256), np.uint8)
    a[0, :128], a[0, 128:] = 0x38, 0x40
    a[1, 0], a[1, 128:] = 0x7E, 0x30
    b = np.zeros((2, 256), np.uint8)
    b[0, :] = 0x38
    b[1, :128] = np.tile(np.array([0x38, 0xB8], np.uint8), 64)
    b[1, 128:] = 0x01
    sfa = W.mn_major(np.array([[0.5, 0.25], [2.0, 1.0]], np.float32))
    sfb = np.array([[4.0, 8.0]], np.float32)
    c = np.array([[1.0, -1.0], [0.5, 0.25]], np.float32)
    d = oracle.fp8_gemm_nt(a, sfa, b, sfb, c)
    for r, col, val in _read_rows("worked_example.txt"):
        assert d[int(r), int(col)] == float(val)


@pytest.mark.parametrize("seed", [3, 4])
def test_oracle_matches_rational_brute_force(seed):
    p = W.make_dense(3, 130, 256, seed=seed, with_c=True, stress=True)   # 2 B block rows, ragged
    d = oracle.fp8_gemm_nt(p.a, p.sfa, p.b, p.sfb, p.c)
    exact = _fraction_gemm(p.a, p.sfa, p.b, p.sfb, p.c)
    for i in range(p.m):
        for j in range(p.n):
            e = exact[i, j]
            err = abs(Fraction(float(d[i, j])) - e)
            assert err <= abs(e) * Fraction(1, 10 ** 14) + Fraction(1, 10 ** 300), (i, j)


# ---------------------------------------------------------------- library routine special case

def test_unit_scales_no_c_equals_numpy_matmul():
    p = W.make_dense(64, 192, 512, seed=5)
    sfa = np.ones_like(p.sfa)
    sfb = np.ones_like(p.sfb)
    d = oracle.fp8_gemm_nt(p.a, sfa, p.b, sfb, None)
    ref = torch_decode(p.a) @ torch_decode(p.b).T          # every partial sum is exact here
    assert np.array_equal(d, ref)


# ---------------------------------------------------------------- closed forms

def test_identity_a():
    rng = np.random.default_rng(6)
    a = np.zeros((128, 128), np.uint8)
    a[np.arange(128), np.arange(128)] = 0x38
    sfa = W.mn_major(np.ones((128, 1), np.float32))
    b = rng.integers(0, 256, size=(256, 128)).astype(np.uint8)
    b[(b & 0x7F) == 0x7F] = 0x00                             # no NaN codes
    sfb = rng.uniform(0.1, 4.0, size=(2, 1)).astype(np.float32)
    d = oracle.fp8_gemm_nt(a, sfa, b, sfb, None)
    ref = (torch_decode(b) * sfb.astype(np.float64)[np.arange(256) // 128]).T
    assert np.array_equal(d, ref)


def test_one_hot_a_and_zero_a():
    p = W.make_dense(16, 256, 384, seed=7, with_c=True)
    a = np.zeros_like(p.a)
    d0 = oracle.fp8_gemm_nt(a, p.sfa, p.b, p.sfb, p.c)
    assert np.array_equal(d0, p.c.astype(np.float64))       # A = 0  =>  D = C
    m0, k0 = 5, 200
    a[m0, k0] = 0xC4                                        # -3.0
    d1 = oracle.fp8_gemm_nt(a, p.sfa, p.b, p.sfb, p.c)
    kb = k0 // 128
    col = (np.float64(p.sfa[kb, m0]) * p.sfb[np.arange(256) // 128, kb].astype(np.float64)
           * -3.0 * torch_decode(p.b[:, k0]))
    assert np.array_equal(d1[m0], col + p.c[m0].astype(np.float64))
    others = np.arange(16) != m0
    assert np.array_equal(d1[others], p.c[others].astype(np.float64))


# ---------------------------------------------------------------- linearity in each scale factor

def test_power_of_two_row_and_block_scaling_is_exact():
    p = W.make_dense(32, 256, 384, seed=8, stress=True)
    d = oracle.fp8_gemm_nt(p.a, p.sfa, p.b, p.sfb, None)
    sfa = p.sfa.copy()
    sfa[:, 9] *= 8.0
    d2 = oracle.fp8_gemm_nt(p.a, sfa, p.b, p.sfb, None)
    assert np.array_equal(d2[9], 8.0 * d[9])
    rest = np.arange(32) != 9
    assert np.array_equal(d2[rest], d[rest])
    sfb = p.sfb.copy()
    sfb[1, :] *= 0.25
    d3 = oracle.fp8_gemm_nt(p.a, p.sfa, p.b, sfb, None)
    assert np.array_equal(d3[:, 128:], 0.25 * d[:, 128:])
    assert np.array_equal(d3[:, :128], d[:, :128])


def test_single_scale_perturbation_is_linear():
    p = W.make_dense(8, 256, 384, seed=9, with_c=True)
    part = oracle.block_partials(p.a, p.b)
    d = oracle.fp8_gemm_nt(p.a, p.sfa, p.b, p.sfb, p.c)
    t = 1.7
    m0, kb0 = 3, 1
    sfa = p.sfa.copy()
    sfa[kb0, m0] = np.float32(sfa[kb0, m0] * t)
    d2 = oracle.fp8_gemm_nt(p.a, sfa, p.b, p.sfb, p.c)
    delta = (np.float64(sfa[kb0, m0]) - np.float64(p.sfa[kb0, m0])) * \
        p.sfb[np.arange(256) // 128, kb0].astype(np.float64) * part[m0, :, kb0]
    assert np.allclose(d2[m0] - d[m0], delta, rtol=0, atol=1e-12 * np.abs(d).max())
    nb0 = 1
    sfb = p.sfb.copy()
    sfb[nb0, kb0] = np.float32(sfb[nb0, kb0] * t)
    d3 = oracle.fp8_gemm_nt(p.a, p.sfa, p.b, sfb, p.c)
    cols = slice(128, 256)
    delta = p.sfa[kb0, :8].astype(np.float64)[:, None] * \
        (np.float64(sfb[nb0, kb0]) - np.float64(p.sfb[nb0, kb0])) * part[:, cols, kb0]
    assert np.allclose(d3[:, cols] - d[:, cols], delta, rtol=0, atol=1e-12 * np.abs(d).max())
    assert np.array_equal(d3[:, :128], d[:, :128])


# ---------------------------------------------------------------- grouped forms

def test_contiguous_equals_per_group_dense_and_skips_padding():
    p = W.make_contiguous(4, 300, 256, 256, seed=10, counts=[0, 130, 41, 129], pad_nan=True)
    d = oracle.m_grouped_contiguous(p.a, p.sfa, p.b, p.sfb, p.m_indices)
    for g in range(p.num_groups):
        rows = np.nonzero(p.m_indices == g)[0]
        assert rows.size == p.counts[g]
        if rows.size == 0:
            continue
        sub = W.mn_major(p.sfa[:, rows].T)
        ref = oracle.fp8_gemm_nt(p.a[rows], sub, p.b[g], p.sfb[g], None)
        assert np.array_equal(d[rows], ref)
    pad = p.m_indices < 0
    assert pad.sum() == p.m_total - 300
    assert np.isnan(d[pad]).all()                  # untouched
    assert np.isfinite(d[~pad]).all()              # NaN padding leaks nowhere


def test_masked_equals_per_group_dense_and_leaves_tail_untouched():
    mm = [0, 1, 255, 256, 130, 999, -3]            # includes the clamp cases
    p = W.make_masked(7, 256, 256, 256, seed=11, masked_m=mm, tail_nan=True)
    d = oracle.m_grouped_masked(p.a, p.sfa, p.b, p.sfb, p.masked_m)
    for g in range(7):
        valid = min(max(mm[g], 0), 256)
        if valid:
            ref = oracle.fp8_gemm_nt(p.a[g, :valid], W.mn_major(p.sfa[g, :, :valid].T),
                                     p.b[g], p.sfb[g], None)
            assert np.array_equal(d[g, :valid], ref)
            assert np.isfinite(d[g, :valid]).all()
        assert np.isnan(d[g, valid:]).all()


# ---------------------------------------------------------------- the tolerance is not vacuous

def _bf16_round(x):
    t = torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16)
    return bf16_bits_to_f64(t.view(torch.int16).numpy().view(np.uint16))


def test_tolerance_accepts_bf16_rounding_of_the_exact_result():
    p = W.make_dense(64, 256, 512, seed=12, with_c=True)
    d = oracle.fp8_gemm_nt(p.a, p.sfa, p.b, p.sfb, p.c)
    assert within_tol(_bf16_round(d), d)


def test_planted_faults_fail_the_tolerance_dense():
    p = W.make_dense(64, 384, 512, seed=13, with_c=True, stress=True)
    ref = oracle.fp8_gemm_nt(p.a, p.sfa, p.b, p.sfb, p.c)
    kb, ld = p.sfa.shape
    faults = {
        # A scales read as if stored [M, K/128] instead of MN-major
        "sfa_transposed": p.sfa.reshape(-1)[:kb * ld].reshape(ld, kb)[:, :].T.copy(),
        "sfa_kb_plus_1": np.roll(p.sfa, -1, axis=0),
        "sfa_kb_minus_1": np.roll(p.sfa, 1, axis=0),
    }
    for name, sfa in faults.items():
        bad = oracle.fp8_gemm_nt(p.a, sfa, p.b, p.sfb, p.c)
        assert not within_tol(_bf16_round(bad), ref), name
    for name, sfb in {"sfb_nb_plus_1": np.roll(p.sfb, -1, axis=0),
                      "sfb_kb_plus_1": np.roll(p.sfb, -1, axis=1)}.items():
        bad = oracle.fp8_gemm_nt(p.a, p.sfa, p.b, sfb, p.c)
        assert not within_tol(_bf16_round(bad), ref), name
    # with C ~ N(0, 0.1) next to |A @ B.T| ~ sqrt(K) a dropped C hides inside the tolerance,
    # so the C fault is planted on an input whose C is as large as the product
    q = W.make_dense(64, 384, 512, seed=13, with_c=True, c_std=30.0)
    refc = oracle.fp8_gemm_nt(q.a, q.sfa, q.b, q.sfb, q.c)
    bad = oracle.fp8_gemm_nt(q.a, q.sfa, q.b, q.sfb, None)
    assert not within_tol(_bf16_round(bad), refc), "c_dropped"


def test_planted_faults_fail_grouped():
    p = W.make_contiguous(4, 512, 256, 256, seed=14, stress=True)
    ref = oracle.m_grouped_contiguous(p.a, p.sfa, p.b, p.sfb, p.m_indices)
    valid = p.m_indices >= 0
    wrong = np.where(valid, (p.m_indices + 1) % 4, -1).astype(np.int32)
    bad = oracle.m_grouped_contiguous(p.a, p.sfa, p.b, p.sfb, wrong)
    assert not within_tol(_bf16_round(bad[valid]), ref[valid]), "wrong expert"
    q = W.make_masked(4, 64, 256, 256, seed=15, masked_m=[10, 0, 64, 33])
    refm = oracle.m_grouped_masked(q.a, q.sfa, q.b, q.sfb, q.masked_m)
    for delta in (+1, -1):
        mm = np.clip(q.masked_m + delta, 0, 64).astype(np.int32)
        badm = oracle.m_grouped_masked(q.a, q.sfa, q.b, q.sfb, mm)
        # an off-by-one valid-row count shows up as a row whose written/untouched state differs
        assert not np.array_equal(np.isnan(badm), np.isnan(refm)), delta


def test_violation_mask_counts_nan():
    assert tol_violations(np.array([np.nan]), np.array([1.0])).all()


# ---------------------------------------------------------------- other dense layouts

@pytest.mark.parametrize("layout", ["nt", "nn", "tn", "tt"])
def test_layouts_with_unit_scales_equal_numpy_matmul(layout):
    # with unit scales and no C, D = dec(A) @ dec(B) in the layout's own storage, computed by
    # numpy's matmul on the stored arrays (their transposes taken as the layout says)
    p = W.stored_layout(W.make_dense(48, 64, 256, seed=30), layout)
    sfa = np.ones_like(p.sfa)
    sfb = np.ones_like(p.sfb)
    da, db = torch_decode(p.a), torch_decode(p.b)
    a_math = da if layout[0] == "n" else da.T          # [M, K]
    b_math = db.T if layout[1] == "t" else db          # [K, N]
    want = a_math @ b_math
    got = oracle.fp8_gemm_layout(layout, p.a, sfa, p.b, sfb)
    assert np.allclose(got, want, rtol=1e-15, atol=0)


@pytest.mark.parametrize("layout", ["nn", "tn", "tt"])
def test_layouts_match_rational_brute_force(layout):
    q = W.make_dense(3, 16, 256, seed=31, with_c=True, stress=True)
    p = W.stored_layout(q, layout)
    got = oracle.fp8_gemm_layout(layout, p.a, p.sfa, p.b, p.sfb, p.c)
    exact = _fraction_gemm(q.a, q.sfa, q.b, q.sfb, q.c)    # the NT storage of the same problem
    for i in range(got.shape[0]):
        for j in range(got.shape[1]):
            e = exact[i, j]
            assert abs(Fraction(float(got[i, j])) - e) <= abs(e) * Fraction(1, 10 ** 14) + Fraction(1, 10 ** 300)


def test_layout_storage_is_transposed_bytes():
    q = W.make_dense(32, 48, 256, seed=32)
    p = W.stored_layout(q, "tn")
    assert p.a.shape == (256, 32) and p.b.shape == (256, 48)
    assert np.array_equal(p.a, q.a.T) and np.array_equal(p.b, q.b.T)
    with pytest.raises(ValueError):
        oracle.fp8_gemm_layout("xx", q.a, q.sfa, q.b, q.sfb)
