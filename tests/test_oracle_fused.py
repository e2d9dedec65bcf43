"""Pins for the oracle's fused reading of the first MoE GEMM with the activation step behind it
(SwiGLU of the unrounded contiguous GEMM result, then the 1x128 FP8 cast): a closed-form case
built from one-hot A rows, agreement with the already pinned activation step whenever the GEMM
result is exactly a bf16 value, the gate/up order, and untouched padding rows.  CPU only."""
import math

import numpy as np

import oracle
import workloads as W

ONE = 0x38      # e4m3 1.0


def _contiguous(a, b, sfb, m_indices):
    m = a.shape[0]
    sfa = W.mn_major(np.ones((m, a.shape[1] // 128), np.float32))
    return oracle.m_grouped_contiguous_swiglu(a, sfa, b, sfb, m_indices)


def test_closed_form_one_hot_rows():
    # row r (group 0) is one-hot at K index r, so D1[r, n] = sfb * dec(B[0, n, r]).  The gate
    # rows hold 3 (0x44) under block scale 1 and the up rows 2 (0x40) under block scale 0.5, so
    # gate = 3 and up = 1 give h = 3 / (1 + e^-3), except at column 7 of row 0, whose up row
    # holds 4 (0x48) there: up = 2 and h doubles.  A segment's scale is its largest h over 448.
    i, k = 128, 128
    a = np.zeros((2, k), np.uint8)
    a[0, 0] = ONE
    a[1, 1] = ONE
    b = np.zeros((1, 2 * i, k), np.uint8)
    b[0, :i, :2] = 0x44                         # gate rows: 3
    b[0, i:, :2] = 0x40                         # up rows: 2
    b[0, i + 7, 0] = 0x48                       # up row 7 at K index 0: 4
    sfb = np.array([[[1.0], [0.5]]], np.float32)  # gate block 1, up block 0.5
    d1, h, sf, q = _contiguous(a, b, sfb, np.array([0, 0], np.int32))
    base = 3.0 / (1.0 + math.exp(-3.0))        # gate 3, up 2 * 0.5 = 1
    assert np.all(d1[:, :i] == 3.0)
    assert d1[0, i + 7] == 2.0 and np.all(np.delete(d1[0, i:], 7) == 1.0)
    assert abs(h[0, 7] - 2 * base) <= 1e-15 * base and abs(h[1, 7] - base) <= 1e-15 * base
    tab = oracle.e4m3_table()
    top = tab[0x7E]
    assert abs(sf[0, 0] * top / (2 * base) - 1) <= 2.0 ** -52
    assert abs(sf[0, 1] * top / base - 1) <= 2.0 ** -52
    # row 0: the doubled column maps to 448, the rest to 224; row 1: all 448
    assert tab[q[0, 7]] == 448.0 and np.all(tab[np.delete(q[0], 7)] == 224.0)
    assert np.all(tab[q[1]] == 448.0)


def test_gate_and_up_halves_are_not_interchangeable():
    # swapping the halves of B swaps gate and up; silu(g) * u != silu(u) * g here
    rng = np.random.default_rng(3)
    a = rng.integers(0, 0x50, size=(128, 256)).astype(np.uint8)
    b = rng.integers(0, 0x50, size=(1, 256, 256)).astype(np.uint8)
    sfb = np.full((1, 2, 2), 2.0 ** -6, np.float32)
    idx = np.zeros(128, np.int32)
    _, h, _, q = _contiguous(a, b, sfb, idx)
    _, h2, _, q2 = _contiguous(a, np.concatenate([b[:, 128:], b[:, :128]], axis=1), sfb, idx)
    assert not np.allclose(h, h2) and (q != q2).any()


def test_equals_the_activation_step_on_bf16_exact_results():
    # unit scales and small integer codes (0, +-1, +-2 as e4m3) give integer GEMM results of
    # magnitude below 256, which bf16 holds exactly: the fused reading then equals the pinned
    # activation step applied to the bf16 of the GEMM result, code for code and scale for scale
    rng = np.random.default_rng(4)
    vals = np.array([0x00, 0x38, 0xB8, 0x40, 0xC0], np.uint8)     # 0, 1, -1, 2, -2
    a = vals[rng.integers(0, 5, size=(256, 128))]
    b = vals[rng.integers(0, 5, size=(2, 512, 128))]
    sfb = np.ones((2, 4, 1), np.float32)
    idx = np.repeat(np.array([0, 1], np.int32), 128)
    d1, h, sf, q = _contiguous(a, b, sfb, idx)
    assert np.all(np.abs(d1) < 256) and np.all(d1 == np.round(d1))
    h_ref, sf_ref, q_ref = oracle.swiglu_quant(W.f32_to_bf16_bits(d1.astype(np.float32)))
    assert np.array_equal(h, h_ref) and np.array_equal(sf, sf_ref) and np.array_equal(q, q_ref)


def test_padding_rows_are_not_computed():
    p = W.make_contiguous(3, 300, 256, 256, seed=5, counts=[100, 0, 200], pad_nan=True)
    d1, h, sf, q = oracle.m_grouped_contiguous_swiglu(p.a, p.sfa, p.b, p.sfb, p.m_indices)
    pad = p.m_indices < 0
    assert np.isnan(d1[pad]).all() and np.isnan(h[pad]).all()
    assert not q[pad].any() and not sf[:, :p.m_total][:, pad].any()
    assert not np.isnan(h[~pad]).any() and (sf[:, :p.m_total][:, ~pad] > 0).all()


def _rule_inputs(p):
    from tolerance import gemm_error_bound
    d1, h, sf, q = oracle.m_grouped_contiguous_swiglu(p.a, p.sfa, p.b, p.sfb, p.m_indices)
    rows = np.nonzero(p.m_indices >= 0)[0]
    tab = oracle.e4m3_table()
    err = gemm_error_bound(p.a[rows], p.sfa[:, rows].T, p.b, p.sfb, p.m_indices[rows], tab)
    return rows, d1[rows], err, h[rows], sf[:, rows].T, q[rows], tab


def test_fused_rule_accepts_the_oracle_and_rejects_planted_faults():
    from tolerance import fused_cast_violations
    p = W.make_contiguous(3, 400, 512, 384, seed=6, counts=[150, 0, 250], stress=True)
    rows, d1, err, h, s, q, tab = _rule_inputs(p)
    bad_s, bad_q, amb = fused_cast_violations(q, s, d1, err, h, s, tab, oracle.e4m3_nearest)
    assert not bad_s.any() and not bad_q.any()
    # the worst-case FP32 bound leaves codes of small |y| (where e4m3 steps are finer than it)
    # undecided; most codes are still decided exactly (under a third without stress inputs,
    # about half with these stress scales)
    assert amb < 0.6 * q.size
    # the rule is not vacuous: a scale off by 2^-10, codes of the neighbouring row, codes one
    # step off and the gate/up halves swapped all fail it
    faults = {
        "scale": (q, s * (1 + 2.0 ** -10)),
        "row_shift": (np.roll(q, 1, axis=0), s),
        "codes_one_step_up": (np.where((q & 0x7F) < 0x7E, q + 1, q - 1).astype(np.uint8), s),
    }
    for name, (qq, ss) in faults.items():
        bs, bq, _ = fused_cast_violations(qq, ss, d1, err, h, s, tab, oracle.e4m3_nearest)
        assert bs.any() or bq.any(), name
    sw = np.concatenate([p.b[:, 256:], p.b[:, :256]], axis=1)
    _, h2, sf2, q2 = oracle.m_grouped_contiguous_swiglu(p.a, p.sfa, sw, p.sfb, p.m_indices)
    bs, bq, _ = fused_cast_violations(q2[rows], sf2[:, rows].T, d1, err, h, s, tab,
                                      oracle.e4m3_nearest)
    assert bs.any() or bq.any(), "gate_up_swapped"


def test_gemm_error_bound_covers_fp32_accumulation():
    # the bound holds for an FP32 evaluation of the GEMM in the kernel's order (block sums
    # accumulated one product at a time in FP32, promoted with an FP32 scale product)
    from tolerance import gemm_error_bound
    p = W.make_contiguous(2, 256, 256, 512, seed=7, counts=[128, 128])
    tab = oracle.e4m3_table()
    rows = np.arange(256)
    d1 = oracle.m_grouped_contiguous(p.a, p.sfa, p.b, p.sfb, p.m_indices)
    err = gemm_error_bound(p.a, p.sfa[:, :256].T, p.b, p.sfb, p.m_indices, tab)
    f32 = np.float32
    got = np.zeros((256, 256), np.float32)
    for r in rows[::17]:
        g = p.m_indices[r]
        a = tab[p.a[r]].astype(f32)
        for n in range(0, 256, 13):
            bvec = tab[p.b[g, n]].astype(f32)
            acc = f32(0)
            for kb in range(4):
                part = f32(0)
                for t in range(kb * 128, kb * 128 + 128):
                    part = f32(part + f32(a[t] * bvec[t]))
                sc = f32(f32(p.sfa[kb, r]) * f32(p.sfb[g, n // 128, kb]))
                acc = f32(acc + f32(part * sc))
            assert abs(float(acc) - d1[r, n]) <= err[r, n], (r, n)
