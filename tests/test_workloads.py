"""The seeded input generator: determinism, layouts and the amax/448 cast (CPU only)."""
import numpy as np
import torch

import workloads as W


def _dec(bits):
    return torch.from_numpy(bits).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def test_dense_is_deterministic_and_shaped():
    p = W.make_config("dense_small", seed=0)
    q = W.make_config("dense_small", seed=0)
    assert np.array_equal(p.a, q.a) and np.array_equal(p.b, q.b)
    assert p.a.shape == (128, 512) and p.b.shape == (256, 512)
    assert p.sfa.shape == (4, 128) and p.sfb.shape == (2, 4) and p.c is None


def test_cast_uses_amax_over_448_and_reconstructs():
    p = W.make_dense(8, 200, 256, seed=1)          # ragged last B block row (72 rows)
    da, db = _dec(p.a), _dec(p.b)
    assert np.abs(da).max() <= 448 and np.abs(db).max() <= 448
    # each segment's largest element maps to +-448 exactly
    seg = np.abs(da.reshape(8, 2, 128)).max(axis=2)
    assert np.all(seg == 448.0)
    blk = [np.abs(db[i * 128:(i + 1) * 128, j * 128:(j + 1) * 128]).max()
           for i in range(2) for j in range(2)]
    assert np.all(np.array(blk) == 448.0)
    assert p.sfb.shape == (2, 2)


def test_contiguous_layout():
    p = W.make_contiguous(5, 1000, 128, 256, seed=2)
    assert p.m_total % 128 == 0 and p.counts.sum() == 1000
    assert p.sfa.shape[1] >= p.m_total
    # groups appear in order, each padded to 128 with -1
    start = 0
    for g in range(5):
        cnt = int(p.counts[g])
        pad = (cnt + 127) // 128 * 128
        assert np.all(p.m_indices[start:start + cnt] == g)
        assert np.all(p.m_indices[start + cnt:start + pad] == -1)
        start += pad
    assert start == p.m_total


def test_masked_counts_inclusive_range_and_replays():
    mm = W.masked_counts(16, 256, seed=0)
    assert mm.dtype == np.int32 and mm.min() >= 0 and mm.max() <= 256
    r1 = W.masked_counts(16, 256, seed=0, replay=1)
    r2 = W.masked_counts(16, 256, seed=0, replay=2)
    assert not np.array_equal(r1, r2)
    draws = W.masked_counts(20000, 256, seed=3)
    assert draws.min() == 0 and draws.max() == 256


def test_new_generators_are_deterministic():
    a = W.make_k_grouped(3, 300, 32, 48, seed=5, counts=[100, 0, 200], with_c=True)
    b = W.make_k_grouped(3, 300, 32, 48, seed=5, counts=[100, 0, 200], with_c=True)
    for f in ("a", "sfa", "b", "sfb", "ks", "c"):
        assert np.array_equal(getattr(a, f), getattr(b, f)), f
    x1 = W.make_swiglu_input(8, 256, seed=6)
    x2 = W.make_swiglu_input(8, 256, seed=6)
    assert x1.dtype == np.uint16 and x1.shape == (8, 512) and np.array_equal(x1, x2)
    u = W.make_dense(64, 128, 512, seed=7, ue8m0=True)
    assert u.sfa.dtype == np.int32 and u.sfa.shape == (1, 64) and u.sfb.shape == (1, 1)


def test_f32_to_bf16_bits_rounds_to_nearest_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 3.0e38], np.float32)
    got = W.f32_to_bf16_bits(x)
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7: to the even mantissa (1.0)
    assert got.tolist() == [0x3F80, 0x3F80, 0x3F82, 0xC020, 0x7F62]


def test_stored_layout_keeps_the_scales():
    q = W.make_dense(32, 64, 256, seed=8)
    for lay in ("nn", "tn", "tt"):
        p = W.stored_layout(q, lay)
        assert p.sfa is q.sfa and p.sfb is q.sfb
