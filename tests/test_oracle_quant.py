"""Pins for the oracle's activation step (SwiGLU, then the 1x128 FP8 cast of the next GEMM's
A): the nearest-e4m3 rounding against torch's float8_e4m3fn cast (a library routine) including
exact ties, bf16 decoding from the format's closed form, SwiGLU identities, and the cast's
invariants (each segment's largest element at +-448, half-step error bound, zero segments,
the MN-major scale layout).  CPU only."""
import numpy as np
import torch

import oracle
import workloads as W


def _torch_cast(y):
    return torch.from_numpy(np.asarray(y, np.float64)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_nearest_e4m3_matches_torch_cast_with_ties():
    rng = np.random.default_rng(0)
    tab = oracle.e4m3_table()
    mags = np.sort(tab[:0x7F])
    mids = (mags[1:] + mags[:-1]) / 2                          # exact ties
    y = np.concatenate([rng.uniform(-448, 448, 20000), rng.standard_normal(20000) * 1e-3,
                        mids, -mids, mags, -mags, [0.0, -0.0, 448.0, -448.0]])
    assert np.array_equal(oracle.e4m3_nearest(y), _torch_cast(y))


def test_bf16_decode_closed_forms():
    bits = np.array([0x3F80, 0xC000, 0x0001, 0x7F7F, 0x8000, 0x4049], np.uint16)
    want = [1.0, -2.0, 2.0 ** -133, (2 - 2 ** -7) * 2.0 ** 127, -0.0, 3.140625]
    got = oracle.bf16_decode(bits)
    assert all(g == w for g, w in zip(got, want)) and np.signbit(got[4])


def _bits(gate, up):
    return W.f32_to_bf16_bits(np.concatenate([np.asarray(gate, np.float32),
                                              np.asarray(up, np.float32)], axis=1))


def test_swiglu_identities():
    g = np.array([[0.0, 1.0, -1.0, 20.0, -20.0, 0.5, 3.0, -3.0]], np.float32)
    u = np.array([[5.0, 2.0, 2.0, 1.5, 1.5, -4.0, 1.0, 1.0]], np.float32)
    h = oracle.swiglu(_bits(g, u))[0]
    assert h[0] == 0.0
    assert abs(h[1] - 2.0 / (1 + np.exp(-1.0))) < 1e-15
    # silu(-x) = silu(x) - x
    assert abs(h[2] - (h[1] - 2.0 * 1.0)) < 1e-15
    assert abs(h[3] - 30.0) < 30.0 * 3e-9 and abs(h[4]) < 30.0 * 3e-9
    assert abs(h[6] - h[7] - 3.0) < 1e-14          # silu(3) - silu(-3) = 3 (times up = 1)


def test_cast_invariants_and_scale_layout():
    x = W.make_swiglu_input(37, 512, seed=3)
    h, sf, q = oracle.swiglu_quant(x)
    assert sf.shape == (4, 40) and not sf[:, 37:].any()
    tab = oracle.e4m3_table()
    seg = h.reshape(37, 4, 128)
    amax = np.abs(seg).max(axis=2)
    scale = sf[:, :37].T
    # the scale maps each segment's largest magnitude onto the format's largest finite value,
    # read off the decode table (0x7E): before any clip, max |h| / scale equals it within one
    # float64 ulp, and no element of the segment exceeds it (a denominator of 447 or 449
    # fails both ways)
    top = oracle.e4m3_table()[0x7E]
    big = amax >= 1e-4
    ratio = amax[big] / scale[big]
    assert np.all(np.abs(ratio - top) <= np.spacing(top)), ratio[np.abs(ratio - top) > np.spacing(top)][:4]
    assert np.all(np.abs(seg / scale[:, :, None]) <= top + np.spacing(top))
    # the largest element of every non-zero segment is cast to +-448
    qs = q.reshape(37, 4, 128)
    for r in range(37):
        for s in range(4):
            if amax[r, s] > 0:
                k = np.argmax(np.abs(seg[r, s]))
                assert tab[qs[r, s, k]] == np.sign(seg[r, s, k]) * 448.0
    # every code is within half an e4m3 step of h / scale (relative 2^-4 for normals, absolute
    # 2^-10 in the subnormal range)
    y = seg / scale[:, :, None]
    err = np.abs(tab[qs] - y)
    assert np.all(err <= np.maximum(np.abs(y) * 2.0 ** -4, 2.0 ** -10))


def test_zero_segments_give_the_floor_scale_and_zero_codes():
    g = np.zeros((2, 256), np.float32)
    u = np.random.default_rng(4).standard_normal((2, 256)).astype(np.float32)
    h, sf, q = oracle.swiglu_quant(_bits(g, u))
    # a zero segment takes the floor: its scale maps 1e-4 onto the largest e4m3 value
    top = oracle.e4m3_table()[0x7E]
    assert np.all(np.abs(1e-4 / sf[:, :2] - top) <= np.spacing(top))
    assert np.all((q == 0) | (q == 0x80))


def test_scale_of_a_known_segment():
    # gate 20 makes silu(gate) = 20 / (1 + e^-20); with up = 2 at one column and 1 elsewhere the
    # segment's largest magnitude is 40 / (1 + e^-20), so the scale is that over 448, and the
    # codes are 448 at that column and the nearest e4m3 of 448 / 2 = 224 elsewhere
    gate = np.full((1, 128), 20.0, np.float32)
    up = np.ones((1, 128), np.float32)
    up[0, 5] = 2.0
    h, sf, q = oracle.swiglu_quant(_bits(gate, up))
    amax = 40.0 / (1.0 + np.exp(-20.0))
    assert abs(sf[0, 0] * 448.0 / amax - 1.0) <= 2.0 ** -52
    tab = oracle.e4m3_table()
    assert tab[q[0, 5]] == 448.0 and np.all(tab[np.delete(q[0], 5)] == 224.0)
