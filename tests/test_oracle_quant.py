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
    assert np.array_equal(scale, np.maximum(amax, 1e-4) / 448.0)
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
    assert np.all(sf[:, :2] == 1e-4 / 448.0)
    assert np.all((q == 0) | (q == 0x80))
