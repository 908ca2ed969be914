"""Pins of the oracle's E4M3 fine-grained quantisation: every code, RNE
midpoints, saturation, and torch's float8_e4m3fn as a library reference.  CPU only."""
import numpy as np
import torch

import oracle as O


def _torch_decode(codes):
    return torch.from_numpy(np.asarray(codes, np.uint8)).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def test_decode_all_codes_matches_torch():
    codes = np.arange(256, dtype=np.uint8)
    mine = O.e4m3_decode(codes)
    ref = _torch_decode(codes)
    nan = np.isnan(ref)
    assert set(np.nonzero(nan)[0].tolist()) == {0x7F, 0xFF}
    np.testing.assert_array_equal(np.isnan(mine), nan)
    np.testing.assert_array_equal(mine[~nan], ref[~nan])
    assert mine[0x7E] == 448.0 and mine[0x01] == 2.0 ** -9 and mine[0x08] == 2.0 ** -6


def test_every_code_roundtrips():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    vals = O.e4m3_decode(codes).astype(np.float32)
    np.testing.assert_array_equal(O.e4m3_quantize(vals), codes)


def test_midpoints_round_to_even_and_saturate():
    pos = np.array([c for c in range(0x7F)], dtype=np.uint8)          # 0 .. 448
    v = O.e4m3_decode(pos)
    mid = ((v[:-1] + v[1:]) / 2).astype(np.float32)
    q = O.e4m3_quantize(mid)
    lo, hi = pos[:-1], pos[1:]
    expect = np.where(lo % 2 == 0, lo, hi)       # even mantissa wins
    np.testing.assert_array_equal(q, expect)
    big = np.array([448.0, 460.0, 464.0, 470.0, 480.0, 1e6, 3e38], np.float32)
    assert np.all(O.e4m3_quantize(big) == 0x7E)
    assert np.all(O.e4m3_quantize(-big) == 0xFE)
    assert O.e4m3_quantize(np.float32(2.0 ** -10)) == 0x00      # half of the smallest subnormal
    assert O.e4m3_quantize(np.float32(-(2.0 ** -10) * 1.01)) == 0x81


def test_quantize_matches_torch_in_range():
    g = np.random.default_rng(7)
    v = (g.standard_normal(200000) * np.exp(g.uniform(-12, 6, 200000))).astype(np.float32)
    v = v[np.abs(v) < 448.0]
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(O.e4m3_quantize(v), ref)


def test_quantize_1x128_scales_and_error_bound():
    g = np.random.default_rng(3)
    a = g.standard_normal((5, 512)).astype(np.float32)
    a[2, 7] = 200.0                       # an outlier only coarsens its own 1x128 tile
    a[4, 128:256] = 0.0                   # all-zero tile: scale 1
    q, s = O.quantize_1x128(a)
    assert s.shape == (5, 4) and s.dtype == np.float32
    amax = np.abs(a.reshape(5, 4, 128)).max(axis=2)
    np.testing.assert_array_equal(s[amax > 0], (amax[amax > 0] / np.float32(448.0)).astype(np.float32))
    assert s[4, 1] == 1.0 and np.all(q[4, 128:256] == 0)
    # the max-abs element of each nonzero tile hits +-448
    dq = O.dequantize_1x128(q, s)
    for r in range(5):
        for t in range(4):
            if amax[r, t] > 0:
                tile = np.abs(O.e4m3_decode(q[r, t * 128:(t + 1) * 128]))
                assert tile.max() == 448.0
    # relative error of normals <= 2^-4, absolute error of subnormals <= 2^-10 * scale
    err = np.abs(dq - a.astype(np.float64))
    bound = np.maximum(np.abs(a) * 2.0 ** -4, np.repeat(s, 128, axis=1) * 2.0 ** -10)
    assert np.all(err <= bound * (1 + 1e-6))
    assert s[2, 0] > 10 * s[2, 1]


def test_fake_quant_is_idempotent():
    g = np.random.default_rng(5)
    a = g.standard_normal((3, 256))
    once = O.fake_quant_1x128(a)
    twice = O.fake_quant_1x128(once)
    np.testing.assert_array_equal(once, twice)


def test_block_dequant_uses_the_right_scale():
    codes = np.full((256, 256), 0x38, np.uint8)     # 1.0
    scales = np.array([[1.0, 2.0], [3.0, 4.0]], np.float32)
    w = O.dequant_blocks(codes, scales)
    assert w[0, 0] == 1.0 and w[0, 200] == 2.0 and w[200, 0] == 3.0 and w[255, 255] == 4.0
