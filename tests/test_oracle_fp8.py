"""Pins for the oracle's E4M3 decode, rounding and block quantisation.

The oracle's decode and round are checked against torch's CPU float8_e4m3fn
casts (a library routine, valid inside +-448), exhaustively over every code
point and every rounding midpoint, and the block quantiser against its
defining invariants.
"""
import math

import numpy as np
import pytest
import torch


def torch_decode(codes):
    t = torch.from_numpy(np.asarray(codes, dtype=np.uint8)).view(torch.float8_e4m3fn)
    return t.to(torch.float32).numpy().astype(np.float64)


def torch_round(values):
    t = torch.from_numpy(np.asarray(values, dtype=np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_decode_all_codes_match_library(orc):
    codes = np.arange(256)
    ours = orc.e4m3_decode(codes)
    ref = torch_decode(codes)
    finite = ~np.isnan(ref)
    assert np.isnan(ours[~finite]).all()
    assert set(codes[~finite]) == {0x7F, 0xFF}
    np.testing.assert_array_equal(ours[finite], ref[finite])


def test_decode_hand_values(orc):
    # format definition: bias 7, 3 mantissa bits, subnormals below 2^-6
    assert orc.e4m3_value(0x7E) == 448.0
    assert orc.e4m3_value(0x38) == 1.0
    assert orc.e4m3_value(0x01) == 2.0 ** -9
    assert orc.e4m3_value(0x07) == 7 * 2.0 ** -9
    assert orc.e4m3_value(0x08) == 2.0 ** -6
    assert orc.e4m3_value(0xB8) == -1.0
    assert orc.e4m3_value(0x3C) == 1.5


def _positive_values(orc):
    return np.array([orc.e4m3_value(c) for c in range(127)])  # 0x00..0x7E


def test_round_exact_code_points(orc):
    vals = _positive_values(orc)
    for c, v in enumerate(vals):
        assert orc.e4m3_round(v) == c
        assert orc.e4m3_round(-v) == (0x80 | c)


def test_round_midpoints_go_to_even(orc):
    vals = _positive_values(orc)
    for c in range(126):
        mid = (vals[c] + vals[c + 1]) / 2.0
        assert float(np.float32(mid)) == mid  # midpoints are exact in binary32
        even = c if c % 2 == 0 else c + 1
        assert orc.e4m3_round(mid) == even, (c, mid)
        assert orc.e4m3_round(-mid) == (0x80 | even)
        below = float(np.nextafter(np.float32(mid), np.float32(0)))
        above = float(np.nextafter(np.float32(mid), np.float32(1e9)))
        assert orc.e4m3_round(below) == c
        assert orc.e4m3_round(above) == c + 1


def test_round_matches_library_on_random_values(orc):
    rng = np.random.default_rng(7)
    v = np.concatenate([
        rng.standard_normal(20000) * 100,
        rng.standard_normal(20000) * 1e-2,
        rng.uniform(-448, 448, 20000),
    ]).astype(np.float32)
    ours = np.array([orc.e4m3_round(x) for x in v], dtype=np.uint8)
    ref = torch_round(v)
    np.testing.assert_array_equal(ours, ref)


def test_round_saturates(orc):
    assert orc.e4m3_round(448.0) == 0x7E
    assert orc.e4m3_round(463.9) == 0x7E
    assert orc.e4m3_round(1e30) == 0x7E
    assert orc.e4m3_round(-1e30) == 0xFE
    assert orc.e4m3_round(0.0) == 0x00
    assert orc.e4m3_round(-0.0) == 0x80
    assert orc.e4m3_round(2.0 ** -11) == 0x00  # below half the smallest subnormal
    assert orc.e4m3_round(-(2.0 ** -11)) == 0x80


@pytest.mark.parametrize("shape,blk", [((3, 300), (1, 128)), ((130, 257), (128, 128)),
                                       ((256, 128), (128, 128))])
def test_quant_blocks_invariants(orc, shape, blk):
    rng = np.random.default_rng(11)
    v = (rng.standard_normal(shape) * rng.uniform(0.01, 10)).astype(np.float32)
    v[: blk[0], : blk[1]] = 0.0  # one all-zero block
    q, s = orc.quant_blocks(v, *blk)
    R, Cn = shape
    br, bc = blk
    assert s.shape == (math.ceil(R / br), math.ceil(Cn / bc))
    assert s[0, 0] == 1.0 and (q[:br, :bc] == 0).all()
    deq = torch_decode(q)
    for rb in range(s.shape[0]):
        for cb in range(s.shape[1]):
            blkv = v[rb * br:(rb + 1) * br, cb * bc:(cb + 1) * bc]
            amax = np.float32(np.abs(blkv).max())
            if amax == 0:
                continue
            assert s[rb, cb] == np.float32(amax / np.float32(448.0))
            sc = s[rb, cb]
            blkq = deq[rb * br:(rb + 1) * br, cb * bc:(cb + 1) * bc]
            # the absmax element lands on +-448
            assert np.abs(blkq).max() == 448.0
            # codes are the library's RNE of the binary32 quotient v / s
            quot = (blkv / sc).astype(np.float32)
            np.testing.assert_array_equal(
                q[rb * br:(rb + 1) * br, cb * bc:(cb + 1) * bc], torch_round(quot))
            # dequantised values within half a code spacing (relative 1/16)
            err = np.abs(blkq * sc - blkv)
            assert (err <= np.abs(blkv) / 16 + sc * 2.0 ** -10 + 1e-30).all()
