"""Pins of the oracle's E4M3FN codec and of the write's fp32 quotient.

The codec follows the OCP E4M3FN definition (the E4M3 format named in
"Optimización de KV Cache con PagedAttention y Cuantización FP8 ...", §6.2 and
§8, whose largest finite value 448 is what an amax/448 scale targets).  It is
checked against a library routine (torch's float8_e4m3fn) and against values
derived by hand from the format definition.
"""
import math

import numpy as np
import pytest
import torch


def test_decode_table_matches_library_view_cast(orc):
    table = orc.e4m3_decode_table()
    lib = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan_o, nan_l = np.isnan(table), np.isnan(lib)
    assert np.array_equal(nan_o, nan_l)
    assert set(np.flatnonzero(nan_o)) == {0x7F, 0xFF}
    assert np.array_equal(table[~nan_o], lib[~nan_l])
    # signs, including the negative zero
    assert np.array_equal(np.signbit(table[~nan_o]), np.signbit(lib[~nan_l]))


@pytest.mark.parametrize("code,value", [
    (0x00, 0.0), (0x01, 2.0 ** -9), (0x07, 7 * 2.0 ** -9), (0x08, 2.0 ** -6),
    (0x0F, 1.875 * 2.0 ** -6), (0x38, 1.0), (0x39, 1.125), (0x3F, 1.875),
    (0x40, 2.0), (0x7E, 448.0), (0x77, 240.0), (0xB8, -1.0), (0xFE, -448.0),
])
def test_decode_landmarks(orc, code, value):
    assert orc.e4m3_decode(code) == value


def test_negative_zero(orc):
    v = orc.e4m3_decode(0x80)
    assert v == 0.0 and math.copysign(1.0, v) < 0
    assert int(orc.e4m3_encode(np.float32(-0.0))) == 0x80


@pytest.mark.parametrize("u,code", [
    (2.0 ** -10, 0x00),            # halfway 0 .. 2^-9: tie to the even code 0
    (3 * 2.0 ** -10, 0x02),        # halfway 2^-9 .. 2^-8: tie to even code 2
    (1.0625, 0x38),                # halfway 1.0 .. 1.125: even code 0x38
    (1.1875, 0x3A),                # halfway 1.125 .. 1.25: even code 0x3A
    (15 * 2.0 ** -10, 0x08),       # halfway 7*2^-9 .. 2^-6: even is 0x08
    (448.0, 0x7E), (464.0, 0x7E), (1000.0, 0x7E), (float("inf"), 0x7E),
    (-1000.0, 0xFE), (float("-inf"), 0xFE),
    (447.9, 0x7E), (416.0, 0x7D), (432.0, 0x7E),  # 432 is the 416/448 midpoint: even 0x7E
    (2.0 ** -20, 0x00), (-(2.0 ** -20), 0x80),
])
def test_encode_hand_cases(orc, u, code):
    assert int(orc.e4m3_encode(np.float32(u))) == code


def test_encode_nan(orc):
    assert int(orc.e4m3_encode(np.float32("nan"))) == 0x7F
    assert int(orc.e4m3_encode(-np.float32("nan"))) == 0xFF


def test_encode_round_trip_all_codes(orc):
    table = orc.e4m3_decode_table()
    for c in range(256):
        if c in (0x7F, 0xFF):
            continue
        assert int(orc.e4m3_encode(np.float32(table[c]))) == c


def _library_cast(u: np.ndarray) -> np.ndarray:
    return torch.from_numpy(u).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_encode_matches_library_on_all_fp16_values(orc):
    u = np.arange(65536, dtype=np.uint16).view(np.float16).astype(np.float32)
    u = u[np.isfinite(u) & (np.abs(u) < 464.0)]
    assert np.array_equal(orc.e4m3_encode(u), _library_cast(u))


def test_encode_matches_library_on_midpoints_and_neighbours(orc):
    table = orc.e4m3_decode_table()[:0x7F]
    mids = ((table[1:] + table[:-1]) / 2).astype(np.float32)
    u = np.concatenate([mids, np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(500))])
    u = np.concatenate([u, -u])
    u = u[np.abs(u) < 464.0]
    assert np.array_equal(orc.e4m3_encode(u), _library_cast(u))


def test_encode_matches_library_on_random_fp32(orc):
    rng = np.random.default_rng(1234)
    mag = np.exp2(rng.uniform(-14, np.log2(463.9), size=200_000)).astype(np.float32)
    u = np.where(rng.random(mag.size) < 0.5, -mag, mag).astype(np.float32)
    assert np.array_equal(orc.e4m3_encode(u), _library_cast(u))


def test_encode_is_monotone(orc):
    u = np.linspace(0, 460, 100_001, dtype=np.float32)
    vals = orc.e4m3_decode_table()[orc.e4m3_encode(u)]
    assert np.all(np.diff(vals) >= 0)


def test_quotient_is_correctly_rounded_fp32_division(orc):
    rng = np.random.default_rng(7)
    x = rng.standard_normal(2000).astype(np.float16)
    s = np.exp2(rng.uniform(-8, 4, size=2000)).astype(np.float32)
    for xi, si in zip(x, s):
        assert orc.quotient(float(xi), float(si)) == np.float32(xi) / si  # numpy: IEEE fp32 division


def test_quantize_f16_equals_elementwise_encode(orc):
    rng = np.random.default_rng(3)
    x = rng.standard_normal(50_000).astype(np.float16)
    scale = np.float32(np.abs(x.astype(np.float32)).max() / np.float32(448.0))
    u = x.astype(np.float32) / scale
    assert np.array_equal(orc.quantize_f16(x, scale), orc.e4m3_encode(u))
    # the amax/448 scale never leaves the finite range: no saturation, no NaN
    assert np.abs(u).max() <= 448.0
