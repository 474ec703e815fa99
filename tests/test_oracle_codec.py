"""Pins for the oracle's element codecs (E4M3FN, f16, bf16).

Checked against torch's own float8_e4m3fn / float16 / bfloat16 conversions
(independent library routines) and the E4M3 range the pages give
("大语言模型推理引擎深度剖析", section 4.2: E4M3 spans +-448)."""
import json
import os

import numpy as np
import pytest
import torch

from oracle import oracle as orc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def torch_e4m3_decode(codes):
    return torch.from_numpy(codes.astype(np.uint8)).view(torch.float8_e4m3fn).double().numpy()


def test_e4m3_decode_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = orc.to_f64(codes, "fp8")
    ref = torch_e4m3_decode(codes)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert set(np.nonzero(nan)[0].tolist()) == {0x7F, 0xFF}
    assert np.array_equal(ours[~nan], ref[~nan])
    # signed zeros decode with their sign
    assert np.signbit(ours[0x80]) and not np.signbit(ours[0x00])


def test_e4m3_range_from_pages():
    with open(os.path.join(GOLDEN, "kv_bytes.json")) as f:
        g = json.load(f)["e4m3_max"]
    vals = orc.to_f64(np.arange(256, dtype=np.uint8), "fp8")
    assert np.nanmax(vals) == g["value"] == 448.0
    assert np.nanmin(vals) == -448.0
    assert orc.to_f64(np.array([0x7E], np.uint8), "fp8")[0] == 448.0


def test_e4m3_special_codes():
    v = orc.to_f64(np.array([0x08, 0x01, 0x07, 0x38, 0x40], np.uint8), "fp8")
    # smallest normal 2^-6, smallest subnormal 2^-9, largest subnormal 7*2^-9,
    # exponent field 7 = bias -> 1.0, exponent 8 -> 2.0
    assert v.tolist() == [2.0 ** -6, 2.0 ** -9, 7 * 2.0 ** -9, 1.0, 2.0]


def test_e4m3_encode_roundtrip_every_finite_code():
    codes = np.array([c for c in range(256) if c & 0x7F != 0x7F], dtype=np.uint8)
    x = orc.to_f64(codes, "fp8").astype(np.float32)
    assert np.array_equal(orc.e4m3_encode(x), codes)


def _midpoints_and_neighbours():
    pos = np.sort(orc.to_f64(np.arange(0, 127, dtype=np.uint8), "fp8"))
    mids = (pos[:-1] + pos[1:]) / 2.0  # exact in float32 (few mantissa bits)
    f = np.concatenate([pos, mids]).astype(np.float32)
    up = np.nextafter(f, np.float32(np.inf))
    dn = np.nextafter(f, np.float32(-np.inf))
    allv = np.concatenate([f, up, dn])
    return np.concatenate([allv, -allv])


def test_e4m3_encode_matches_torch_in_range():
    rs = np.random.default_rng(7)
    x = np.concatenate([
        _midpoints_and_neighbours(),
        rs.standard_normal(200000).astype(np.float32) * np.float32(50.0),
        rs.uniform(-0.02, 0.02, 100000).astype(np.float32),
    ]).astype(np.float32)
    # torch's cast does not saturate: compare only where no overflow happens
    x = x[np.abs(x) < 464.0]
    ours = orc.e4m3_encode(x)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)


def test_e4m3_encode_ties_to_even_examples():
    # 17 lies halfway between 16 (code 0x58, mantissa 0) and 18 (0x59): even wins
    # 19 lies halfway between 18 (0x59) and 20 (0x5A): even wins
    assert orc.e4m3_encode(np.array([17.0, 19.0, -17.0], np.float32)).tolist() == [0x58, 0x5A, 0xD8]
    # half of the smallest subnormal rounds to zero, slightly more rounds up
    tiny = np.float32(2.0 ** -10)
    assert orc.e4m3_encode(np.array([tiny, np.nextafter(tiny, np.float32(1))], np.float32)).tolist() == [0, 1]


def test_e4m3_encode_saturates_and_nan():
    x = np.array([464.0, 1e6, np.inf, -464.0, -np.inf, np.nan, 449.0], np.float32)
    assert orc.e4m3_encode(x).tolist() == [0x7E, 0x7E, 0x7E, 0xFE, 0xFE, 0x7F, 0x7E]


def test_e4m3_encode_saturates_every_large_magnitude():
    # every bf16 magnitude from 448 to the largest finite float (the whole
    # exponent range beyond the codes), both signs
    pat = np.arange(0x43E0, 0x7F80, dtype=np.uint32) << np.uint32(16)
    x = pat.view(np.float32)
    x = np.concatenate([x, np.nextafter(x, np.float32(np.inf)), np.float32(3.4028235e38)[None]])
    x = x[np.isfinite(x)]
    assert np.all(orc.e4m3_encode(x) == 0x7E)
    assert np.all(orc.e4m3_encode(-x) == 0xFE)


def test_e4m3_encode_is_monotone_over_every_bf16_pattern():
    # nearest-code rounding never decreases as the input grows
    x = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16).view(np.uint16)
    f = (x.astype(np.uint32) << np.uint32(16)).view(np.float32)
    f = np.sort(f[np.isfinite(f)])
    dec = orc.to_f64(orc.e4m3_encode(f), "fp8")
    assert np.all(np.diff(dec) >= 0)
    assert dec[0] == -448.0 and dec[-1] == 448.0


@pytest.mark.parametrize("dtype,tdt", [("f16", torch.float16), ("bf16", torch.bfloat16)])
def test_16bit_decode_all_patterns_match_torch(dtype, tdt):
    pats = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = orc.to_f64(pats, dtype)
    ref = torch.from_numpy(pats.view(np.int16)).view(tdt).double().numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])


def test_f32_decode_is_identity():
    x = np.random.default_rng(3).standard_normal(1000).astype(np.float32)
    assert np.array_equal(orc.to_f64(x, "f32"), x.astype(np.float64))


# -- INT8 codes (symmetric, one scale per tensor) -----------------------------

def test_int8_encode_matches_numpy_rint_and_clip():
    """Nearest integer with ties to even (numpy's rint), saturated to +-127,
    on a dense grid, every half-integer tie in range and beyond the range."""
    grid = np.linspace(-140.0, 140.0, 280001, dtype=np.float32)
    ties = np.arange(-130, 130, dtype=np.float32) + np.float32(0.5)
    x = np.concatenate([grid, ties, np.float32([3e38, -3e38, 127.49, 127.5, -127.5, 0.0, -0.0])])
    got = orc.int8_encode(x)
    ref = np.clip(np.rint(x), -127, 127).astype(np.int8)
    assert np.array_equal(got, ref)


def test_int8_encode_specials():
    got = orc.int8_encode(np.float32([np.nan, np.inf, -np.inf, 0.5, 1.5, 2.5, -0.5, -1.5]))
    assert got.tolist() == [0, 127, -127, 0, 2, 2, 0, -2]
    # -128 is never produced
    assert orc.int8_encode(np.float32([-128.0, -1e9])).tolist() == [-127, -127]
