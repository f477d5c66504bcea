"""Pins for the oracle's number formats (bfloat16, OCP E4M3).

The oracle writes both codecs from their definitions; here they are checked
against torch's own conversions (a library routine, independent code) over
every pattern and over every rounding midpoint, and against closed forms.
"""
import numpy as np
import pytest
import torch

import oracle


def _torch_bf16_bits(v32: np.ndarray) -> np.ndarray:
    return torch.from_numpy(v32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_bf16_decode_all_patterns():
    pats = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(pats.view(np.int16)).view(torch.bfloat16).to(torch.float32).numpy()
    got = oracle.bf16_decode(pats)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan].astype(np.float64))


def test_bf16_encode_matches_library_rne():
    rng = np.random.default_rng(0)
    bits = rng.integers(0, 1 << 32, size=1 << 20, dtype=np.uint64).astype(np.uint32)
    v = bits.view(np.float32)
    v = v[np.isfinite(v)]
    assert np.array_equal(oracle.bf16_encode(v), _torch_bf16_bits(v))


def test_bf16_encode_midpoints_tie_to_even():
    # every midpoint between two adjacent positive finite bf16 values
    pats = np.arange(0, 0x7F7F, dtype=np.uint32)
    mid = ((pats << 16) | 0x8000).view(np.float32)          # exact midpoint pattern
    got = oracle.bf16_encode(mid)
    want = np.where(pats & 1, pats + 1, pats).astype(np.uint16)
    assert np.array_equal(got, want)
    assert np.array_equal(got, _torch_bf16_bits(mid))
    # just above / below a midpoint go up / down
    above = ((pats << 16) | 0x8001).view(np.float32)
    below = ((pats << 16) | 0x7FFF).view(np.float32)
    assert np.array_equal(oracle.bf16_encode(above), (pats + 1).astype(np.uint16))
    assert np.array_equal(oracle.bf16_encode(below), pats.astype(np.uint16))


def test_bf16_encode_specials():
    v = np.array([0.0, -0.0, np.inf, -np.inf, 3.3895314e38, np.float32(3.4028235e38)], np.float32)
    got = oracle.bf16_encode(v)
    assert got[0] == 0x0000 and got[1] == 0x8000
    assert got[2] == 0x7F80 and got[3] == 0xFF80
    assert got[4] == 0x7F7F                      # largest finite bf16 stays
    assert got[5] == 0x7F80                      # past max + half ulp -> inf
    assert np.isnan(oracle.bf16_decode(oracle.bf16_encode(np.array([np.nan], np.float32))))[0]


def _e4m3_table():
    return torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn) \
        .to(torch.float32).numpy().astype(np.float64)


def test_e4m3_decode_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ref = _e4m3_table()
    got = oracle.e4m3_decode(codes)
    nan = np.isnan(ref)
    assert nan.sum() == 2 and np.isnan(got[0x7F]) and np.isnan(got[0xFF])
    assert np.array_equal(got[~nan], ref[~nan])
    assert got[0x7E] == 448.0 and got[0x01] == 2.0 ** -9 and got[0x08] == 2.0 ** -6


def test_e4m3_roundtrip_and_midpoints():
    codes = np.arange(0, 0x7F, dtype=np.uint8)                 # non-negative finite
    vals = oracle.e4m3_decode(codes)
    assert np.array_equal(oracle.e4m3_encode(vals.astype(np.float32)), codes)
    assert np.array_equal(oracle.e4m3_encode(-vals[1:].astype(np.float32)), codes[1:] | 0x80)
    # exact midpoints between neighbours round to the even code
    mids = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)
    assert np.array_equal(mids.astype(np.float64), (vals[:-1] + vals[1:]) / 2)   # exact in fp32
    want = np.where(codes[:-1] & 1, codes[:-1] + 1, codes[:-1]).astype(np.uint8)
    got = oracle.e4m3_encode(mids)
    assert np.array_equal(got, want)
    lib = torch.from_numpy(mids).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(got, lib)


def test_e4m3_encode_matches_library_in_range():
    rng = np.random.default_rng(1)
    v = np.concatenate([rng.uniform(-448, 448, 200000), rng.normal(0, 1, 200000),
                        rng.normal(0, 0.01, 100000), rng.uniform(-2e-3, 2e-3, 100000)]).astype(np.float32)
    lib = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = oracle.e4m3_encode(v)
    # the library may keep the sign of a value that rounds to zero; compare values
    assert np.array_equal(oracle.e4m3_decode(got), oracle.e4m3_decode(lib))


def test_e4m3_saturates():
    v = np.array([448.0, 463.9, 464.0, 1e6, np.inf, -500.0, -np.inf], np.float32)
    got = oracle.e4m3_encode(v)
    assert list(got) == [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0xFE]
    assert oracle.e4m3_encode(np.array([np.nan], np.float32))[0] == 0x7F


# OCP Microscaling Formats (MX) v1.0, FP4 E2M1 element values by code (sign
# bit 3): the eight non-negative magnitudes of the format.
E2M1_MAGNITUDES = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def test_e2m1_decode_matches_the_format_table():
    got = oracle.e2m1_decode(np.arange(16, dtype=np.uint8))
    want = np.array(E2M1_MAGNITUDES + [-m for m in E2M1_MAGNITUDES])
    assert np.array_equal(got, want)
    assert np.signbit(got[8]) and not np.signbit(got[0])      # code 8 is -0


def test_e8m0_decode_is_a_power_of_two():
    e = np.arange(256, dtype=np.uint8)
    got = oracle.e8m0_decode(e)
    assert np.array_equal(got[:255], np.ldexp(1.0, e[:255].astype(np.int64) - 127))
    assert np.isnan(got[255])
