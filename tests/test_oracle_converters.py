"""Pins of the oracle's scalar converters against torch's CPU casts (a
library routine independent of the oracle), exhaustively where the domain
is small and on dense random plus tie samples where it is not."""
import numpy as np
import pytest
import torch

import oracle


def _torch_cast_bits(x32, dtype):
    t = torch.from_numpy(np.ascontiguousarray(x32, np.float32)).to(dtype)
    if dtype == torch.float8_e4m3fn:
        return t.view(torch.uint8).numpy()
    return t.view(torch.int16).numpy().view(np.uint16)


def _samples(rng, lo_exp, hi_exp, n):
    mant = rng.uniform(1.0, 2.0, n).astype(np.float32)
    e = rng.integers(lo_exp, hi_exp, n)
    s = rng.choice([-1.0, 1.0], n).astype(np.float32)
    return (s * np.ldexp(mant, e)).astype(np.float32)


def _midpoints(codes_f32):
    """fp32 values exactly halfway between consecutive representable values
    of a narrower format (ties), when representable in fp32."""
    v = np.sort(np.unique(codes_f32[np.isfinite(codes_f32)].astype(np.float64)))
    mid = (v[:-1] + v[1:]) / 2
    m32 = mid.astype(np.float32)
    return m32[m32.astype(np.float64) == mid]


def test_bf16_all_patterns_roundtrip_and_ties():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    f = oracle.bf16_to_f32(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float32).numpy()
    fin = np.isfinite(ref)
    np.testing.assert_array_equal(f.view(np.uint32)[fin], ref.view(np.uint32)[fin])
    back = oracle.f32_to_bf16(f[fin])
    np.testing.assert_array_equal(back, bits[fin])
    mids = _midpoints(ref)
    np.testing.assert_array_equal(oracle.f32_to_bf16(mids), _torch_cast_bits(mids, torch.bfloat16))


def test_bf16_random():
    x = _samples(np.random.default_rng(0), -130, 127, 1_000_000)
    np.testing.assert_array_equal(oracle.f32_to_bf16(x), _torch_cast_bits(x, torch.bfloat16))


def test_f16_all_patterns_roundtrip_and_ties():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    f = oracle.f16_to_f32(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.float16).to(torch.float32).numpy()
    fin = np.isfinite(ref)
    np.testing.assert_array_equal(f.view(np.uint32)[fin], ref.view(np.uint32)[fin])
    np.testing.assert_array_equal(oracle.f32_to_f16(f[fin]), bits[fin])
    mids = _midpoints(ref)
    np.testing.assert_array_equal(oracle.f32_to_f16(mids), _torch_cast_bits(mids, torch.float16))


def test_f16_random_including_subnormal_and_overflow():
    x = _samples(np.random.default_rng(1), -30, 18, 1_000_000)
    np.testing.assert_array_equal(oracle.f32_to_f16(x), _torch_cast_bits(x, torch.float16))


def test_e4m3_decode_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    f = oracle.e4m3_to_f32(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float32).numpy()
    nan = np.isnan(ref)
    assert nan.sum() == 2 and np.isnan(f[nan]).all()  # S.1111.111 only
    np.testing.assert_array_equal(f[~nan], ref[~nan])
    assert np.nanmax(f) == 448.0 and np.nanmin(f) == -448.0
    assert f[1] == 2.0 ** -9  # smallest subnormal


def test_e4m3_encode_in_range_random_and_ties():
    rng = np.random.default_rng(2)
    x = rng.uniform(-448, 448, 2_000_000).astype(np.float32)
    x = np.concatenate([x, _samples(rng, -12, 8, 1_000_000)])
    x = x[np.abs(x) <= 448]
    np.testing.assert_array_equal(oracle.f32_to_e4m3(x), _torch_cast_bits(x, torch.float8_e4m3fn))
    ref = torch.from_numpy(np.arange(256, dtype=np.uint8)).view(torch.float8_e4m3fn).to(torch.float32).numpy()
    mids = _midpoints(ref)
    np.testing.assert_array_equal(oracle.f32_to_e4m3(mids), _torch_cast_bits(mids, torch.float8_e4m3fn))
    # every finite code round-trips
    fin = np.isfinite(ref)
    np.testing.assert_array_equal(oracle.f32_to_e4m3(ref[fin]), np.arange(256, dtype=np.uint8)[fin])


def test_e4m3_keeps_signed_zero():
    assert oracle.f32_to_e4m3(np.array([-0.0], np.float32))[0] == 0x80
    assert oracle.f32_to_e4m3(np.array([0.0], np.float32))[0] == 0x00
