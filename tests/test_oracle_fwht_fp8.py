"""Pins of the oracle's Hadamard-128 + power-of-two-scale FP8 quantizer
(kpool_compress.py, _fwht_quant_kernel / fwht128_quant_fp8).

Exact on integer-valued rows, where the fp32 butterflies are exact and the
whole pipeline reduces to library routines: scipy's Hadamard matrix, an
fp32 multiply by the page's 1/sqrt(128) constant, torch's bf16 and
float8_e4m3fn casts, and an exact power-of-two ceiling from math.frexp.
Properties on random rows: the scale is a power of two, the row maximum
lands in (224, 448], every code is finite E4M3, and code*scale tracks the
normalized transform. The power-of-two rule is also checked over every
positive finite bf16 absmax value.
"""
import json
import math
import os

import numpy as np
import scipy.linalg
import torch

import oracle
from quantized_paged_kv_tq_amd import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _consts():
    g = json.load(open(os.path.join(GOLDEN, "page_constants.json")))
    return {k: np.uint32(int(v["fp32_bits"], 16)).view(np.float32) for k, v in g["constants"].items()}


def _exact_pow2_ceil(t):
    m, e = math.frexp(t)  # t = m * 2^e, 0.5 <= m < 1
    return 2.0 ** (e - 1) if m == 0.5 else 2.0 ** e


def test_page_constants_are_the_fp32_roundings():
    c = _consts()
    assert c["inv_sqrt128"] == np.float32(0.08838834764831845)
    assert c["inv_448"] == np.float32(1.0 / 448.0)
    assert c["absmax_floor"] == np.float32(1e-4)
    assert c["int4_scale_floor"] == np.float32(1e-6)


def test_integer_rows_exact_pipeline():
    c = _consts()
    rng = np.random.default_rng(0)
    x = rng.integers(-64, 64, size=(3000, 128)).astype(np.float32)
    x[0] = 0.0
    x[1] = 0.0
    x[1, 5] = 1.0
    bits = W.to_bits(x, "bf16")
    assert np.array_equal(W.bits_to_f32(bits, "bf16"), x)
    y, s = oracle.fwht128_quant_fp8(bits)
    H = scipy.linalg.hadamard(128).astype(np.float64)
    hx = (x.astype(np.float64) @ H.T).astype(np.float32)  # exact integers
    xr = torch.from_numpy(hx * c["inv_sqrt128"]).to(torch.bfloat16).to(torch.float32).numpy()
    amax = np.maximum(np.abs(xr).max(1), c["absmax_floor"])
    want_s = np.array([_exact_pow2_ceil(float(np.float32(a * c["inv_448"]))) for a in amax], np.float32)
    np.testing.assert_array_equal(s, want_s)
    yy = np.clip(xr / want_s[:, None], -448, 448)
    want_y = torch.from_numpy(yy).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(y, want_y)


def test_random_rows_properties():
    bits = W.fwht_rows(rows=4096, wid=77)
    y, s = oracle.fwht128_quant_fp8(bits)
    m, e = np.frexp(s)
    assert np.all(m == 0.5)  # powers of two
    dec = torch.from_numpy(y).view(torch.float8_e4m3fn).to(torch.float32).numpy()
    assert np.all(np.isfinite(dec))
    amax = np.abs(dec).max(1)
    assert np.all(amax <= 448) and np.all(amax > 224 * (1 - 2 ** -3))
    x = W.bits_to_f32(bits, "bf16").astype(np.float64)
    ref = x @ scipy.linalg.hadamard(128).T / np.sqrt(128)
    err = np.abs(dec * s[:, None] - ref)
    assert np.all(err <= np.abs(ref) * (2 ** -4 + 2 ** -8) + s[:, None] * 2 ** -9 + 1e-6)


def test_pow2_scale_rule_over_all_bf16_absmax():
    c = _consts()
    bits = np.arange(0x0001, 0x7F80, dtype=np.uint16)  # positive finite bf16
    vals = W.bits_to_f32(bits, "bf16")
    for a in vals[::1]:
        got = oracle.fp8_pow2_scale(a)
        t = float(np.float32(max(a, c["absmax_floor"]) * c["inv_448"]))
        assert got == _exact_pow2_ceil(t), a


def test_empty_and_zero_rows():
    y, s = oracle.fwht128_quant_fp8(np.zeros((0, 128), np.uint16))
    assert y.shape == (0, 128) and s.shape == (0,)
    y, s = oracle.fwht128_quant_fp8(np.zeros((2, 128), np.uint16))
    assert np.all(y == 0)
    assert s[0] == _exact_pow2_ceil(float(np.float32(np.float32(1e-4) * np.float32(1 / 448))))
