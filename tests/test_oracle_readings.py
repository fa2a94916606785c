"""Hand-derived pins of the rounding readings of the quantizers.

Each row in golden/rounding_readings.json is built so that the reading
taken and its plausible alternative give different codes, with the exact
binary arithmetic written out in the file:
  * INT4 (int4_per_token_head.py, _reshape_cache_int4_kernel): the
    quantizer's x * inv + zp is one fused multiply-add, and "+-0.5 then
    truncate" is an fp32 add followed by truncation (not roundf / rint);
  * TurboQuant slot encoder (the reader is triton_turboquant_decode.py,
    _tq_decode_stage1; the pages show no encoder): u = (y r) / ||k|| and
    (v - zero16) / scale16 are divisions per element, and the key norm sums
    the squares pairwise in the butterfly order.
tests/test_oracle_mutants.py compiles the oracle with each alternative and
shows that these rows fail it.
"""
import json
import os

import numpy as np

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden():
    return json.load(open(os.path.join(GOLDEN, "rounding_readings.json")))


def _f32(hexes):
    return np.array([int(h, 16) for h in hexes], np.uint32).view(np.float32)


def _nibbles(packed):
    q = np.empty(2 * packed.size, np.int64)
    q[0::2] = packed & 0xF
    q[1::2] = packed >> 4
    return q


def _int4_row(name):
    g = _golden()[name]
    packed, word = oracle.int4_quantize_row(_f32(g["x_f32_hex"]))
    assert "0x%08X" % int(np.float32(word).view(np.uint32)) == g["word_hex"]
    np.testing.assert_array_equal(_nibbles(packed), np.array(g["q"]))


def test_int4_half_add_then_truncate():
    _int4_row("int4_half_add_truncate")


def test_int4_single_fused_multiply_add():
    _int4_row("int4_fused_multiply_add")


def _bits_lsb_first(buf, n, b):
    bits = np.unpackbits(buf, bitorder="little")[: n * b].reshape(n, b)
    return (bits * (1 << np.arange(b))).sum(1)


def test_tq_encoder_divisions_and_norm_order():
    g = _golden()["tq_slot_division_and_norm_order"]
    d = 64
    k = _f32(g["key_f32_hex"]).reshape(1, 1, d)
    v = _f32(g["value_f32_hex"]).reshape(1, 1, d)
    cen = np.array(g["centroids"], np.float32)
    sb = oracle.tq_slot_bytes(d, oracle.KEY_MSE3, oracle.VAL_U4)
    cache = np.zeros((1, 1, 1, sb), np.uint8)
    oracle.tq_encode(k, v, oracle.KEY_MSE3, oracle.VAL_U4, cen, None,
                     np.zeros(1, np.int64), cache)
    s = cache[0, 0, 0]
    mb = d * 3 // 8
    np.testing.assert_array_equal(_bits_lsb_first(s[:mb], d, 3), np.array(g["key_index"]))
    assert "0x%04X" % int(s[mb:mb + 2].view(np.uint16)[0]) == g["norm_f16_hex"]
    vd = s[mb + 2:]
    np.testing.assert_array_equal(_bits_lsb_first(vd[:d // 2], d, 4), np.array(g["value_index"]))
    assert "0x%04X" % int(vd[d // 2:d // 2 + 2].view(np.uint16)[0]) == g["scale_f16_hex"]
    assert "0x%04X" % int(vd[d // 2 + 2:d // 2 + 4].view(np.uint16)[0]) == g["zero_f16_hex"]
