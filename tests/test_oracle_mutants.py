"""Planted mistakes: each pin must catch a plausible error in the oracle.

Every case copies oracle/tq_oracle.c, replaces one expression with a
plausible wrong one (a reading not taken, a dropped term, an index off by
one), compiles the copy with the oracle's own flags into a temporary
directory, routes the oracle through it (oracle.use_library) and runs the
pins that should notice. The case passes when at least one of them fails.
Each replaced expression must occur in the source exactly as written, so a
case cannot silently stop applying after an edit of the oracle.
"""
import os

import pytest

import oracle
import test_oracle_fwht_int4 as P_int4
import test_oracle_kpool as P_kpool
import test_oracle_prefill as P_prefill
import test_oracle_readings as P_read

SRC = os.path.join(os.path.dirname(oracle.__file__), "tq_oracle.c")


def _calls(fn, *param_sets):
    if not param_sets:
        return [lambda: fn()]
    return [lambda kw=kw: fn(**kw) for kw in param_sets]


_PREFILL_ALL = (
    _calls(P_prefill.test_brute_force_tiny,
           *[dict(window=w, softcap=c, sinks=s)
             for (w, c, s) in ((0, 0.0, False), (5, 0.0, False), (0, 7.5, False),
                               (0, 0.0, True), (9, 30.0, True))])
    + _calls(P_prefill.test_last_query_token_is_decode)
    + _calls(P_prefill.test_window_of_one_returns_own_value_row)
    + _calls(P_prefill.test_causality_and_empty_sequences)
    + _calls(P_prefill.test_sink_limits))

_KPOOL_ALL = (
    _calls(P_kpool.test_exp_is_correctly_rounded_fp32)
    + _calls(P_kpool.test_equal_weights_exact_pipeline,
             *[dict(P=p, round_scale=r) for p in (1, 2, 4, 8) for r in (True, False)])
    + _calls(P_kpool.test_dominant_slot_per_dimension,
             *[dict(P=p, round_scale=r) for p in (2, 3) for r in (True, False)])
    + _calls(P_kpool.test_indexer_page_layout_mask_and_skips))

# name -> (replacements [(old, new, count)], pins)
MUTANTS = {
    # INT4 quantizer (int4_per_token_head.py, _reshape_cache_int4_kernel)
    "int4_mul_then_add": (
        [("fmaf(x[2 * j], inv, zp)", "(x[2 * j] * inv + zp)", 1),
         ("fmaf(x[2 * j + 1], inv, zp)", "(x[2 * j + 1] * inv + zp)", 1)],
        _calls(P_read.test_int4_single_fused_multiply_add)),
    "int4_roundf": (
        [("int32_t i = (t >= 0.0f) ? trunc_sat(t + 0.5f) : trunc_sat(t - 0.5f);",
          "int32_t i = trunc_sat(roundf(t));", 1)],
        _calls(P_read.test_int4_half_add_then_truncate)),
    "int4_rint": (
        [("int32_t i = (t >= 0.0f) ? trunc_sat(t + 0.5f) : trunc_sat(t - 0.5f);",
          "int32_t i = trunc_sat(rintf(t));", 1)],
        _calls(P_read.test_int4_half_add_then_truncate)
        + _calls(P_int4.test_int4_nibble_order_and_half_away_ties)),
    "int4_scale_over_16": (
        [("float scale = (mx - mn) / 15.0f;", "float scale = (mx - mn) / 16.0f;", 1)],
        _calls(P_int4.test_int4_quantizer_nearest_grid_and_error_bound)),
    "int4_zero_point_sign": (
        [("float u = -mn / scale;", "float u = mn / scale;", 1)],
        _calls(P_int4.test_int4_quantizer_nearest_grid_and_error_bound)),
    "int4_nibbles_swapped": (
        [("packed[j] = (uint8_t)(((uint32_t)qe & 0xFu) | (((uint32_t)qo & 0xFu) << 4));",
          "packed[j] = (uint8_t)(((uint32_t)qo & 0xFu) | (((uint32_t)qe & 0xFu) << 4));", 1)],
        _calls(P_int4.test_int4_nibble_order_and_half_away_ties)),
    "fwht_stage_order_reversed": (
        [("void orc_fwht_f32(float* x, int d) {\n  for (int h = 1; h < d; h <<= 1)",
          "void orc_fwht_f32(float* x, int d) {\n  for (int h = d / 2; h >= 1; h >>= 1)", 1)],
        _calls(P_int4.test_fwht_fp32_stage_order_hand_example)),
    # TurboQuant slot encoder (readings of the absent encoder)
    "tq_value_reciprocal": (
        [("nearbyintf((v[i] - zr) / scr)", "nearbyintf((v[i] - zr) * (1.0f / scr))", 1)],
        _calls(P_read.test_tq_encoder_divisions_and_norm_order)),
    "tq_key_reciprocal": (
        [("(y[i] * r) / nrm", "y[i] * (r / nrm)", 1)],
        _calls(P_read.test_tq_encoder_divisions_and_norm_order)),
    "tq_norm_sequential": (
        [("  for (int h = 1; h < d; h <<= 1)\n    for (int i = 0; i < d; i += 2 * h) s[i] = s[i] + s[i + h];\n  return s[0];",
          "  for (int i = 1; i < d; ++i) s[0] = s[0] + s[i];\n  return s[0];", 1)],
        _calls(P_read.test_tq_encoder_divisions_and_norm_order)),
    # multi-query INT4 attention (int4_per_token_head.py, _attn_packed)
    "prefill_window_off_by_one": (
        [("lo = pos - window + 1;", "lo = pos - window;", 1)], _PREFILL_ALL),
    "prefill_causal_off_by_one": (
        [("int64_t hi = pos + 1 < seq ? pos + 1 : seq;", "int64_t hi = pos < seq ? pos : seq;", 1)],
        _PREFILL_ALL),
    "prefill_no_context_offset": (
        [("int64_t pos = seq - qlen + i;", "int64_t pos = i;", 1)], _PREFILL_ALL),
    "prefill_sink_dropped": (
        [("double l = sinks ? exp((double)sinks[h] - m) : 0.0;", "double l = 0.0;", 1)],
        _PREFILL_ALL),
    "prefill_softcap_dropped": (
        [("if (softcap > 0) st = softcap * tanh(st / softcap);", "(void)softcap;", 2)],
        _PREFILL_ALL),
    # pooled key compression (kpool_compress.py, _kpool_softmax_rotate_write_cache_kernel)
    "kpool_bias_dropped": (
        [(" + ape[s * 128 + d];", ";", 2)], _KPOOL_ALL),
    "kpool_exponent_sign": (
        [("float p = orc_exp_f32(v - m);", "float p = orc_exp_f32(m - v);", 1)], _KPOOL_ALL),
    "kpool_no_bf16_round_of_mean": (
        [("x[d] = orc_bf16_to_f32(orc_f32_to_bf16(acc / den));", "x[d] = acc / den;", 1)],
        _KPOOL_ALL),
    "kpool_wrong_entry": (
        [("memcpy(page + off * 128, q, 128);",
          "memcpy(page + ((off + 1) % block_size) * 128, q, 128);", 1)], _KPOOL_ALL),
    "kpool_libm_expf": (
        [("float p = orc_exp_f32(v - m);", "float p = expf(v - m);", 1),
         ("float orc_exp_f32(float x) {", "float orc_exp_f32(float x) {\n  return expf(x);", 1)],
        _KPOOL_ALL),
    "kpool_divide_by_448": (
        [("sc = amax * inv_448;", "sc = amax / 448.0f;", 1)], _KPOOL_ALL),
    "kpool_short_scale_store": (
        [("memcpy(page + (int64_t)block_size * 128 + off * 4, &sc, 4);",
          "memcpy(page + (int64_t)block_size * 128 + off * 4, &sc, 2);", 1)], _KPOOL_ALL),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name, tmp_path):
    reps, pins = MUTANTS[name]
    src = open(SRC).read()
    for old, new, count in reps:
        assert src.count(old) == count, (name, old)
        src = src.replace(old, new)
    path = tmp_path / "mutant.c"
    path.write_text(src)
    so = oracle.compile_source(str(path), str(tmp_path / "libmutant.so"),
                              ["-w", "-I", os.path.dirname(SRC)])
    failures = 0
    with oracle.use_library(so):
        for pin in pins:
            try:
                pin()
            except AssertionError:
                failures += 1
                break
    assert failures, "no pin noticed the planted mistake " + name
