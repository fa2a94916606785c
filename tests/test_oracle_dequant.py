"""Pins of the oracle's bulk TurboQuant dequant (triton_turboquant_decode.py,
_tq_full_dequant_kv): every (b, kv head, position) slot rebuilt as fp16 K
and V rows.

- FP8 keys: torch's float8_e4m3fn -> float16 cast, bit for bit.
- Centroid keys and uniform values: an independent NumPy unpacking of the
  LSB-first index stream (np.unpackbits) and IEEE fp32 products cast to
  fp16, bit for bit (the value's fma is exact in fp64 here: a 4-bit index
  times an fp16 scale plus an fp16 zero needs fewer than 53 bits).
- Norm correction: within one fp16 step of an fp64 computation.
- FP8 values and pages outside the pool give zeros.
- Consistency with the decode oracle: attention over the dequantized rows
  matches tq_decode within the fp16 rounding of K and V.
"""
import numpy as np
import pytest
import torch

import oracle
from quantized_paged_kv_tq_amd import workloads as W


def _f16(bits):
    return np.ascontiguousarray(bits, np.uint16).view(np.float16).astype(np.float64)


def _setup(key_fmt, val_fmt, d=128, wid=120):
    w = W.custom_decode_workload(wid, 2, 8, 2, d, 16, 1, [37, 70], extra_pages=2)
    sb = oracle.tq_slot_bytes(d, key_fmt, val_fmt)
    cache = W.random_tq_cache(w, key_fmt, val_fmt, sb)
    cen = None
    if key_fmt != oracle.KEY_FP8:
        levels = 8 if key_fmt == oracle.KEY_MSE3 else 16
        cen = (oracle.lloyd_max_gaussian(levels) / np.sqrt(d)).astype(np.float32)
    return w, cache, cen


def _slots(w, cache):
    """[B, Hk, max_seq, slot] bytes gathered through the block table."""
    ms = int(w.seq_lens.max())
    t = np.arange(ms)
    out = np.zeros((w.B, w.hk, ms, cache.shape[-1]), np.uint8)
    for b in range(w.B):
        pg = w.block_table[b, t // w.block_size]
        out[b] = cache[pg, t % w.block_size].transpose(1, 0, 2)
    return out


def _indices(bytes_, d, bits):
    stream = np.unpackbits(bytes_, axis=-1, bitorder="little")[..., :d * bits]
    stream = stream.reshape(bytes_.shape[:-1] + (d, bits)).astype(np.int64)
    return (stream << np.arange(bits)).sum(-1)


def test_fp8_keys_and_u4_values_bit_exact():
    w, cache, _ = _setup(oracle.KEY_FP8, oracle.VAL_U4)
    ms = int(w.seq_lens.max())
    k, v = oracle.tq_full_dequant(cache, w.block_table, w.d, oracle.KEY_FP8, oracle.VAL_U4, ms)
    s = _slots(w, cache)
    want_k = torch.from_numpy(s[..., :w.d].copy()).view(torch.float8_e4m3fn).to(torch.float16)
    np.testing.assert_array_equal(k, want_k.view(torch.int16).numpy().view(np.uint16))
    idx = _indices(s[..., w.d:w.d + w.d // 2], w.d, 4)
    sc = _f16(s[..., w.d + 64:w.d + 66].copy().view(np.uint16))
    zr = _f16(s[..., w.d + 66:w.d + 68].copy().view(np.uint16))
    exact = idx * sc + zr
    want_v = exact.astype(np.float32).astype(np.float16).view(np.uint16)
    np.testing.assert_array_equal(v, want_v)


@pytest.mark.parametrize("key_fmt,val_fmt,kb,vb", [(2, 1, 3, 3), (3, 2, 4, 4), (2, 2, 3, 4)])
def test_centroid_keys_and_values_bit_exact(key_fmt, val_fmt, kb, vb):
    w, cache, cen = _setup(key_fmt, val_fmt, d=64, wid=121 + key_fmt)
    ms = int(w.seq_lens.max())
    k, v = oracle.tq_full_dequant(cache, w.block_table, w.d, key_fmt, val_fmt, ms, centroids=cen)
    s = _slots(w, cache)
    mse = w.d * kb // 8
    kidx = _indices(s[..., :mse], w.d, kb)
    nrm = s[..., mse:mse + 2].copy().view(np.float16).astype(np.float32)
    want_k = (nrm * cen[kidx]).astype(np.float32).astype(np.float16).view(np.uint16)
    np.testing.assert_array_equal(k, want_k)
    vo, vdb = mse + 2, w.d * vb // 8
    vidx = _indices(s[..., vo:vo + vdb], w.d, vb)
    sc = _f16(s[..., vo + vdb:vo + vdb + 2].copy().view(np.uint16))
    zr = _f16(s[..., vo + vdb + 2:vo + vdb + 4].copy().view(np.uint16))
    want_v = (vidx * sc + zr).astype(np.float32).astype(np.float16).view(np.uint16)
    np.testing.assert_array_equal(v, want_v)


def test_norm_correction_within_one_fp16_step():
    w, cache, cen = _setup(oracle.KEY_MSE3, oracle.VAL_U3, d=128, wid=125)
    ms = int(w.seq_lens.max())
    k, _ = oracle.tq_full_dequant(cache, w.block_table, w.d, 2, 1, ms, centroids=cen,
                                  norm_correction=True)
    s = _slots(w, cache)
    c = cen[_indices(s[..., :48], w.d, 3)].astype(np.float64)
    c = c / np.sqrt((c * c).sum(-1, keepdims=True) + 1e-16)
    want = s[..., 48:50].copy().view(np.float16).astype(np.float64) * c
    got = _f16(k)
    step = np.abs(np.spacing(want.astype(np.float16))).astype(np.float64)
    assert np.all(np.abs(got - want) <= step)
    norms = np.linalg.norm(got, axis=-1) / s[..., 48:50].copy().view(np.float16).astype(np.float64)[..., 0]
    np.testing.assert_allclose(norms, 1.0, atol=2e-3)


def test_fp8_values_and_outside_pages_are_zero():
    w, cache, cen = _setup(oracle.KEY_MSE4, oracle.VAL_FP8, d=64, wid=126)
    ms = int(w.seq_lens.max())
    bt = w.block_table.copy()
    bt[1, 1] = w.num_blocks      # a page outside the pool
    bt[0, 0] = -3
    k, v = oracle.tq_full_dequant(cache, bt, w.d, 3, 3, ms, centroids=cen)
    assert np.all(v == 0)
    assert np.all(k[1, :, 16:32] == 0) and np.all(k[0, :, 0:16] == 0)
    assert np.any(k[1, :, 0:16] != 0)


@pytest.mark.parametrize("key_fmt,val_fmt", [(1, 2), (2, 1)])
def test_attention_over_dequantized_rows_matches_decode(key_fmt, val_fmt):
    w, cache, cen = _setup(key_fmt, val_fmt, d=128, wid=127 + key_fmt)
    ms = int(w.seq_lens.max())
    k, v = oracle.tq_full_dequant(cache, w.block_table, w.d, key_fmt, val_fmt, ms, centroids=cen)
    kf, vf = _f16(k), _f16(v)
    q = W.query(w)
    out, _ = oracle.tq_decode(q, cache, w.block_table, w.seq_lens, cen, None, key_fmt, val_fmt,
                              False, 0, w.sm_scale)
    out = out.reshape(w.B, w.hq, w.d)
    g = w.hq // w.hk
    qq = q.astype(np.float64)
    if key_fmt != 1:
        import scipy.linalg
        H = scipy.linalg.hadamard(w.d) / np.sqrt(w.d)
        qq = qq @ H.T
    for b in range(w.B):
        n = int(w.seq_lens[b])
        for h in range(w.hq):
            sc = (kf[b, h // g, :n] @ qq[b, h]) * w.sm_scale
            p = np.exp(sc - sc.max())
            o = p @ vf[b, h // g, :n] / p.sum()
            np.testing.assert_allclose(o, out[b, h], rtol=0, atol=5e-3)
