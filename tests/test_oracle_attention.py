"""Pins of the oracle's decode attention (fp64).

INT4 (int4_per_token_head.py, unified_attention_int4): brute force through
library routines (scipy's Hadamard matrix, scipy.special.softmax and
logsumexp, numpy matmul) in the ORIGINAL, unrotated domain -- which pins the
rotation bookkeeping (score scale / d, output / d) as well as paging and GQA;
seq_len = 1 returns the dequantized value; identical keys average the
values; num_kv_splits does not change the result (split-KV + log-sum-exp
merge of triton_turboquant_decode.py); seq_len = 0 gives zeros and -inf.

TurboQuant (triton_turboquant_decode.py, _tq_decode_stage1): FP8 keys
through torch's float8_e4m3fn decode, fp16 fields through numpy's float16,
bit fields through numpy.unpackbits; centroids against Max's 8-level
Gaussian quantizer table and the Lloyd-Max optimality conditions.
"""
import json
import os

import numpy as np
import pytest
import scipy.linalg
import scipy.special
import scipy.stats
import torch

import oracle
from quantized_paged_kv_tq_amd import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _int4_case(wid, B, hq, hk, d, bs, seq, extra_pages=3, dtype="f16"):
    w = W.custom_decode_workload(wid, B, hq, hk, d, bs, 4, seq, extra_pages, dtype)
    kb, vb = W.kv_source(w)
    kc = np.zeros((w.num_blocks, bs, hk, d // 2), np.uint8)
    vc = np.zeros_like(kc)
    ks = np.zeros((w.num_blocks, bs, hk), np.float32)
    vs = np.zeros_like(ks)
    code = {"f32": oracle.DT_F32, "f16": oracle.DT_F16, "bf16": oracle.DT_BF16}[dtype]
    s = W.rht_signs(d)
    oracle.reshape_and_cache_int4(kb, vb, code, w.slot_mapping, s, kc, vc, ks, vs)
    q = W.query(w)
    return w, q, kc, vc, ks, vs, s


def _brute_int4(w, q, kc, vc, ks, vs, s):
    d = w.d
    H = scipy.linalg.hadamard(d).astype(np.float64)
    g = w.hq // w.hk
    out = np.zeros((w.B * w.hq, d))
    lse = np.zeros(w.B * w.hq)
    for b in range(w.B):
        n = int(w.seq_lens[b])
        for h in range(w.hq):
            kvh = h // g
            K = np.zeros((n, d))
            V = np.zeros((n, d))
            for t in range(n):
                page = w.block_table[b, t // w.block_size]
                off = t % w.block_size
                kr = oracle.int4_dequant_row(kc[page, off, kvh], ks[page, off, kvh], d)
                vr = oracle.int4_dequant_row(vc[page, off, kvh], vs[page, off, kvh], d)
                # stored rows are H diag(s) x: undo with diag(s) H / d
                K[t] = (H @ kr) * s / d
                V[t] = (H @ vr) * s / d
            sc = (K @ q[b, h].astype(np.float64)) * w.sm_scale
            out[b * w.hq + h] = scipy.special.softmax(sc) @ V
            lse[b * w.hq + h] = scipy.special.logsumexp(sc)
    return out, lse


@pytest.mark.parametrize("shape", [
    (2, 4, 1, 64, 16, [37, 100]),
    (3, 8, 2, 64, 8, [1, 17, 40]),
    (2, 6, 3, 128, 16, [33, 5]),
])
def test_int4_decode_matches_unrotated_brute_force(shape):
    B, hq, hk, d, bs, seq = shape
    w, q, kc, vc, ks, vs, s = _int4_case(10 + d + B, B, hq, hk, d, bs, seq)
    ref, ref_lse = _brute_int4(w, q, kc, vc, ks, vs, s)
    for S in (0, 1, 3, 4):
        out, lse = oracle.int4_decode(q, kc, vc, ks, vs, w.block_table, w.seq_lens, s, S, w.sm_scale)
        np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse, ref_lse, rtol=1e-13, atol=1e-12)


def test_int4_split_invariance_and_rows():
    w, q, kc, vc, ks, vs, s = _int4_case(21, 2, 4, 1, 64, 16, [37, 100])
    base, blse = oracle.int4_decode(q, kc, vc, ks, vs, w.block_table, w.seq_lens, s, 0, w.sm_scale)
    for S in (1, 2, 3, 4, 8, 37, 100, 105):
        out, lse = oracle.int4_decode(q, kc, vc, ks, vs, w.block_table, w.seq_lens, s, S, w.sm_scale)
        np.testing.assert_allclose(out, base, rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse, blse, rtol=0, atol=1e-12)
    rows = np.array([5, 0, 7], np.int32)
    out, lse = oracle.int4_decode(q, kc, vc, ks, vs, w.block_table, w.seq_lens, s, 4, w.sm_scale, rows)
    np.testing.assert_allclose(out, base[rows], rtol=0, atol=1e-12)


def test_int4_seq_len_one_returns_value_and_zero_len():
    w, q, kc, vc, ks, vs, s = _int4_case(22, 2, 4, 2, 64, 16, [1, 3])
    seq = np.array([1, 0], np.int32)
    out, lse = oracle.int4_decode(q, kc, vc, ks, vs, w.block_table, seq, s, 4, w.sm_scale)
    H = scipy.linalg.hadamard(64).astype(np.float64)
    page = w.block_table[0, 0]
    for h in range(4):
        vr = oracle.int4_dequant_row(vc[page, 0, h // 2], vs[page, 0, h // 2], 64)
        np.testing.assert_allclose(out[h], (H @ vr) * s / 64, rtol=0, atol=1e-14)
    assert np.all(out[4:] == 0) and np.all(np.isneginf(lse[4:]))


def test_int4_identical_keys_average_values():
    w, q, kc, vc, ks, vs, s = _int4_case(23, 1, 2, 1, 64, 16, [20])
    page0 = w.block_table[0, 0]
    for t in range(20):  # copy token 0's key into every token
        p, o = w.block_table[0, t // 16], t % 16
        kc[p, o] = kc[page0, 0]
        ks[p, o] = ks[page0, 0]
    out, _ = oracle.int4_decode(q, kc, vc, ks, vs, w.block_table, w.seq_lens, s, 3, w.sm_scale)
    H = scipy.linalg.hadamard(64).astype(np.float64)
    vals = [(H @ oracle.int4_dequant_row(vc[w.block_table[0, t // 16], t % 16, 0],
                                         vs[w.block_table[0, t // 16], t % 16, 0], 64)) * s / 64
            for t in range(20)]
    np.testing.assert_allclose(out[0], np.mean(vals, 0), rtol=0, atol=1e-13)
    np.testing.assert_allclose(out[1], np.mean(vals, 0), rtol=0, atol=1e-13)


# ------------------------------------------------------------------ TurboQuant
def test_lloyd_max_textbook_and_optimality():
    g = json.load(open(os.path.join(GOLDEN, "lloyd_max_gaussian.json")))
    c = oracle.lloyd_max_gaussian(8)
    np.testing.assert_allclose(c[4:], g["levels8_positive"], atol=1e-4)
    np.testing.assert_allclose(c[:4], -np.array(g["levels8_positive"])[::-1], atol=1e-4)
    for L in (4, 8, 16):
        c = oracle.lloyd_max_gaussian(L)
        b = np.concatenate([[-np.inf], (c[1:] + c[:-1]) / 2, [np.inf]])
        mass = scipy.stats.norm.cdf(b[1:]) - scipy.stats.norm.cdf(b[:-1])
        mean = (scipy.stats.norm.pdf(b[:-1]) - scipy.stats.norm.pdf(b[1:])) / mass
        np.testing.assert_allclose(c, mean, atol=1e-12)


def test_tq_slot_sizes():
    assert oracle.tq_slot_bytes(128, oracle.KEY_FP8, oracle.VAL_U4) == 208
    assert oracle.tq_slot_bytes(128, oracle.KEY_MSE3, oracle.VAL_U3) == 112
    assert oracle.tq_slot_bytes(128, oracle.KEY_MSE4, oracle.VAL_U4) == 144
    assert oracle.tq_slot_bytes(64, oracle.KEY_FP8, oracle.VAL_U3) == 96
    # FP8 values: D E4M3 codes, no scale or zero
    assert oracle.tq_slot_bytes(128, oracle.KEY_FP8, oracle.VAL_FP8) == 256
    assert oracle.tq_slot_bytes(128, oracle.KEY_MSE3, oracle.VAL_FP8) == 192   # 50 + 128
    assert oracle.tq_slot_bytes(256, oracle.KEY_MSE4, oracle.VAL_FP8) == 400   # 130 + 256
    assert oracle.tq_slot_bytes(256, oracle.KEY_MSE3, oracle.VAL_U3) == 208    # 98 + 96 + 4
    assert oracle.tq_slot_bytes(128, oracle.KEY_FP8, 4) == -1


def _tq_case(key_fmt, val_fmt, wid=30, B=2, hq=4, hk=2, d=128, bs=16, seq=(40, 19)):
    w = W.custom_decode_workload(wid, B, hq, hk, d, bs, 4, list(seq), 3, "bf16")
    kb, vb = W.kv_source(w)
    k = W.bits_to_f32(kb, "bf16")
    v = W.bits_to_f32(vb, "bf16")
    sb = oracle.tq_slot_bytes(d, key_fmt, val_fmt)
    cache = np.zeros((w.num_blocks, bs, hk, sb), np.uint8)
    kbits = {oracle.KEY_FP8: 8, oracle.KEY_MSE3: 3, oracle.KEY_MSE4: 4}[key_fmt]
    cen = None if key_fmt == oracle.KEY_FP8 else \
        (oracle.lloyd_max_gaussian(1 << kbits) / np.sqrt(d)).astype(np.float32)
    oracle.tq_encode(k, v, key_fmt, val_fmt, cen, None, w.slot_mapping, cache)
    q = W.query(w, bf16_valued=True)
    return w, q, cache, cen, k, v


def _tq_fields(cache, key_fmt, val_fmt, d, cen):
    """Decode one slot array [.., sb] with numpy/torch library routines."""
    kb = {oracle.KEY_FP8: 8, oracle.KEY_MSE3: 3, oracle.KEY_MSE4: 4}[key_fmt]
    vb = {oracle.VAL_U3: 3, oracle.VAL_U4: 4, oracle.VAL_FP8: 8}[val_fmt]
    if key_fmt == oracle.KEY_FP8:
        kps = d
        kv = torch.from_numpy(cache[..., :d].copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
        norm = None
    else:
        mb = (d * kb + 7) // 8
        kps = mb + 2
        bits = np.unpackbits(cache[..., :mb], axis=-1, bitorder="little")
        idx = (bits.reshape(*bits.shape[:-1], d, kb) * (1 << np.arange(kb))).sum(-1)
        kv = cen.astype(np.float64)[idx]
        norm = cache[..., mb:mb + 2].copy().view(np.float16)[..., 0].astype(np.float64)
    vdb = (d * vb + 7) // 8
    if val_fmt == oracle.VAL_FP8:
        vals = torch.from_numpy(cache[..., kps:kps + d].copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
        return kv, norm, vals
    bits = np.unpackbits(cache[..., kps:kps + vdb], axis=-1, bitorder="little")
    vidx = (bits.reshape(*bits.shape[:-1], d, vb) * (1 << np.arange(vb))).sum(-1)
    f16 = cache[..., kps + vdb:kps + vdb + 4].copy().view(np.float16).astype(np.float64)
    vals = vidx * f16[..., 0:1] + f16[..., 1:2]
    return kv, norm, vals


@pytest.mark.parametrize("fmt", [(oracle.KEY_FP8, oracle.VAL_U4), (oracle.KEY_MSE3, oracle.VAL_U3),
                                 (oracle.KEY_MSE4, oracle.VAL_U4), (oracle.KEY_FP8, oracle.VAL_U3),
                                 (oracle.KEY_FP8, oracle.VAL_FP8), (oracle.KEY_MSE3, oracle.VAL_FP8)])
@pytest.mark.parametrize("norm_correction", [0, 1])
@pytest.mark.parametrize("d", [128, 256])
def test_tq_decode_matches_library_brute_force(fmt, norm_correction, d):
    key_fmt, val_fmt = fmt
    if key_fmt == oracle.KEY_FP8 and norm_correction:
        pytest.skip("norm correction applies to centroid keys only")
    w, q, cache, cen, k, v = _tq_case(key_fmt, val_fmt, d=d)
    d = w.d
    H = scipy.linalg.hadamard(d).astype(np.float64) / np.sqrt(d)
    kv, norm, vals = _tq_fields(cache, key_fmt, val_fmt, d, cen)
    g = w.hq // w.hk
    for S in (0, 1, 4, 7):
        out, lse = oracle.tq_decode(q, cache, w.block_table, w.seq_lens, cen, None, key_fmt,
                                    val_fmt, norm_correction, S, w.sm_scale)
        for b in range(w.B):
            n = int(w.seq_lens[b])
            t = np.arange(n)
            pages = w.block_table[b, t // w.block_size]
            offs = t % w.block_size
            for h in range(w.hq):
                kvh = h // g
                Kd = kv[pages, offs, kvh]
                Vd = vals[pages, offs, kvh]
                qq = q[b, h].astype(np.float64)
                if key_fmt == oracle.KEY_FP8:
                    sc = Kd @ qq
                else:
                    if norm_correction:
                        Kd = Kd / np.sqrt((Kd ** 2).sum(1, keepdims=True) + 1e-16)
                    sc = norm[pages, offs, kvh] * (Kd @ (H @ qq))
                sc = sc * w.sm_scale
                np.testing.assert_allclose(out[b * w.hq + h], scipy.special.softmax(sc) @ Vd,
                                           rtol=0, atol=1e-12)
                np.testing.assert_allclose(lse[b * w.hq + h], scipy.special.logsumexp(sc), rtol=1e-13)


def test_tq_encoder_round_trip_quality():
    """Encoded fields approximate the source: FP8 keys within half an e4m3
    step, uniform values within scale/2, centroid keys reconstruct the key
    direction (cosine close to 1 for 3 bits per coordinate)."""
    for key_fmt, val_fmt in ((oracle.KEY_FP8, oracle.VAL_U4), (oracle.KEY_MSE3, oracle.VAL_U3)):
        w, q, cache, cen, k, v = _tq_case(key_fmt, val_fmt, wid=31)
        kv, norm, vals = _tq_fields(cache, key_fmt, val_fmt, w.d, cen)
        H = scipy.linalg.hadamard(w.d).astype(np.float64) / np.sqrt(w.d)
        for t in range(w.total_tokens):
            p, o = divmod(int(w.slot_mapping[t]), w.block_size)
            for h in range(w.hk):
                vb = 3 if val_fmt == oracle.VAL_U3 else 4
                span = (v[t, h].max() - v[t, h].min()) / ((1 << vb) - 1)
                assert np.abs(vals[p, o, h] - v[t, h]).max() <= span * 0.51 + 1e-2
                if key_fmt == oracle.KEY_FP8:
                    assert np.all(np.abs(kv[p, o, h] - k[t, h]) <= np.abs(k[t, h]) * 2 ** -4 + 2 ** -10)
                else:
                    rec = norm[p, o, h] * (H.T @ kv[p, o, h])
                    cos = rec @ k[t, h] / (np.linalg.norm(rec) * np.linalg.norm(k[t, h]))
                    assert cos > 0.95
                    assert abs(norm[p, o, h] - np.linalg.norm(k[t, h])) <= 1e-3 * np.linalg.norm(k[t, h])


@pytest.mark.parametrize("key_fmt,bits", [(oracle.KEY_MSE3, 3), (oracle.KEY_MSE4, 4)])
@pytest.mark.parametrize("d", [64, 128])
def test_tq_centroid_encoder_fp32_agrees_with_fp64(key_fmt, bits, d):
    """The fp32 centroid encoder picks the fp64 nearest centroid of
    u = H diag(s) k / (sqrt(d) ||k||) wherever u is not within 1e-5 of a
    decision boundary, and stores ||k|| rounded to fp16 (within one fp16 ulp
    of the fp64 norm's rounding). Special rows: a zero key (norm 0, every
    index the centroid nearest 0) and a one-hot key (u = +-1/sqrt(d))."""
    rng = np.random.default_rng(50 + d + bits)
    hk, T = 2, 300
    k = rng.standard_normal((T, hk, d)).astype(np.float32)
    k[:, :, :4] *= 10.0
    k[5, 0] = 0.0
    k[6, 1] = 0.0
    k[6, 1, 3] = -2.5
    v = rng.standard_normal((T, hk, d)).astype(np.float32)
    cen = (oracle.lloyd_max_gaussian(1 << bits) / np.sqrt(d)).astype(np.float32)
    H = scipy.linalg.hadamard(d).astype(np.float64)
    mids = (cen[1:].astype(np.float64) + cen[:-1]) / 2
    for rs in (None, W.rht_signs(d, round_idx=2)):
        sb = oracle.tq_slot_bytes(d, key_fmt, oracle.VAL_U4)
        cache = np.zeros((T, 1, hk, sb), np.uint8)
        oracle.tq_encode(k, v, key_fmt, oracle.VAL_U4, cen, rs, np.arange(T, dtype=np.int64), cache)
        mb = (d * bits + 7) // 8
        got = np.unpackbits(cache[:, 0, :, :mb], axis=-1, bitorder="little")
        got = (got.reshape(T, hk, d, bits) * (1 << np.arange(bits))).sum(-1)
        n16 = cache[:, 0, :, mb:mb + 2].copy().view(np.float16)[..., 0]
        k64 = k.astype(np.float64) * (1.0 if rs is None else rs.astype(np.float64))
        nrm = np.linalg.norm(k.astype(np.float64), axis=-1)
        u = (k64 @ H.T) / np.sqrt(d) / np.where(nrm > 0, nrm, 1.0)[..., None]
        u[nrm == 0] = 0.0
        ref = np.abs(u[..., None] - cen.astype(np.float64)).argmin(-1)
        far = np.abs(u[..., None] - mids).min(-1) > 1e-5
        far[5, 0] = far[6, 1] = False  # the special rows are checked below
        assert far.mean() > 0.99
        assert np.array_equal(got[far], ref[far])
        assert np.array_equal(got[5, 0], np.full(d, np.abs(cen).argmin()))
        assert n16[5, 0] == 0
        # one-hot row: |u| = 1/sqrt(d) everywhere, sign = sign(k) * s_3 * H[:, 3]
        s3 = 1.0 if rs is None else float(rs[3])
        sign = -s3 * H[:, 3]
        one = np.where(sign > 0, np.abs(cen - 1 / np.sqrt(d)).argmin(), np.abs(cen + 1 / np.sqrt(d)).argmin())
        assert np.array_equal(got[6, 1], one)
        assert float(n16[6, 1]) == 2.5
        want16 = nrm.astype(np.float16)
        ulp = np.spacing(np.abs(want16).astype(np.float16)).astype(np.float64)
        assert np.all(np.abs(n16.astype(np.float64) - want16.astype(np.float64)) <= ulp)
        assert (n16 == want16).mean() > 0.99


@pytest.mark.parametrize("d", [64, 128, 256])
def test_tq_fp8_value_bytes_are_library_e4m3(d):
    """FP8 values (value bits 8): the D bytes after the key region are
    torch's float8_e4m3fn codes of clamp(v, +-448), the rest of the slot is
    zero (no scale or zero point)."""
    rng = np.random.default_rng(40 + d)
    T, hk = 20, 2
    k = rng.standard_normal((T, hk, d)).astype(np.float32)
    v = (rng.standard_normal((T, hk, d)) * rng.choice([1e-3, 1.0, 100.0, 1e3], (T, hk, 1))).astype(np.float32)
    v[0, 0, :4] = [500.0, -600.0, 0.0, -0.0]
    sb = oracle.tq_slot_bytes(d, oracle.KEY_FP8, oracle.VAL_FP8)
    cache = np.full((2, 16, hk, sb), 0xA5, np.uint8)
    slots = np.arange(T, dtype=np.int64)
    slots[3] = -1
    oracle.tq_encode(k, v, oracle.KEY_FP8, oracle.VAL_FP8, None, None, slots, cache)
    want_v = torch.from_numpy(np.clip(v, -448, 448)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    want_k = torch.from_numpy(np.clip(k, -448, 448)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    flat = cache.reshape(32, hk, sb)
    for t in range(T):
        if t == 3:
            assert np.all(flat[t] == 0xA5)
            continue
        np.testing.assert_array_equal(flat[t, :, :d], want_k[t])
        np.testing.assert_array_equal(flat[t, :, d:2 * d], want_v[t])
        assert np.all(flat[t, :, 2 * d:] == 0)
