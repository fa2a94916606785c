"""GPU parity of the cache writers against the CPU oracle (bit-exact):
tq_reshape_and_cache_int4 and fwht128_quant_fp8, through the C ABI."""
import os

import numpy as np
import pytest
import torch

import oracle
from quantized_paged_kv_tq_amd import workloads as W

from gpu_cases import DEV, DT_CODE, src_to_dev, to_dev

pytestmark = pytest.mark.gpu


def _write_both(kb, vb, dtype, slots, nb, bs, hk, d, canary=True):
    import quantized_paged_kv_tq_amd as tq
    s = W.rht_signs(d)
    shape = (nb, bs, hk, d // 2)
    fill = (0xA5, 0x5A, 7.0, 9.0) if canary else (0, 0, 0.0, 0.0)
    kc_o = np.full(shape, fill[0], np.uint8)
    vc_o = np.full(shape, fill[1], np.uint8)
    ks_o = np.full(shape[:3], fill[2], np.float32)
    vs_o = np.full(shape[:3], fill[3], np.float32)
    kc, vc, ks, vs = (to_dev(a) for a in (kc_o, vc_o, ks_o, vs_o))
    oracle.reshape_and_cache_int4(kb, vb, DT_CODE[dtype], slots, s, kc_o, vc_o, ks_o, vs_o)
    tq.tq_reshape_and_cache_int4(src_to_dev(kb, dtype), src_to_dev(vb, dtype), kc, vc,
                                 to_dev(slots), k_scale_cache=ks, v_scale_cache=vs,
                                 rht_signs=to_dev(s))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(kc.cpu().numpy(), kc_o)
    np.testing.assert_array_equal(vc.cpu().numpy(), vc_o)
    np.testing.assert_array_equal(ks.cpu().numpy().view(np.uint32), ks_o.view(np.uint32))
    np.testing.assert_array_equal(vs.cpu().numpy().view(np.uint32), vs_o.view(np.uint32))


def test_write_tiny_f16_d64():
    w = W.decode_workload("tiny_int4")
    kb, vb = W.kv_source(w)
    _write_both(kb, vb, "f16", w.slot_mapping, w.num_blocks, w.block_size, w.hk, w.d)


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("d,hk,T", [(128, 8, 300), (64, 3, 257), (128, 1, 33), (64, 5, 1)])
def test_write_dtypes_shapes_and_skips(dtype, d, hk, T):
    wl = W.write_workload(num_tokens=T, hk=hk, d=d, block_size=16, skip_frac=0.1, dtype=dtype,
                          wid=50 + d + hk)
    _write_both(wl["key"], wl["value"], dtype, wl["slot_mapping"], wl["num_blocks"], 16, hk, d)


def test_write_scaled_and_outlier_rows():
    # large and tiny magnitudes, constant rows and single spikes
    rng = np.random.default_rng(9)
    T, hk, d = 64, 2, 128
    k = rng.standard_normal((T, hk, d)).astype(np.float32)
    k[0] = 0.0
    k[1] = 3.0
    k[2] *= 1e-6
    k[3] *= 1e4
    k[4, :, 7] = 500.0
    # rows whose rotated values are one-signed (every code above 15 before
    # the clamp, or below 0): the source is the inverse rotation of a
    # chosen row, x = signs * H y / d (H the Sylvester Hadamard matrix)
    sg = W.rht_signs(d).astype(np.float64)
    h = np.array([[1.0]])
    while h.shape[0] < d:
        h = np.block([[h, h], [h, -h]])
    for r, y in ((5, 5.0 + 0.1 * rng.standard_normal(d)),
                 (6, -5.0 + 0.1 * rng.standard_normal(d)),
                 (7, np.full(d, 2.5)),
                 (8, 1e3 + rng.standard_normal(d)),
                 (9, np.where(np.arange(d) % 3 == 0, 7.0, 0.0) + 0.01 * rng.standard_normal(d))):
        k[r] = (sg * (h @ y) / d).astype(np.float32)
    v = np.flip(k, 0).copy()
    slots = np.arange(T, dtype=np.int64)[::-1].copy()
    for dtype in ("bf16", "f16", "f32"):
        kb, vb = W.to_bits(k, dtype), W.to_bits(v, dtype)
        _write_both(kb, vb, dtype, slots, 4, 16, hk, d)


def test_write_out_of_range_slots_are_skipped():
    wl = W.write_workload(num_tokens=40, hk=2, d=64, block_size=8, skip_frac=0.0, dtype="bf16", wid=58)
    slots = wl["slot_mapping"].copy()
    slots[3] = 40 * 1000  # beyond the cache: must not be written
    slots[5] = -7
    _write_both(wl["key"], wl["value"], "bf16", slots, wl["num_blocks"], 8, 2, 64)


def test_write_full_size_65536x8x128_bf16():
    wl = W.write_workload()
    _write_both(wl["key"], wl["value"], "bf16", wl["slot_mapping"], wl["num_blocks"], 16, 8, 128,
                canary=False)


def _fwht_both(bits):
    import quantized_paged_kv_tq_amd as tq
    y_o, s_o = oracle.fwht128_quant_fp8(bits)
    y, s = tq.fwht128_quant_fp8(to_dev(bits.view(np.int16), torch.bfloat16))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(y.view(torch.uint8).cpu().numpy(), y_o)
    np.testing.assert_array_equal(s.cpu().numpy().ravel().view(np.uint32), s_o.view(np.uint32))


@pytest.mark.parametrize("rows", [1, 15, 17, 1000])
def test_fwht_ragged_rows(rows):
    _fwht_both(W.fwht_rows(rows=rows, wid=60 + rows))


def test_fwht_special_rows():
    rng = np.random.default_rng(12)
    x = rng.standard_normal((64, 128)).astype(np.float32)
    x[0] = 0.0                       # absmax floor
    x[1] *= 1e-8                     # tiny row: subnormal FP8 codes
    x[2] *= 3e4                      # large row
    x[3] = 0.0
    x[3, 0] = 1.75 * 2 ** 3 * np.sqrt(128)   # transform is constant: exact powers
    x[4, :] = rng.integers(-3, 4, 128)       # integer row
    x[5] = x[4] * 2.0 ** -20
    _fwht_both(W.to_bits(x, "bf16"))


def test_fwht_full_size_1m_rows():
    _fwht_both(W.fwht_rows())


def test_fwht_empty():
    import quantized_paged_kv_tq_amd as tq
    y, s = tq.fwht128_quant_fp8(torch.empty(0, 128, dtype=torch.bfloat16, device=DEV))
    assert y.shape == (0, 128) and s.shape == (0, 1)


# ---------------------------------------------------------------------------
# TurboQuant combined-slot writer (tq_encode_and_cache)

TQ_FMTS = [(oracle.KEY_FP8, oracle.VAL_U4), (oracle.KEY_FP8, oracle.VAL_U3),
           (oracle.KEY_MSE3, oracle.VAL_U3), (oracle.KEY_MSE3, oracle.VAL_U4),
           (oracle.KEY_MSE4, oracle.VAL_U4), (oracle.KEY_MSE4, oracle.VAL_U3)]


def _centroids(key_fmt, d):
    if key_fmt == oracle.KEY_FP8:
        return None
    bits = 3 if key_fmt == oracle.KEY_MSE3 else 4
    return (oracle.lloyd_max_gaussian(1 << bits) / np.sqrt(d)).astype(np.float32)


def _encode_both(kb, vb, dtype, slots, nb, bs, hk, d, key_fmt, val_fmt, rot_signs=None,
                 extra_pad=0, cen=None):
    import quantized_paged_kv_tq_amd as tq
    sb = oracle.tq_slot_bytes(d, key_fmt, val_fmt) + extra_pad
    if cen is None:
        cen = _centroids(key_fmt, d)
    want = np.full((nb, bs, hk, sb), 0xA5, np.uint8)  # canary: skipped slots keep it
    got = to_dev(want)
    k32 = W.bits_to_f32(kb, dtype)
    v32 = W.bits_to_f32(vb, dtype)
    oracle.tq_encode(k32, v32, key_fmt, val_fmt, cen, rot_signs, slots, want)
    tq.tq_encode_and_cache(src_to_dev(kb, dtype), src_to_dev(vb, dtype), got, to_dev(slots),
                           key_fmt=key_fmt, val_fmt=val_fmt,
                           centroids=None if cen is None else to_dev(cen),
                           rot_signs=None if rot_signs is None else to_dev(rot_signs))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(got.cpu().numpy(), want)


@pytest.mark.parametrize("fmt", TQ_FMTS, ids=[str(f) for f in TQ_FMTS])
@pytest.mark.parametrize("d,hk,T", [(128, 4, 300), (64, 3, 257)])
def test_tq_encode_formats_bit_exact(fmt, d, hk, T):
    wl = W.write_workload(num_tokens=T, hk=hk, d=d, block_size=16, skip_frac=0.1, dtype="bf16",
                          wid=60 + d + hk + 7 * fmt[0] + fmt[1])
    _encode_both(wl["key"], wl["value"], "bf16", wl["slot_mapping"], wl["num_blocks"], 16, hk, d,
                 *fmt)


@pytest.mark.parametrize("dtype", ["f16", "f32"])
@pytest.mark.parametrize("key_fmt", [oracle.KEY_FP8, oracle.KEY_MSE4])
def test_tq_encode_dtypes_rot_signs_and_padding(dtype, key_fmt):
    d, hk, T = 128, 2, 129
    wl = W.write_workload(num_tokens=T, hk=hk, d=d, block_size=16, skip_frac=0.05, dtype=dtype,
                          wid=70 + key_fmt)
    rs = None if key_fmt == oracle.KEY_FP8 else W.rht_signs(d, round_idx=3)
    _encode_both(wl["key"], wl["value"], dtype, wl["slot_mapping"], wl["num_blocks"], 16, hk, d,
                 key_fmt, oracle.VAL_U4, rot_signs=rs, extra_pad=32)


@pytest.mark.parametrize("fmt", TQ_FMTS[:3], ids=[str(f) for f in TQ_FMTS[:3]])
def test_tq_encode_special_rows(fmt):
    """Zero and constant rows (norm 0, value range 0), FP8 saturation beyond
    +-448, tiny and huge magnitudes, single spikes."""
    rng = np.random.default_rng(11)
    T, hk, d = 64, 2, 128
    k = rng.standard_normal((T, hk, d)).astype(np.float32)
    k[0] = 0.0
    k[1] = 3.0
    k[2] *= 1e-6
    k[3] *= 1e3
    k[4, :, 7] = 500.0
    k[5, :, 9] = -1e5
    v = np.flip(k, 0).copy()
    slots = np.arange(T, dtype=np.int64)[::-1].copy()
    slots[10] = -1
    slots[11] = 10 ** 6  # beyond the cache: skipped
    _encode_both(k, v, "f32", slots, 4, 16, hk, d, *fmt)


def _table_cases(d):
    """Centroid tables for the nearest-centroid search: the writer takes
    decision thresholds for sorted tables with gaps >= 2^-20 inside [-1, 1]
    and scans every centroid otherwise."""
    lm = (oracle.lloyd_max_gaussian(8) / np.sqrt(d)).astype(np.float32)
    rs = np.float32(1.0 / np.sqrt(d))
    # c[4] and c[5] straddle rs = u of a one-hot key exactly: a tie, which
    # goes to the lower index
    tie = lm.copy()
    tie[4], tie[5] = rs - np.float32(0.03125), rs + np.float32(0.03125)
    tie[6], tie[7] = np.float32(0.25), np.float32(0.5)
    near = lm.copy()
    near[5] = np.nextafter(near[4], np.float32(1))  # gap of one ulp: scanned
    big = lm.copy()
    big[7] = np.float32(1.5)  # beyond [-1, 1]: scanned
    perm = lm[[3, 0, 7, 1, 6, 2, 5, 4]].copy()  # unsorted: scanned
    return {"lloyd_max": lm, "tie": tie, "near_duplicate": near, "outside_unit": big,
            "unsorted": perm}


@pytest.mark.parametrize("case", ["lloyd_max", "tie", "near_duplicate", "outside_unit", "unsorted"])
def test_tq_encode_centroid_tables(case):
    """Threshold and scan forms of the nearest-centroid search against the
    oracle's scan: random rows, one-hot rows (every coordinate of u is
    +-1/sqrt(D) exactly) and rows of one repeated value."""
    d, hk, T = 128, 2, 96
    rng = np.random.default_rng(21)
    k = rng.standard_normal((T, hk, d)).astype(np.float32)
    for t in range(0, 32):
        k[t] = 0.0
        k[t, :, t % d] = np.float32(2.0 ** (t % 3 - 1))  # u = +-1/sqrt(D) exactly
    k[32:40] = np.float32(0.75)
    v = rng.standard_normal((T, hk, d)).astype(np.float32)
    slots = rng.permutation(T).astype(np.int64)
    cen = _table_cases(d)[case]
    _encode_both(k, v, "f32", slots, 6, 16, hk, d, oracle.KEY_MSE3, oracle.VAL_U3, cen=cen)



N2_FMTS = [(oracle.KEY_FP8, oracle.VAL_FP8), (oracle.KEY_MSE3, oracle.VAL_FP8),
           (oracle.KEY_MSE4, oracle.VAL_FP8)]


@pytest.mark.parametrize("fmt", N2_FMTS, ids=[str(f) for f in N2_FMTS])
@pytest.mark.parametrize("d,hk,T", [(128, 4, 300), (64, 3, 257), (256, 2, 129)])
def test_tq_encode_fp8_values_bit_exact(fmt, d, hk, T):
    """FP8 values (D E4M3 codes after the key region, no scale or zero)."""
    wl = W.write_workload(num_tokens=T, hk=hk, d=d, block_size=16, skip_frac=0.1, dtype="bf16",
                          wid=80 + d + hk + 7 * fmt[0])
    _encode_both(wl["key"], wl["value"], "bf16", wl["slot_mapping"], wl["num_blocks"], 16, hk, d,
                 *fmt)


@pytest.mark.parametrize("fmt", TQ_FMTS, ids=[str(f) for f in TQ_FMTS])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_tq_encode_head_dim_256(fmt, dtype):
    """D = 256: sixteen lanes per row; rot signs on centroid keys."""
    d, hk, T = 256, 2, 133
    wl = W.write_workload(num_tokens=T, hk=hk, d=d, block_size=16, skip_frac=0.05, dtype=dtype,
                          wid=90 + 7 * fmt[0] + fmt[1])
    rs = None if fmt[0] == oracle.KEY_FP8 else W.rht_signs(d, round_idx=5)
    _encode_both(wl["key"], wl["value"], dtype, wl["slot_mapping"], wl["num_blocks"], 16, hk, d,
                 *fmt, rot_signs=rs)


def test_tq_encode_rounding_boundaries():
    """Rows that sit on the encoder's rounding boundaries: the hand-derived
    slot of golden/rounding_readings.json (a key coordinate 2^-25 above a
    decision threshold, a value quotient 4.3e-7 above a half-integer), keys
    whose rotated coordinates cluster at a threshold (four nearly equal
    entries: u = 1/4 + O(1e-4)), and value rows whose quotients lie within a
    few ulps of half-integers (both sides of the rounding check)."""
    import json
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden",
                                    "rounding_readings.json")))["tq_slot_division_and_norm_order"]
    d, hk = 64, 1
    rng = np.random.default_rng(77)
    T = 2048
    k = np.zeros((T, hk, d), np.float32)
    k[:, 0, :4] = (1 + rng.uniform(-1e-3, 1e-3, (T, 4))).astype(np.float32)
    k[0, 0] = np.array([int(h, 16) for h in g["key_f32_hex"]], np.uint32).view(np.float32)
    v = np.empty((T, hk, d), np.float32)
    for t in range(T):
        s16 = np.float16(rng.uniform(0.05, 3.0))
        z16 = np.float16(rng.uniform(-4.0, 0.0))
        s, z = np.float32(s16), np.float32(z16)
        row = np.empty(d, np.float32)
        row[0], row[1] = z, np.float32(z + np.float32(15) * s)
        kk = rng.integers(0, 15, d - 2).astype(np.float32)
        base = (z + (kk + np.float32(0.5)) * s).astype(np.float32)
        steps = rng.integers(-3, 4, d - 2)
        for i in range(d - 2):
            x = base[i]
            for _ in range(abs(int(steps[i]))):
                x = np.nextafter(x, np.float32(np.inf) if steps[i] > 0 else np.float32(-np.inf))
            row[2 + i] = x
        v[t, 0] = row
    v[0, 0] = np.array([int(h, 16) for h in g["value_f32_hex"]], np.uint32).view(np.float32)
    slots = rng.permutation(T).astype(np.int64)
    step = np.array(g["centroids"], np.float32)
    lm = (oracle.lloyd_max_gaussian(8) / np.sqrt(d)).astype(np.float32)
    for cen in (step, lm):
        _encode_both(k, v, "f32", slots, T // 16, 16, hk, d, oracle.KEY_MSE3, oracle.VAL_U4, cen=cen)
    _encode_both(k, v, "f32", slots, T // 16, 16, hk, d, oracle.KEY_MSE3, oracle.VAL_U3, cen=step)
