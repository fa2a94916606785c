"""Pins of the oracle's Walsh-Hadamard transform, randomized Hadamard
rotation and INT4 per-(token, head) quantizer.

FWHT: equals scipy's Sylvester Hadamard matrix times x (a library routine),
exactly on integer inputs; H*H = n*I; Parseval. INT4: brute-force nearest
grid point, the scale/2 error bound, closed-form special cases (constant
rows, one-signed rows, exact .5 ties, nibble order) and the scale-word
round trip. The page claims pinned are from int4_per_token_head.py:
fast_hadamard_transform ("H_d x H_d = d x I"), single_rht,
_reshape_cache_int4_kernel and _attn_packed's scale-word reader.
"""
import json
import os

import numpy as np
import pytest
import scipy.linalg

import oracle
from quantized_paged_kv_tq_amd import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.mark.parametrize("n", [1, 2, 4, 8, 16, 32, 64, 128, 256])
def test_fwht_equals_sylvester_matrix_exact_on_integers(n):
    rng = np.random.default_rng(n)
    x = rng.integers(-1000, 1000, size=(20, n)).astype(np.float64)
    H = scipy.linalg.hadamard(n).astype(np.float64)
    ref = x @ H.T
    np.testing.assert_array_equal(oracle.fwht_f64(x), ref)
    np.testing.assert_array_equal(oracle.fwht_f32(x.astype(np.float32)), ref.astype(np.float32))


def test_fwht_matrix_matches_page_doubling_construction():
    # the page builds H by doubling [[H, H], [H, -H]] (_get_hadamard_matrix);
    # the golden file holds H_4 and H_8 written out by hand
    g = json.load(open(os.path.join(GOLDEN, "hadamard_small.json")))
    for key in ("H4", "H8"):
        H = np.array(g[key], np.float64)
        n = H.shape[0]
        np.testing.assert_array_equal(oracle.fwht_f64(np.eye(n)), H.T)


def test_fwht_involution_and_parseval():
    rng = np.random.default_rng(5)
    for n in (64, 128):
        x = rng.standard_normal((50, n))
        y = oracle.fwht_f64(x)
        np.testing.assert_allclose(oracle.fwht_f64(y), n * x, rtol=0, atol=1e-11)
        np.testing.assert_allclose((y ** 2).sum(1), n * (x ** 2).sum(1), rtol=1e-12)
        H = oracle.fwht_f64(np.eye(n))
        np.testing.assert_array_equal(H @ H, n * np.eye(n))


def test_rht_signs_deterministic_pm1():
    # the page draws them with torch's CPU generator seeded 0x9E3779B9
    for d in (64, 128):
        s = W.rht_signs(d)
        assert s.shape == (d,) and set(np.unique(s)) == {-1.0, 1.0}
        np.testing.assert_array_equal(s, W.rht_signs(d))


def _grid_ok(x, packed, word):
    """Brute force over the 16 grid points (q - zp) * scale'."""
    d = x.shape[0]
    bits = np.float32(word).view(np.uint32)
    zp = int(bits & 0xF)
    sc = float(np.uint32(bits & 0xFFFFFFF0).view(np.float32))
    q = np.empty(d, np.int64)
    q[0::2] = packed & 0xF
    q[1::2] = packed >> 4
    grid = (np.arange(16) - zp) * sc
    dist = np.abs(x[:, None].astype(np.float64) - grid[None, :])
    best = dist.min(1)
    chosen = dist[np.arange(d), q]
    # chosen grid point is a nearest one up to rounding of the fp32 pipeline
    return np.all(chosen <= best + 1e-6 * sc), q, zp, sc


def test_int4_quantizer_nearest_grid_and_error_bound():
    rng = np.random.default_rng(11)
    for trial in range(2000):
        d = 128 if trial % 2 else 64
        x = (rng.standard_normal(d) * rng.uniform(0.01, 100)).astype(np.float32)
        if trial % 7 == 0:
            x[rng.integers(d)] *= 30  # outlier
        packed, word = oracle.int4_quantize_row(x)
        ok, q, zp, sc = _grid_ok(x, packed, word)
        assert ok, trial
        assert 0 <= zp <= 15 and q.min() >= 0 and q.max() <= 15
        mn, mx = float(x.min()), float(x.max())
        # scale spans the row's range in 15 steps (fp32 division, 1e-6 floor)
        assert abs(15 * sc - (mx - mn)) <= 1e-5 * (mx - mn) + 15 * 2.0 ** -19 * sc
        if mn <= 0 <= mx:
            err = np.abs(x.astype(np.float64) - (q - zp) * sc)
            assert err.max() <= sc / 2 * (1 + 2.0 ** -20), trial


def test_int4_constant_rows():
    for v, want_q, want_zp in ((0.0, 0, 0), (3.0, 15, 0), (-3.0, 0, 15)):
        x = np.full(64, v, np.float32)
        packed, word = oracle.int4_quantize_row(x)
        bits = np.float32(word).view(np.uint32)
        assert bits & 0xF == want_zp
        assert np.uint32(bits & 0xFFFFFFF0) == (np.float32(1e-6).view(np.uint32) & np.uint32(0xFFFFFFF0))
        assert np.all(packed == want_q * 17)


def test_int4_nibble_order_and_half_away_ties():
    # min 0, max 15 -> scale exactly 1, zp 0, q_i = round_half_away(x_i)
    x = np.array([0, 15] + [i % 16 for i in range(2, 62)] + [2.5, 3.5], np.float32)
    packed, word = oracle.int4_quantize_row(x)
    assert np.float32(word).view(np.uint32) == np.float32(1.0).view(np.uint32)
    q = np.empty(64, np.int64)
    q[0::2] = packed & 0xF
    q[1::2] = packed >> 4
    np.testing.assert_array_equal(q[:62], x[:62].astype(np.int64))
    assert packed[0] == 0xF0  # element 0 low nibble, element 1 high nibble
    assert q[62] == 3 and q[63] == 4  # .5 rounds away from zero, not to even


def test_int4_one_signed_row_saturates():
    # all values in [1, 2]: zp clamps to 0 and values above max-min saturate
    x = np.linspace(1.0, 2.0, 64).astype(np.float32)
    packed, word = oracle.int4_quantize_row(x)
    assert np.float32(word).view(np.uint32) & 0xF == 0
    q = np.empty(64, np.int64)
    q[0::2] = packed & 0xF
    q[1::2] = packed >> 4
    assert q[-1] == 15 and q[0] == 15


def test_int4_zero_point_is_nearest_integer_of_minus_min_over_scale():
    rng = np.random.default_rng(3)
    for _ in range(500):
        x = rng.standard_normal(128).astype(np.float32)
        x -= np.float32(rng.uniform(-1, 1) * x.std())
        _, word = oracle.int4_quantize_row(x)
        zp = int(np.float32(word).view(np.uint32) & 0xF)
        sc = (float(x.max()) - float(x.min())) / 15.0
        u = -float(x.min()) / sc
        if 0.0 <= u <= 15.0:
            assert abs(zp - u) <= 0.5 + 1e-5
        else:
            assert zp == (0 if u < 0 else 15)


def test_scale_word_round_trip():
    rng = np.random.default_rng(4)
    x = rng.standard_normal(128).astype(np.float32)
    packed, word = oracle.int4_quantize_row(x)
    deq = oracle.int4_dequant_row(packed, word, 128)
    bits = np.float32(word).view(np.uint32)
    sc = float(np.uint32(bits & 0xFFFFFFF0).view(np.float32))
    zp = int(bits & 0xF)
    np.testing.assert_array_equal(deq[0::2], ((packed & 0xF).astype(np.float64) - zp) * sc)
    np.testing.assert_array_equal(deq[1::2], ((packed >> 4).astype(np.float64) - zp) * sc)


@pytest.mark.parametrize("dtype", ["f16", "bf16", "f32"])
def test_reshape_and_cache_rotation_and_layout(dtype):
    """The written row dequantizes to RHT(x) rounded to the source dtype,
    within scale/2; RHT^-1 of it returns x (scaled by d). Skipped slots
    leave canary bytes untouched."""
    rng = np.random.default_rng(6)
    T, hk, d, bs, nb = 40, 3, 64, 16, 4
    k32 = rng.standard_normal((T, hk, d)).astype(np.float32)
    v32 = rng.standard_normal((T, hk, d)).astype(np.float32)
    kb, vb = W.to_bits(k32, dtype), W.to_bits(v32, dtype)
    kx, vx = W.bits_to_f32(kb, dtype), W.bits_to_f32(vb, dtype)
    slots = rng.permutation(nb * bs)[:T].astype(np.int64)
    slots[::5] = -1
    s = W.rht_signs(d)
    kc = np.full((nb, bs, hk, d // 2), 0xA5, np.uint8)
    vc = np.full_like(kc, 0x5A)
    ks = np.full((nb, bs, hk), 7.0, np.float32)
    vs = np.full_like(ks, 9.0)
    code = {"f32": oracle.DT_F32, "f16": oracle.DT_F16, "bf16": oracle.DT_BF16}[dtype]
    oracle.reshape_and_cache_int4(kb, vb, code, slots, s, kc, vc, ks, vs)
    H = scipy.linalg.hadamard(d).astype(np.float64)
    written = set()
    for t in range(T):
        if slots[t] < 0:
            continue
        blk, off = divmod(int(slots[t]), bs)
        written.add((blk, off))
        for h in range(hk):
            for src, cache, sc in ((kx, kc, ks), (vx, vc, vs)):
                rot = H @ (src[t, h].astype(np.float64) * s)
                deq = oracle.int4_dequant_row(cache[blk, off, h], sc[blk, off, h], d)
                word_bits = np.float32(sc[blk, off, h]).view(np.uint32)
                step = float(np.uint32(word_bits & np.uint32(0xFFFFFFF0)).view(np.float32))
                tol = step / 2 * 1.001 + (np.abs(rot).max() * 2 ** -7 if dtype != "f32" else 1e-5)
                assert np.abs(deq - rot).max() <= tol
                back = (H @ deq) * s / d
                assert np.abs(back - src[t, h]).max() <= tol * np.sqrt(d) / d * 4 + 1e-6
    for blk in range(nb):
        for off in range(bs):
            if (blk, off) not in written:
                assert np.all(kc[blk, off] == 0xA5) and np.all(vc[blk, off] == 0x5A)
                assert np.all(ks[blk, off] == 7.0) and np.all(vs[blk, off] == 9.0)


def test_fwht_fp32_stage_order_hand_example():
    g = json.load(open(os.path.join(GOLDEN, "fwht_stage_order.json")))
    x = np.array([int(h, 16) for h in g["input_f32_hex"]], np.uint32).view(np.float32)
    want = np.array([int(h, 16) for h in g["expected_f32_hex"]], np.uint32)
    np.testing.assert_array_equal(oracle.fwht_f32(x).view(np.uint32), want)
