"""Pins of the oracle's pooled-softmax key compressor (kpool_compress.py,
_kpool_softmax_rotate_write_cache_kernel and kpool_compress_and_write_cache).

- The softmax exponential is the correctly rounded fp32 e^x: checked against
  Python's decimal module at 60 digits.
- Exact pipelines from library routines: with equal weights or one slot
  dominating each dimension (chosen partly by the position bias), the pooled
  value is exact, and the entry must equal scipy's Hadamard matrix, an fp32
  multiply by the page's 1/sqrt(128), torch's bf16 and float8_e4m3fn casts and
  either scale rule (power of two by math.frexp, or absmax * fl32(1/448)).
- Brute force in fp64 on random pools (scores with offsets up to 150, where
  an unshifted exponential overflows): the decoded entry, rotated back, is
  within the bf16 and E4M3 error bound of the softmax-weighted mean.
- Layout of the indexer page (codes first, fp32 scales after block_size*128
  bytes), write mask, skipped locations, score dtypes and argument errors.
"""
import math
from decimal import Decimal, localcontext

import numpy as np
import pytest
import scipy.linalg
import scipy.special
import torch

import oracle
from quantized_paged_kv_tq_amd import workloads as W

INV_SQRT128 = np.float32(0.08838834764831845)
INV_448 = np.float32(1.0 / 448.0)
H = scipy.linalg.hadamard(128).astype(np.float64)


def _cr_exp_f32(x):
    """Nearest fp32 to e^x, decided in exact decimal arithmetic."""
    with localcontext() as ctx:
        ctx.prec = 60
        e = Decimal(float(x)).exp()
        f = np.float32(float(e))
        cands = [np.nextafter(f, np.float32(-np.inf)), f, np.nextafter(f, np.float32(np.inf))]
        return min(cands, key=lambda c: abs(Decimal(float(c)) - e))


def test_exp_is_correctly_rounded_fp32():
    g = np.random.default_rng(1)
    xs = np.concatenate([
        g.uniform(-105, 0, 2000), g.uniform(-1, 0, 2000), g.uniform(0, 88, 300),
        -np.exp2(g.uniform(-30, 0, 300)),
        [0.0, -0.0, -1e-30, -87.3, -88.7, -103.0, -103.9, -104.0, -110.0, 88.7]]).astype(np.float32)
    for x in xs:
        got = np.float32(oracle.exp_f32(x))
        want = _cr_exp_f32(x)
        assert got == want, (float(x), float(got), float(want))
    assert oracle.exp_f32(0.0) == 1.0
    assert oracle.exp_f32(-np.inf) == 0.0


def _exact_pow2_ceil(t):
    m, e = math.frexp(t)
    return 2.0 ** (e - 1) if m == 0.5 else 2.0 ** e


def _entry_from_x(x, round_scale):
    """Library-routine pipeline from pooled values x [n, 128] that are bf16
    multiples of 1/8 below 2^9, so the Hadamard sums are exact in fp32."""
    hx = (x.astype(np.float64) @ H.T).astype(np.float32)
    xr = torch.from_numpy(hx * INV_SQRT128).to(torch.bfloat16).to(torch.float32).numpy()
    amax = np.maximum(np.abs(xr).max(1), np.float32(1e-4))
    if round_scale:
        s = np.array([_exact_pow2_ceil(float(np.float32(a * INV_448))) for a in amax], np.float32)
    else:
        s = (amax * INV_448).astype(np.float32)
    q = np.clip(xr / s[:, None], -448, 448).astype(np.float32)
    codes = torch.from_numpy(q).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return codes, s


def _int_pools(n, P, seed):
    g = np.random.default_rng(seed)
    k = g.integers(-64, 64, size=(n, P, 128)).astype(np.float32)
    return k, W.to_bits(k, "bf16")


@pytest.mark.parametrize("P", [1, 2, 4, 8])
@pytest.mark.parametrize("round_scale", [True, False])
def test_equal_weights_exact_pipeline(P, round_scale):
    k, kb = _int_pools(300, P, 10 + P)
    g = np.random.default_rng(20 + P)
    ape = g.integers(-8, 8, size=(P, 128)).astype(np.float32)
    c = g.integers(-4, 4, size=(300, 1, 128)).astype(np.float32)
    score = (c - ape[None]).astype(np.float32)  # score + ape = c for every slot
    codes, s = oracle.kpool_compress_and_write(kb, score, ape, round_scale=round_scale,
                                               return_compressed=True)
    x = (k.sum(1) / P).astype(np.float32)  # exact in fp32, then the bf16 rounding
    x = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    want_c, want_s = _entry_from_x(x, round_scale)
    np.testing.assert_array_equal(s, want_s)
    np.testing.assert_array_equal(codes, want_c)


@pytest.mark.parametrize("P", [2, 3, 5])
@pytest.mark.parametrize("round_scale", [True, False])
def test_dominant_slot_per_dimension(P, round_scale):
    n = 200
    k, kb = _int_pools(n, P, 30 + P)
    g = np.random.default_rng(40 + P)
    win = g.integers(0, P, size=(n, 128))
    by_ape = g.random(128) < 0.5  # dims whose winner is set by the position bias
    score = g.standard_normal((n, P, 128)).astype(np.float32)
    ape = g.standard_normal((P, 128)).astype(np.float32)
    for d in np.nonzero(by_ape)[0]:
        win[:, d] = d % P
        ape[d % P, d] += 120.0
    rows = np.arange(n)[:, None]
    dims = np.arange(128)[None, :]
    score[rows, win, dims] += np.where(by_ape[None, :], 0.0, 120.0).astype(np.float32)
    codes, s = oracle.kpool_compress_and_write(kb, score, ape, round_scale=round_scale,
                                               return_compressed=True)
    x = k[rows, win, dims]  # e^-110 and below round to 0 in fp32
    want_c, want_s = _entry_from_x(x, round_scale)
    np.testing.assert_array_equal(s, want_s)
    np.testing.assert_array_equal(codes, want_c)


@pytest.mark.parametrize("P,offset,sdt", [(1, 0.0, "bf16"), (3, 0.0, "f32"), (4, 150.0, "f32"),
                                          (8, -40.0, "f16"), (16, 0.0, "bf16")])
@pytest.mark.parametrize("round_scale", [True, False])
def test_brute_force_fp64_bound(P, offset, sdt, round_scale):
    w = W.kpool_workload(n_pools=500, pool_size=P, score_dtype=sdt, score_offset=offset, wid=12)
    codes, s = oracle.kpool_compress_and_write(w["slot_k"], w["slot_score"], w["ape"],
                                               round_scale=round_scale, return_compressed=True,
                                               score_dtype=sdt)
    kk = W.bits_to_f32(w["slot_k"], "bf16").astype(np.float64)
    sc = W.bits_to_f32(w["slot_score"], sdt).astype(np.float64) + w["ape"][None]
    wts = scipy.special.softmax(sc, axis=1)
    xt = (wts * kk).sum(1)
    dec = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float32).numpy().astype(np.float64)
    yh = dec * s[:, None]
    xh = yh @ H / np.sqrt(128)
    err = np.linalg.norm(xh - xt, axis=1)
    nx = np.linalg.norm(xt, axis=1)
    q_err = np.linalg.norm(2.0 ** -4 * np.abs(yh) / (1 - 2.0 ** -4) + 2.0 ** -10 * s[:, None], axis=1)
    bound = 1.05 * ((2 * 2.0 ** -9 + 1e-5) * nx + q_err) + 1e-6
    assert np.all(err <= bound), (err / bound).max()
    # the rule of each scale mode
    if round_scale:
        m, _ = np.frexp(s)
        assert np.all(m == 0.5)
        assert np.all(np.abs(dec).max(1) > 224 * (1 - 2.0 ** -3))
    else:
        assert np.all(np.abs(dec).max(1) == 448)


def test_indexer_page_layout_mask_and_skips():
    bs, nb, P = 16, 5, 4
    n = nb * bs
    w = W.kpool_workload(n_pools=n, pool_size=P, score_dtype="f32", block_size=bs, wid=13)
    codes, s = oracle.kpool_compress_and_write(w["slot_k"], w["slot_score"], w["ape"],
                                               return_compressed=True)
    g = np.random.default_rng(5)
    loc = g.permutation(n).astype(np.int64)
    loc[3] = -1
    loc[7] = n          # outside the cache
    loc[11] = n + 500
    mask = g.random(n) >= 0.2
    cache = np.full((nb, bs, 132), 0xA5, np.uint8)
    oracle.kpool_compress_and_write(w["slot_k"], w["slot_score"], w["ape"], loc, cache,
                                    write_mask=mask)
    flat = cache.reshape(nb, bs * 132)
    written = np.zeros((nb, bs), bool)
    for i in range(n):
        if not mask[i] or not (0 <= loc[i] < n):
            continue
        pg, off = divmod(int(loc[i]), bs)
        written[pg, off] = True
        assert np.array_equal(flat[pg, off * 128:(off + 1) * 128], codes[i])
        sb = flat[pg, bs * 128 + 4 * off:bs * 128 + 4 * off + 4].view(np.float32)[0]
        assert sb == s[i]
    for pg in range(nb):
        for off in range(bs):
            if not written[pg, off]:
                assert np.all(flat[pg, off * 128:(off + 1) * 128] == 0xA5)
                assert np.all(flat[pg, bs * 128 + 4 * off:bs * 128 + 4 * off + 4] == 0xA5)
    assert written.sum() == sum(1 for i in range(n) if mask[i] and 0 <= loc[i] < n)


def test_score_dtypes_agree_on_representable_values():
    w = W.kpool_workload(n_pools=64, pool_size=4, score_dtype="f32", wid=14)
    s16 = W.to_bits(w["slot_score"], "f16")
    s32 = W.bits_to_f32(s16, "f16")
    a = oracle.kpool_compress_and_write(w["slot_k"], s32, w["ape"], return_compressed=True)
    b = oracle.kpool_compress_and_write(w["slot_k"], s16, w["ape"], return_compressed=True,
                                        score_dtype="f16")
    sb = W.to_bits(w["slot_score"], "bf16")
    c = oracle.kpool_compress_and_write(w["slot_k"], W.bits_to_f32(sb, "bf16"), w["ape"],
                                        return_compressed=True)
    d = oracle.kpool_compress_and_write(w["slot_k"], sb, w["ape"], return_compressed=True,
                                        score_dtype="bf16")
    for x, y in ((a, b), (c, d)):
        np.testing.assert_array_equal(x[0], y[0])
        np.testing.assert_array_equal(x[1], y[1])


def test_zero_pools_and_argument_errors():
    z = np.zeros((0, 4, 128), np.uint16)
    codes, s = oracle.kpool_compress_and_write(z, z.astype(np.float32), np.zeros((4, 128), np.float32),
                                               return_compressed=True)
    assert codes.shape == (0, 128) and s.shape == (0,)
    k = np.zeros((2, 4, 64), np.uint16)
    with pytest.raises(ValueError):  # the Hadamard-128 entry needs head_dim 128
        oracle.kpool_compress_and_write(k, k.astype(np.float32), np.zeros((4, 64), np.float32),
                                        return_compressed=True)
    k = np.zeros((2, 4, 128), np.uint16)
    with pytest.raises(ValueError):  # neither output
        oracle.kpool_compress_and_write(k, k.astype(np.float32), np.zeros((4, 128), np.float32))
    with pytest.raises(ValueError):  # write mask with the compressed output
        oracle.kpool_compress_and_write(k, k.astype(np.float32), np.zeros((4, 128), np.float32),
                                        write_mask=np.ones(2, bool), return_compressed=True)
    # an all-zero pool: the 1e-4 absmax floor, every code 0
    codes, s = oracle.kpool_compress_and_write(k, k.astype(np.float32), np.zeros((4, 128), np.float32),
                                               return_compressed=True)
    assert np.all(codes == 0)
    assert s[0] == _exact_pow2_ceil(float(np.float32(np.float32(1e-4) * INV_448)))
