"""GPU parity of tq_decode_attention against the CPU oracle (fp64), through
the C ABI: max |err| <= 1e-3 and relative L2 <= 1e-4 on the output, lse
within 1e-4. Caches are written by the oracle. Covers the INT4 format on
both kernels (matrix-core and generic), the TurboQuant formats, ragged and
degenerate sequence lengths, every split count regime, and the full-size
workloads on sampled rows."""
import numpy as np
import pytest

import oracle
import quantized_paged_kv_tq_amd as tq
from quantized_paged_kv_tq_amd import workloads as W

from gpu_cases import (assert_close, gpu_int4_decode, gpu_tq_decode, int4_caches, oracle_rows,
                       tq_case)

pytestmark = pytest.mark.gpu


def _oracle_int4(w, q, c, splits=None, rows=None, seq_lens=None):
    return oracle.int4_decode(q, c["kc"], c["vc"], c["ks"], c["vs"], w.block_table,
                              w.seq_lens if seq_lens is None else seq_lens, c["signs"],
                              w.num_splits if splits is None else splits, w.sm_scale, rows)


@pytest.mark.parametrize("flags", [0, tq.FLAG_GENERIC])
def test_int4_tiny_workload(flags):
    w = W.decode_workload("tiny_int4")
    c = int4_caches(w)
    q = W.query(w)
    ref, ref_lse = _oracle_int4(w, q, c)
    got, lse = gpu_int4_decode(w, q, c, flags=flags)
    assert_close(got, ref, lse, ref_lse, "tiny_int4")


SHAPES = [
    # B, hq, hk, d, bs, seq_lens, splits
    (3, 8, 2, 128, 16, [1, 70, 333], 4),
    (2, 32, 8, 128, 16, [1024, 517], 8),
    (2, 64, 8, 128, 64, [700, 4096], 16),
    (4, 8, 8, 128, 16, [15, 16, 17, 200], 3),
    (2, 16, 1, 128, 16, [300, 129], 5),
    (2, 12, 4, 64, 16, [111, 64], 2),
    (1, 6, 2, 64, 7, [100], 9),
    (2, 16, 16, 64, 32, [65, 1], 1),
    (2, 2, 2, 128, 1, [19, 40], 64),
    (2, 40, 4, 128, 16, [90, 160], 4),
]


@pytest.mark.parametrize("flags", [0, tq.FLAG_GENERIC, tq.FLAG_WIDE],
                         ids=["mfma", "generic", "mfma_wide"])
@pytest.mark.parametrize("shape", SHAPES, ids=[str(i) for i in range(len(SHAPES))])
def test_int4_shapes(shape, flags):
    B, hq, hk, d, bs, seq, S = shape
    w = W.custom_decode_workload(100 + len(seq) * 7 + hq + d, B, hq, hk, d, bs, S, seq, 5, "bf16")
    c = int4_caches(w)
    q = W.query(w)
    ref, ref_lse = _oracle_int4(w, q, c)
    got, lse = gpu_int4_decode(w, q, c, flags=flags)
    assert_close(got, ref, lse, ref_lse, str(shape))


@pytest.mark.parametrize("hq,hk", [(24, 2), (32, 2), (40, 2), (56, 2), (64, 2), (96, 2)],
                         ids=["g12", "g16", "g20", "g28", "g32", "g48"])
def test_int4_query_groups_above_eight(hq, hk):
    """g = 9 .. 32 on the matrix-core path: ceil(g / 4) waves of four query
    heads per kv head (workgroups of 3 .. 8 waves, the last wave padded);
    g = 48 goes to the generic kernel. Empty, one-token and long sequences."""
    seq = [0, 1, 300, 777, 65, 2000]
    w = W.custom_decode_workload(330 + hq, len(seq), hq, hk, 128, 16, 3, seq, 6, "bf16")
    c = int4_caches(w)
    q = W.query(w)
    ref, ref_lse = _oracle_int4(w, q, c)
    for flags in (0, tq.FLAG_WIDE):
        got, lse = gpu_int4_decode(w, q, c, flags=flags)
        assert_close(got, ref, lse, ref_lse, "hq=%d hk=%d flags=%d" % (hq, hk, flags))


def test_int4_split_invariance_and_empty_splits():
    w = W.custom_decode_workload(140, 2, 8, 2, 128, 16, 4, [37, 100], 2, "bf16")
    c = int4_caches(w)
    q = W.query(w)
    ref, ref_lse = _oracle_int4(w, q, c, splits=0)
    for S in (1, 2, 8, 37, 64, 100, 105, 256):
        got, lse = gpu_int4_decode(w, q, c, num_splits=S)
        assert_close(got, ref, lse, ref_lse, "S=%d" % S)


def test_int4_zero_and_one_token_sequences():
    w = W.custom_decode_workload(141, 3, 8, 2, 128, 16, 4, [1, 1, 40], 2, "bf16")
    c = int4_caches(w)
    q = W.query(w)
    seq = np.array([1, 0, 40], np.int32)
    ref, ref_lse = _oracle_int4(w, q, c, seq_lens=seq)
    got, lse = gpu_int4_decode(w, q, c, seq_lens=seq)
    assert_close(got, ref, lse, ref_lse, "seq 1/0")
    assert np.all(got[8:16] == 0) and np.all(np.isneginf(lse[8:16]))


def test_int4_random_cache_bytes():
    """Uniformly random nibbles and scale words (no writer involved)."""
    w = W.custom_decode_workload(142, 2, 16, 4, 128, 16, 4, [300, 77], 4, "bf16")
    kc, vc, ks, vs = W.random_int4_cache(w)
    c = dict(kc=kc, vc=vc, ks=ks, vs=vs, signs=W.rht_signs(128))
    q = W.query(w)
    ref, ref_lse = _oracle_int4(w, q, c)
    for flags in (0, tq.FLAG_GENERIC, tq.FLAG_WIDE):
        got, lse = gpu_int4_decode(w, q, c, flags=flags)
        assert_close(got, ref, lse, ref_lse, "random bytes")


def test_int4_balanced_many_sequences():
    """More sequences than threads per workgroup (two per thread in the
    prefix sums), empty ones interleaved, ranges that cross many sequence
    and split boundaries, and workgroups with empty ranges."""
    rng = np.random.default_rng(143)
    seq = rng.choice([0, 1, 5, 63, 64, 65, 130, 200, 777], size=600).astype(np.int32)
    w = W.custom_decode_workload(143, 600, 8, 2, 128, 16, 3, seq, 7, "bf16")
    kc, vc, ks, vs = W.random_int4_cache(w)
    c = dict(kc=kc, vc=vc, ks=ks, vs=vs, signs=W.rht_signs(128))
    q = W.query(w)
    ref, ref_lse = _oracle_int4(w, q, c)
    got, lse = gpu_int4_decode(w, q, c)
    assert_close(got, ref, lse, ref_lse, "600 sequences")


@pytest.mark.parametrize("seq,S", [([1, 3], 2), ([64, 65, 1], 7), ([2000], 1), ([2000], 256)])
def test_int4_balanced_few_tiles(seq, S):
    """Fewer tiles than workgroups (most ranges empty), single-tile splits and
    one split spread over many workgroups."""
    w = W.custom_decode_workload(144 + len(seq) + S, len(seq), 32, 8, 128, 16, S, seq, 3, "bf16")
    c = int4_caches(w)
    q = W.query(w)
    ref, ref_lse = _oracle_int4(w, q, c)
    got, lse = gpu_int4_decode(w, q, c)
    assert_close(got, ref, lse, ref_lse, "seq %s S=%d" % (seq, S))


def test_int4_balanced_chunked_range():
    """Ranges longer than the 64 tiles a workgroup resolves at a time: one
    sequence of 1,056,896 tokens over 8 kv heads (16,514 tiles on 256
    workgroups), random cache bytes, sampled rows."""
    seq = [64 * 64 * 256 + 64 * 130]
    w = W.custom_decode_workload(145, 1, 32, 8, 128, 64, 4, seq, 0, "bf16")
    kc, vc, ks, vs = W.random_int4_cache(w)
    c = dict(kc=kc, vc=vc, ks=ks, vs=vs, signs=W.rht_signs(128))
    q = W.query(w)
    got, lse = gpu_int4_decode(w, q, c)
    rows = np.array([0, 13, 31], np.int32)
    ref, ref_lse = _oracle_int4(w, q, c, rows=rows)
    assert_close(got[rows], ref, lse[rows], ref_lse, "chunked range")
    assert np.all(np.isfinite(got))


@pytest.mark.parametrize("name", ["llama8b_int4", "long_int4"])
def test_int4_full_size_all_rows(name):
    """Every (batch, query head) row of the full-size workloads, in the
    launch configuration the benchmark times, against the fp64 oracle."""
    w = W.decode_workload(name)
    c = int4_caches(w)
    q = W.query(w)
    got, lse = gpu_int4_decode(w, q, c)
    ref, ref_lse = oracle_rows(lambda r: _oracle_int4(w, q, c, rows=r), w.B * w.hq)
    assert_close(got, ref, lse, ref_lse, name)


TQ_FORMATS = [(oracle.KEY_FP8, oracle.VAL_U4), (oracle.KEY_MSE3, oracle.VAL_U3),
              (oracle.KEY_FP8, oracle.VAL_U3), (oracle.KEY_MSE4, oracle.VAL_U4),
              (oracle.KEY_MSE3, oracle.VAL_U4), (oracle.KEY_MSE4, oracle.VAL_U3)]


@pytest.mark.parametrize("fmt", TQ_FORMATS, ids=[str(f) for f in TQ_FORMATS])
@pytest.mark.parametrize("d", [128, 64])
def test_tq_formats_small(fmt, d):
    key_fmt, val_fmt = fmt
    w = W.custom_decode_workload(150 + d, 2, 8, 2, d, 16, 4, [150, 33], 3, "bf16")
    cache, cen = tq_case(w, key_fmt, val_fmt)
    q = W.query(w, bf16_valued=True)
    ref, ref_lse = oracle.tq_decode(q, cache, w.block_table, w.seq_lens, cen, None, key_fmt,
                                    val_fmt, 0, w.num_splits, w.sm_scale)
    got, lse = gpu_tq_decode(w, q, cache, cen, key_fmt, val_fmt)
    assert_close(got, ref, lse, ref_lse, str(fmt))


@pytest.mark.parametrize("key_fmt", [oracle.KEY_MSE3, oracle.KEY_MSE4])
def test_tq_norm_correction_and_rot_signs(key_fmt):
    w = W.custom_decode_workload(160, 2, 8, 4, 128, 16, 5, [90, 211], 3, "bf16")
    rs = W.rht_signs(128, round_idx=1)
    cache, cen = tq_case(w, key_fmt, oracle.VAL_U3, rot_signs=rs)
    q = W.query(w, bf16_valued=True)
    for nc in (0, 1):
        ref, ref_lse = oracle.tq_decode(q, cache, w.block_table, w.seq_lens, cen, rs, key_fmt,
                                        oracle.VAL_U3, nc, w.num_splits, w.sm_scale)
        got, lse = gpu_tq_decode(w, q, cache, cen, key_fmt, oracle.VAL_U3, rot_signs=rs,
                                 norm_correction=nc)
        assert_close(got, ref, lse, ref_lse, "nc=%d" % nc)


@pytest.mark.parametrize("fmt", [(oracle.KEY_FP8, oracle.VAL_U4), (oracle.KEY_MSE3, oracle.VAL_U3),
                                 (oracle.KEY_FP8, oracle.VAL_FP8)],
                         ids=["A_fp8_u4", "B_mse3_u3", "fp8_fp8"])
def test_tq_full_size_all_rows(fmt):
    """Every row of the full tq_mixed shape (B = 16, Hq = 32, 16384 tokens,
    S = 32) against the fp64 oracle."""
    key_fmt, val_fmt = fmt
    w = W.decode_workload("tq_mixed")
    cache, cen = tq_case(w, key_fmt, val_fmt)
    q = W.query(w, bf16_valued=True)
    got, lse = gpu_tq_decode(w, q, cache, cen, key_fmt, val_fmt)
    ref, ref_lse = oracle_rows(
        lambda r: oracle.tq_decode(q, cache, w.block_table, w.seq_lens, cen, None, key_fmt,
                                   val_fmt, 0, w.num_splits, w.sm_scale, r), w.B * w.hq)
    assert_close(got, ref, lse, ref_lse, "tq_mixed %s" % (fmt,))


def _oracle_tq(w, q, cache, cen, key_fmt, val_fmt, splits=None, rows=None, seq_lens=None):
    return oracle.tq_decode(q, cache, w.block_table, w.seq_lens if seq_lens is None else seq_lens,
                            cen, None, key_fmt, val_fmt, 0,
                            w.num_splits if splits is None else splits, w.sm_scale, rows)


A_FMT = (oracle.KEY_FP8, oracle.VAL_U4)


@pytest.mark.parametrize("flags", [0, tq.FLAG_GENERIC, tq.FLAG_WIDE],
                         ids=["mfma", "generic", "mfma_wide"])
@pytest.mark.parametrize("shape", SHAPES, ids=[str(i) for i in range(len(SHAPES))])
def test_tq_fp8_u4_shapes(shape, flags):
    """FP8 keys / 4-bit values on the matrix-core kernel (D = 128, up to
    8 query heads per kv head) and on the generic one, same shapes as the
    INT4 cases (the others fall back to the generic kernel)."""
    B, hq, hk, d, bs, seq, S = shape
    w = W.custom_decode_workload(200 + len(seq) * 7 + hq + d, B, hq, hk, d, bs, S, seq, 5, "bf16")
    cache, cen = tq_case(w, *A_FMT)
    q = W.query(w, bf16_valued=True)
    ref, ref_lse = _oracle_tq(w, q, cache, cen, *A_FMT)
    got, lse = gpu_tq_decode(w, q, cache, cen, *A_FMT, flags=flags)
    assert_close(got, ref, lse, ref_lse, str(shape))


def test_tq_fp8_u4_split_invariance_and_degenerate_lengths():
    w = W.custom_decode_workload(240, 3, 8, 2, 128, 16, 4, [37, 1, 100], 2, "bf16")
    cache, cen = tq_case(w, *A_FMT)
    q = W.query(w, bf16_valued=True)
    seq = np.array([37, 0, 100], np.int32)
    ref, ref_lse = _oracle_tq(w, q, cache, cen, *A_FMT, splits=0, seq_lens=seq)
    for S in (1, 2, 8, 37, 64, 100, 105, 256):
        got, lse = gpu_tq_decode(w, q, cache, cen, *A_FMT, num_splits=S, seq_lens=seq)
        assert_close(got, ref, lse, ref_lse, "S=%d" % S)
        assert np.all(got[8:16] == 0) and np.all(np.isneginf(lse[8:16]))


def test_tq_fp8_u4_random_slot_bytes():
    """Random slots (no writer): every finite E4M3 key code, value scales of
    both signs (negative ones take the signed-digit path), random zeros."""
    w = W.custom_decode_workload(241, 2, 16, 4, 128, 16, 4, [300, 77], 4, "bf16")
    cache = W.random_tq_fp8_u4_cache(w, oracle.tq_slot_bytes(128, *A_FMT))
    q = W.query(w) / 16  # random codes reach 448: keep scores O(10)
    ref, ref_lse = _oracle_tq(w, q, cache, None, *A_FMT)
    for flags in (0, tq.FLAG_GENERIC, tq.FLAG_WIDE):
        got, lse = gpu_tq_decode(w, q, cache, None, *A_FMT, flags=flags)
        assert_close(got, ref, lse, ref_lse, "random slots flags=%d" % flags)


def test_tq_fp8_u4_balanced_many_sequences():
    """600 sequences (two per thread in the prefix sums), empty ones
    interleaved, ranges over many sequence and split boundaries."""
    rng = np.random.default_rng(242)
    seq = rng.choice([0, 1, 5, 63, 64, 65, 130, 200, 777], size=600).astype(np.int32)
    w = W.custom_decode_workload(242, 600, 8, 2, 128, 16, 3, seq, 7, "bf16")
    cache = W.random_tq_fp8_u4_cache(w, oracle.tq_slot_bytes(128, *A_FMT))
    q = W.query(w) / 16  # random codes reach 448: keep scores O(10)
    ref, ref_lse = _oracle_tq(w, q, cache, None, *A_FMT)
    got, lse = gpu_tq_decode(w, q, cache, None, *A_FMT)
    assert_close(got, ref, lse, ref_lse, "600 sequences")


@pytest.mark.parametrize("seq,S", [([1, 3], 2), ([64, 65, 1], 7), ([2000], 1), ([2000], 256)])
def test_tq_fp8_u4_balanced_few_tiles(seq, S):
    w = W.custom_decode_workload(243 + len(seq) + S, len(seq), 32, 8, 128, 16, S, seq, 3, "bf16")
    cache, cen = tq_case(w, *A_FMT)
    q = W.query(w, bf16_valued=True)
    ref, ref_lse = _oracle_tq(w, q, cache, cen, *A_FMT)
    got, lse = gpu_tq_decode(w, q, cache, cen, *A_FMT)
    assert_close(got, ref, lse, ref_lse, "seq %s S=%d" % (seq, S))


# ---------------------------------------------------------------------------
# 3-bit centroid keys + 3-bit values (matrix-core path for D = 128, g <= 8)

B_FMT = (oracle.KEY_MSE3, oracle.VAL_U3)


@pytest.mark.parametrize("flags", [0, tq.FLAG_GENERIC, tq.FLAG_WIDE],
                         ids=["mfma", "generic", "mfma_wide"])
@pytest.mark.parametrize("shape", SHAPES, ids=[str(i) for i in range(len(SHAPES))])
def test_tq_mse3_u3_shapes(shape, flags):
    B, hq, hk, d, bs, seq, S = shape
    w = W.custom_decode_workload(300 + len(seq) * 7 + hq + d, B, hq, hk, d, bs, S, seq, 5, "bf16")
    cache, cen = tq_case(w, *B_FMT)
    q = W.query(w, bf16_valued=True)
    ref, ref_lse = _oracle_tq(w, q, cache, cen, *B_FMT)
    got, lse = gpu_tq_decode(w, q, cache, cen, *B_FMT, flags=flags)
    assert_close(got, ref, lse, ref_lse, str(shape))


def test_tq_mse3_u3_rot_signs_split_invariance_and_degenerate_lengths():
    w = W.custom_decode_workload(340, 3, 8, 2, 128, 16, 4, [37, 1, 100], 2, "bf16")
    rs = W.rht_signs(128, round_idx=4)
    cache, cen = tq_case(w, *B_FMT, rot_signs=rs)
    q = W.query(w)
    seq = np.array([37, 0, 100], np.int32)
    ref, ref_lse = oracle.tq_decode(q, cache, w.block_table, seq, cen, rs, *B_FMT, 0, 0, w.sm_scale)
    for S in (1, 2, 8, 37, 64, 100, 105, 256):
        got, lse = gpu_tq_decode(w, q, cache, cen, *B_FMT, rot_signs=rs, num_splits=S, seq_lens=seq)
        assert_close(got, ref, lse, ref_lse, "S=%d" % S)
        assert np.all(got[8:16] == 0) and np.all(np.isneginf(lse[8:16]))


def _random_centroids(seed, antisymmetric=False):
    """A sorted random table; ``antisymmetric`` mirrors its upper half so that
    c[7 - j] == -c[j] holds exactly (the shape of every Lloyd-Max table)."""
    rng = np.random.default_rng(seed)
    c = np.sort(rng.uniform(-0.3, 0.3, 8)).astype(np.float32)
    if antisymmetric:
        c[:4] = -c[4:][::-1]
    return c


@pytest.mark.parametrize("antisymmetric", [False, True], ids=["general", "antisymmetric"])
def test_tq_mse3_u3_random_slot_bytes_and_table(antisymmetric):
    """Random slots (no writer) and an arbitrary centroid table: every index
    pattern, value scales of both signs, random norms and zeros.  The matrix
    kernel has one score form for any table and a shorter one for tables with
    c[7 - j] == -c[j]; both are run."""
    w = W.custom_decode_workload(341, 2, 16, 4, 128, 16, 4, [300, 77], 4, "bf16")
    cache = W.random_tq_mse3_u3_cache(w, oracle.tq_slot_bytes(128, *B_FMT))
    cen = _random_centroids(341, antisymmetric)
    assert np.array_equal(cen[::-1] == -cen, np.full(8, antisymmetric))
    q = W.query(w) / 4
    ref, ref_lse = _oracle_tq(w, q, cache, cen, *B_FMT)
    for flags in (0, tq.FLAG_GENERIC, tq.FLAG_WIDE):
        got, lse = gpu_tq_decode(w, q, cache, cen, *B_FMT, flags=flags)
        assert_close(got, ref, lse, ref_lse, "random slots flags=%d" % flags)


def test_tq_mse3_u3_balanced_many_sequences():
    rng = np.random.default_rng(342)
    seq = rng.choice([0, 1, 5, 63, 64, 65, 130, 200, 777], size=600).astype(np.int32)
    w = W.custom_decode_workload(342, 600, 8, 2, 128, 16, 3, seq, 7, "bf16")
    cache = W.random_tq_mse3_u3_cache(w, oracle.tq_slot_bytes(128, *B_FMT))
    cen = _random_centroids(342)
    q = W.query(w) / 4
    ref, ref_lse = _oracle_tq(w, q, cache, cen, *B_FMT)
    got, lse = gpu_tq_decode(w, q, cache, cen, *B_FMT)
    assert_close(got, ref, lse, ref_lse, "600 sequences")


@pytest.mark.parametrize("seq,S", [([1, 3], 2), ([64, 65, 1], 7), ([2000], 1), ([2000], 256)])
def test_tq_mse3_u3_balanced_few_tiles(seq, S):
    w = W.custom_decode_workload(343 + len(seq) + S, len(seq), 32, 8, 128, 16, S, seq, 3, "bf16")
    cache, cen = tq_case(w, *B_FMT)
    q = W.query(w, bf16_valued=True)
    ref, ref_lse = _oracle_tq(w, q, cache, cen, *B_FMT)
    got, lse = gpu_tq_decode(w, q, cache, cen, *B_FMT)
    assert_close(got, ref, lse, ref_lse, "seq %s S=%d" % (seq, S))


@pytest.mark.parametrize("antisymmetric", [False, True], ids=["general", "antisymmetric"])
@pytest.mark.parametrize("hq,hk", [(10, 2), (12, 2), (14, 2), (16, 2), (32, 4)],
                         ids=["g5", "g6", "g7", "g8", "g8x4"])
def test_tq_mse3_u3_query_groups_of_five_to_eight(hq, hk, antisymmetric):
    """g = 5 .. 8 on the matrix-core path: one wave serves all query heads
    of a kv head (two MFMA row sets; heads past g padded); random slots,
    empty and one-token sequences, split and range boundaries."""
    seq = [0, 1, 300, 777, 65, 2000]
    w = W.custom_decode_workload(350 + hq, len(seq), hq, hk, 128, 16, 3, seq, 6, "bf16")
    cache = W.random_tq_mse3_u3_cache(w, oracle.tq_slot_bytes(128, *B_FMT))
    cen = _random_centroids(350 + hq, antisymmetric)
    q = W.query(w) / 4
    ref, ref_lse = _oracle_tq(w, q, cache, cen, *B_FMT)
    for flags in (0, tq.FLAG_WIDE):
        got, lse = gpu_tq_decode(w, q, cache, cen, *B_FMT, flags=flags)
        assert_close(got, ref, lse, ref_lse, "hq=%d hk=%d" % (hq, hk))


@pytest.mark.parametrize("hq,hk", [(10, 2), (12, 2), (14, 2), (16, 2), (32, 4)],
                         ids=["g5", "g6", "g7", "g8", "g8x4"])
def test_tq_fp8_u4_query_groups_of_five_to_eight(hq, hk):
    """FP8 keys + 4-bit values at g = 5 .. 8: one wave serves all query
    heads of a kv head; random slots, empty and one-token sequences."""
    seq = [0, 1, 300, 777, 65, 2000]
    w = W.custom_decode_workload(360 + hq, len(seq), hq, hk, 128, 16, 3, seq, 6, "bf16")
    cache = W.random_tq_fp8_u4_cache(w, oracle.tq_slot_bytes(128, *A_FMT))
    q = W.query(w) / 16  # random codes reach 448: keep scores O(10)
    ref, ref_lse = _oracle_tq(w, q, cache, None, *A_FMT)
    for flags in (0, tq.FLAG_WIDE):
        got, lse = gpu_tq_decode(w, q, cache, None, *A_FMT, flags=flags)
        assert_close(got, ref, lse, ref_lse, "hq=%d hk=%d" % (hq, hk))



# 4-bit centroid keys and 4-bit values on the same matrix-core kernel
# (D = 128, g <= 8): every combination of 3- and 4-bit keys and values

C_FMTS = [(oracle.KEY_MSE4, oracle.VAL_U4), (oracle.KEY_MSE3, oracle.VAL_U4),
          (oracle.KEY_MSE4, oracle.VAL_U3)]


def _random_table(seed, n, antisymmetric=False):
    """A sorted random table of n centroids; ``antisymmetric`` mirrors its
    upper half so that c[n - 1 - j] == -c[j] holds exactly."""
    rng = np.random.default_rng(seed)
    c = np.sort(rng.uniform(-0.3, 0.3, n)).astype(np.float32)
    if antisymmetric:
        c[:n // 2] = -c[n // 2:][::-1]
    return c


@pytest.mark.parametrize("flags", [0, tq.FLAG_GENERIC, tq.FLAG_WIDE],
                         ids=["mfma", "generic", "mfma_wide"])
@pytest.mark.parametrize("fmt", C_FMTS, ids=["mse4_u4", "mse3_u4", "mse4_u3"])
@pytest.mark.parametrize("shape", SHAPES[:5], ids=[str(i) for i in range(5)])
def test_tq_centroid_bits_shapes(shape, fmt, flags):
    """Oracle-encoded caches (Lloyd-Max tables) on the shapes of the other
    formats: GQA 1 .. 16, block sizes 16 and 64, split counts 3 .. 16."""
    B, hq, hk, d, bs, seq, S = shape
    w = W.custom_decode_workload(900 + len(seq) * 7 + hq + 3 * fmt[0] + fmt[1], B, hq, hk, d, bs, S,
                                 seq, 5, "bf16")
    cache, cen = tq_case(w, *fmt)
    q = W.query(w, bf16_valued=True)
    ref, ref_lse = _oracle_tq(w, q, cache, cen, *fmt)
    got, lse = gpu_tq_decode(w, q, cache, cen, *fmt, flags=flags)
    assert_close(got, ref, lse, ref_lse, "%s %s" % (shape, fmt))


@pytest.mark.parametrize("antisymmetric", [False, True], ids=["general", "antisymmetric"])
@pytest.mark.parametrize("fmt", C_FMTS, ids=["mse4_u4", "mse3_u4", "mse4_u3"])
def test_tq_centroid_bits_random_slots_and_table(fmt, antisymmetric):
    """Random slots (no writer): every index pattern, value scales of both
    signs, random norms and zeros, and an arbitrary centroid table, in the
    general (Moebius) and the antisymmetric (Walsh) score forms."""
    w = W.custom_decode_workload(910 + 3 * fmt[0] + fmt[1], 2, 16, 4, 128, 16, 4, [300, 77], 4, "bf16")
    cache = W.random_tq_cache(w, *fmt, oracle.tq_slot_bytes(128, *fmt))
    n = 16 if fmt[0] == oracle.KEY_MSE4 else 8
    cen = _random_table(911 + fmt[1], n, antisymmetric)
    assert np.array_equal(cen[::-1] == -cen, np.full(n, antisymmetric))
    q = W.query(w) / 4
    ref, ref_lse = _oracle_tq(w, q, cache, cen, *fmt)
    for flags in (0, tq.FLAG_GENERIC, tq.FLAG_WIDE):
        got, lse = gpu_tq_decode(w, q, cache, cen, *fmt, flags=flags)
        assert_close(got, ref, lse, ref_lse, "random slots %s flags=%d" % (fmt, flags))


@pytest.mark.parametrize("antisymmetric", [False, True], ids=["general", "antisymmetric"])
@pytest.mark.parametrize("hq,hk", [(10, 2), (16, 2), (32, 4), (6, 1), (21, 3)],
                         ids=["g5", "g8", "g8x4", "g6x1", "g7x3"])
def test_tq_mse4_u4_query_groups_of_five_to_eight(hq, hk, antisymmetric):
    """4-bit keys and values at g = 5 .. 8 (two waves per kv head splitting
    the head dims, both MFMA row sets; workgroups of one and two kv heads;
    the 64-bit variant splits by one wave per kv head); random slots, empty
    and one-token sequences, split and range boundaries."""
    fmt = (oracle.KEY_MSE4, oracle.VAL_U4)
    seq = [0, 1, 300, 777, 65, 2000]
    w = W.custom_decode_workload(920 + hq, len(seq), hq, hk, 128, 16, 3, seq, 6, "bf16")
    cache = W.random_tq_cache(w, *fmt, oracle.tq_slot_bytes(128, *fmt))
    cen = _random_table(920 + hq, 16, antisymmetric)
    q = W.query(w) / 4
    ref, ref_lse = _oracle_tq(w, q, cache, cen, *fmt)
    for flags in (0, tq.FLAG_WIDE):
        got, lse = gpu_tq_decode(w, q, cache, cen, *fmt, flags=flags)
        assert_close(got, ref, lse, ref_lse, "hq=%d hk=%d" % (hq, hk))


def test_tq_mse4_u4_rot_signs_split_invariance_and_degenerate_lengths():
    fmt = (oracle.KEY_MSE4, oracle.VAL_U4)
    w = W.custom_decode_workload(930, 3, 8, 2, 128, 16, 4, [37, 1, 100], 2, "bf16")
    rs = W.rht_signs(128, round_idx=5)
    cache, cen = tq_case(w, *fmt, rot_signs=rs)
    q = W.query(w)
    seq = np.array([37, 0, 100], np.int32)
    ref, ref_lse = oracle.tq_decode(q, cache, w.block_table, seq, cen, rs, *fmt, 0, 0, w.sm_scale)
    for S in (1, 2, 8, 37, 64, 100, 105, 256):
        got, lse = gpu_tq_decode(w, q, cache, cen, *fmt, rot_signs=rs, num_splits=S, seq_lens=seq)
        assert_close(got, ref, lse, ref_lse, "S=%d" % S)
        assert np.all(got[8:16] == 0) and np.all(np.isneginf(lse[8:16]))


def test_tq_mse4_u4_balanced_many_sequences():
    fmt = (oracle.KEY_MSE4, oracle.VAL_U4)
    rng = np.random.default_rng(940)
    seq = rng.choice([0, 1, 5, 63, 64, 65, 130, 200, 777], size=600).astype(np.int32)
    w = W.custom_decode_workload(940, 600, 8, 2, 128, 16, 3, seq, 7, "bf16")
    cache = W.random_tq_cache(w, *fmt, oracle.tq_slot_bytes(128, *fmt))
    cen = _random_table(940, 16, True)
    q = W.query(w) / 4
    ref, ref_lse = _oracle_tq(w, q, cache, cen, *fmt)
    got, lse = gpu_tq_decode(w, q, cache, cen, *fmt)
    assert_close(got, ref, lse, ref_lse, "600 sequences")


# ---------------------------------------------------------------------------
# Read-side variants on the generic kernel: FP8 values, D = 256

N2_FMTS = [(oracle.KEY_FP8, oracle.VAL_FP8), (oracle.KEY_MSE3, oracle.VAL_FP8),
           (oracle.KEY_MSE4, oracle.VAL_FP8), (oracle.KEY_MSE4, oracle.VAL_U3)]


@pytest.mark.parametrize("fmt", N2_FMTS, ids=[str(f) for f in N2_FMTS])
@pytest.mark.parametrize("d", [64, 128, 256])
def test_tq_fp8_values_and_head_dims(fmt, d):
    seq = [0, 1, 77, 300]
    w = W.custom_decode_workload(370 + d + 3 * fmt[0] + fmt[1], len(seq), 8, 2, d, 16, 3, seq, 4, "bf16")
    rs = None if fmt[0] == oracle.KEY_FP8 else W.rht_signs(d, round_idx=6)
    cache, cen = tq_case(w, *fmt, rot_signs=rs)
    q = W.query(w, bf16_valued=True)
    ref, ref_lse = oracle.tq_decode(q, cache, w.block_table, w.seq_lens, cen, rs, *fmt, 0,
                                    w.num_splits, w.sm_scale)
    got, lse = gpu_tq_decode(w, q, cache, cen, *fmt, rot_signs=rs)
    assert_close(got, ref, lse, ref_lse, "fmt %s d=%d" % (fmt, d))


@pytest.mark.parametrize("fmt", [(oracle.KEY_FP8, oracle.VAL_U4), (oracle.KEY_MSE3, oracle.VAL_U3)],
                         ids=["fp8_u4", "mse3_u3"])
@pytest.mark.parametrize("norm_correction", [False, True])
def test_tq_head_dim_256_shapes(fmt, norm_correction):
    """D = 256 on the formats the matrix-core kernels take at D = 128 (the
    generic kernel serves D = 256), g from 1 to 8, norm correction."""
    if fmt[0] == oracle.KEY_FP8 and norm_correction:
        pytest.skip("norm correction applies to centroid keys only")
    for (B, hq, hk, seq, S) in [(2, 8, 8, [300, 1], 4), (3, 16, 2, [129, 0, 640], 5)]:
        w = W.custom_decode_workload(380 + hq + S, B, hq, hk, 256, 16, S, seq, 3, "bf16")
        cache, cen = tq_case(w, *fmt)
        q = W.query(w, bf16_valued=True)
        ref, ref_lse = oracle.tq_decode(q, cache, w.block_table, w.seq_lens, cen, None, *fmt,
                                        int(norm_correction), S, w.sm_scale)
        got, lse = gpu_tq_decode(w, q, cache, cen, *fmt, norm_correction=norm_correction)
        assert_close(got, ref, lse, ref_lse, "fmt %s B=%d" % (fmt, B))


ALL_C_FMTS = [(oracle.KEY_MSE3, oracle.VAL_U3)] + C_FMTS


@pytest.mark.parametrize("flags", [0, tq.FLAG_GENERIC, tq.FLAG_WIDE],
                         ids=["mfma", "generic", "mfma_wide"])
@pytest.mark.parametrize("fmt", ALL_C_FMTS, ids=["mse3_u3", "mse4_u4", "mse3_u4", "mse4_u3"])
def test_tq_centroid_head_dim_256(fmt, flags):
    """D = 256 on the centroid-key matrix-core kernel (four query heads per
    wave, one wave per SIMD): oracle-encoded caches, g = 1, 4, 8, ragged,
    empty and one-token sequences."""
    for (B, hq, hk, seq, S) in [(2, 8, 8, [300, 1], 4), (3, 16, 2, [129, 0, 640], 5),
                                (2, 16, 4, [1000, 65], 7)]:
        w = W.custom_decode_workload(960 + hq + S + 3 * fmt[0] + fmt[1], B, hq, hk, 256, 16, S, seq, 3,
                                     "bf16")
        cache, cen = tq_case(w, *fmt)
        q = W.query(w, bf16_valued=True)
        ref, ref_lse = _oracle_tq(w, q, cache, cen, *fmt)
        got, lse = gpu_tq_decode(w, q, cache, cen, *fmt, flags=flags)
        assert_close(got, ref, lse, ref_lse, "fmt %s B=%d hq=%d" % (fmt, B, hq))


def test_tq_centroid_one_wave_layout_at_the_batch_limit():
    """3-bit centroid keys and values at g = 8 with four kv heads (one wave
    per kv head, four per workgroup: the layout whose value sums keep an LDS
    base) at the largest batch the decode accepts, 4096 sequences of 0 .. 40
    tokens, every row against the oracle."""
    rng = np.random.default_rng(4096)
    seq = [int(x) for x in rng.integers(0, 41, 4096)]
    fmt = (oracle.KEY_MSE3, oracle.VAL_U3)
    w = W.custom_decode_workload(4096, 4096, 32, 4, 128, 16, 2, seq, 3, "bf16")
    cache, cen = tq_case(w, *fmt)
    q = W.query(w, bf16_valued=True)
    ref, ref_lse = _oracle_tq(w, q, cache, cen, *fmt)
    got, lse = gpu_tq_decode(w, q, cache, cen, *fmt)
    assert_close(got, ref, lse, ref_lse, "B=4096 centroid keys")


@pytest.mark.parametrize("fmt", ALL_C_FMTS, ids=["mse3_u3", "mse4_u4", "mse3_u4", "mse4_u3"])
def test_tq_centroid_head_dim_256_query_groups_of_five_to_eight(fmt):
    """D = 256 with g = 5 .. 8, where the two waves of a kv head split the
    head dims: one and three kv heads (workgroups of one and two kv heads),
    padded query-head groups, ragged and empty sequences, against the oracle
    and against the 64-bit variant (which splits by query heads)."""
    for (B, hq, hk, seq, S) in [(2, 5, 1, [300, 0], 3), (2, 6, 1, [1, 257], 4), (3, 7, 1, [64, 65, 200], 2),
                                (2, 8, 1, [500, 129], 5), (2, 24, 3, [190, 33], 6)]:
        w = W.custom_decode_workload(990 + hq + 7 * hk + 3 * fmt[0] + fmt[1], B, hq, hk, 256, 16, S, seq, 3,
                                     "bf16")
        cache, cen = tq_case(w, *fmt)
        q = W.query(w, bf16_valued=True)
        ref, ref_lse = _oracle_tq(w, q, cache, cen, *fmt)
        got, lse = gpu_tq_decode(w, q, cache, cen, *fmt)
        assert_close(got, ref, lse, ref_lse, "fmt %s B=%d hq=%d hk=%d" % (fmt, B, hq, hk))
        got_w, lse_w = gpu_tq_decode(w, q, cache, cen, *fmt, flags=tq.FLAG_WIDE)
        assert_close(got_w, ref, lse_w, ref_lse, "wide fmt %s B=%d hq=%d hk=%d" % (fmt, B, hq, hk))


@pytest.mark.parametrize("antisymmetric", [False, True], ids=["general", "antisymmetric"])
@pytest.mark.parametrize("fmt", ALL_C_FMTS, ids=["mse3_u3", "mse4_u4", "mse3_u4", "mse4_u3"])
def test_tq_centroid_head_dim_256_random_slots(fmt, antisymmetric):
    """D = 256, random slots and random tables (both score forms), split
    counts 1 .. 256."""
    w = W.custom_decode_workload(970 + 3 * fmt[0] + fmt[1], 3, 16, 2, 256, 16, 4, [300, 77, 1], 4, "bf16")
    cache = W.random_tq_cache(w, *fmt, oracle.tq_slot_bytes(256, *fmt))
    n = 16 if fmt[0] == oracle.KEY_MSE4 else 8
    cen = _random_table(971 + fmt[1], n, antisymmetric)
    q = W.query(w) / 4
    ref, ref_lse = _oracle_tq(w, q, cache, cen, *fmt, splits=0)
    for S in (1, 4, 37, 256):
        for flags in (0, tq.FLAG_WIDE):
            got, lse = gpu_tq_decode(w, q, cache, cen, *fmt, num_splits=S, flags=flags)
            assert_close(got, ref, lse, ref_lse, "random slots %s S=%d flags=%d" % (fmt, S, flags))


NC_FMTS = ALL_C_FMTS + [(oracle.KEY_MSE3, oracle.VAL_FP8), (oracle.KEY_MSE4, oracle.VAL_FP8)]


@pytest.mark.parametrize("d", [128, 256])
@pytest.mark.parametrize("antisymmetric", [False, True], ids=["general", "antisymmetric"])
@pytest.mark.parametrize("fmt", NC_FMTS, ids=["mse3_u3", "mse4_u4", "mse3_u4", "mse4_u3", "mse3_fp8", "mse4_fp8"])
def test_tq_centroid_norm_correction(fmt, antisymmetric, d):
    """The norm-corrected read on the matrix-core kernel (the sum of c[idx]^2
    over a token's dims from parity-plane counts): random slots, random
    tables in both forms, g = 4 and 8, against the oracle and with the
    64-bit variant and the generic kernel."""
    for (hq, hk) in [(16, 4), (16, 2)]:
        w = W.custom_decode_workload(980 + hq + hk + d + 3 * fmt[0] + fmt[1], 3, hq, hk, d, 16, 4,
                                     [300, 77, 1], 4, "bf16")
        cache = W.random_tq_cache(w, *fmt, oracle.tq_slot_bytes(d, *fmt))
        n = 16 if fmt[0] == oracle.KEY_MSE4 else 8
        cen = _random_table(981 + fmt[1] + hq, n, antisymmetric)
        q = W.query(w)
        ref, ref_lse = oracle.tq_decode(q, cache, w.block_table, w.seq_lens, cen, None, *fmt, 1,
                                        w.num_splits, w.sm_scale)
        for flags in (0, tq.FLAG_WIDE, tq.FLAG_GENERIC):
            got, lse = gpu_tq_decode(w, q, cache, cen, *fmt, norm_correction=True, flags=flags)
            assert_close(got, ref, lse, ref_lse, "%s hq=%d hk=%d flags=%d" % (fmt, hq, hk, flags))


@pytest.mark.parametrize("antisymmetric", [False, True], ids=["general", "antisymmetric"])
@pytest.mark.parametrize("key_fmt", [oracle.KEY_MSE3, oracle.KEY_MSE4], ids=["mse3", "mse4"])
def test_tq_centroid_keys_fp8_values(key_fmt, antisymmetric):
    """Centroid keys with FP8 values on the centroid-key matrix-core kernel
    (D = 128): random slots (every E4M3 code but NaN) and random tables, g =
    2, 4, 8, split counts 1 .. 256, the 64-bit variant and the generic kernel
    alongside."""
    fmt = (key_fmt, oracle.VAL_FP8)
    for (hq, hk) in [(4, 2), (16, 4), (16, 2)]:
        w = W.custom_decode_workload(990 + hq + hk + key_fmt, 3, hq, hk, 128, 16, 4, [300, 77, 1], 4, "bf16")
        cache = W.random_tq_cache(w, *fmt, oracle.tq_slot_bytes(128, *fmt))
        n = 16 if key_fmt == oracle.KEY_MSE4 else 8
        cen = _random_table(991 + hq + key_fmt, n, antisymmetric)
        q = W.query(w) / 4
        ref, ref_lse = _oracle_tq(w, q, cache, cen, *fmt, splits=0)
        for S in (1, 4, 256):
            for flags in (0, tq.FLAG_WIDE, tq.FLAG_GENERIC):
                got, lse = gpu_tq_decode(w, q, cache, cen, *fmt, num_splits=S, flags=flags)
                assert_close(got, ref, lse, ref_lse, "%s hq=%d S=%d flags=%d" % (fmt, hq, S, flags))


@pytest.mark.parametrize("key_fmt", [oracle.KEY_MSE3, oracle.KEY_MSE4], ids=["mse3", "mse4"])
@pytest.mark.parametrize("shape", SHAPES[:5], ids=[str(i) for i in range(5)])
def test_tq_centroid_keys_fp8_values_shapes(shape, key_fmt):
    """Oracle-encoded caches (Lloyd-Max tables) on the other formats' shapes."""
    B, hq, hk, d, bs, seq, S = shape
    fmt = (key_fmt, oracle.VAL_FP8)
    w = W.custom_decode_workload(995 + len(seq) * 7 + hq + key_fmt, B, hq, hk, d, bs, S, seq, 5, "bf16")
    cache, cen = tq_case(w, *fmt)
    q = W.query(w, bf16_valued=True)
    ref, ref_lse = _oracle_tq(w, q, cache, cen, *fmt)
    got, lse = gpu_tq_decode(w, q, cache, cen, *fmt)
    assert_close(got, ref, lse, ref_lse, "%s %s" % (shape, fmt))


@pytest.mark.parametrize("val_fmt", [oracle.VAL_U4, oracle.VAL_FP8], ids=["u4", "fp8"])
def test_tq_fp8_keys_head_dim_256(val_fmt):
    """FP8 keys at D = 256 on the FP8-key matrix-core kernel (four query
    heads per wave): random slots, g = 1, 4, 8, split counts 1 .. 256, the
    64-bit and generic paths alongside, and oracle-encoded caches."""
    fmt = (oracle.KEY_FP8, val_fmt)
    for (B, hq, hk, seq, S) in [(2, 8, 8, [300, 1], 4), (3, 16, 4, [129, 0, 640], 5),
                                (2, 16, 2, [1000, 65], 7)]:
        w = W.custom_decode_workload(1000 + hq + hk + S + val_fmt, B, hq, hk, 256, 16, S, seq, 3, "bf16")
        cache = W.random_tq_cache(w, *fmt, oracle.tq_slot_bytes(256, *fmt))
        q = W.query(w) / 16  # random codes reach 448: keep scores O(10)
        ref, ref_lse = _oracle_tq(w, q, cache, None, *fmt, splits=0)
        for Sx in (1, S, 256):
            for flags in (0, tq.FLAG_WIDE, tq.FLAG_GENERIC):
                got, lse = gpu_tq_decode(w, q, cache, None, *fmt, num_splits=Sx, flags=flags)
                assert_close(got, ref, lse, ref_lse, "%s hq=%d S=%d flags=%d" % (fmt, hq, Sx, flags))
        cache, cen = tq_case(w, *fmt)
        q = W.query(w, bf16_valued=True)
        ref, ref_lse = _oracle_tq(w, q, cache, cen, *fmt)
        got, lse = gpu_tq_decode(w, q, cache, cen, *fmt)
        assert_close(got, ref, lse, ref_lse, "encoded %s hq=%d" % (fmt, hq))


# ---------------------------------------------------------------------------
# FP8 keys + FP8 values (matrix-core path for D = 128, g <= 8)

F8_FMT = (oracle.KEY_FP8, oracle.VAL_FP8)


@pytest.mark.parametrize("flags", [0, tq.FLAG_GENERIC, tq.FLAG_WIDE],
                         ids=["mfma", "generic", "mfma_wide"])
@pytest.mark.parametrize("shape", SHAPES, ids=[str(i) for i in range(len(SHAPES))])
def test_tq_fp8_fp8_shapes(shape, flags):
    """FP8 keys and FP8 values on the matrix-core kernel (values as exact
    bf16, weights in three bf16 parts) and on the generic one."""
    B, hq, hk, d, bs, seq, S = shape
    w = W.custom_decode_workload(420 + len(seq) * 7 + hq + d, B, hq, hk, d, bs, S, seq, 5, "bf16")
    cache, cen = tq_case(w, *F8_FMT)
    q = W.query(w, bf16_valued=True)
    ref, ref_lse = _oracle_tq(w, q, cache, cen, *F8_FMT)
    got, lse = gpu_tq_decode(w, q, cache, cen, *F8_FMT, flags=flags)
    assert_close(got, ref, lse, ref_lse, str(shape))


@pytest.mark.parametrize("hq,hk", [(2, 2), (4, 2), (8, 2), (10, 2), (12, 2), (14, 2), (16, 2), (32, 4)],
                         ids=["g1", "g2", "g4", "g5", "g6", "g7", "g8", "g8x4"])
def test_tq_fp8_fp8_query_groups(hq, hk):
    """g = 1 .. 8 (one wave per kv head from g = 5), empty and one-token
    sequences, sequences over many tiles and splits."""
    seq = [0, 1, 300, 777, 65, 2000]
    w = W.custom_decode_workload(430 + hq, len(seq), hq, hk, 128, 16, 3, seq, 6, "bf16")
    cache, cen = tq_case(w, *F8_FMT)
    q = W.query(w, bf16_valued=True)
    ref, ref_lse = _oracle_tq(w, q, cache, cen, *F8_FMT)
    for flags in (0, tq.FLAG_WIDE):
        got, lse = gpu_tq_decode(w, q, cache, cen, *F8_FMT, flags=flags)
        assert_close(got, ref, lse, ref_lse, "hq=%d hk=%d" % (hq, hk))


def test_tq_fp8_fp8_split_invariance_and_degenerate_lengths():
    w = W.custom_decode_workload(440, 3, 8, 2, 128, 16, 4, [37, 1, 100], 2, "bf16")
    cache, cen = tq_case(w, *F8_FMT)
    q = W.query(w, bf16_valued=True)
    seq = np.array([37, 0, 100], np.int32)
    ref, ref_lse = _oracle_tq(w, q, cache, cen, *F8_FMT, splits=0, seq_lens=seq)
    for S in (1, 2, 8, 37, 64, 100, 105, 256):
        got, lse = gpu_tq_decode(w, q, cache, cen, *F8_FMT, num_splits=S, seq_lens=seq)
        assert_close(got, ref, lse, ref_lse, "S=%d" % S)
        assert np.all(got[8:16] == 0) and np.all(np.isneginf(lse[8:16]))


@pytest.mark.parametrize("hq,hk", [(8, 2), (16, 2)], ids=["g4", "g8"])
def test_tq_fp8_fp8_random_slot_bytes_wide_scores(hq, hk):
    """Random slots (no writer): key bytes over every finite E4M3 code, so
    scores spread over tens of units and the running maximum moves often
    along a sequence; value codes kept below 2 in magnitude (exponent field
    at most 7) so the outputs stay O(1). Matrix-core and generic paths."""
    seq = [0, 1, 300, 2000, 777]
    w = W.custom_decode_workload(450 + hq, len(seq), hq, hk, 128, 16, 3, seq, 6, "bf16")
    cache = W.random_tq_cache(w, *F8_FMT, oracle.tq_slot_bytes(128, *F8_FMT))
    cache[..., 128:256] &= 0xBF
    q = W.query(w) / 8
    ref, ref_lse = _oracle_tq(w, q, cache, None, *F8_FMT)
    for flags in (0, tq.FLAG_GENERIC, tq.FLAG_WIDE):
        got, lse = gpu_tq_decode(w, q, cache, None, *F8_FMT, flags=flags)
        assert_close(got, ref, lse, ref_lse, "wide scores flags=%d" % flags)
