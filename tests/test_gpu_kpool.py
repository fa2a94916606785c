"""GPU parity of the pooled-softmax key compressor against the CPU oracle
(kpool_compress.py, kpool_compress_and_write_cache): every byte of the
indexer cache and of the compressed output, bit-exact, through the C ABI."""
import numpy as np
import pytest
import torch

import oracle
from quantized_paged_kv_tq_amd import workloads as W

from gpu_cases import DEV, src_to_dev, to_dev

pytestmark = pytest.mark.gpu


def _run_both(w, round_scale=True, compressed=False, write_cache=True, mask=None, loc=None,
              fill=0xA5):
    import quantized_paged_kv_tq_amd as tq
    sdt = w["score_dtype"]
    n, P = w["slot_k"].shape[:2]
    loc = w["loc"] if loc is None else loc
    print("kpool case: n=%d P=%d score=%s round_scale=%s compressed=%s cache=%s mask=%s"
          % (n, P, sdt, round_scale, compressed, write_cache, mask is not None), flush=True)
    cache_o = np.full((w["num_blocks"], w["block_size"], 132), fill, np.uint8)
    cache = to_dev(cache_o)
    ref = oracle.kpool_compress_and_write(
        w["slot_k"], w["slot_score"], w["ape"], loc, cache_o if write_cache else None,
        write_mask=mask, round_scale=round_scale, return_compressed=compressed, score_dtype=sdt)
    got = tq.tq_kpool_compress_and_write_cache(
        cache, src_to_dev(w["slot_k"], "bf16"), src_to_dev(w["slot_score"], sdt), to_dev(w["ape"]),
        to_dev(loc), write_mask=None if mask is None else to_dev(mask),
        round_scale=round_scale, return_compressed=compressed, write_cache=write_cache)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(cache.cpu().numpy(), cache_o)
    if compressed:
        np.testing.assert_array_equal(got[0].view(torch.uint8).cpu().numpy(), ref[0])
        np.testing.assert_array_equal(got[1].cpu().numpy().view(np.uint32), ref[1].view(np.uint32))


@pytest.mark.parametrize("P,sdt", [(1, "bf16"), (2, "f32"), (3, "bf16"), (4, "bf16"), (4, "f32"),
                                   (4, "f16"), (5, "f16"), (8, "bf16"), (16, "f32")])
@pytest.mark.parametrize("round_scale", [True, False])
def test_pool_sizes_and_score_dtypes(P, sdt, round_scale):
    w = W.kpool_workload(n_pools=1013, pool_size=P, score_dtype=sdt, block_size=64,
                         skip_frac=0.05, wid=60 + P)
    _run_both(w, round_scale=round_scale)


@pytest.mark.parametrize("P", [4, 6])
def test_write_mask_and_compressed_output(P):
    w = W.kpool_workload(n_pools=777, pool_size=P, score_dtype="bf16", block_size=16,
                         mask_frac=0.3, skip_frac=0.02, wid=70 + P)
    _run_both(w, mask=w["write_mask"])
    _run_both(w, compressed=True)
    _run_both(w, compressed=True, write_cache=False)
    _run_both(w, compressed=True, round_scale=False)


def test_out_of_range_locations_and_odd_page():
    w = W.kpool_workload(n_pools=300, pool_size=4, score_dtype="f32", block_size=7, wid=80)
    loc = w["loc"].copy()
    nent = w["num_blocks"] * 7
    loc[::17] = nent          # one past the cache
    loc[5::23] = nent + 1000
    loc[9::31] = -7
    _run_both(w, loc=loc)


@pytest.mark.parametrize("offset", [150.0, -60.0])
def test_score_offsets(offset):
    w = W.kpool_workload(n_pools=256, pool_size=4, score_dtype="f32", score_offset=offset, wid=81)
    _run_both(w)


def test_tiny_and_subnormal_weights():
    # exponent arguments in [-104, -85]: probabilities in the fp32 subnormal
    # range, and some that round to zero
    w = W.kpool_workload(n_pools=512, pool_size=4, score_dtype="f32", wid=82)
    g = np.random.default_rng(3)
    sc = w["slot_score"].copy()
    sc[:, 0, :] = 0.0
    sc[:, 1:, :] = -g.uniform(85.0, 104.5, size=sc[:, 1:, :].shape).astype(np.float32)
    w["slot_score"] = sc
    w["ape"] = np.zeros_like(w["ape"])
    _run_both(w, compressed=True)


def test_degenerate_pools():
    w = W.kpool_workload(n_pools=96, pool_size=4, score_dtype="bf16", wid=83)
    k = w["slot_k"].copy()
    k[0:8] = 0                    # zero pools: the 1e-4 absmax floor
    k[8:16] = W.to_bits(np.full((8, 4, 128), 3.0, np.float32), "bf16")
    w["slot_k"] = k
    sc = w["slot_score"].copy()
    sc[16:32] = W.to_bits(np.zeros((16, 4, 128), np.float32), "bf16")  # equal weights
    w["slot_score"] = sc
    _run_both(w, compressed=True)
    _run_both(w, round_scale=False)


@pytest.mark.parametrize("n", [0, 1, 31, 33])
def test_small_counts(n):
    w = W.kpool_workload(n_pools=max(n, 1), pool_size=4, score_dtype="bf16", wid=84)
    if n == 0:
        for key in ("slot_k", "slot_score"):
            w[key] = w[key][:0]
        w["loc"] = w["loc"][:0]
    _run_both(w, compressed=n > 0)


def test_full_size_prefill_bit_exact():
    # 262144 pools of 4 tokens (1M tokens), bf16 scores: the benchmark shape
    w = W.kpool_workload(n_pools=262144, pool_size=4, score_dtype="bf16", block_size=64, wid=11)
    _run_both(w, fill=0)
