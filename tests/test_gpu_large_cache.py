"""Caches of more than 2 GiB: pages beyond the 2^31-byte mark are addressed
64-bit (the pages' kernels address slots in int64: triton_turboquant_decode.py,
_tq_decode_stage1's page gather, and int4_per_token_head.py's cache
strides). A few sequences' pages are placed across a pool of more than
2.5 GiB per cache tensor, below and far above 2 GiB; every output row is
compared with the fp64 oracle run on the same pages in a compact pool (the
same data under a renumbered block table)."""
import numpy as np
import pytest
import torch

import oracle
import quantized_paged_kv_tq_amd as tq
from quantized_paged_kv_tq_amd import workloads as W

from gpu_cases import DEV, assert_close, int4_caches, tq_case, to_dev

pytestmark = pytest.mark.gpu

GiB = 1 << 30


def _spread_pages(w, nb_big, seed):
    """Big-pool page of each compact page: half below 2 GiB / 4, half in
    the top part of the pool, in a seeded order."""
    rng = np.random.default_rng(seed)
    n = w.num_blocks
    low = rng.choice(nb_big // 8, n // 2, replace=False)
    high = nb_big - 1 - rng.choice(nb_big // 8, n - n // 2, replace=False)
    big = np.concatenate([low, high])
    rng.shuffle(big)
    return big.astype(np.int64)


def _big_table(w, big):
    bt = w.block_table.copy()
    used = bt >= 0
    bt[used] = big[bt[used]]
    return bt


def test_int4_cache_above_2gib_all_rows():
    w = W.custom_decode_workload(970, 3, 32, 8, 128, 16, 8, [700, 1500, 333], 6, "bf16")
    c = int4_caches(w)
    q = W.query(w)
    ref, ref_lse = oracle.int4_decode(q, c["kc"], c["vc"], c["ks"], c["vs"], w.block_table,
                                      w.seq_lens, c["signs"], w.num_splits, w.sm_scale)
    page_bytes = w.block_size * w.hk * (w.d // 2)
    nb_big = (5 * GiB // 2) // page_bytes + 1  # > 2.5 GiB per cache tensor
    big = _spread_pages(w, nb_big, 971)
    assert big.max() * page_bytes > 2 * GiB
    shape = (nb_big, w.block_size, w.hk, w.d // 2)
    kc = torch.zeros(shape, dtype=torch.uint8, device=DEV)
    vc = torch.zeros_like(kc)
    ks = torch.zeros(shape[:3], dtype=torch.float32, device=DEV)
    vs = torch.zeros_like(ks)
    idx = to_dev(big)
    kc[idx] = to_dev(c["kc"])
    vc[idx] = to_dev(c["vc"])
    ks[idx] = to_dev(c["ks"])
    vs[idx] = to_dev(c["vs"])
    print("[large cache] INT4 pool of %d pages, %.2f GiB per cache" % (nb_big, kc.numel() / GiB),
          flush=True)
    out, lse = tq.tq_decode_attention(to_dev(q), to_dev(_big_table(w, big)), to_dev(w.seq_lens),
                                      num_kv_splits=w.num_splits, key_cache=kc, value_cache=vc,
                                      k_scale_cache=ks, v_scale_cache=vs,
                                      rht_signs=to_dev(c["signs"]))
    torch.cuda.synchronize()
    got = out.cpu().numpy().reshape(-1, w.d).astype(np.float64)
    assert_close(got, ref, lse.cpu().numpy().ravel(), ref_lse, "INT4 > 2 GiB")
    del kc, vc, ks, vs
    torch.cuda.empty_cache()


@pytest.mark.parametrize("fmt", [(oracle.KEY_FP8, oracle.VAL_U4), (oracle.KEY_MSE3, oracle.VAL_U3)],
                         ids=["fp8_u4", "mse3_u3"])
def test_tq_cache_above_2gib_all_rows(fmt):
    key_fmt, val_fmt = fmt
    w = W.custom_decode_workload(975, 3, 32, 4, 128, 16, 6, [900, 64, 1700], 6, "bf16")
    cache, cen = tq_case(w, key_fmt, val_fmt)
    q = W.query(w, bf16_valued=True)
    ref, ref_lse = oracle.tq_decode(q, cache, w.block_table, w.seq_lens, cen, None, key_fmt,
                                    val_fmt, 0, w.num_splits, w.sm_scale)
    sb = cache.shape[-1]
    page_bytes = w.block_size * w.hk * sb
    nb_big = (5 * GiB // 2) // page_bytes + 1
    big = _spread_pages(w, nb_big, 976)
    assert big.max() * page_bytes > 2 * GiB
    kv = torch.zeros((nb_big, w.block_size, w.hk, sb), dtype=torch.uint8, device=DEV)
    kv[to_dev(big)] = to_dev(cache)
    print("[large cache] %s pool of %d pages, %.2f GiB" % (fmt, nb_big, kv.numel() / GiB), flush=True)
    out, lse = tq.tq_decode_attention(
        to_dev(q), to_dev(_big_table(w, big)), to_dev(w.seq_lens), num_kv_splits=w.num_splits,
        kv_cache=kv, key_fmt=key_fmt, val_fmt=val_fmt,
        centroids=None if cen is None else to_dev(cen))
    torch.cuda.synchronize()
    got = out.cpu().numpy().reshape(-1, w.d).astype(np.float64)
    assert_close(got, ref, lse.cpu().numpy().ravel(), ref_lse, "%s > 2 GiB" % (fmt,))
    del kv
    torch.cuda.empty_cache()
