"""tq_decode_attention_static (the entry point for callers that cannot
allocate: its workspace is the library's static device array) against
tq_decode_attention with a caller workspace, through the C ABI: two calls
in a row on the INT4 format, the second with a smaller batch, fewer splits
and shorter sequences, then one TurboQuant-format call. The static array
keeps the previous call's partials, so the later calls also show that
nothing stale is read. Both entry points run the same kernels on the same
partition, so the outputs must agree bit for bit (and hence within the
attention tolerance)."""
import numpy as np
import pytest
import torch

import oracle
import quantized_paged_kv_tq_amd as tq
from quantized_paged_kv_tq_amd import workloads as W

from gpu_cases import assert_close, int4_caches, tq_case, to_dev

pytestmark = pytest.mark.gpu


def _both(w, q, **caches):
    args = (to_dev(q), to_dev(w.block_table), to_dev(w.seq_lens))
    out_ws, lse_ws = tq.tq_decode_attention(*args, num_kv_splits=w.num_splits, **caches)
    torch.cuda.synchronize()
    out_st, lse_st = tq.tq_decode_attention_static(*args, num_kv_splits=w.num_splits, **caches)
    torch.cuda.synchronize()
    return (out_ws.cpu().numpy(), lse_ws.cpu().numpy(), out_st.cpu().numpy(), lse_st.cpu().numpy())


def _int4(w):
    c = int4_caches(w)
    q = W.query(w)
    res = _both(w, q, key_cache=to_dev(c["kc"]), value_cache=to_dev(c["vc"]),
                k_scale_cache=to_dev(c["ks"]), v_scale_cache=to_dev(c["vs"]),
                rht_signs=to_dev(c["signs"]))
    return res, w


def _check(res, w, what):
    out_ws, lse_ws, out_st, lse_st = res
    d = w.d
    assert_close(out_st.reshape(-1, d).astype(np.float64), out_ws.reshape(-1, d).astype(np.float64),
                 lse_st.ravel(), lse_ws.ravel(), what)
    np.testing.assert_array_equal(out_st, out_ws, err_msg=what)
    np.testing.assert_array_equal(lse_st, lse_ws, err_msg=what)


def test_static_workspace_matches_caller_workspace():
    print("[no-alloc] INT4 B=8 Hq=32 Hk=8 D=128 S=8", flush=True)
    big = W.custom_decode_workload(901, 8, 32, 8, 128, 16, 8,
                                   [3000, 1, 777, 2048, 64, 1500, 999, 2500], 5, "bf16")
    res, w = _int4(big)
    _check(res, w, "first call")
    print("[no-alloc] INT4 B=3 Hq=8 Hk=2 D=128 S=3 (smaller)", flush=True)
    small = W.custom_decode_workload(902, 3, 8, 2, 128, 16, 3, [300, 17, 129], 5, "bf16")
    res, w = _int4(small)
    _check(res, w, "second call (smaller)")
    print("[no-alloc] FP8 keys + 4-bit values B=2 Hq=16 Hk=4 D=128 S=4", flush=True)
    tw = W.custom_decode_workload(903, 2, 16, 4, 128, 16, 4, [700, 90], 5, "bf16")
    cache, cen = tq_case(tw, oracle.KEY_FP8, oracle.VAL_U4)
    res = _both(tw, W.query(tw), kv_cache=to_dev(cache), key_fmt=tq.KEY_FP8, val_fmt=tq.VAL_U4)
    _check(res, tw, "TurboQuant call")


def test_static_workspace_limit_is_reported():
    # a batch whose partials exceed the static array: rejected, nothing launched
    w = W.custom_decode_workload(904, 1, 8, 2, 128, 16, 2, [40], 5, "bf16")
    c = int4_caches(w)
    q = np.zeros((4096, 64, 128), np.float32)
    bt = np.zeros((4096, 4), np.int32)
    sl = np.ones(4096, np.int32)
    with pytest.raises(tq.TQError, match="static maximum"):
        tq.tq_decode_attention_static(
            to_dev(q), to_dev(bt), to_dev(sl), num_kv_splits=64,
            key_cache=to_dev(np.zeros((w.num_blocks, 16, 8, 64), np.uint8)),
            value_cache=to_dev(np.zeros((w.num_blocks, 16, 8, 64), np.uint8)),
            k_scale_cache=to_dev(np.zeros((w.num_blocks, 16, 8), np.float32)),
            v_scale_cache=to_dev(np.zeros((w.num_blocks, 16, 8), np.float32)),
            rht_signs=to_dev(c["signs"]))
