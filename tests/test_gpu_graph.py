"""Graph capture of the decode step: tq_reshape_and_cache_int4 followed by
tq_decode_attention (and its static-workspace variant), captured into one
HIP graph with every buffer allocated beforehand, replayed several times
with new queries written eagerly between the replays. The pages fix the
split count and pre-allocate the outputs so that the call can be captured
(triton_turboquant_decode.py, triton_turboquant_decode_attention). Every
replay is checked against the eager result and the fp64 oracle; the
captured region holds kernel nodes only (no memset nodes)."""
import numpy as np
import pytest
import torch

import oracle
import quantized_paged_kv_tq_amd as tq
from quantized_paged_kv_tq_amd import workloads as W

from gpu_cases import DEV, assert_close, to_dev

pytestmark = pytest.mark.gpu


def test_capture_write_and_decode_replays():
    w = W.custom_decode_workload(950, 4, 32, 8, 128, 16, 8, [1500, 17, 900, 2048], 6, "bf16")
    kb, vb = W.kv_source(w)
    signs = W.rht_signs(w.d)
    shape = (w.num_blocks, w.block_size, w.hk, w.d // 2)
    # the cache holds every token but each sequence's last; the captured
    # step writes the last tokens, then decodes
    last = np.cumsum(w.seq_lens.astype(np.int64)) - 1
    first_slots = w.slot_mapping.copy()
    first_slots[last] = -1
    kc_o = np.zeros(shape, np.uint8); vc_o = np.zeros(shape, np.uint8)
    ks_o = np.zeros(shape[:3], np.float32); vs_o = np.zeros(shape[:3], np.float32)
    oracle.reshape_and_cache_int4(kb, vb, oracle.DT_BF16, w.slot_mapping, signs, kc_o, vc_o, ks_o, vs_o)
    kc = torch.zeros(shape, dtype=torch.uint8, device=DEV); vc = torch.zeros_like(kc)
    ks = torch.zeros(shape[:3], dtype=torch.float32, device=DEV); vs = torch.zeros_like(ks)
    key = to_dev(kb.view(np.int16), torch.bfloat16)
    val = to_dev(vb.view(np.int16), torch.bfloat16)
    sg = to_dev(signs)
    tq.tq_reshape_and_cache_int4(key, val, kc, vc, to_dev(first_slots), k_scale_cache=ks,
                                 v_scale_cache=vs, rht_signs=sg)
    new_k, new_v = key[last].contiguous(), val[last].contiguous()
    new_slots = to_dev(w.slot_mapping[last])
    q = torch.zeros(w.B, w.hq, w.d, dtype=torch.float32, device=DEV)
    bt, sl = to_dev(w.block_table), to_dev(w.seq_lens)
    ws = torch.empty(tq.tq_decode_workspace_bytes(w.B, w.hq, w.hk, w.d, w.num_splits) // 4,
                     dtype=torch.float32, device=DEV)
    out = torch.empty(w.B, w.hq, w.d, dtype=torch.float32, device=DEV)
    lse = torch.empty(w.B, w.hq, dtype=torch.float32, device=DEV)
    out2 = torch.empty_like(out)
    lse2 = torch.empty_like(lse)
    write = tq.prepare_reshape(new_k, new_v, kc, vc, new_slots, k_scale_cache=ks,
                               v_scale_cache=vs, rht_signs=sg)
    caches = dict(key_cache=kc, value_cache=vc, k_scale_cache=ks, v_scale_cache=vs, rht_signs=sg)
    dec = tq.prepare_decode(q, bt, sl, num_kv_splits=w.num_splits, workspace=ws, out=out, lse=lse,
                            **caches)[0]
    dec_static = tq.prepare_decode(q, bt, sl, num_kv_splits=w.num_splits, out=out2, lse=lse2,
                                   static_workspace=True, **caches)[0]
    torch.cuda.synchronize()
    # warm the calls once outside the capture (first-use set-up happens here)
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        write.run()
        dec.run()
        dec_static.run()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        write.run()
        dec.run()
        dec_static.run()
    torch.cuda.synchronize()
    for rep in range(4):
        qh = W.query(w) * np.float32(1 + rep)
        q.copy_(torch.from_numpy(qh))      # eager work between the replays
        torch.cuda.synchronize()
        out.fill_(np.nan); out2.fill_(np.nan)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got, got_lse = out.cpu().numpy().reshape(-1, w.d), lse.cpu().numpy().ravel()
        got2, got2_lse = out2.cpu().numpy().reshape(-1, w.d), lse2.cpu().numpy().ravel()
        assert np.array_equal(kc.cpu().numpy(), kc_o) and np.array_equal(vc.cpu().numpy(), vc_o)
        assert np.array_equal(ks.cpu().numpy().view(np.uint32), ks_o.view(np.uint32))
        # eager call on the same inputs
        e_out, e_lse = tq.tq_decode_attention(q, bt, sl, num_kv_splits=w.num_splits, **caches)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(got, e_out.cpu().numpy().reshape(-1, w.d))
        np.testing.assert_array_equal(got2, got)
        np.testing.assert_array_equal(got2_lse, got_lse)
        ref, ref_lse = oracle.int4_decode(qh, kc_o, vc_o, ks_o, vs_o, w.block_table, w.seq_lens,
                                          signs, w.num_splits, w.sm_scale)
        assert_close(got.astype(np.float64), ref, got_lse, ref_lse, "replay %d" % rep)
